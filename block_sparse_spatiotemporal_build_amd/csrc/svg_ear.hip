// Centroid linear compensation with error-aware routing for gfx950.
//
// Source: "SVG-EAR: Parameter-Free Linear Compensation for Sparse Video
// Generation via Error-aware Routing", technical summary section 2 Method.
// Tokens arrive ordered by cluster (query cluster a = rows [q_off[a],
// q_off[a+1]); key cluster b = rows [k_off[b], k_off[b+1]) of K and V).  A block
// is a (query cluster, key cluster) pair with cost n_a * n_b.
//
//   centroids (idea 1)   c^_a, c_b, vbar_b: fp32 segmented means.
//   route probe (idea 2) for every proxy c^_a and key cluster b, the squared
//                        norm of the compensation error of block (a, b),
//                          e_ab = (sum_{j in b} exp(l_aj - m_a) v_j
//                                  - n_b exp(s c^_a.c_b - m_a) vbar_b) / Z_a
//                               = sum_{j in b} (exp(l_aj - m_a) - exp(s c^_a.c_b - m_a)) v_j / Z_a
//                        (n_b vbar_b = sum_j v_j), accumulated in the second
//                        form so that rounding acts on the difference itself;
//                        score = |e_ab|^2 / n_b.  Streamed over key clusters
//                        (logits are never stored): each workgroup keeps an
//                        online max per proxy, stores |.|^2 of each finished
//                        cluster with the max it was taken at, and a finalize
//                        pass rescales with the combined (m_a, Z_a).
//   route select         per head: keep the longest prefix of blocks ordered by
//                        (score desc, a*Ck + b asc) whose cost fits the density
//                        budget floor(N*N*ppm/1e6).  Radix select on the score
//                        bits with integer (exact) cost sums, then the tie group
//                        in index order; output CSR with ascending columns.
//   compensated attention (idea 1) one softmax per query over the exact keys of
//                        the kept clusters of its row and one virtual key per
//                        skipped non-empty cluster (key c_b, value vbar_b,
//                        logit bias ln n_b).  Same MFMA core as the block-sparse
//                        kernel, with a gathered key-row map.

#include "launch.h"

namespace bsa {

struct SvgArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  int64_t sb, sh, sn;
  int B, H, N;
  const int32_t* q_off;  // [BH][Cq+1]
  const int32_t* k_off;  // [BH][Ck+1]
  int Cq, Ck;
};

__device__ __forceinline__ const uint16_t* head_ptr(const uint16_t* base, const SvgArgs& a, int bh) {
  return base + (int64_t)(bh / a.H) * a.sb + (int64_t)(bh % a.H) * a.sh;
}

// ---------------------------------------------------------------------------
// centroids
// ---------------------------------------------------------------------------

// Workgroup (c0 + blockIdx.x, bh): query cluster c < Cq, else key cluster
// c - Cq (whose key and value means it takes together).  Four rows per
// thread are loaded before they are summed, so each thread keeps four loads in
// flight.
template <int D>
__global__ void __launch_bounds__(256) centroid_kernel(SvgArgs a, float* q_cent, float* k_cent, float* v_cent,
                                                       int c0) {
  constexpr int CH = D / 8, RS = 256 / CH, U = 4;
  __shared__ float red[2][RS][D];
  const int bh = blockIdx.y, c = c0 + blockIdx.x, tid = threadIdx.x;
  const bool is_q = c < a.Cq;
  const int idx = is_q ? c : c - a.Cq;
  const int32_t* off = is_q ? a.q_off + (int64_t)bh * (a.Cq + 1) : a.k_off + (int64_t)bh * (a.Ck + 1);
  const int r0 = off[idx], r1 = off[idx + 1];
  const uint16_t* X = head_ptr(is_q ? a.q : a.k, a, bh);
  const uint16_t* V = head_ptr(a.v, a, bh);
  const int cc = tid % CH, rg = tid / CH;
  float s1[8], s2[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) s1[e] = s2[e] = 0.f;
  for (int r = r0 + rg; r < r1; r += U * RS) {
    u32x4 x[U], y[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int rr = r + u * RS;
      x[u] = rr < r1 ? *(const u32x4*)(X + (int64_t)rr * a.sn + cc * 8) : u32x4{0, 0, 0, 0};
      y[u] = (!is_q && rr < r1) ? *(const u32x4*)(V + (int64_t)rr * a.sn + cc * 8) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        s1[2 * w] += bf16_lo(x[u][w]);
        s1[2 * w + 1] += bf16_hi(x[u][w]);
        s2[2 * w] += bf16_lo(y[u][w]);
        s2[2 * w + 1] += bf16_hi(y[u][w]);
      }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    red[0][rg][cc * 8 + e] = s1[e];
    red[1][rg][cc * 8 + e] = s2[e];
  }
  __syncthreads();
  if (tid < D) {
    float t1 = 0.f, t2 = 0.f;
    for (int g = 0; g < RS; ++g) {
      t1 += red[0][g][tid];
      t2 += red[1][g][tid];
    }
    const int n = r1 - r0;
    const float inv = n > 0 ? 1.f / (float)n : 0.f;
    if (is_q) {
      q_cent[((int64_t)bh * a.Cq + idx) * D + tid] = t1 * inv;
    } else {
      k_cent[((int64_t)bh * a.Ck + idx) * D + tid] = t1 * inv;
      v_cent[((int64_t)bh * a.Ck + idx) * D + tid] = t2 * inv;
    }
  }
}

// ---------------------------------------------------------------------------
// route probe (streaming over key clusters)
// ---------------------------------------------------------------------------

constexpr int kPrBN = 32;  // keys per probe sub-tile

struct ProbeArgs {
  SvgArgs s;
  const float* q_cent;
  const float* k_cent;
  const float* v_cent;
  float* e_buf;     // [BH][Cq][Ck]  squared error norm at the recorded max
  float* m_buf;     // [BH][Cq][Ck]  the max (log2 units) it was taken at
  float* m_split;   // [BH][splits][Cq]
  float* z_split;   // [BH][splits][Cq]
  int splits, cps;  // splits per head, clusters per split
  float c2;         // scale * log2(e)
};

template <int D>
__global__ void __launch_bounds__(256) probe_kernel(ProbeArgs p) {
  constexpr int KT = D / 16, DT = D / 32, CH = D / 8;
  constexpr int KST = D + 8, VST = D + 32;
  constexpr int LCH = kPrBN * CH / 256;
  static_assert(LCH >= 1 && LCH * 256 == kPrBN * CH, "probe tile/thread mismatch");
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kPrBN * KST];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][kPrBN * VST];

  const SvgArgs& a = p.s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hi = lane >> 5;
  const int split = blockIdx.x, bh = blockIdx.y;
  const int prox = blockIdx.z * 128 + wave * 32 + l32;  // proxy (query cluster) of this lane
  const bool pvalid = prox < a.Cq;
  const int32_t* koff = a.k_off + (int64_t)bh * (a.Ck + 1);
  const uint16_t* Kh = head_ptr(a.k, a, bh);
  const uint16_t* Vh = head_ptr(a.v, a, bh);

  // proxy fragments (B operand): c^ = hi + lo, both bf16, so that the logits
  // are accurate to about 2^-16 relative (the score is a small difference of
  // nearly equal weights on data where the logits barely vary)
  bf16x8 cf[KT], cl_[KT];
  {
    const float* src = p.q_cent + ((int64_t)bh * a.Cq + (pvalid ? prox : 0)) * D + hi * 8;
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      u32x4 wh, wl;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = pvalid ? src[t * 16 + 2 * e] : 0.f, x1 = pvalid ? src[t * 16 + 2 * e + 1] : 0.f;
        wh[e] = pack_bf16x2(x0, x1);
        wl[e] = pack_bf16x2(x0 - bf16_lo(wh[e]), x1 - bf16_hi(wh[e]));
      }
      cf[t] = __builtin_bit_cast(bf16x8, wh);
      cl_[t] = __builtin_bit_cast(bf16x8, wl);
    }
  }

  const int b0 = split * p.cps, b1 = min(b0 + p.cps, a.Ck);
  // flattened (cluster, sub-tile) sequence of this split
  auto ntiles_of = [&](int b) { return (koff[b + 1] - koff[b] + kPrBN - 1) / kPrBN; };
  int total = 0;
  for (int b = b0; b < b1; ++b) total += ntiles_of(b);

  u32x4 kreg[LCH], vreg[LCH];
  auto fetch = [&](int row0, int rend) {
#pragma unroll
    for (int i = 0; i < LCH; ++i) {
      const int c = tid + 256 * i;
      const int row = c / CH, col = (c % CH) * 8;
      const int64_t off = (int64_t)min(row0 + row, rend - 1) * a.sn + col;
      kreg[i] = *(const u32x4*)(Kh + off);
      vreg[i] = *(const u32x4*)(Vh + off);
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LCH; ++i) {
      const int c = tid + 256 * i;
      const int row = c / CH, col = (c % CH) * 8;
      *(u32x4*)&Ks[buf][row * KST + col] = kreg[i];
      *(u32x4*)&Vs[buf][row * VST + col] = vreg[i];
    }
  };

  f32x16 U[DT];
  float m_run = -1e30f, l_run = 0.f, lc2 = 0.f;
  const int g16 = lane >> 4, j16 = lane & 15;
  const int v_row = 4 * hi + (j16 >> 2);
  const int v_col = 16 * (g16 & 1) + 4 * (j16 & 3);

  // walk state: current cluster and sub-tile within it (for the tile being computed)
  int cb = b0, cst = 0;
  while (cb < b1 && ntiles_of(cb) == 0) ++cb;
  int nb_ = cb < b1 ? ntiles_of(cb) : 0;
  // prefetch cursor
  int fb = cb, fst = 0;
  auto advance = [&](int& bb, int& st) {
    ++st;
    if (st >= ntiles_of(bb)) {
      st = 0;
      ++bb;
      while (bb < b1 && ntiles_of(bb) == 0) ++bb;
    }
  };
  if (total > 0) {
    fetch(koff[fb] + fst * kPrBN, koff[fb + 1]);
    stage(0);
    advance(fb, fst);
  }
  __syncthreads();

  for (int u = 0; u < total; ++u) {
    const int buf = u & 1;
    const int kbeg = koff[cb], kend = koff[cb + 1];
    const int key0 = kbeg + cst * kPrBN;
    if (u + 1 < total) fetch(koff[fb] + fst * kPrBN, koff[fb + 1]);
    if (cst == 0) {
#pragma unroll
      for (int i = 0; i < DT; ++i) U[i] = f32x16{};
      // centroid logit of this cluster for the lane's proxy (log2 units)
      const float* cbp = p.k_cent + ((int64_t)bh * a.Ck + cb) * D;
      float dot = 0.f;
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        const u32x4 wh = __builtin_bit_cast(u32x4, cf[t]), wl = __builtin_bit_cast(u32x4, cl_[t]);
        const float4 c0 = *(const float4*)(cbp + t * 16 + hi * 8);
        const float4 c1 = *(const float4*)(cbp + t * 16 + hi * 8 + 4);
        const float cv[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dot = __builtin_fmaf(bf16_lo(wh[e]) + bf16_lo(wl[e]), cv[2 * e], dot);
          dot = __builtin_fmaf(bf16_hi(wh[e]) + bf16_hi(wl[e]), cv[2 * e + 1], dot);
        }
      }
      lc2 = pair_sum(dot) * p.c2;
    }
    // S^T (32 keys x 32 proxies): s[r] = S^T[key 8*(r/4) + 4*hi + r%4][proxy l32]
    f32x16 s = f32x16{};
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      const bf16x8 kf = *(const bf16x8*)&Ks[buf][l32 * KST + t * 16 + hi * 8];
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, cf[t], s, 0, 0, 0);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, cl_[t], s, 0, 0, 0);
    }
    if (key0 + kPrBN > kend) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (key0 + 8 * (r >> 2) + 4 * hi + (r & 3) >= kend) s[r] = -__builtin_inff();
    }
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    const float m_new = fmaxf(m_run, pair_max(mx) * p.c2);
    if (__any(m_new > m_run)) {
      const float alpha = fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DT; ++i) U[i] *= alpha;
      m_run = m_new;
    }
    // weights relative to the centroid weight: U accumulates
    // sum_j (p_j - p_c) v_j = sum_j p_j v_j - n_b p_c vbar_b directly
    const float pc = fast_exp2(lc2 - m_run);
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float pr = fast_exp2(__builtin_fmaf(s[r], p.c2, -m_run));
      psum += pr;
      s[r] = (s[r] == -__builtin_inff()) ? 0.f : pr - pc;
    }
    l_run += psum;
    // P' = hi + lo (bf16 each): the difference keeps about 16 significant bits
    bf16x8 pf[2], pl[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 wh, wl;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = s[8 * ks + 2 * e], x1 = s[8 * ks + 2 * e + 1];
        wh[e] = pack_bf16x2(x0, x1);
        wl[e] = pack_bf16x2(x0 - bf16_lo(wh[e]), x1 - bf16_hi(wh[e]));
      }
      pf[ks] = __builtin_bit_cast(bf16x8, wh);
      pl[ks] = __builtin_bit_cast(bf16x8, wl);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint16_t* p0 = &Vs[buf][(ks * 16 + v_row) * VST + dt * 32 + v_col];
        const u32x2 lo = lds_tr16(p0), hi2 = lds_tr16(p0 + 8 * VST);
        const u32x4 w = {lo[0], lo[1], hi2[0], hi2[1]};
        const bf16x8 vf = __builtin_bit_cast(bf16x8, w);
        U[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ks], U[dt], 0, 0, 0);
        U[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pl[ks], U[dt], 0, 0, 0);
      }
    }

    if (cst + 1 == nb_) {
      // cluster finished: squared norm of the accumulated error (at max m_run)
      float e2 = 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) e2 = __builtin_fmaf(U[dt][r], U[dt][r], e2);
      e2 = pair_sum(e2);
      if (pvalid && hi == 0) {
        const int64_t o = ((int64_t)bh * a.Cq + prox) * a.Ck + cb;
        p.e_buf[o] = e2;
        p.m_buf[o] = m_run;
      }
      cst = 0;
      ++cb;
      while (cb < b1 && ntiles_of(cb) == 0) ++cb;
      nb_ = cb < b1 ? ntiles_of(cb) : 0;
    } else {
      ++cst;
    }
    if (u + 1 < total) {
      stage(buf ^ 1);
      advance(fb, fst);
    }
    __syncthreads();
  }
  const float z = pair_sum(l_run);
  if (pvalid && hi == 0) {
    p.m_split[((int64_t)bh * p.splits + split) * a.Cq + prox] = m_run;
    p.z_split[((int64_t)bh * p.splits + split) * a.Cq + prox] = z;
  }
}

// ---------------------------------------------------------------------------
// fused route probe, head_dim 128
// ---------------------------------------------------------------------------
// One pass over the keys of a split of key clusters.  Split s of S takes the
// clusters whose first key lies in [K0 + s T / S, K0 + (s + 1) T / S) (T keys
// in the head, K0 its first), so splits hold about equal numbers of keys.
// Each cluster's keys are cut into groups of 16, the k-step of the value
// product; the last group of a cluster is padded with copies of its last key,
// and two consecutive groups form one 32-key tile, so a tile may hold two
// clusters but a k-step never does.  Per tile:
//   S^T = K (c^_hi + c^_lo)^T for the workgroup's 128 proxies (4 waves x 32),
//         with c^ scaled by c2 = scale log2(e) beforehand, so S is the logit t
//         in log2 units;
//   one lazily moved reference m_run and a sum l_run per proxy over every key
//   of the split (the proxy softmax of idea 2); and per group g:
//     U  += V_g^T P_g   (P = exp2(t - m_run) as bf16 hi + lo)
//     sv += column sums of V_g, sk += column sums of K_g, both over this
//           wave's 32 dims (v_dot2 with 0/1 masks that drop the padding)
//     ls += sum of t over the group's keys.
// When cluster b (n_b keys) ends, the waves exchange their sv through LDS and
//   lc = ls / n_b = c2 c^ . c_b   (the mean logit is the logit of the mean key)
//   e  = U - exp2(lc - m_run) sv = sum_j (p_j - p_c) v_j,  e2 = |e|^2
// at reference m_run.  The key and value centroids come out of the same pass
// (c_b = sk / n_b, vbar_b = sv / n_b), so K and V are read once.  Padding
// copies a key of the same tile, so the tile maximum needs no mask.  Four LDS
// stages, three tile copies in flight.
constexpr int kFpTK = 32, kFpGK = 16;


struct FusedProbeArgs {
  SvgArgs s;
  const float* q_cent;  // [BH][Cq][D]
  float* e_buf;         // [BH][Cq][Ck]
  float* m_buf;         // [BH][Cq][Ck]
  float* m_split;       // [BH][splits][Cq]
  float* z_split;       // [BH][splits][Cq]
  float* k_cent;        // [BH][Ck][D] output
  float* v_cent;        // [BH][Ck][D] output
  uint16_t* kc_bf;      // [BH][Ck][D] bf16 copy (nullable)
  uint16_t* vc_bf;      // [BH][Ck][D] bf16 copy (nullable)
  int splits;
  float c2;  // scale * log2(e)
};

// Position of a group walk: local cluster c, key offset off of the group in
// it, and the cluster's key range [k0, k1).  c == nclu: past the last cluster.
struct FpCursor {
  int c, off, k0, k1;
};


__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
probe_fused_d128_kernel(FusedProbeArgs p) {
  constexpr int D = 128, KT = 8, DT = 4, TILE = kFpTK * D;
  __shared__ __attribute__((aligned(1024))) uint16_t K0[TILE], K1[TILE], K2[TILE], K3[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t V0[TILE], V1[TILE], V2[TILE], V3[TILE];
  __shared__ float svx[2][D];  // value column sums of a finished cluster (two slots)

  const SvgArgs& a = p.s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hi = lane >> 5;
  const int split = blockIdx.x, bh = blockIdx.y;
  const int prow = wave * 32 + l32;
  const int prox = blockIdx.z * 128 + prow;  // proxy (query cluster) of this lane
  const bool pvalid = prox < a.Cq;
  const bool write_cent = blockIdx.z == 0;
  // the head's cluster offsets, read through the constant address space
  // (scalar loads, uniform across the workgroup)
  const cint_ptr koffs = (cint_ptr)(a.k_off + (int64_t)bh * (a.Ck + 1));
  const uint16_t* Kh = head_ptr(a.k, a, bh);
  const uint16_t* Vh = head_ptr(a.v, a, bh);
  int b0, nclu;
  {
    // clusters whose first key lies below each bound (offsets ascend): every
    // lane tests 1/64 of the offsets, the ballots count
    const int kfirst = koffs[0], total = koffs[a.Ck] - kfirst;
    const int lo = kfirst + (int)((int64_t)split * total / p.splits);
    const int hi_k = kfirst + (int)((int64_t)(split + 1) * total / p.splits);
    const int32_t* offs = a.k_off + (int64_t)bh * (a.Ck + 1);
    int n_lo = 0, n_hi = 0;
#pragma unroll 8
    for (int base = 0; base < a.Ck; base += 64) {
      const int i = base + lane;
      const int o = i < a.Ck ? offs[i] : INT32_MAX;
      n_lo += __popcll(__ballot(o < lo));
      n_hi += __popcll(__ballot(o < hi_k));
    }
    b0 = split == 0 ? 0 : n_lo;
    const int b1 = split + 1 == p.splits ? a.Ck : n_hi;
    nclu = max(b1 - b0, 0);
  }
  auto koff = [&](int c) -> int { return koffs[b0 + c]; };

  // proxy fragments (MFMA B operands, in registers): c2 c^ = hi + lo, both
  // bf16 (about 2^-16 relative), so the logits keep the small spread of a
  // tight cluster
  bf16x8 cf[KT], cl[KT];
  {
    // invalid proxies read proxy 0 (in bounds) and use zeros
    const float* src = p.q_cent + ((int64_t)bh * a.Cq + (pvalid ? prox : 0)) * D + hi * 8;
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      const f32x4 y0 = *(const f32x4*)&src[t * 16], y1 = *(const f32x4*)&src[t * 16 + 4];
      const float yv[8] = {y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
      u32x4 wh, wl;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = pvalid ? p.c2 * yv[2 * e] : 0.f, x1 = pvalid ? p.c2 * yv[2 * e + 1] : 0.f;
        wh[e] = pack_bf16x2(x0, x1);
        wl[e] = pack_bf16x2(x0 - bf16_lo(wh[e]), x1 - bf16_hi(wh[e]));
      }
      cf[t] = __builtin_bit_cast(bf16x8, wh);
      cl[t] = __builtin_bit_cast(bf16x8, wl);
    }
  }
  __syncthreads();
  retire_loads();
  const int K1k = nclu > 0 ? koff(nclu) : 0;

  // cluster walk: start at cluster c (key k0), skipping empty clusters
  auto enter = [&](FpCursor& g, int c, int k0) {
    g.c = c;
    g.off = 0;
    g.k0 = k0;
    g.k1 = c < nclu ? max(koff(c + 1), k0) : k0;
  };
  auto skip_empty = [&](FpCursor& g) {
    while (g.c < nclu && g.k1 == g.k0) enter(g, g.c + 1, g.k1);
  };
  // keys in the group at the cursor (0 past the last cluster)
  auto count_of = [&](const FpCursor& g) { return g.c < nclu ? min(kFpGK, g.k1 - g.k0 - g.off) : 0; };

  // copy roles: wave w, instruction j covers tile rows 8w + 4j + lane / 16, so
  // waves 0-1 copy the tile's first group and waves 2-3 its second
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t row_bytes = (uint32_t)a.sn * 2u;
  const i32x4 krs = raw_buffer_desc(Kh, 0x7fffffffu), vrs = raw_buffer_desc(Vh, 0x7fffffffu);
  FpCursor dg;  // first group of the next tile to copy
  enter(dg, 0, nclu > 0 ? koff(0) : 0);
  skip_empty(dg);
  auto dma_next = [&](FpCursor& g) {
    if (g.c >= nclu) return;
    g.off += kFpGK;
    if (g.k0 + g.off >= g.k1) {
      enter(g, g.c + 1, g.k1);
      skip_empty(g);
    }
  };
  int issued = 0;  // tiles whose copies have been issued
  auto dma = [&](uint16_t* kst, uint16_t* vst) __attribute__((always_inline)) {
    if (dg.c >= nclu) return;  // the split's groups are all copied
    ++issued;
    FpCursor g = dg;
    dma_next(dg);
    if (wv >= 2) g = dg;
    dma_next(dg);
    const int cnt = count_of(g), start = g.k0 + g.off;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int row = 8 * wv + 4 * j + (lane >> 4);
      // padding repeats the group's last key; an empty group (past the
      // split's last cluster) repeats the split's last key
      const int r = 8 * (wv & 1) + 4 * j + (lane >> 4);
      const int key = cnt > 0 ? start + min(r, cnt - 1) : K1k - 1;
      const uint32_t ro = (uint32_t)key * row_bytes;
      lds_copy16(krs, ro + (uint32_t)(((lane & 15) ^ swz_k(row)) * 16),
                 __builtin_amdgcn_readfirstlane(lds_addr(&kst[(8 * wv + 4 * j) * D])));
      lds_copy16(vrs, ro + (uint32_t)(((lane & 15) ^ swz_v(row)) * 16),
                 __builtin_amdgcn_readfirstlane(lds_addr(&vst[(8 * wv + 4 * j) * D])));
    }
  };

  f32x16 U[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) U[i] = f32x16{};
  float sv = 0.f, sk = 0.f, ls = 0.f;  // sv, sk: dim 32 wave + lane % 32
  float m_run = -1e30f, l_run = 0.f;
  int par = 0;  // svx slot of the next finished cluster
  const int g16 = lane >> 4, j16 = lane & 15;
  // per-lane LDS byte offsets within a stage; every read is base ^ immediate,
  // the identities are checked for every lane on the host:
  //   K row fragment of k-step t:            kb2 ^ 32 t
  //   V transposed reads (ks, dt):           va2 ^ (4096 ks + 64 dt), rows + 8: ^ 2080 more
  //   V column sums of this wave's 32 dims:  the (ks, dt = wave) reads
  //   K transposed reads (same dims):        kt2 ^ 4096 ks, rows + 8: ^ 2176 more
  const int q4 = j16 >> 2, c0 = 2 * (g16 & 1) + ((j16 >> 1) & 1), half4 = (j16 & 1) * 4;
  const uint32_t kb2 = 2 * (l32 * D + 16 * ((l32 & 15) >> 1) + 8 * (hi ^ (l32 & 1)));
  const uint32_t va2 = 2 * ((4 * hi + q4) * D + 32 * q4 + 8 * (c0 ^ hi) + half4);
  const uint32_t vw2 = va2 ^ (64 * wave);
  const uint32_t kt2 = 2 * ((4 * hi + q4) * D + 8 * (4 * (wave ^ hi) + (c0 ^ q4)) + half4);

  // cluster c (local index, n_b keys) is complete: its error and centroids.
  // The correction U -= sv (x) p_c is one MFMA per 32 dims: A holds sv of the
  // lane's row (dim 32 dt + lane % 32) and B holds -p_c of its column (the
  // proxy), each split into three bf16 pieces (24 bits; each of the nine
  // products is exact in fp32), so e = U - p_c sv keeps fp32 accuracy and
  // |e|^2 is a lane-local sum.  Called at the same point by every wave.
  auto split3 = [](float x, float (&o)[3]) {
    o[0] = bf16_lo(f2bf(x));
    o[1] = bf16_lo(f2bf(x - o[0]));
    o[2] = bf16_lo(f2bf(x - o[0] - o[1]));
  };
  auto finish = [&](int c, int nb) __attribute__((always_inline)) {
    const int bg = b0 + c;
    const float svo = pair_sum(sv), skf = pair_sum(sk);
    float e2 = 0.f;
    if (nb > 0) {
      if (lane < 32) svx[par][32 * wave + lane] = svo;
      // wait for this wave's LDS write only, then meet the other waves: a
      // fence would also wait for the tile copies in flight (they write LDS)
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      float svf[DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) svf[dt] = svx[par][32 * dt + l32];
      par ^= 1;
      const float lc = pair_sum(ls) / (float)nb;
      float b3[3];
      split3(-fast_exp2(lc - m_run), b3);
      // k slots 0..8: (h,h) (h,m) (h,l) (m,h) (m,m) (m,l) (l,h) (l,m) (l,l);
      // lanes 0..31 hold slots 0..7, lanes 32..63 slots 8..15
      uint32_t bw[4];
      if (hi == 0) {
        bw[0] = pack_bf16x2(b3[0], b3[1]);
        bw[1] = pack_bf16x2(b3[2], b3[0]);
        bw[2] = pack_bf16x2(b3[1], b3[2]);
        bw[3] = pack_bf16x2(b3[0], b3[1]);
      } else {
        bw[0] = pack_bf16x2(b3[2], 0.f);
        bw[1] = bw[2] = bw[3] = 0u;
      }
      const bf16x8 bf = __builtin_bit_cast(bf16x8, (u32x4){bw[0], bw[1], bw[2], bw[3]});
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        float a3[3];
        split3(svf[dt], a3);
        uint32_t aw[4];
        if (hi == 0) {
          aw[0] = pack_bf16x2(a3[0], a3[0]);
          aw[1] = pack_bf16x2(a3[0], a3[1]);
          aw[2] = pack_bf16x2(a3[1], a3[1]);
          aw[3] = pack_bf16x2(a3[2], a3[2]);
        } else {
          aw[0] = pack_bf16x2(a3[2], 0.f);
          aw[1] = aw[2] = aw[3] = 0u;
        }
        const bf16x8 af = __builtin_bit_cast(bf16x8, (u32x4){aw[0], aw[1], aw[2], aw[3]});
        U[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf, U[dt], 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) e2 = __builtin_fmaf(U[dt][r], U[dt][r], e2);
      }
      e2 = pair_sum(e2);
    }
    if (pvalid && hi == 0) {
      const int64_t o = ((int64_t)bh * a.Cq + prox) * a.Ck + bg;
      p.e_buf[o] = e2;
      p.m_buf[o] = nb > 0 ? m_run : -1e30f;
    }
    if (write_cent && lane < 32) {
      const float inv = nb > 0 ? 1.f / (float)nb : 0.f;
      const int64_t o = ((int64_t)bh * a.Ck + bg) * D + 32 * wave + lane;
      const float kc = skf * inv, vc = svo * inv;
      p.k_cent[o] = kc;
      p.v_cent[o] = vc;
      if (p.kc_bf) p.kc_bf[o] = (uint16_t)f2bf(kc);
      if (p.vc_bf) p.vc_bf[o] = (uint16_t)f2bf(vc);
    }
#pragma unroll
    for (int i = 0; i < DT; ++i) U[i] = f32x16{};
    sv = sk = ls = 0.f;
  };

  // compute walk: the group being accumulated; leading empty clusters finish
  // at once
  FpCursor cg;
  enter(cg, 0, nclu > 0 ? koff(0) : 0);
  while (cg.c < nclu && cg.k1 == cg.k0) {
    finish(cg.c, 0);
    enter(cg, cg.c + 1, cg.k1);
  }

  // group ks (keys 16 ks .. 16 ks + 15 of the tile) at the compute cursor;
  // s holds the tile's logits, the bases are per-step opaque copies
  auto group = [&](const uint16_t* Kb, const uint16_t* Vb, const f32x16& s, int ks, uint32_t va,
                   uint32_t vw, uint32_t kt) __attribute__((always_inline)) {
    const int cnt = count_of(cg);
    if (cnt == 0) return;
    // the group's V^T operands and the column-sum reads go out first; P is
    // built while they are in flight
    u32x4 vfr[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint32_t o = 4096 * ks + 64 * dt;
      const u32x2 v0 = lds_tr16(lds_byte(Vb, va ^ o)), v1 = lds_tr16(lds_byte(Vb, va ^ (o + 2080)));
      vfr[dt] = u32x4{v0[0], v0[1], v1[0], v1[1]};
    }
    u32x4 wvv, wk;
    {
      const u32x2 v0 = lds_tr16(lds_byte(Vb, vw ^ (4096 * ks))), v1 = lds_tr16(lds_byte(Vb, vw ^ (4096 * ks + 2080)));
      const u32x2 k0 = lds_tr16(lds_byte(Kb, kt ^ (4096 * ks))), k1 = lds_tr16(lds_byte(Kb, kt ^ (4096 * ks + 2176)));
      wvv = u32x4{v0[0], v0[1], v1[0], v1[1]};
      wk = u32x4{k0[0], k0[1], k1[0], k1[1]};
    }
    __builtin_amdgcn_sched_barrier(0);
    // this lane's 8 keys of the group: 4 hi + (e & 3) + 8 (e >> 2), e = 0..7,
    // logits s[8 ks + e]
    u32x4 wh, wl, mw;
    float lsum = 0.f, psum = 0.f;
    if (cnt == kFpGK) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float t0 = s[8 * ks + 2 * e], t1 = s[8 * ks + 2 * e + 1];
        const float x0 = fast_exp2(t0 - m_run), x1 = fast_exp2(t1 - m_run);
        lsum += t0 + t1;
        psum += x0 + x1;
        wh[e] = pack_bf16x2(x0, x1);
        wl[e] = pack_bf16x2(x0 - bf16_lo(wh[e]), x1 - bf16_hi(wh[e]));
        mw[e] = 0x3f803f80u;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int k0 = 4 * hi + ((2 * e) & 3) + 8 * ((2 * e) >> 2);
        const bool in0 = k0 < cnt, in1 = k0 + 1 < cnt;
        const float t0 = s[8 * ks + 2 * e], t1 = s[8 * ks + 2 * e + 1];
        const float x0 = in0 ? fast_exp2(t0 - m_run) : 0.f, x1 = in1 ? fast_exp2(t1 - m_run) : 0.f;
        lsum += (in0 ? t0 : 0.f) + (in1 ? t1 : 0.f);
        psum += x0 + x1;
        wh[e] = pack_bf16x2(x0, x1);
        wl[e] = pack_bf16x2(x0 - bf16_lo(wh[e]), x1 - bf16_hi(wh[e]));
        mw[e] = (in0 ? 0x3f80u : 0u) | (in1 ? 0x3f800000u : 0u);
      }
    }
    ls += lsum;
    l_run += psum;
    const bf16x8 pf = __builtin_bit_cast(bf16x8, wh), plf = __builtin_bit_cast(bf16x8, wl);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const bf16x8 vf = __builtin_bit_cast(bf16x8, vfr[dt]);
      U[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, U[dt], 0, 0, 0);
      U[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, plf, U[dt], 0, 0, 0);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sv = dot2_bf16(wvv[e], mw[e], sv);
      sk = dot2_bf16(wk[e], mw[e], sk);
    }
    // advance; the group that ends a cluster finishes it (and any empty
    // clusters after it)
    cg.off += kFpGK;
    if (cg.k0 + cg.off >= cg.k1) {
      finish(cg.c, cg.k1 - cg.k0);
      enter(cg, cg.c + 1, cg.k1);
      while (cg.c < nclu && cg.k1 == cg.k0) {
        finish(cg.c, 0);
        enter(cg, cg.c + 1, cg.k1);
      }
    }
  };

  auto step = [&](const uint16_t* Kb, const uint16_t* Vb, uint16_t* Kn, uint16_t* Vn, int u)
                  __attribute__((always_inline)) {
    // tile u landed.  Loads return in order, so while a copy of tile u is
    // outstanding all copies of the later tiles (issued after it, four per
    // tile) are too: waiting until at most 4 (one later tile issued) or 8 (two)
    // operations remain covers tile u even with result stores in between
    // (which only make it wait longer)
    const int ahead = issued - u - 1;
    if (ahead >= 2) asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else if (ahead == 1) asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // the bases are opaque here, so the XORed offsets are formed next to their
    // reads instead of being held across the loop
    uint32_t kb = kb2, va = va2, vw = vw2, kt = kt2;
    asm volatile("" : "+v"(kb), "+v"(va), "+v"(vw), "+v"(kt));
    // S^T (32 keys x 32 proxies) = K (c_hi + c_lo)^T, in log2 units: all K
    // reads first, then the MFMA chain
    bf16x8 kf[KT];
#pragma unroll
    for (int t = 0; t < KT; ++t) kf[t] = *(const bf16x8*)lds_byte(Kb, kb ^ (32 * t));
    __builtin_amdgcn_sched_barrier(0);
    f32x16 s = f32x16{};
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[t], cf[t], s, 0, 0, 0);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[t], cl[t], s, 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // the next copy (tile u + 3, if any) goes out while the chain runs (stage
    // Kn was released by the barrier above)
    dma(Kn, Vn);
    // key row of s[r]: 8 (r / 4) + 4 hi + r % 4; padding rows repeat a key of
    // this tile, so they never raise the maximum
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    const float m_new = fmaxf(m_run, pair_max(mx));
    if (__any(m_new - m_run > kLazyRescaleLog2)) {
      const float alpha = fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DT; ++i) U[i] *= alpha;
      m_run = m_new;
    }
    group(Kb, Vb, s, 0, va, vw, kt);
    group(Kb, Vb, s, 1, va, vw, kt);
  };

  dma(K0, V0);
  dma(K1, V1);
  dma(K2, V2);
  // tile u exists iff u < issued (copies run three tiles ahead); issued is
  // uniform, so every wave leaves at the same step
  for (int u = 0;; u += 4) {
    if (u >= issued) break;
    step(K0, V0, K3, V3, u);
    if (u + 1 >= issued) break;
    step(K1, V1, K0, V0, u + 1);
    if (u + 2 >= issued) break;
    step(K2, V2, K1, V1, u + 2);
    if (u + 3 >= issued) break;
    step(K3, V3, K2, V2, u + 3);
  }

  const float z = pair_sum(l_run);
  if (pvalid && hi == 0) {
    p.m_split[((int64_t)bh * p.splits + split) * a.Cq + prox] = m_run;
    p.z_split[((int64_t)bh * p.splits + split) * a.Cq + prox] = z;
  }
}

// ---------------------------------------------------------------------------
// route select
// ---------------------------------------------------------------------------

constexpr int kSelThreads = 1024, kSelWaves = kSelThreads / 64, kSelMaxCk = 4096;
constexpr int kSelBatch = 8;  // 64-column chunks whose loads are issued together

__device__ __forceinline__ long long wave_sum64(long long x) {
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}
__device__ __forceinline__ long long wave_incl_scan64(long long x, int lane) {
  for (int off = 1; off < 64; off <<= 1) {
    const long long y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

// ---------------------------------------------------------------------------
// scores and their cost histogram
// ---------------------------------------------------------------------------
// score_ab = e2_ab 2^(2 (m_ab - M_a)) / Z_a^2 / n_b, with (M_a, Z_a) the proxy's
// softmax reference and normaliser combined over the probe's splits (the
// finalize of the streamed probe), or scores given by the caller.  Each of
// kHistGroups workgroups per (batch, head) takes a range of rows and adds the
// cost n_a n_b of every non-empty block to a histogram over bits 30..20 of
// the score (non-negative floats order like their bit patterns); the
// histograms are written per workgroup and summed by the selection in a fixed
// order (integer sums: exact, so the cut does not depend on the order).
constexpr int kHistBins = 2048, kHistGroups = 32;

struct ScoreHistArgs {
  const int32_t* q_off;
  const int32_t* k_off;
  const float* e_buf;    // null: the scores are given in `score`
  const float* m_buf;
  const float* m_split;
  const float* z_split;
  float* score;          // [BH][Cq][Ck]
  unsigned long long* hist;  // [BH][kHistGroups][kHistBins]
  int Cq, Ck, splits;
};

__device__ __forceinline__ int score_bin(uint32_t bits) {
  return (int)min(bits >> 20, (uint32_t)(kHistBins - 1));
}

__global__ void __launch_bounds__(256) score_hist_kernel(ScoreHistArgs f) {
  constexpr int kRows = 64;  // rows whose (M_a, 1 / Z_a^2) are combined per round
  __shared__ unsigned long long h[kHistBins];
  __shared__ float rm[kRows], rz[kRows];
  const int g = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rpg = (f.Cq + kHistGroups - 1) / kHistGroups;
  const int a0 = min(g * rpg, f.Cq), a1 = min(a0 + rpg, f.Cq);
  const int32_t* qo = f.q_off + (int64_t)bh * (f.Cq + 1);
  const int32_t* ko = f.k_off + (int64_t)bh * (f.Ck + 1);
  for (int i = tid; i < kHistBins; i += 256) h[i] = 0;
  for (int r0 = a0; r0 < a1; r0 += kRows) {
    const int nr = min(kRows, a1 - r0);
    if (f.e_buf) {
      // combine the splits' (reference, normaliser) pairs of each row, one wave
      // per row, all rows of the round in parallel
      for (int i = wave; i < nr; i += 4) {
        const int a = r0 + i;
        float mm = -1e30f;
        for (int s = lane; s < f.splits; s += 64) mm = fmaxf(mm, f.m_split[((int64_t)bh * f.splits + s) * f.Cq + a]);
        for (int off = 32; off > 0; off >>= 1) mm = fmaxf(mm, __shfl_xor(mm, off, 64));
        float z = 0.f;
        for (int s = lane; s < f.splits; s += 64) {
          const int64_t o = ((int64_t)bh * f.splits + s) * f.Cq + a;
          z += f.z_split[o] * fast_exp2(f.m_split[o] - mm);
        }
        for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off, 64);
        if (lane == 0) {
          rm[i] = mm;
          rz[i] = z > 0.f ? 1.f / (z * z) : 0.f;
        }
      }
    }
    __syncthreads();
    // every block of the round's rows, four per thread in flight
    const int n = nr * f.Ck;
    for (int e0 = tid; e0 < n; e0 += 4 * 256) {
      float ev[4], mv[4];
      int64_t ov[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = min(e0 + 256 * j, n - 1);
        const int i = e / f.Ck, b = e - i * f.Ck;
        ov[j] = ((int64_t)bh * f.Cq + r0 + i) * f.Ck + b;
        if (f.e_buf) {
          ev[j] = f.e_buf[ov[j]];
          mv[j] = f.m_buf[ov[j]];
        } else {
          ev[j] = f.score[ov[j]];
          mv[j] = 0.f;
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = e0 + 256 * j;
        if (e >= n) break;
        const int i = e / f.Ck, b = e - i * f.Ck;
        const long long na = qo[r0 + i + 1] - qo[r0 + i], nb = ko[b + 1] - ko[b];
        float sc = ev[j];
        if (f.e_buf) {
          sc = 0.f;
          if (na > 0 && nb > 0) sc = ev[j] * fast_exp2(2.f * (mv[j] - rm[i])) * rz[i] / (float)nb;
          f.score[ov[j]] = sc;
        }
        const long long cost = na * nb;
        if (cost > 0) atomicAdd(&h[score_bin(__float_as_uint(sc))], (unsigned long long)cost);
      }
    }
    __syncthreads();
  }
  unsigned long long* out = f.hist + ((int64_t)bh * kHistGroups + g) * kHistBins;
  for (int i = tid; i < kHistBins; i += 256) out[i] = h[i];
}

// First selection level from the histograms (one workgroup of kSelThreads):
// the total cost of the non-empty blocks, and, unless all of them fit the
// budget, the cut bin d (bits 30..20): the blocks of bins above d cost at most
// the budget, adding d's blocks would exceed it.  Returns take_all; otherwise
// sets pre = d << 20 and R = budget - (cost of the bins above d).  Thread t
// holds bins 2t and 2t + 1.
__device__ bool select_level1(const unsigned long long* hist, long long budget, long long* wred, long long* sh_R,
                              unsigned* sh_prefix, unsigned& pre, long long& R) {
  static_assert(kSelThreads * 2 == kHistBins, "two bins per thread");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  unsigned long long h0 = 0, h1 = 0;
  for (int gg = 0; gg < kHistGroups; ++gg) {
    h0 += hist[gg * kHistBins + 2 * tid];
    h1 += hist[gg * kHistBins + 2 * tid + 1];
  }
  const long long own = (long long)(h0 + h1);
  long long suf = own;  // inclusive suffix over the lanes >= this one
  for (int off = 1; off < 64; off <<= 1) {
    const long long y = __shfl_down(suf, off, 64);
    if (lane + off < 64) suf += y;
  }
  if (lane == 0) wred[wave] = suf;
  __syncthreads();
  long long total = 0, above = suf - own;
  for (int w = 0; w < kSelWaves; ++w) {
    total += wred[w];
    if (w > wave) above += wred[w];
  }
  const bool take_all = total <= budget;
  if (!take_all) {
    if (above <= budget && above + (long long)h1 > budget) {
      *sh_R = budget - above;
      *sh_prefix = (unsigned)(2 * tid + 1) << 20;
    } else if (above + (long long)h1 <= budget && above + (long long)(h0 + h1) > budget) {
      *sh_R = budget - above - (long long)h1;
      *sh_prefix = (unsigned)(2 * tid) << 20;
    }
  }
  __syncthreads();
  pre = take_all ? 0u : *sh_prefix;
  R = take_all ? budget : *sh_R;
  __syncthreads();
  return take_all;
}

// Selection state of one (batch, head), written by the level-1 and resolve
// kernels: a block of cost > 0 is kept iff take_all, or its score bits are
// above Tb, or equal to Tb with an index a * Ck + b up to tie_cut.
struct SelState {
  long long R;    // budget left for the cut bin
  unsigned pre;   // cut bin << 20
  int take_all;
  unsigned Tb;
  int tie_cut;
  int count;      // blocks gathered from the cut bin
  int pad;
};

struct SelectArgs {
  const float* score;   // [BH][Cq][Ck]
  const int32_t* q_off;
  const int32_t* k_off;
  int32_t* rrow;        // [BH][Cq+1]
  int32_t* rcol;        // [BH][Cq*Ck]
  const unsigned long long* hist;  // [BH][kHistGroups][kHistBins]
  SelState* state;      // [BH]
  unsigned long long* cand;        // [BH][kSelCand] cut-bin keys ~bits << 32 | index
  int32_t* counts;      // [BH][Cq] kept blocks per row
  int Cq, Ck, N;
  long long budget;
};

// Blocks are ranked by (score descending, index a * Ck + b ascending); the
// kept set is the longest prefix of that order whose total cost n_a n_b fits
// the budget.  Non-negative floats order like their bit patterns.  Six short
// launches, the row-wise ones one wave per query cluster:
//   score_hist_kernel     scores and their cost histograms (bits 30..20);
//   select_level1_kernel  per head: the cut bin and the budget R left for it;
//   select_gather_kernel  per row: the cut bin's blocks into a per-head list;
//   select_resolve_kernel per head: the list sorted by (bits descending, index
//                         ascending) as 64-bit keys (bitonic in LDS, kSelCand
//                         at most); the kept ones are the longest prefix whose
//                         cost fits R, which fixes Tb and tie_cut.  A cut bin
//                         of more blocks (many equal scores) is resolved by
//                         radix passes of 8, 8 and 4 bits over the head's
//                         scores, the blocks equal to the final pattern taken
//                         in index order while R lasts;
//   select_count_kernel   per row: kept blocks;
//   select_emit_kernel    per row: its CSR offset (sum of the earlier rows'
//                         counts) and its ascending kept columns.
constexpr int kSelCand = 4096;

__device__ __forceinline__ bool sel_keep(const SelState& st, unsigned bits, int idx, long long cost) {
  return cost > 0 && (st.take_all || bits > st.Tb || (bits == st.Tb && idx <= st.tie_cut));
}

__global__ void __launch_bounds__(kSelThreads) select_level1_kernel(SelectArgs s) {
  __shared__ long long wred[kSelWaves];
  __shared__ long long sh_R;
  __shared__ unsigned sh_prefix;
  const int bh = blockIdx.x;
  unsigned pre = 0;
  long long R = s.budget;
  const bool take_all = select_level1(s.hist + (int64_t)bh * kHistGroups * kHistBins, s.budget, wred, &sh_R,
                                      &sh_prefix, pre, R);
  if (threadIdx.x == 0) {
    SelState st;
    st.R = R;
    st.pre = pre;
    st.take_all = take_all ? 1 : 0;
    st.Tb = 0;
    st.tie_cut = 0x7fffffff;
    st.count = 0;
    st.pad = 0;
    s.state[bh] = st;
  }
}

// one wave per row: visit the row's blocks in column order, the loads of a
// batch of 64-column chunks in flight together: f(b, bits, cost)
template <typename F>
__device__ __forceinline__ void sel_row(const SelectArgs& s, int bh, int a, F&& f) {
  const int lane = threadIdx.x & 63;
  const int32_t* qo = s.q_off + (int64_t)bh * (s.Cq + 1);
  const int32_t* ko = s.k_off + (int64_t)bh * (s.Ck + 1);
  const long long na = qo[a + 1] - qo[a];
  const unsigned* row = (const unsigned*)s.score + ((int64_t)bh * s.Cq + a) * s.Ck;
  for (int b0 = 0; b0 < s.Ck; b0 += 64 * kSelBatch) {
    unsigned bits[kSelBatch];
    int nb[kSelBatch];
#pragma unroll
    for (int j = 0; j < kSelBatch; ++j) {
      const int b = b0 + 64 * j + lane;
      bits[j] = b < s.Ck ? row[b] : 0u;
      nb[j] = b < s.Ck ? ko[b + 1] - ko[b] : 0;
    }
#pragma unroll
    for (int j = 0; j < kSelBatch; ++j) {
      if (b0 + 64 * j >= s.Ck) break;  // wave-uniform
      f(b0 + 64 * j + lane, bits[j], na * nb[j]);
    }
  }
}

__global__ void __launch_bounds__(256) select_gather_kernel(SelectArgs s) {
  const int bh = blockIdx.y, a = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  const SelState st = s.state[bh];
  if (st.take_all || a >= s.Cq) return;
  unsigned long long* cand = s.cand + (int64_t)bh * kSelCand;
  const int32_t* qo = s.q_off + (int64_t)bh * (s.Cq + 1);
  const int32_t* ko = s.k_off + (int64_t)bh * (s.Ck + 1);
  const long long na = qo[a + 1] - qo[a];
  if (na == 0) return;
  const unsigned* row = (const unsigned*)s.score + ((int64_t)bh * s.Cq + a) * s.Ck;
  for (int b0 = 0; b0 < s.Ck; b0 += 64 * kSelBatch) {
    // the batch's cut-bin blocks, then one counter atomic for all of them
    unsigned bits[kSelBatch];
    bool in[kSelBatch];
#pragma unroll
    for (int j = 0; j < kSelBatch; ++j) {
      const int b = b0 + 64 * j + lane;
      bits[j] = b < s.Ck ? row[b] : 0u;
      in[j] = b < s.Ck && ko[b + 1] > ko[b] && (bits[j] >> 20) == (st.pre >> 20);
    }
    int total = 0;
#pragma unroll
    for (int j = 0; j < kSelBatch; ++j) total += __popcll(__ballot(in[j]));
    if (total == 0) continue;
    int base = 0;
    if (lane == 0) base = atomicAdd(&s.state[bh].count, total);
    base = __shfl(base, 0, 64);
#pragma unroll
    for (int j = 0; j < kSelBatch; ++j) {
      const unsigned long long bal = __ballot(in[j]);
      const int pos = base + __popcll(bal & ((1ull << lane) - 1ull));
      if (in[j] && pos < kSelCand)
        cand[pos] = ((unsigned long long)(~bits[j]) << 32) | (unsigned)(a * s.Ck + b0 + 64 * j + lane);
      base += __popcll(bal);
    }
  }
}

__global__ void __launch_bounds__(kSelThreads) select_resolve_kernel(SelectArgs s) {
  __shared__ unsigned long long keys[kSelCand];  // the gathered bin; the radix passes' histograms
  __shared__ unsigned long long hc[kSelCand];    // level-2 / level-3 histograms; the sorted ties
  __shared__ long long wred[kSelWaves];
  __shared__ int wcnt[kSelWaves];
  __shared__ long long sh_R;
  __shared__ unsigned sh_prefix;
  __shared__ int sh_tie;
  const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const SelState st = s.state[bh];
  if (st.take_all) return;
  const int Cq = s.Cq, Ck = s.Ck;
  const int32_t* qo = s.q_off + (int64_t)bh * (Cq + 1);
  const int32_t* ko = s.k_off + (int64_t)bh * (Ck + 1);
  long long R = st.R;
  unsigned Tb;
  int tie_cut;
  const int count = st.count;
  if (count <= kSelCand) {
    // levels 2 and 3 (bits 19..8, then 7..0) as cost histograms over the
    // gathered blocks, each candidate staying in LDS: keys[] holds them, hc[]
    // the histogram; then the blocks equal to the final pattern in index order
    const unsigned long long* cand = s.cand + (int64_t)bh * kSelCand;
    for (int i = tid; i < count; i += kSelThreads) keys[i] = cand[i];
    unsigned pre = st.pre, msk = 0xfff00000u;
    for (int level = 0; level < 2; ++level) {
      const int width = level == 0 ? 12 : 8, shift = level == 0 ? 8 : 0;
      const int nbins = 1 << width;
      for (int i = tid; i < nbins; i += kSelThreads) hc[i] = 0;
      __syncthreads();
      for (int i = tid; i < count; i += kSelThreads) {
        const unsigned long long key = keys[i];
        const unsigned bits = ~(unsigned)(key >> 32), idx = (unsigned)key;
        if ((bits & msk) == pre) {
          const int a = (int)(idx / (unsigned)Ck), b = (int)(idx % (unsigned)Ck);
          atomicAdd(&hc[(bits >> shift) & (nbins - 1)],
                    (unsigned long long)((long long)(qo[a + 1] - qo[a]) * (ko[b + 1] - ko[b])));
        }
      }
      __syncthreads();
      // thread t holds bins [t * per, (t + 1) * per); the cut bin d: the bins
      // above it fit R, adding d's cost exceeds R (bin 0 if none does)
      const int per = nbins / kSelThreads > 0 ? nbins / kSelThreads : 1;
      unsigned long long own = 0;
      for (int e = 0; e < per; ++e) {
        const int d = tid * per + e;
        own += d < nbins ? hc[d] : 0;
      }
      long long suf = (long long)own;  // inclusive suffix over lanes >= this one
      for (int o = 1; o < 64; o <<= 1) {
        const long long y = __shfl_down(suf, o, 64);
        if (lane + o < 64) suf += y;
      }
      if (lane == 0) wred[wave] = suf;
      __syncthreads();
      long long above = suf - (long long)own;
      for (int w = wave + 1; w < kSelWaves; ++w) above += wred[w];
      for (int e = per - 1; e >= 0; --e) {
        const int d = tid * per + e;
        if (d >= nbins) continue;
        const long long h = (long long)hc[d];
        if (above <= R && (above + h > R || d == 0)) {
          sh_R = R - above;
          sh_prefix = pre | ((unsigned)d << shift);
        }
        above += h;
      }
      __syncthreads();
      R = sh_R;
      pre = sh_prefix;
      msk |= (unsigned)(nbins - 1) << shift;
      __syncthreads();
    }
    Tb = pre;
    // ties: the gathered blocks equal to Tb, in index order, while R lasts.
    // Compact their indices (usually one) and sort them (bitonic, in hc[]).
    if (tid == 0) sh_tie = 0;
    __syncthreads();
    for (int i = tid; i < count; i += kSelThreads) {
      const unsigned long long key = keys[i];
      if (~(unsigned)(key >> 32) == Tb) hc[atomicAdd(&sh_tie, 1)] = (unsigned)key;
    }
    __syncthreads();
    const int nt = sh_tie;
    int P = 1;
    while (P < nt) P <<= 1;
    for (int i = nt + tid; i < P; i += kSelThreads) hc[i] = ~0ull;
    __syncthreads();
    for (int k = 2; k <= P; k <<= 1)
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < P; i += kSelThreads) {
          const int l = i ^ j;
          if (l > i) {
            const unsigned long long x = hc[i], y = hc[l];
            if ((x > y) == ((i & k) == 0)) {
              hc[i] = y;
              hc[l] = x;
            }
          }
        }
        __syncthreads();
      }
    // the last tie whose inclusive prefix cost fits R (thread t: ties 4t..4t+3)
    long long c4[4], run = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * tid + e;
      long long cc = 0;
      if (i < nt) {
        const unsigned idx = (unsigned)hc[i];
        const int a = (int)(idx / (unsigned)Ck), b = (int)(idx % (unsigned)Ck);
        cc = (long long)(qo[a + 1] - qo[a]) * (ko[b + 1] - ko[b]);
      }
      run += cc;
      c4[e] = run;
    }
    const long long inc = wave_incl_scan64(run, lane);
    if (lane == 63) wred[wave] = inc;
    __syncthreads();
    long long off = 0;
    for (int w = 0; w < wave; ++w) off += wred[w];
    const long long excl = off + inc - run;
    int kept = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) kept += (4 * tid + e < nt && excl + c4[e] <= R) ? 1 : 0;
    kept = (int)wave_sum64(kept);
    if (lane == 0) wcnt[wave] = kept;
    __syncthreads();
    int cut = 0;
    for (int w = 0; w < kSelWaves; ++w) cut += wcnt[w];
    tie_cut = cut > 0 ? (int)(unsigned)hc[cut - 1] : -1;
  } else {
    // many equal scores in the cut bin: radix passes below the first level
    // over the head's scores (wave w takes rows [w rpw, (w + 1) rpw)), one
    // cost histogram per wave
    unsigned long long* hist = keys;  // [kSelWaves][256]
    const int rpw = (Cq + kSelWaves - 1) / kSelWaves;
    const int ra0 = min(wave * rpw, Cq), ra1 = min(ra0 + rpw, Cq);
    unsigned pre = st.pre, msk = 0xfff00000u;
    for (int low = 20; low > 0;) {
      const int width = min(8, low);
      const int shift = low - width;
      const unsigned dmask = (1u << width) - 1u;
      low = shift;
      for (int i = lane; i < 256; i += 64) hist[wave * 256 + i] = 0;
      __builtin_amdgcn_wave_barrier();
      for (int a = ra0; a < ra1; ++a)
        sel_row(s, bh, a, [&](int, unsigned bits, long long c) {
          if (c > 0 && (bits & msk) == pre) atomicAdd(&hist[wave * 256 + ((bits >> shift) & dmask)], (unsigned long long)c);
        });
      __syncthreads();
      if (wave == 0) {
        // lane l holds digits 4l .. 4l+3; the cut digit is the first from the
        // top whose own cost takes the cost above it past R (digit 0 if none)
        unsigned long long h[4], own = 0;
        for (int i = 0; i < 4; ++i) {
          unsigned long long t = 0;
          for (int w = 0; w < kSelWaves; ++w) t += hist[w * 256 + 4 * lane + i];
          h[i] = t;
          own += t;
        }
        long long above = (long long)own;
        for (int o = 1; o < 64; o <<= 1) {
          const long long y = __shfl_down(above, o, 64);
          if (lane + o < 64) above += y;
        }
        above -= (long long)own;
        for (int i = 3; i >= 0; --i) {
          const int d = 4 * lane + i;
          const bool cut = (above + (long long)h[i] > R) || d == 0;
          if (cut && above <= R) {
            sh_R = R - above;
            sh_prefix = pre | ((unsigned)d << shift);
            break;
          }
          above += (long long)h[i];
        }
      }
      __syncthreads();
      R = sh_R;
      pre = sh_prefix;
      msk |= dmask << shift;
      __syncthreads();
    }
    Tb = pre;
    // blocks equal to Tb in index order while R lasts: the last kept index
    long long tc = 0;
    for (int a = ra0; a < ra1; ++a)
      sel_row(s, bh, a, [&](int, unsigned bits, long long c) {
        if (c > 0 && bits == Tb) tc += c;
      });
    tc = wave_sum64(tc);
    if (lane == 0) wred[wave] = tc;
    if (tid == 0) sh_tie = -1;
    __syncthreads();
    long long carry = 0;
    for (int w = 0; w < wave; ++w) carry += wred[w];
    int last = -1;
    for (int a = ra0; a < ra1; ++a)
      sel_row(s, bh, a, [&](int b, unsigned bits, long long c) {
        const bool tie = c > 0 && bits == Tb;
        long long incl = 0;
        if (__any(tie)) incl = wave_incl_scan64(tie ? c : 0, lane);
        if (tie && carry + incl <= R) last = max(last, a * Ck + b);
        carry += __shfl(incl, 63, 64);
      });
    for (int o = 32; o > 0; o >>= 1) last = max(last, __shfl_xor(last, o, 64));
    if (lane == 0) atomicMax(&sh_tie, last);
    __syncthreads();
    tie_cut = sh_tie;
  }
  if (tid == 0) {
    s.state[bh].Tb = Tb;
    s.state[bh].tie_cut = tie_cut;
  }
}

__global__ void __launch_bounds__(256) select_count_kernel(SelectArgs s) {
  const int bh = blockIdx.y, a = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (a >= s.Cq) return;
  const SelState st = s.state[bh];
  int kept = 0;
  sel_row(s, bh, a, [&](int b, unsigned bits, long long c) {
    kept += __popcll(__ballot(sel_keep(st, bits, a * s.Ck + b, c)));
  });
  if (lane == 0) s.counts[(int64_t)bh * s.Cq + a] = kept;
}

__global__ void __launch_bounds__(256) select_emit_kernel(SelectArgs s) {
  const int bh = blockIdx.y, a = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (a >= s.Cq) return;
  const SelState st = s.state[bh];
  const int32_t* cnt = s.counts + (int64_t)bh * s.Cq;
  int start = 0;
  for (int i = lane; i < a; i += 64) start += cnt[i];
  for (int o = 32; o > 0; o >>= 1) start += __shfl_xor(start, o, 64);
  int32_t* rr = s.rrow + (int64_t)bh * (s.Cq + 1);
  int32_t* rc = s.rcol + (int64_t)bh * s.Cq * s.Ck;
  if (lane == 0) {
    if (a == 0) rr[0] = 0;
    rr[a + 1] = start + cnt[a];
  }
  sel_row(s, bh, a, [&](int b, unsigned bits, long long c) {
    const bool keep = sel_keep(st, bits, a * s.Ck + b, c);
    const unsigned long long bal = __ballot(keep);
    if (keep) rc[start + __popcll(bal & ((1ull << lane) - 1ull))] = b;
    start += __popcll(bal);
  });
}

// ---------------------------------------------------------------------------
// compensated attention
// ---------------------------------------------------------------------------

constexpr int kCaBN = 64;

struct CompArgs {
  SvgArgs s;
  uint16_t* o;
  float* lse;
  const int32_t* rrow;
  const int32_t* rcol;
  const float* k_cent;
  const float* v_cent;
  float scale, c2;
  const uint16_t* kc_bf;  // head_dim 128 path: bf16 copies of k_cent / v_cent, [BH][Ck][D]
  const uint16_t* vc_bf;
  const int32_t* tile_item;   // head_dim 128 path: tile schedule, longest first: item bh * Cq + a,
  const int32_t* tile_x;      // tile x of that cluster (rows q_off[a] + 128 x ...),
  const int32_t* tile_count;  // and the number of tiles
  const int32_t* runs;        // head_dim 128 path: run tables of the route rows (see comp_steps_kernel)
};

template <int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
comp_attn_kernel(CompArgs p) {
  constexpr int KT = D / 16, DT = D / 32, CH = D / 8;
  constexpr int KST = D + 8, VST = D + 32;
  constexpr int LCH = kCaBN * CH / 256;
  constexpr int MAXCK = 512;  // key clusters (the host rejects more)
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kCaBN * KST];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][kCaBN * VST];
  __shared__ int cum[MAXCK + 1];     // prefix of kept cluster sizes
  __shared__ float bias[MAXCK];      // virtual-key logit bias (raw units) or -inf
  __shared__ int sh_tile[3];

  const SvgArgs& a = p.s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hi = lane >> 5;
  const int bh = blockIdx.y;
  const int32_t* qo = a.q_off + (int64_t)bh * (a.Cq + 1);
  const int32_t* ko = a.k_off + (int64_t)bh * (a.Ck + 1);

  if (tid == 0) {
    int x = blockIdx.x, ca = -1, t0 = 0;
    for (int c = 0; c < a.Cq; ++c) {
      const int nt = (qo[c + 1] - qo[c] + 127) / 128;
      if (x < t0 + nt) {
        ca = c;
        break;
      }
      t0 += nt;
    }
    sh_tile[0] = ca;
    sh_tile[1] = ca >= 0 ? qo[ca] + 128 * (x - t0) : 0;
    sh_tile[2] = ca >= 0 ? qo[ca + 1] : 0;
  }
  __syncthreads();
  const int ca = sh_tile[0];
  if (ca < 0) return;  // beyond the last query tile of this head (uniform)
  const int r0 = sh_tile[1], r1 = sh_tile[2];

  // route row of this cluster; a caller-given route is clamped into range so
  // that the tables below and the offset reads stay in bounds
  const int rb = max(0, min(p.rrow[(int64_t)bh * (a.Cq + 1) + ca], a.Cq * a.Ck));
  const int nk = max(0, min(p.rrow[(int64_t)bh * (a.Cq + 1) + ca + 1] - rb, min(a.Ck, a.Cq * a.Ck - rb)));
  const int32_t* cl = p.rcol + (int64_t)bh * a.Cq * a.Ck + rb;
  for (int b = tid; b < a.Ck; b += 256) {
    const int n = ko[b + 1] - ko[b];
    bias[b] = n > 0 ? __logf((float)n) / p.scale : -__builtin_inff();
  }
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int i = 0; i < nk; ++i) {
      cum[i] = acc;
      const int b = max(0, min(cl[i], a.Ck - 1));
      acc += ko[b + 1] - ko[b];
      bias[b] = -__builtin_inff();  // kept clusters are exact, never virtual
    }
    cum[nk] = acc;
  }
  __syncthreads();
  const int E = cum[nk];
  const int ne = (E + kCaBN - 1) / kCaBN;
  const int nv = (a.Ck + kCaBN - 1) / kCaBN;
  const int nsub = ne + nv;

  const uint16_t* Qh = head_ptr(a.q, a, bh);
  const uint16_t* Kh = head_ptr(a.k, a, bh);
  const uint16_t* Vh = head_ptr(a.v, a, bh);
  const int qrow = r0 + wave * 32 + l32;
  const bool qok = qrow < r1;
  bf16x8 qf[KT];
  {
    const uint16_t* src = Qh + (int64_t)(qok ? qrow : r0) * a.sn + hi * 8;
#pragma unroll
    for (int t = 0; t < KT; ++t) qf[t] = __builtin_bit_cast(bf16x8, *(const u32x4*)(src + t * 16));
  }

  u32x4 kreg[LCH], vreg[LCH];
  auto fetch = [&](int u) {
#pragma unroll
    for (int i = 0; i < LCH; ++i) {
      const int c = tid + 256 * i;
      const int row = c / CH, col = (c % CH) * 8;
      if (u < ne) {
        const int slot = min(u * kCaBN + row, E - 1);
        int lo = 0, hi_ = nk - 1;  // largest i with cum[i] <= slot
        while (lo < hi_) {
          const int mid = (lo + hi_ + 1) >> 1;
          if (cum[mid] <= slot) lo = mid;
          else hi_ = mid - 1;
        }
        const int key = ko[max(0, min(cl[lo], a.Ck - 1))] + slot - cum[lo];
        kreg[i] = *(const u32x4*)(Kh + (int64_t)key * a.sn + col);
        vreg[i] = *(const u32x4*)(Vh + (int64_t)key * a.sn + col);
      } else {
        const int b = min((u - ne) * kCaBN + row, a.Ck - 1);
        const float* kc = p.k_cent + ((int64_t)bh * a.Ck + b) * D + col;
        const float* vc = p.v_cent + ((int64_t)bh * a.Ck + b) * D + col;
        const float4 k0 = *(const float4*)kc, k1 = *(const float4*)(kc + 4);
        const float4 v0 = *(const float4*)vc, v1 = *(const float4*)(vc + 4);
        kreg[i] = u32x4{pack_bf16x2(k0.x, k0.y), pack_bf16x2(k0.z, k0.w), pack_bf16x2(k1.x, k1.y),
                        pack_bf16x2(k1.z, k1.w)};
        vreg[i] = u32x4{pack_bf16x2(v0.x, v0.y), pack_bf16x2(v0.z, v0.w), pack_bf16x2(v1.x, v1.y),
                        pack_bf16x2(v1.z, v1.w)};
      }
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LCH; ++i) {
      const int c = tid + 256 * i;
      const int row = c / CH, col = (c % CH) * 8;
      *(u32x4*)&Ks[buf][row * KST + col] = kreg[i];
      *(u32x4*)&Vs[buf][row * VST + col] = vreg[i];
    }
  };

  f32x16 o[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) o[i] = f32x16{};
  float m_run = -1e30f, l_run = 0.f;
  const int g16 = lane >> 4, j16 = lane & 15;
  const int v_row = 4 * hi + (j16 >> 2);
  const int v_col = 16 * (g16 & 1) + 4 * (j16 & 3);

  fetch(0);
  stage(0);
  __syncthreads();
  for (int u = 0; u < nsub; ++u) {
    const int buf = u & 1;
    if (u + 1 < nsub) fetch(u + 1);
    f32x16 s[2];
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int t = 0; t < KT; ++t)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const bf16x8 kf = *(const bf16x8*)&Ks[buf][(kt * 32 + l32) * KST + t * 16 + hi * 8];
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[t], s[kt], 0, 0, 0);
      }
    if (u < ne) {
      if ((u + 1) * kCaBN > E) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (u * kCaBN + kt * 32 + 8 * (r >> 2) + 4 * hi + (r & 3) >= E) s[kt][r] = -__builtin_inff();
      }
    } else {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int b = (u - ne) * kCaBN + kt * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          s[kt][r] = b < a.Ck ? s[kt][r] + bias[b] : -__builtin_inff();
        }
    }
    float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int r = 2; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
    const float m_new = fmaxf(m_run, pair_max(mx));
    if (__any(m_new > m_run)) {
      const float alpha = fast_exp2((m_run - m_new) * p.c2);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DT; ++i) o[i] *= alpha;
      m_run = m_new;
    }
    const float mc = m_run * p.c2;
    float psum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = fast_exp2(__builtin_fmaf(s[kt][r], p.c2, -mc));
        s[kt][r] = pr;
        psum += pr;
      }
    l_run += psum;
    bf16x8 pf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kt = ks >> 1, q0 = (ks & 1) * 8;
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(s[kt][q0 + 2 * e], s[kt][q0 + 2 * e + 1]);
      pf[ks] = __builtin_bit_cast(bf16x8, w);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint16_t* p0 = &Vs[buf][(ks * 16 + v_row) * VST + dt * 32 + v_col];
        const u32x2 lo = lds_tr16(p0), hi2 = lds_tr16(p0 + 8 * VST);
        const u32x4 w = {lo[0], lo[1], hi2[0], hi2[1]};
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w), pf[ks], o[dt], 0, 0, 0);
      }
    if (u + 1 < nsub) stage(buf ^ 1);
    __syncthreads();
  }

  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qok) {
    uint16_t* dst = p.o + (int64_t)(bh / a.H) * a.sb + (int64_t)(bh % a.H) * a.sh + (int64_t)qrow * a.sn;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = dt * 32 + 8 * g + 4 * hi;
        u32x2 w = {pack_bf16x2(o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv),
                   pack_bf16x2(o[dt][4 * g + 2] * inv, o[dt][4 * g + 3] * inv)};
        *(u32x2*)(dst + d0) = w;
      }
    if (p.lse != nullptr && hi == 0)
      p.lse[(int64_t)bh * a.N + qrow] =
          l_tot > 0.f ? (m_run * p.c2 + __builtin_log2f(l_tot)) * kLn2 : -__builtin_inff();
  }
}

// bf16 copies of the key / value centroids (the virtual keys and values of the
// head_dim-128 compensated attention are staged from them like real rows).
__global__ void __launch_bounds__(256) centroid_bf16_kernel(const float* k_cent, const float* v_cent,
                                                            uint16_t* kc_bf, uint16_t* vc_bf, int64_t n2) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // pair of elements
  if (i < n2) {
    const float2 k = reinterpret_cast<const float2*>(k_cent)[i];
    const float2 v = reinterpret_cast<const float2*>(v_cent)[i];
    reinterpret_cast<uint32_t*>(kc_bf)[i] = pack_bf16x2(k.x, k.y);
    reinterpret_cast<uint32_t*>(vc_bf)[i] = pack_bf16x2(v.x, v.y);
  }
}

// Tile schedule of the head_dim-128 compensated attention, longest first.  A
// tile is 128 query rows of one cluster; its work is its number of 64-key
// sub-tiles, ceil(E_a / 64) + ceil(Ck / 64), E_a = the exact keys of the kept
// clusters of row a.  Launching the longest tiles first keeps the launch's
// tail short (the lengths vary by a factor of about 4 on the clustered
// workload).  The schedule only decides which workgroup runs a tile and when;
// no result depends on it.
constexpr int kOrdBuckets = 4096;  // work is bucketed by min(sub-tiles, 4095)

struct CompOrderArgs {
  const int32_t* q_off;
  const int32_t* k_off;
  const int32_t* rrow;
  const int32_t* rcol;
  int Cq, Ck, BH, cap;  // cap: capacity of the schedule arrays
  int32_t* work;   // [BH * Cq] sub-tiles of a tile of cluster (bh, a)
  int32_t* ntile;  // [BH * Cq] tiles of cluster (bh, a)
  int32_t* tile_item;
  int32_t* tile_x;
  int32_t* tile_count;
  int32_t* runs;   // [BH][Cq * Ck] pairs, indexed like the route columns
};

// one wave per (head, cluster a): from the route row (indices clamped like the
// attention kernel clamps them) E_a and the row's run table.  The exact keys
// of cluster a are the key rows of its kept clusters concatenated in route
// order; entry i of the table describes the i-th kept cluster b as the pair
// (end slot, key row minus slot): slots [end_{i-1}, end_i) of the
// concatenation hold key rows slot + delta_i, delta_i = k_off[b] - end_{i-1}.
__global__ void __launch_bounds__(256) comp_steps_kernel(CompOrderArgs o) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int bh = blockIdx.y, ca = blockIdx.x * 4 + wave;
  if (ca >= o.Cq) return;
  const int32_t* qo = o.q_off + (int64_t)bh * (o.Cq + 1);
  const int32_t* ko = o.k_off + (int64_t)bh * (o.Ck + 1);
  const int rb = max(0, min(o.rrow[(int64_t)bh * (o.Cq + 1) + ca], o.Cq * o.Ck));
  const int nk = max(0, min(o.rrow[(int64_t)bh * (o.Cq + 1) + ca + 1] - rb, min(o.Ck, o.Cq * o.Ck - rb)));
  const int32_t* cl = o.rcol + (int64_t)bh * o.Cq * o.Ck + rb;
  int32_t* runs = o.runs + 2 * ((int64_t)bh * o.Cq * o.Ck + rb);
  int e = 0;  // slots before this 64-entry chunk
  for (int i0 = 0; i0 < nk; i0 += 64) {
    const int i = i0 + lane;
    int b = 0, sz = 0;
    if (i < nk) {
      b = max(0, min(cl[i], o.Ck - 1));
      sz = ko[b + 1] - ko[b];
    }
    int inc = sz;  // inclusive prefix over the chunk
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(inc, off, 64);
      if (lane >= off) inc += y;
    }
    if (i < nk) {
      runs[2 * i] = e + inc;
      runs[2 * i + 1] = ko[b] - (e + inc - sz);
    }
    e += __shfl(inc, 63, 64);
  }
  if (lane == 0) {
    const int i = bh * o.Cq + ca;
    o.work[i] = (e + kCaBN - 1) / kCaBN + (o.Ck + kCaBN - 1) / kCaBN;
    o.ntile[i] = max(0, (qo[ca + 1] - qo[ca] + 127) / 128);
  }
}

// one workgroup: histogram of tiles by work, bucket starts in descending work
// order, then every cluster's tiles are placed at its bucket's cursor
__global__ void __launch_bounds__(1024) comp_order_kernel(CompOrderArgs o) {
  __shared__ int hist[kOrdBuckets];
  __shared__ int part[1024];
  const int tid = threadIdx.x, n = o.BH * o.Cq;
  for (int b = tid; b < kOrdBuckets; b += 1024) hist[b] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += 1024) atomicAdd(&hist[min(o.work[i], kOrdBuckets - 1)], o.ntile[i]);
  __syncthreads();
  // exclusive prefix from the top bucket down: thread t owns buckets
  // kOrdBuckets - 4 (t + 1) .. kOrdBuckets - 4 t - 1, taken from the top
  constexpr int per = kOrdBuckets / 1024;
  const int top = kOrdBuckets - per * tid;
  int sum = 0;
  for (int q = 1; q <= per; ++q) sum += hist[top - q];
  part[tid] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int add = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  int run = part[tid] - sum;
  for (int q = 1; q <= per; ++q) {
    const int c = hist[top - q];
    hist[top - q] = run;  // now the cursor of the bucket
    run += c;
  }
  if (tid == 1023) *o.tile_count = min(part[1023], o.cap);
  __syncthreads();
  for (int i = tid; i < n; i += 1024) {
    const int nt = o.ntile[i];
    const int base = atomicAdd(&hist[min(o.work[i], kOrdBuckets - 1)], nt);
    for (int x = 0; x < nt && base + x < o.cap; ++x) {  // (cap holds for offsets within [0, N])
      o.tile_item[base + x] = i;
      o.tile_x[base + x] = x;
    }
  }
}

// head_dim 128 compensated attention.  Same online-softmax core and staging
// as attn_bf16_d128_kernel: 64-key sub-tiles copied straight to two swizzled
// LDS stages (separate objects, loop unrolled by two).  Sub-tile u < ne holds
// slots 64 u .. 64 u + 63 of the concatenated keys of the kept clusters of the
// row's query cluster (each staged row is gathered through the row's run
// table); sub-tiles u >= ne hold the virtual keys, one per key cluster b (bf16
// centroid rows), whose logit gets the bias ln(n_b) / scale, or -inf when b is
// kept or empty.
constexpr int kCaMaxCk = 512;

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
comp_attn_d128_kernel(CompArgs p) {
  constexpr int D = 128, KT = 8, DT = 4, TILE = kCaBN * D;
  __shared__ __attribute__((aligned(1024))) uint16_t K0[TILE], K1[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t V0[TILE], V1[TILE];
  // virtual-key logit bias (raw units), -inf for kept or empty clusters and
  // for the padding of the last virtual sub-tile
  __shared__ __attribute__((aligned(16))) float bias[kCaMaxCk];

  const SvgArgs& a = p.s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hi = lane >> 5;
  // Tile of this workgroup from the longest-first schedule.  Three consecutive
  // schedule entries (usually the tiles of one query cluster, which stage the
  // same kept keys) go to workgroups that the hardware deals to one XCD, so
  // they share its L2: within each run of 24 workgroups, workgroup r takes
  // entry 3 (r % 8) + r / 8.
  const int pid = blockIdx.x, r24 = pid % 24;
  const int j = pid - r24 + 3 * (r24 % 8) + r24 / 8;
  if (j >= *p.tile_count) return;  // uniform
  const int item = __builtin_amdgcn_readfirstlane(p.tile_item[j]);
  const int tx = __builtin_amdgcn_readfirstlane(p.tile_x[j]);
  const int bh = item / a.Cq, ca = item % a.Cq;
  const int32_t* qo = a.q_off + (int64_t)bh * (a.Cq + 1);
  const int32_t* ko = a.k_off + (int64_t)bh * (a.Ck + 1);
  const int r0 = __builtin_amdgcn_readfirstlane(qo[ca] + 128 * tx);
  const int r1 = __builtin_amdgcn_readfirstlane(qo[ca + 1]);

  // ---- kept clusters of row ca (a caller-given route is clamped into range so
  // every table index and every staged row stays in bounds)
  const int rb = __builtin_amdgcn_readfirstlane(max(0, min(p.rrow[(int64_t)bh * (a.Cq + 1) + ca], a.Cq * a.Ck)));
  const int nk = __builtin_amdgcn_readfirstlane(
      max(0, min(p.rrow[(int64_t)bh * (a.Cq + 1) + ca + 1] - rb, min(a.Ck, a.Cq * a.Ck - rb))));
  const int32_t* cl = p.rcol + (int64_t)bh * a.Cq * a.Ck + rb;
  for (int b = tid; b < kCaMaxCk; b += 256) {
    const int n = b < a.Ck ? ko[b + 1] - ko[b] : 0;
    bias[b] = n > 0 ? __logf((float)n) / p.scale : -__builtin_inff();
  }
  __syncthreads();
  for (int i = tid; i < nk; i += 256) bias[max(0, min(cl[i], a.Ck - 1))] = -__builtin_inff();
  // run table of the row, read with scalar loads: entry i = (end slot, delta)
  const cint_ptr runs = (cint_ptr)(p.runs + 2 * ((int64_t)bh * a.Cq * a.Ck + rb));
  const int E = nk > 0 ? max(runs[2 * (nk - 1)], 0) : 0;
  const int ne = (E + kCaBN - 1) / kCaBN;
  const int nv = (a.Ck + kCaBN - 1) / kCaBN;
  const int nsub = ne + nv;

  // ---- query fragments (rows past the cluster end are computed, not stored)
  const int64_t head_off = (int64_t)(bh / a.H) * a.sb + (int64_t)(bh % a.H) * a.sh;
  const int qrow = r0 + wave * 32 + l32;
  bf16x8 qf[KT];
  {
    const uint16_t* src = a.q + head_off + (int64_t)min(qrow, a.N - 1) * a.sn + hi * 8;
#pragma unroll
    for (int t = 0; t < KT; ++t) qf[t] = __builtin_bit_cast(bf16x8, *(const u32x4*)(src + t * 16));
  }
  retire_loads();
  __syncthreads();  // bias complete

  // ---- copy roles: wave w, instruction j covers tile rows 16w + 4j + lane/16
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t row_bytes = (uint32_t)a.sn * 2u;
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.k + head_off), (short)0, 0x7fffffff, kBufferWord3);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.v + head_off), (short)0, 0x7fffffff, kBufferWord3);
  const __amdgpu_buffer_rsrc_t kcs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.kc_bf + (int64_t)bh * a.Ck * D), (short)0, a.Ck * D * 2, kBufferWord3);
  const __amdgpu_buffer_rsrc_t vcs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.vc_bf + (int64_t)bh * a.Ck * D), (short)0, a.Ck * D * 2, kBufferWord3);
  // A wave stages rows 16w + 4j + lane/16 (j = 0..3) of a sub-tile, i.e. the
  // 16 consecutive slots s0 .. s0 + 15 (s0 = 64 u + 16 w).  A wave-uniform
  // cursor over the run table (in scalar registers, the next entry loaded one
  // move ahead) names the kept cluster holding s0; while the wave's slots lie
  // in one cluster, the rows are s0 + delta + 4j + lane/16: one scalar offset
  // and per-lane constants, as in the block-sparse kernel.  A cluster boundary
  // inside the 16 slots (about one wave-step in four) or the end of the keys
  // takes a per-lane path.  For these rows swz_k(row) = 4j + lane/16 and
  // swz_v(row) = 4 (lane/16) + j, so the swizzled chunk offsets are one
  // per-lane base XOR an immediate.
  // Past the last kept cluster the cursor sees an end of INT_MAX, so the
  // loops compare one value; slots at or past E only occur in the last exact
  // sub-tile, whose rows take the clamped per-lane path.
  const cint64_ptr runs2 = (cint64_ptr)runs;
  auto entry = [&](int i, int& end, int& d) __attribute__((always_inline)) {
    if (i < nk) {
      const int64_t x = runs2[i];
      end = (int)(uint32_t)x;
      d = (int)(x >> 32);
    } else {
      end = 0x7fffffff;
      d = 0;
    }
  };
  int cur = 0, end_cur, d_cur, end_nxt, d_nxt;
  entry(0, end_cur, d_cur);
  entry(1, end_nxt, d_nxt);
  auto advance = [&]() __attribute__((always_inline)) {
    ++cur;
    end_cur = end_nxt;
    d_cur = d_nxt;
    entry(cur + 1, end_nxt, d_nxt);
  };
  const int g4 = lane >> 4;
  const uint32_t rbase = (uint32_t)g4 * row_bytes;
  const uint32_t kbase = (uint32_t)(((lane & 15) ^ (lane >> 4)) * 16);
  const uint32_t vbase = (uint32_t)(((lane & 15) ^ (4 * (lane >> 4))) * 16);
  auto dma = [&](uint16_t* kst, uint16_t* vst, int u) __attribute__((always_inline)) {
    if (u < ne) {
      const int s0 = u * kCaBN + 16 * wv;
      while (end_cur <= s0) advance();
      if (end_cur >= s0 + 16 && s0 + 16 <= E) {
        // one cluster holds all 16 slots
        const uint32_t so = (uint32_t)(s0 + d_cur) * row_bytes;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t ro = rbase + (uint32_t)(4 * j) * row_bytes;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)&kst[(16 * wv + 4 * j) * D], 16,
                                                   ro + (kbase ^ (64u * j)), so, 0, 0);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)&vst[(16 * wv + 4 * j) * D], 16,
                                                   ro + (vbase ^ (16u * j)), so, 0, 0);
        }
      } else {
        // per-lane deltas: each boundary end_cur inside the slots moves the
        // lanes at or past it to the next kept cluster's delta (empty kept
        // clusters are passed over the same way)
        int dl[4] = {d_cur, d_cur, d_cur, d_cur};
        while (end_cur < s0 + 16) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (s0 + 4 * j + g4 >= end_cur) dl[j] = d_nxt;
          advance();
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // slots past E are masked below; their rows are clamped into the sequence
          const int row = min(max(min(s0 + 4 * j + g4, E - 1) + dl[j], 0), a.N - 1);
          const uint32_t ro = (uint32_t)row * row_bytes;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)&kst[(16 * wv + 4 * j) * D], 16,
                                                   ro + (kbase ^ (64u * j)), 0, 0, 0);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)&vst[(16 * wv + 4 * j) * D], 16,
                                                   ro + (vbase ^ (16u * j)), 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = 16 * wv + 4 * j + (lane >> 4);
        const int b = min((u - ne) * kCaBN + row, a.Ck - 1);  // clusters past Ck are masked below
        const uint32_t ro = (uint32_t)b * (D * 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kcs, (lds_void*)&kst[(16 * wv + 4 * j) * D], 16,
                                                 ro + (kbase ^ (64u * j)), 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vcs, (lds_void*)&vst[(16 * wv + 4 * j) * D], 16,
                                                 ro + (vbase ^ (16u * j)), 0, 0, 0);
      }
    }
  };

  f32x16 o[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) o[i] = f32x16{};
  float m_run = -1e30f, l_run = 0.f;
  const float c2 = p.c2;
  const int g16 = lane >> 4, j16 = lane & 15;
  // LDS element offsets of the swizzled stage reads, as one per-lane base and
  // an XOR / add of immediates (keeps a handful of address registers live):
  //   K fragment (kt, t):        4096 kt + (kaddr ^ 16 t)
  //   V transpose read (ks, dt): 2048 ks + (vaddr ^ 32 dt)  (+ vdelta for rows + 8)
  const int kaddr = l32 * 128 + 16 * ((l32 & 15) >> 1) + 8 * (hi ^ (l32 & 1));
  const int vq = j16 >> 2, vc1 = (2 * (g16 & 1) + ((j16 >> 1) & 1)) ^ hi;
  const int vaddr = (4 * hi + vq) * 128 + 32 * vq + 8 * vc1 + (j16 & 1) * 4;
  const int vdelta = 1024 + 8 * ((vc1 ^ 2) - vc1);

  // a wave whose 32 rows all lie past the cluster end (the ragged last tile of
  // a cluster) only takes its share of the copies: its SIMD is left to the
  // co-resident wave of another workgroup
  const bool wave_live = r0 + 32 * wv < r1;
  auto step = [&](const uint16_t* Kb, const uint16_t* Vb, uint16_t* Kn, uint16_t* Vn, int u) {
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0): sub-tile u landed, other stage drained
    __builtin_amdgcn_s_barrier();
    if (u + 1 < nsub) dma(Kn, Vn, u + 1);
    if (!wave_live) return;

    f32x16 s[2];
    s[0] = f32x16{};
    s[1] = f32x16{};
    bf16x8 kfr[2][KT];
#pragma unroll
    for (int t = 0; t < KT; ++t)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) kfr[kt][t] = *(const bf16x8*)&Kb[4096 * kt + (kaddr ^ (16 * t))];
#pragma unroll
    for (int t = 0; t < KT; ++t)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfr[kt][t], qf[t], s[kt], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 12; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);

    // key of s[kt][r]: tile row kt 32 + 8 (r / 4) + 4 hi + r % 4
    if (u < ne) {
      if ((u + 1) * kCaBN > E) {
        const uint32_t vm = tile_row_mask(E - u * kCaBN, hi);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (!((vm >> (16 * kt + r)) & 1u)) s[kt][r] = -__builtin_inff();
      }
    } else {
      // bias of clusters b = 64 (u - ne) + 32 kt + 8 g + 4 hi + 0..3 (-inf past Ck)
      const int bb = (u - ne) * kCaBN + 4 * hi;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 bv = *(const f32x4*)&bias[bb + kt * 32 + 8 * g];
#pragma unroll
          for (int e = 0; e < 4; ++e) s[kt][4 * g + e] += bv[e];
        }
    }
    float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int r = 2; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
    const float m_new = fmaxf(m_run, pair_max(mx));
    if (__any((m_new - m_run) * c2 > kLazyRescaleLog2)) {
      const float alpha = fast_exp2((m_run - m_new) * c2);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DT; ++i) o[i] *= alpha;
      m_run = m_new;
    }
    const float mc = m_run * c2;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kt][r] = fast_exp2(__builtin_fmaf(s[kt][r], c2, -mc));
    // P as bf16 (the operand of the value product); the row sum is taken over
    // the same rounded values with v_dot2 against bf16 ones
    bf16x8 pf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kt = ks >> 1, q0 = (ks & 1) * 8;
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w[e] = pack_bf16x2(s[kt][q0 + 2 * e], s[kt][q0 + 2 * e + 1]);
        l_run = dot2_bf16(w[e], 0x3f803f80u, l_run);
      }
      pf[ks] = __builtin_bit_cast(bf16x8, w);
    }
    // raised issue priority over the PV block (co-resident waves drift out of
    // phase, softmax under matrix work)
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int va = 2048 * ks + (vaddr ^ (32 * dt));
        const u32x2 lo = lds_tr16(&Vb[va]);
        const u32x2 h2 = lds_tr16(&Vb[va + vdelta]);
        const u32x4 w = {lo[0], lo[1], h2[0], h2[1]};
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w), pf[ks], o[dt], 0, 0, 0);
      }
    __builtin_amdgcn_s_setprio(0);
  };

  dma(K0, V0, 0);  // nsub >= 1 (Ck >= 1)
  int u = 0;
  for (; u + 2 <= nsub; u += 2) {
    step(K0, V0, K1, V1, u);
    step(K1, V1, K0, V0, u + 1);
  }
  if (u < nsub) step(K0, V0, K1, V1, u);

  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qrow < r1) {
    uint16_t* dst = p.o + head_off + (int64_t)qrow * a.sn;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = dt * 32 + 8 * g + 4 * hi;
        u32x2 w = {pack_bf16x2(o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv),
                   pack_bf16x2(o[dt][4 * g + 2] * inv, o[dt][4 * g + 3] * inv)};
        *(u32x2*)(dst + d0) = w;
      }
    if (p.lse != nullptr && hi == 0)
      p.lse[(int64_t)bh * a.N + qrow] =
          l_tot > 0.f ? (m_run * c2 + __builtin_log2f(l_tot)) * kLn2 : -__builtin_inff();
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

static SvgArgs svg_args(const void* q, const void* k, const void* v, const bsa_shape& s, const int32_t* q_off,
                        int Cq, const int32_t* k_off, int Ck) {
  SvgArgs a;
  a.q = (const uint16_t*)q; a.k = (const uint16_t*)k; a.v = (const uint16_t*)v;
  a.sb = s.stride_b; a.sh = s.stride_h; a.sn = s.stride_n;
  a.B = s.B; a.H = s.H; a.N = s.N;
  a.q_off = q_off; a.k_off = k_off; a.Cq = Cq; a.Ck = Ck;
  return a;
}

bsa_status launch_centroids(const void* q, const void* k, const void* v, const bsa_shape& s, const int32_t* q_off,
                            int Cq, const int32_t* k_off, int Ck, float* qc, float* kc, float* vc,
                            hipStream_t stream, CentroidSet which) {
  SvgArgs a = svg_args(q, k, v, s, q_off, Cq, k_off, Ck);
  const int c0 = which == kCentKey ? Cq : 0;
  const int n = which == kCentAll ? Cq + Ck : (which == kCentQuery ? Cq : Ck);
  dim3 grid(n, s.B * s.H);
  if (s.D == 128) hipLaunchKernelGGL(centroid_kernel<128>, grid, dim3(256), 0, stream, a, qc, kc, vc, c0);
  else if (s.D == 64) hipLaunchKernelGGL(centroid_kernel<64>, grid, dim3(256), 0, stream, a, qc, kc, vc, c0);
  else return BSA_ERR_UNSUPPORTED;
  return launch_ok("cluster_centroids") ? BSA_OK : BSA_ERR_HIP;
}

static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

// selection scratch: cost histograms [BH][8][2048] u64 | state [BH] |
// cut-bin keys [BH][kSelCand] u64 | kept counts [BH][Cq] int32
struct SelScratch {
  size_t hist, state, cand, counts, total;
};
static SelScratch sel_scratch(const bsa_shape& s, int Cq) {
  SelScratch w;
  const size_t bh = (size_t)s.B * s.H;
  w.hist = 0;
  w.state = al256(bh * kHistGroups * kHistBins * sizeof(unsigned long long));
  w.cand = w.state + al256(bh * sizeof(SelState));
  w.counts = w.cand + al256(bh * kSelCand * sizeof(unsigned long long));
  w.total = w.counts + al256(bh * Cq * sizeof(int32_t));
  return w;
}
size_t route_hist_bytes(const bsa_shape& s, int Cq) { return sel_scratch(s, Cq).total; }

ProbePlan probe_plan(const bsa_shape& s, int Cq, int Ck) {
  ProbePlan p;
  const int bh = s.B * s.H;
  const int groups = (Cq + 127) / 128;
  // the fused head_dim-128 kernel addresses a head with 32-bit offsets
  p.fused = s.D == 128 && ((int64_t)s.N + kFpTK) * s.stride_n * 2 < ((int64_t)1 << 31);
  // about 512 workgroups: two resident on each of the 256 compute units (the
  // fused kernel's LDS and registers allow two), rounded down so that no
  // workgroup waits for a second round
  int want = 512 / (bh * groups);
  if (want > Ck) want = Ck;
  if (want < 1) want = 1;
  // the fused kernel balances its splits by key count, the general one by
  // cluster count (cps clusters per split)
  p.cps = (Ck + want - 1) / want;
  p.splits = p.fused ? want : (Ck + p.cps - 1) / p.cps;
  const size_t blocks = (size_t)bh * Cq * Ck;
  p.off_e = 0;
  p.off_m = al256(p.off_e + blocks * 4);
  p.off_ms = al256(p.off_m + blocks * 4);
  p.off_zs = al256(p.off_ms + (size_t)bh * p.splits * Cq * 4);
  p.off_hist = al256(p.off_zs + (size_t)bh * p.splits * Cq * 4);
  p.total = p.off_hist + route_hist_bytes(s, Cq);
  return p;
}

bsa_status launch_route_scores(const void* k, const void* v, const bsa_shape& s, const int32_t* q_off, int Cq,
                               const int32_t* k_off, int Ck, const float* qc, float* kc, float* vc, float scale,
                               float* score, void* ws, hipStream_t stream, uint16_t* kc_bf, uint16_t* vc_bf) {
  const ProbePlan pl = probe_plan(s, Cq, Ck);
  char* w = (char*)ws;
  float* e_buf = (float*)(w + pl.off_e);
  float* m_buf = (float*)(w + pl.off_m);
  float* m_split = (float*)(w + pl.off_ms);
  float* z_split = (float*)(w + pl.off_zs);
  const float c2 = scale * kLog2e;
  dim3 grid(pl.splits, s.B * s.H, (Cq + 127) / 128);
  if (pl.fused) {
    FusedProbeArgs f;
    f.s = svg_args(nullptr, k, v, s, q_off, Cq, k_off, Ck);
    f.q_cent = qc; f.e_buf = e_buf; f.m_buf = m_buf; f.m_split = m_split; f.z_split = z_split;
    f.k_cent = kc; f.v_cent = vc; f.kc_bf = kc_bf; f.vc_bf = vc_bf;
    f.splits = pl.splits; f.c2 = c2;
    hipLaunchKernelGGL(probe_fused_d128_kernel, grid, dim3(256), 0, stream, f);
  } else {
    // the general probe takes the key and value centroids as inputs
    bsa_status st = launch_centroids(nullptr, k, v, s, q_off, Cq, k_off, Ck, nullptr, kc, vc, stream, kCentKey);
    if (st != BSA_OK) return st;
    ProbeArgs p;
    p.s = svg_args(nullptr, k, v, s, q_off, Cq, k_off, Ck);
    p.q_cent = qc; p.k_cent = kc; p.v_cent = vc;
    p.e_buf = e_buf; p.m_buf = m_buf; p.m_split = m_split; p.z_split = z_split;
    p.splits = pl.splits; p.cps = pl.cps; p.c2 = c2;
    if (s.D == 128) hipLaunchKernelGGL(probe_kernel<128>, grid, dim3(256), 0, stream, p);
    else if (s.D == 64) hipLaunchKernelGGL(probe_kernel<64>, grid, dim3(256), 0, stream, p);
    else return BSA_ERR_UNSUPPORTED;
  }
  ScoreHistArgs h{q_off, k_off, e_buf, m_buf, m_split, z_split, score,
                  (unsigned long long*)(w + pl.off_hist), Cq, Ck, pl.splits};
  hipLaunchKernelGGL(score_hist_kernel, dim3(kHistGroups, s.B * s.H), dim3(256), 0, stream, h);
  return launch_ok("route_scores") ? BSA_OK : BSA_ERR_HIP;
}

bsa_status launch_route_select(const float* score, const bsa_shape& s, const int32_t* q_off, int Cq,
                               const int32_t* k_off, int Ck, long long budget, int32_t* rrow, int32_t* rcol,
                               void* scratch, bool hist_ready, hipStream_t stream) {
  const SelScratch w = sel_scratch(s, Cq);
  char* base = (char*)scratch;
  unsigned long long* hs = (unsigned long long*)(base + w.hist);
  const int bh = s.B * s.H;
  if (!hist_ready) {
    ScoreHistArgs h{q_off, k_off, nullptr, nullptr, nullptr, nullptr, (float*)score, hs, Cq, Ck, 0};
    hipLaunchKernelGGL(score_hist_kernel, dim3(kHistGroups, bh), dim3(256), 0, stream, h);
  }
  SelectArgs a{score, q_off, k_off, rrow, rcol, hs, (SelState*)(base + w.state),
               (unsigned long long*)(base + w.cand), (int32_t*)(base + w.counts), Cq, Ck, s.N, budget};
  const dim3 rows((Cq + 3) / 4, bh);
  hipLaunchKernelGGL(select_level1_kernel, dim3(bh), dim3(kSelThreads), 0, stream, a);
  hipLaunchKernelGGL(select_gather_kernel, rows, dim3(256), 0, stream, a);
  hipLaunchKernelGGL(select_resolve_kernel, dim3(bh), dim3(kSelThreads), 0, stream, a);
  hipLaunchKernelGGL(select_count_kernel, rows, dim3(256), 0, stream, a);
  hipLaunchKernelGGL(select_emit_kernel, rows, dim3(256), 0, stream, a);
  return launch_ok("route_select") ? BSA_OK : BSA_ERR_HIP;
}

static bool comp_d128(const bsa_shape& s) {
  return s.D == 128 && ((int64_t)s.N + kCaBN) * s.stride_n * 2 < ((int64_t)1 << 31);
}

// head_dim-128 workspace: bf16 k_cent, bf16 v_cent, per-cluster work and tile
// counts, the tile schedule (item, x) and its length, the run tables
struct CompWs {
  size_t kb, vb, work, ntile, item, x, count, runs, total;
  int cap;  // upper bound of the tiles of all heads
};
static CompWs comp_ws(const bsa_shape& s, int Cq, int Ck) {
  CompWs w;
  const size_t bh = (size_t)s.B * s.H;
  w.cap = (int)(bh * ((s.N + 127) / 128 + Cq));
  w.kb = 0;
  w.vb = al256(bh * Ck * s.D * 2);
  w.work = w.vb + al256(bh * Ck * s.D * 2);
  w.ntile = w.work + al256(bh * Cq * 4);
  w.item = w.ntile + al256(bh * Cq * 4);
  w.x = w.item + al256((size_t)w.cap * 4);
  w.count = w.x + al256((size_t)w.cap * 4);
  w.runs = w.count + 256;
  w.total = w.runs + al256(bh * Cq * Ck * 8);
  return w;
}
size_t comp_attn_workspace(const bsa_shape& s, int Cq, int Ck) {
  if (!comp_d128(s)) return 0;
  return comp_ws(s, Cq, Ck).total;
}

void comp_attn_bf16_slots(const bsa_shape& s, int Cq, int Ck, void* ws, uint16_t** kb, uint16_t** vb) {
  if (!comp_d128(s)) {
    *kb = *vb = nullptr;
    return;
  }
  const CompWs w = comp_ws(s, Cq, Ck);
  *kb = (uint16_t*)((char*)ws + w.kb);
  *vb = (uint16_t*)((char*)ws + w.vb);
}

bsa_status launch_comp_attn(const void* q, const void* k, const void* v, void* o, float* lse, const bsa_shape& s,
                            const int32_t* q_off, int Cq, const int32_t* k_off, int Ck, const int32_t* rrow,
                            const int32_t* rcol, const float* kc, const float* vc, float scale, void* ws,
                            hipStream_t stream, bool bf16_ready) {
  CompArgs p;
  p.s = svg_args(q, k, v, s, q_off, Cq, k_off, Ck);
  p.o = (uint16_t*)o; p.lse = lse; p.rrow = rrow; p.rcol = rcol; p.k_cent = kc; p.v_cent = vc;
  p.scale = scale; p.c2 = scale * kLog2e;
  p.kc_bf = nullptr; p.vc_bf = nullptr; p.runs = nullptr;
  const int max_tiles = (s.N + 127) / 128 + Cq;
  dim3 grid(max_tiles, s.B * s.H);
  if (comp_d128(s)) {
    const CompWs w = comp_ws(s, Cq, Ck);
    char* base = (char*)ws;
    uint16_t* kb = (uint16_t*)(base + w.kb);
    uint16_t* vb = (uint16_t*)(base + w.vb);
    const int64_t n2 = (int64_t)s.B * s.H * Ck * s.D / 2;
    if (!bf16_ready)
      hipLaunchKernelGGL(centroid_bf16_kernel, dim3((unsigned)((n2 + 255) / 256)), dim3(256), 0, stream, kc, vc,
                         kb, vb, n2);
    CompOrderArgs oa{q_off, k_off, rrow, rcol, Cq, Ck, s.B * s.H, w.cap, (int32_t*)(base + w.work),
                     (int32_t*)(base + w.ntile), (int32_t*)(base + w.item), (int32_t*)(base + w.x),
                     (int32_t*)(base + w.count), (int32_t*)(base + w.runs)};
    hipLaunchKernelGGL(comp_steps_kernel, dim3((Cq + 3) / 4, s.B * s.H), dim3(256), 0, stream, oa);
    hipLaunchKernelGGL(comp_order_kernel, dim3(1), dim3(1024), 0, stream, oa);
    p.kc_bf = kb; p.vc_bf = vb;
    p.tile_item = oa.tile_item; p.tile_x = oa.tile_x; p.tile_count = oa.tile_count; p.runs = oa.runs;
    // 1-D grid, a multiple of 24 covering every schedule entry (see the kernel)
    const int wgs = (w.cap + 23) / 24 * 24;
    hipLaunchKernelGGL(comp_attn_d128_kernel, dim3(wgs), dim3(256), 0, stream, p);
  } else if (s.D == 128) {
    hipLaunchKernelGGL(comp_attn_kernel<128>, grid, dim3(256), 0, stream, p);
  } else if (s.D == 64) {
    hipLaunchKernelGGL(comp_attn_kernel<64>, grid, dim3(256), 0, stream, p);
  } else {
    return BSA_ERR_UNSUPPORTED;
  }
  return launch_ok("compensated_attn_fwd") ? BSA_OK : BSA_ERR_HIP;
}

}  // namespace bsa
