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

template <int D>
__global__ void __launch_bounds__(256) centroid_kernel(SvgArgs a, float* q_cent, float* k_cent, float* v_cent) {
  constexpr int CH = D / 8, RS = 256 / CH;
  __shared__ float red[2][RS][D];
  const int bh = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
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
  for (int r = r0 + rg; r < r1; r += RS) {
    const u32x4 x = *(const u32x4*)(X + (int64_t)r * a.sn + cc * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      s1[2 * w] += bf16_lo(x[w]);
      s1[2 * w + 1] += bf16_hi(x[w]);
    }
    if (!is_q) {
      const u32x4 y = *(const u32x4*)(V + (int64_t)r * a.sn + cc * 8);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        s2[2 * w] += bf16_lo(y[w]);
        s2[2 * w + 1] += bf16_hi(y[w]);
      }
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
  const float* lc;  // [BH][Ck][Cq] proxy-centroid logits (log2 units), head_dim 128 path
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

// Proxy-centroid logits lc[b][a] = s log2(e) c^_a . c_b in fp32, with c^_a
// taken as the same bf16 hi + lo pair the probe multiplies the keys with, so
// that the centroid weight and the key weights of the difference form share
// one proxy.  A workgroup covers 16 proxies x 64 key clusters; thread
// (a = tid / 16, tx = tid % 16) computes the clusters tx, tx + 16, tx + 32,
// tx + 48 with float4 reads (row stride D + 4 floats: conflict-free).
template <int D>
__global__ void __launch_bounds__(256) proxy_logit_kernel(const float* q_cent, const float* k_cent, float* lc,
                                                          int Cq, int Ck, float c2) {
  constexpr int ST = D + 4;
  __shared__ __attribute__((aligned(16))) float qs[16][ST];
  __shared__ __attribute__((aligned(16))) float ks[64][ST];
  const int bh = blockIdx.z, a0 = blockIdx.y * 16, b0 = blockIdx.x * 64, tid = threadIdx.x;
  for (int i = tid; i < 16 * D / 4; i += 256) {
    const int r = i / (D / 4), d = (i % (D / 4)) * 4;
    const int a = a0 + r;
    float4 x = {0.f, 0.f, 0.f, 0.f};
    if (a < Cq) x = *(const float4*)&q_cent[((int64_t)bh * Cq + a) * D + d];
    float4 y;
    float* xs = &x.x;
    float* ys = &y.x;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float h = bf16_lo(pack_bf16x2(xs[e], 0.f));
      ys[e] = h + bf16_lo(pack_bf16x2(xs[e] - h, 0.f));
    }
    *(float4*)&qs[r][d] = y;
  }
  for (int i = tid; i < 64 * D / 4; i += 256) {
    const int r = i / (D / 4), d = (i % (D / 4)) * 4;
    const int bb = b0 + r;
    float4 x = {0.f, 0.f, 0.f, 0.f};
    if (bb < Ck) x = *(const float4*)&k_cent[((int64_t)bh * Ck + bb) * D + d];
    *(float4*)&ks[r][d] = x;
  }
  __syncthreads();
  const int ty = tid >> 4, tx = tid & 15;
  float dot[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int d = 0; d < D; d += 4) {
    const float4 q = *(const float4*)&qs[ty][d];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 k = *(const float4*)&ks[tx + 16 * j][d];
      dot[j] = __builtin_fmaf(q.x, k.x, dot[j]);
      dot[j] = __builtin_fmaf(q.y, k.y, dot[j]);
      dot[j] = __builtin_fmaf(q.z, k.z, dot[j]);
      dot[j] = __builtin_fmaf(q.w, k.w, dot[j]);
    }
  }
  const int a = a0 + ty;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int bb = b0 + tx + 16 * j;
    if (a < Cq && bb < Ck) lc[((int64_t)bh * Ck + bb) * Cq + a] = dot[j] * c2;
  }
}

// head_dim 128 probe: same computation as probe_kernel, with K/V staged by
// buffer loads straight to LDS (two swizzled stages as separate LDS objects,
// loop unrolled by two), the bf16 lo halves of the proxies in LDS instead of
// registers, the split's cluster offsets and proxy-centroid logits in LDS.
// This keeps two waves per SIMD, so one wave's softmax overlaps the other's
// MFMAs and the copies overlap both.
constexpr int kPrMaxCps = 16;  // clusters per split (the plan keeps cps <= this)

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) probe_d128_kernel(ProbeArgs p) {
  constexpr int D = 128, KT = 8, DT = 4, TILE = kPrBN * D;
  __shared__ __attribute__((aligned(1024))) uint16_t K0[TILE], K1[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t V0[TILE], V1[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t CL[128 * D];  // proxy lo halves, rows swizzled (swz_k)
  __shared__ float lcs[kPrMaxCps][128];
  __shared__ int koffs[kPrMaxCps + 1];

  const SvgArgs& a = p.s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hi = lane >> 5;
  const int split = blockIdx.x, bh = blockIdx.y;
  const int prow = wave * 32 + l32;
  const int prox = blockIdx.z * 128 + prow;  // proxy (query cluster) of this lane
  const bool pvalid = prox < a.Cq;
  const int32_t* koff_g = a.k_off + (int64_t)bh * (a.Ck + 1);
  const uint16_t* Kh = head_ptr(a.k, a, bh);
  const uint16_t* Vh = head_ptr(a.v, a, bh);
  const int b0 = split * p.cps, b1 = min(b0 + p.cps, a.Ck), nclu = b1 - b0;

  // proxy fragments: c^ = hi + lo (bf16 each); hi is the MFMA B operand in
  // registers, lo is read from LDS per tile
  bf16x8 cf[KT];
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
      *(u32x4*)&CL[prow * D + (((2 * t + hi) ^ swz_k(prow)) << 3)] = wl;
    }
  }
  for (int i = tid; i <= nclu; i += 256) koffs[i] = koff_g[b0 + i];
  for (int i = wave; i < nclu; i += 4)
    for (int j = lane; j < 128; j += 64) {
      const int px = blockIdx.z * 128 + j;
      lcs[i][j] = px < a.Cq ? p.lc[((int64_t)bh * a.Ck + b0 + i) * a.Cq + px] : 0.f;
    }
  __syncthreads();
  retire_loads();

  auto ntiles_of = [&](int i) { return (koffs[i + 1] - koffs[i] + kPrBN - 1) / kPrBN; };
  int total = 0;
  for (int i = 0; i < nclu; ++i) total += ntiles_of(i);

  // copy roles: wave w, instruction j covers tile rows 8w + 4j + lane/16
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t row_bytes = (uint32_t)a.sn * 2u;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)Kh, (short)0, 0x7fffffff, kBufferWord3);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)Vh, (short)0, 0x7fffffff, kBufferWord3);
  uint32_t koff[2], voff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = 8 * wv + 4 * j + (lane >> 4);
    koff[j] = (uint32_t)row * row_bytes + (uint32_t)(((lane & 15) ^ swz_k(row)) * 16);
    voff[j] = (uint32_t)row * row_bytes + (uint32_t)(((lane & 15) ^ swz_v(row)) * 16);
  }
  auto dma = [&](uint16_t* kst, uint16_t* vst, int key0, int kend) {
    if (key0 + kPrBN <= kend) {
      const uint32_t so = (uint32_t)key0 * row_bytes;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)&kst[(8 * wv + 4 * j) * D], 16, koff[j], so, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)&vst[(8 * wv + 4 * j) * D], 16, voff[j], so, 0, 0);
      }
    } else {  // last tile of a cluster: rows past its end are clamped to its last key (masked below)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = 8 * wv + 4 * j + (lane >> 4);
        const uint32_t ro = (uint32_t)min(key0 + row, kend - 1) * row_bytes;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)&kst[(8 * wv + 4 * j) * D], 16,
                                                 ro + (uint32_t)(((lane & 15) ^ swz_k(row)) * 16), 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)&vst[(8 * wv + 4 * j) * D], 16,
                                                 ro + (uint32_t)(((lane & 15) ^ swz_v(row)) * 16), 0, 0, 0);
      }
    }
  };

  f32x16 U[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) U[i] = f32x16{};
  float m_run = -1e30f, l_run = 0.f, lc2 = 0.f;
  const int g16 = lane >> 4, j16 = lane & 15;

  // walk state: cluster (local index) and sub-tile of the tile being computed,
  // and the prefetch cursor one tile ahead
  int cb = 0, cst = 0;
  while (cb < nclu && ntiles_of(cb) == 0) ++cb;
  int fb = cb, fst = 0;
  auto advance = [&](int& bb, int& st) {
    ++st;
    if (st >= ntiles_of(bb)) {
      st = 0;
      ++bb;
      while (bb < nclu && ntiles_of(bb) == 0) ++bb;
    }
  };

  auto step = [&](const uint16_t* Kb, const uint16_t* Vb, uint16_t* Kn, uint16_t* Vn, int u) {
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0): tile u landed, other stage drained
    __builtin_amdgcn_s_barrier();
    if (u + 1 < total) {
      dma(Kn, Vn, koffs[fb] + fst * kPrBN, koffs[fb + 1]);
      advance(fb, fst);
    }
    const int kend = koffs[cb + 1];
    const int key0 = koffs[cb] + cst * kPrBN;
    if (cst == 0) {
#pragma unroll
      for (int i = 0; i < DT; ++i) U[i] = f32x16{};
      lc2 = lcs[cb][prow];
    }
    // S^T (32 keys x 32 proxies) = K (c_hi + c_lo)^T
    f32x16 s = f32x16{};
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      const bf16x8 kf = *(const bf16x8*)&Kb[l32 * D + (((2 * t + hi) ^ swz_k(l32)) << 3)];
      const bf16x8 cl = *(const bf16x8*)&CL[prow * D + (((2 * t + hi) ^ swz_k(prow)) << 3)];
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, cf[t], s, 0, 0, 0);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, cl, s, 0, 0, 0);
    }
    if (key0 + kPrBN > kend) {  // key of s[r]: key0 + 8 (r / 4) + 4 hi + r % 4
      const int lim = kend - key0 - 4 * hi;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + (r & 3) >= lim) s[r] = -__builtin_inff();
    }
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    const float m_new = fmaxf(m_run, pair_max(mx) * p.c2);
    if (__any(m_new - m_run > kLazyRescaleLog2)) {
      const float alpha = fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DT; ++i) U[i] *= alpha;
      m_run = m_new;
    }
    // U accumulates sum_j (p_j - p_c) v_j (the difference form)
    const float pc = fast_exp2(lc2 - m_run);
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float pr = fast_exp2(__builtin_fmaf(s[r], p.c2, -m_run));
      psum += pr;
      s[r] = (s[r] == -__builtin_inff()) ? 0.f : pr - pc;
    }
    l_run += psum;
    // P' = hi + lo (bf16 each)
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
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int r0 = ks * 16 + 4 * hi + (j16 >> 2), r1 = r0 + 8;
        const int lcn = 4 * dt + 2 * (g16 & 1) + ((j16 & 3) >> 1);
        const int half = (j16 & 1) * 4;
        const u32x2 lo = lds_tr16(&Vb[r0 * D + ((lcn ^ swz_v(r0)) << 3) + half]);
        const u32x2 h2 = lds_tr16(&Vb[r1 * D + ((lcn ^ swz_v(r1)) << 3) + half]);
        const u32x4 w = {lo[0], lo[1], h2[0], h2[1]};
        const bf16x8 vf = __builtin_bit_cast(bf16x8, w);
        U[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ks], U[dt], 0, 0, 0);
        U[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pl[ks], U[dt], 0, 0, 0);
      }

    if (cst + 1 == ntiles_of(cb)) {
      // cluster finished: squared norm of the accumulated error (at reference m_run)
      float e2 = 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) e2 = __builtin_fmaf(U[dt][r], U[dt][r], e2);
      e2 = pair_sum(e2);
      if (pvalid && hi == 0) {
        const int64_t o = ((int64_t)bh * a.Cq + prox) * a.Ck + b0 + cb;
        p.e_buf[o] = e2;
        p.m_buf[o] = m_run;
      }
      cst = 0;
      ++cb;
      while (cb < nclu && ntiles_of(cb) == 0) ++cb;
    } else {
      ++cst;
    }
  };

  if (total > 0) {
    dma(K0, V0, koffs[fb] + fst * kPrBN, koffs[fb + 1]);
    advance(fb, fst);
  }
  int u = 0;
  for (; u + 2 <= total; u += 2) {
    step(K0, V0, K1, V1, u);
    step(K1, V1, K0, V0, u + 1);
  }
  if (u < total) step(K0, V0, K1, V1, u);

  const float z = pair_sum(l_run);
  if (pvalid && hi == 0) {
    p.m_split[((int64_t)bh * p.splits + split) * a.Cq + prox] = m_run;
    p.z_split[((int64_t)bh * p.splits + split) * a.Cq + prox] = z;
  }
}

struct FinalizeArgs {
  const int32_t* q_off;
  const int32_t* k_off;
  const float* e_buf;
  const float* m_buf;
  const float* m_split;
  const float* z_split;
  float* score;  // [BH][Cq][Ck]
  int Cq, Ck, splits;
};

__global__ void __launch_bounds__(256) probe_finalize_kernel(FinalizeArgs f) {
  const int a = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  __shared__ float mz[2];
  if (tid < 64) {
    // combine the splits' (max, normaliser) pairs of proxy a, one wave
    float m = -1e30f;
    for (int s = lane; s < f.splits; s += 64) m = fmaxf(m, f.m_split[((int64_t)bh * f.splits + s) * f.Cq + a]);
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    float z = 0.f;
    for (int s = lane; s < f.splits; s += 64) {
      const int64_t o = ((int64_t)bh * f.splits + s) * f.Cq + a;
      z += f.z_split[o] * fast_exp2(f.m_split[o] - m);
    }
    for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off, 64);
    if (lane == 0) {
      mz[0] = m;
      mz[1] = z;
    }
  }
  __syncthreads();
  const float m = mz[0], z = mz[1];
  const int32_t* qo = f.q_off + (int64_t)bh * (f.Cq + 1);
  const int32_t* ko = f.k_off + (int64_t)bh * (f.Ck + 1);
  const int na = qo[a + 1] - qo[a];
  const float inv_z2 = z > 0.f ? 1.f / (z * z) : 0.f;
  for (int b = tid; b < f.Ck; b += 256) {
    const int nb = ko[b + 1] - ko[b];
    const int64_t o = ((int64_t)bh * f.Cq + a) * f.Ck + b;
    float sc = 0.f;
    if (na > 0 && nb > 0) sc = f.e_buf[o] * fast_exp2(2.f * (f.m_buf[o] - m)) * inv_z2 / (float)nb;
    f.score[o] = sc;
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

struct SelectArgs {
  const float* score;   // [BH][Cq][Ck]
  const int32_t* q_off;
  const int32_t* k_off;
  int32_t* rrow;        // [BH][Cq+1]
  int32_t* rcol;        // [BH][Cq*Ck]
  uint8_t* flags;       // [BH][Cq*Ck] workspace
  int Cq, Ck, N;
  long long budget;
};

// One workgroup per (batch, head).  Blocks are ranked by (score descending,
// index a * Ck + b ascending); the kept set is the longest prefix of that order
// whose total cost n_a n_b fits the budget.  Non-negative floats order like
// their bit patterns, so the cut is a threshold pattern T found by a
// cost-weighted radix select (4 passes of 8 bits, one histogram per wave):
// every block above T is kept, and blocks equal to T are kept in index order
// while the remaining budget lasts.  Wave w owns the contiguous rows
// [w * rpw, (w + 1) * rpw), so index order is wave order, then row order, then
// column order.
__global__ void __launch_bounds__(kSelThreads) select_kernel(SelectArgs s) {
  __shared__ unsigned long long hist[kSelWaves][256];
  __shared__ unsigned long long htot[256];
  __shared__ long long wred[kSelWaves];
  __shared__ int nbk[kSelMaxCk];
  __shared__ int wcnt[kSelWaves];
  __shared__ unsigned wmin[kSelWaves], wmax[kSelWaves];
  __shared__ long long sh_R;
  __shared__ unsigned int sh_prefix;
  const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Cq = s.Cq, Ck = s.Ck;
  const int64_t M = (int64_t)Cq * Ck;
  const unsigned* sc = (const unsigned*)(s.score + (int64_t)bh * M);
  const int32_t* qo = s.q_off + (int64_t)bh * (Cq + 1);
  const int32_t* ko = s.k_off + (int64_t)bh * (Ck + 1);
  uint8_t* fl = s.flags + (int64_t)bh * M;
  int32_t* rr = s.rrow + (int64_t)bh * (Cq + 1);
  int32_t* rc = s.rcol + (int64_t)bh * M;

  const bool nb_lds = Ck <= kSelMaxCk;
  if (nb_lds)
    for (int b = tid; b < Ck; b += kSelThreads) nbk[b] = ko[b + 1] - ko[b];
  __syncthreads();
  auto nb_of = [&](int b) -> int { return nb_lds ? nbk[b] : ko[b + 1] - ko[b]; };
  const int rpw = (Cq + kSelWaves - 1) / kSelWaves;
  const int ra0 = min(wave * rpw, Cq), ra1 = min(ra0 + rpw, Cq);

  // total cost of all non-empty blocks, and the range of their score bits
  long long part = 0;
  unsigned bmin = 0xffffffffu, bmax = 0u;
  for (int a = ra0; a < ra1; ++a) {
    const long long na = qo[a + 1] - qo[a];
    if (na == 0) continue;
    const unsigned* row = sc + (int64_t)a * Ck;
    for (int b0 = 0; b0 < Ck; b0 += 64 * kSelBatch) {
      unsigned bits[kSelBatch];
#pragma unroll
      for (int j = 0; j < kSelBatch; ++j) {
        const int b = b0 + 64 * j + lane;
        bits[j] = b < Ck ? row[b] : 0u;
      }
#pragma unroll
      for (int j = 0; j < kSelBatch; ++j) {
        const int b = b0 + 64 * j + lane;
        const int nbv = b < Ck ? nb_of(b) : 0;
        if (nbv > 0) {
          part += na * nbv;
          bmin = min(bmin, bits[j]);
          bmax = max(bmax, bits[j]);
        }
      }
    }
  }
  part = wave_sum64(part);
  for (int off = 32; off > 0; off >>= 1) {
    bmin = min(bmin, (unsigned)__shfl_xor((int)bmin, off, 64));
    bmax = max(bmax, (unsigned)__shfl_xor((int)bmax, off, 64));
  }
  if (lane == 0) {
    wred[wave] = part;
    wmin[wave] = bmin;
    wmax[wave] = bmax;
  }
  __syncthreads();
  long long total = 0;
  unsigned gmin = 0xffffffffu, gmax = 0u;
  for (int w = 0; w < kSelWaves; ++w) {
    total += wred[w];
    gmin = min(gmin, wmin[w]);
    gmax = max(gmax, wmax[w]);
  }
  const bool take_all = total <= s.budget;

  unsigned T = 0;
  long long R = s.budget;
  if (!take_all) {
    // every counted block shares the leading bits where gmin and gmax agree,
    // so the digits start right below them (the first digit is then spread
    // over many bins instead of piling onto one)
    const int lead = gmin == gmax ? 32 : __clz((int)(gmin ^ gmax));
    unsigned msk = lead == 0 ? 0u : (lead == 32 ? 0xffffffffu : ~0u << (32 - lead));
    unsigned pre = gmin & msk;
    for (int low = 32 - lead; low > 0;) {
      const int width = min(8, low);
      const int shift = low - width;
      const unsigned dmask = (1u << width) - 1u;
      low = shift;
      for (int i = lane; i < 256; i += 64) hist[wave][i] = 0;
      __builtin_amdgcn_wave_barrier();
      for (int a = ra0; a < ra1; ++a) {
        const long long na = qo[a + 1] - qo[a];
        if (na == 0) continue;
        const unsigned* row = sc + (int64_t)a * Ck;
        for (int b0 = 0; b0 < Ck; b0 += 64 * kSelBatch) {
          // the batch's loads are independent of the atomics below, so they are
          // all in flight together instead of one memory latency per element
          unsigned bits[kSelBatch];
#pragma unroll
          for (int j = 0; j < kSelBatch; ++j) {
            const int b = b0 + 64 * j + lane;
            bits[j] = b < Ck ? row[b] : 0u;
          }
#pragma unroll
          for (int j = 0; j < kSelBatch; ++j) {
            const int b = b0 + 64 * j + lane;
            const int nbv = b < Ck ? nb_of(b) : 0;
            const bool in = nbv > 0 && (bits[j] & msk) == pre;
            const unsigned dig = (bits[j] >> shift) & dmask;
            const unsigned long long inb = __ballot(in);
            if (inb == 0) continue;
            const unsigned d0 = (unsigned)__shfl((int)dig, __ffsll((long long)inb) - 1, 64);
            if (__ballot(in && dig == d0) == inb) {
              // the whole batch element falls into one bin: one atomic for the wave
              const long long c = wave_sum64(in ? na * nbv : 0);
              if (lane == 0) atomicAdd(&hist[wave][d0], (unsigned long long)c);
            } else if (in) {
              atomicAdd(&hist[wave][dig], (unsigned long long)(na * nbv));
            }
          }
        }
      }
      __syncthreads();
      if (tid < 256) {
        unsigned long long t = 0;
        for (int w = 0; w < kSelWaves; ++w) t += hist[w][tid];
        htot[tid] = t;
      }
      __syncthreads();
      if (wave == 0) {
        // lane l holds digits 4l .. 4l+3; the cut digit d is the first one from
        // the top where the cost of the digits above stays within R but adding
        // d's own cost exceeds it (digit 0 if none does)
        unsigned long long h[4], own = 0;
        for (int i = 0; i < 4; ++i) {
          h[i] = htot[4 * lane + i];
          own += h[i];
        }
        long long above = (long long)own;  // becomes: cost of all digits held by higher lanes
        for (int off = 1; off < 64; off <<= 1) {
          const long long y = __shfl_down(above, off, 64);
          if (lane + off < 64) above += y;
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
    T = pre;
  }

  // keep flags; ties at T in index order within the remaining budget
  long long tc = 0;
  if (!take_all)
    for (int a = ra0; a < ra1; ++a) {
      const long long na = qo[a + 1] - qo[a];
      if (na == 0) continue;
      const unsigned* row = sc + (int64_t)a * Ck;
      for (int b0 = 0; b0 < Ck; b0 += 64 * kSelBatch) {
        unsigned bits[kSelBatch];
#pragma unroll
        for (int j = 0; j < kSelBatch; ++j) {
          const int b = b0 + 64 * j + lane;
          bits[j] = b < Ck ? row[b] : 0u;
        }
#pragma unroll
        for (int j = 0; j < kSelBatch; ++j) {
          const int b = b0 + 64 * j + lane;
          const int nbv = b < Ck ? nb_of(b) : 0;
          if (nbv > 0 && bits[j] == T) tc += na * nbv;
        }
      }
    }
  tc = wave_sum64(tc);
  if (lane == 0) wred[wave] = tc;
  __syncthreads();
  long long carry = 0;
  for (int w = 0; w < wave; ++w) carry += wred[w];
  int wave_kept = 0;
  for (int a = ra0; a < ra1; ++a) {
    const long long na = qo[a + 1] - qo[a];
    const unsigned* row = sc + (int64_t)a * Ck;
    unsigned bits_b[kSelBatch];
    for (int b0 = 0; b0 < Ck; b0 += 64) {
      const int jb = (b0 / 64) % kSelBatch;
      if (jb == 0) {
#pragma unroll
        for (int j = 0; j < kSelBatch; ++j) {
          const int bb = b0 + 64 * j + lane;
          bits_b[j] = bb < Ck ? row[bb] : 0u;
        }
      }
      const int b = b0 + lane;
      const bool valid = b < Ck;
      const long long c = valid ? na * nb_of(b) : 0;
      unsigned bits = 0u;
#pragma unroll
      for (int j = 0; j < kSelBatch; ++j)
        if (j == jb) bits = bits_b[j];
      const bool tie = !take_all && c > 0 && bits == T;
      long long incl = 0;
      if (__any(tie)) incl = wave_incl_scan64(tie ? c : 0, lane);
      const bool keep = take_all ? c > 0 : (c > 0 && (bits > T || (tie && carry + incl <= R)));
      carry += __shfl(incl, 63, 64);
      if (valid) fl[(int64_t)a * Ck + b] = keep ? 1 : 0;
      wave_kept += __popcll(__ballot(keep));
    }
  }
  if (lane == 0) wcnt[wave] = wave_kept;
  __syncthreads();
  // CSR: wave w's rows start after the blocks kept by waves < w; columns
  // ascending, 64 at a time with ballots (each lane re-reads only flags it wrote)
  int start = 0;
  for (int w = 0; w < wave; ++w) start += wcnt[w];
  if (tid == 0) rr[0] = 0;
  for (int a = ra0; a < ra1; ++a) {
    for (int b0 = 0; b0 < Ck; b0 += 64 * kSelBatch) {
      bool keep[kSelBatch];
#pragma unroll
      for (int j = 0; j < kSelBatch; ++j) {
        const int b = b0 + 64 * j + lane;
        keep[j] = b < Ck && fl[(int64_t)a * Ck + b] != 0;
      }
#pragma unroll
      for (int j = 0; j < kSelBatch; ++j) {
        const int b = b0 + 64 * j + lane;
        const unsigned long long bal = __ballot(keep[j]);
        if (keep[j]) rc[start + __popcll(bal & ((1ull << lane) - 1ull))] = b;
        start += __popcll(bal);
      }
    }
    if (lane == 0) rr[a + 1] = start;
  }
}

// Register-resident form of select_kernel for Cq <= 16 * kSrRows and
// Ck <= 64 * kSrCpl: the same selection and the same CSR, with every score of
// the head loaded once into registers (lane l of wave w holds the columns
// 64 c + l of its rows ra0 + r) and every pass run from there, instead of
// re-reading the scores from memory in each radix pass.
constexpr int kSrRows = 8, kSrCpl = 8;

__global__ void __launch_bounds__(kSelThreads) select_reg_kernel(SelectArgs s) {
  __shared__ unsigned long long hist[kSelWaves][256];
  __shared__ unsigned long long htot[256];
  __shared__ long long wred[kSelWaves];
  __shared__ int wcnt[kSelWaves];
  __shared__ unsigned wmin[kSelWaves], wmax[kSelWaves];
  __shared__ long long sh_R;
  __shared__ unsigned int sh_prefix;
  __shared__ int nbk[64 * kSrCpl];
  const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Cq = s.Cq, Ck = s.Ck;
  const int64_t M = (int64_t)Cq * Ck;
  const unsigned* sc = (const unsigned*)(s.score + (int64_t)bh * M);
  const int32_t* qo = s.q_off + (int64_t)bh * (Cq + 1);
  const int32_t* ko = s.k_off + (int64_t)bh * (Ck + 1);
  int32_t* rr = s.rrow + (int64_t)bh * (Cq + 1);
  int32_t* rc = s.rcol + (int64_t)bh * M;
  const int rpw = (Cq + kSelWaves - 1) / kSelWaves;
  const int ra0 = min(wave * rpw, Cq), nrow = min(ra0 + rpw, Cq) - ra0;

  // scores in registers; key-cluster sizes in LDS (read at each use, so the
  // compiler does not keep 64 per-lane costs live across the passes)
  unsigned sb[kSrRows][kSrCpl];
  int nar[kSrRows];
  for (int b = tid; b < 64 * kSrCpl; b += kSelThreads) nbk[b] = b < Ck ? ko[b + 1] - ko[b] : 0;
#pragma unroll
  for (int r = 0; r < kSrRows; ++r) nar[r] = r < nrow ? qo[ra0 + r + 1] - qo[ra0 + r] : 0;
#pragma unroll
  for (int r = 0; r < kSrRows; ++r)
#pragma unroll
    for (int c = 0; c < kSrCpl; ++c) {
      const int b = 64 * c + lane;
      sb[r][c] = (r < nrow && b < Ck) ? sc[(int64_t)(ra0 + r) * Ck + b] : 0u;
    }
  __syncthreads();
  auto cost = [&](int r, int c) -> long long { return (long long)nar[r] * nbk[64 * c + lane]; };

  // total cost of the non-empty blocks and the range of their score bits
  long long part = 0;
  unsigned bmin = 0xffffffffu, bmax = 0u;
#pragma unroll
  for (int r = 0; r < kSrRows; ++r)
#pragma unroll
    for (int c = 0; c < kSrCpl; ++c) {
      const long long w = cost(r, c);
      if (w > 0) {
        part += w;
        bmin = min(bmin, sb[r][c]);
        bmax = max(bmax, sb[r][c]);
      }
    }
  part = wave_sum64(part);
  for (int off = 32; off > 0; off >>= 1) {
    bmin = min(bmin, (unsigned)__shfl_xor((int)bmin, off, 64));
    bmax = max(bmax, (unsigned)__shfl_xor((int)bmax, off, 64));
  }
  if (lane == 0) {
    wred[wave] = part;
    wmin[wave] = bmin;
    wmax[wave] = bmax;
  }
  __syncthreads();
  long long total = 0;
  unsigned gmin = 0xffffffffu, gmax = 0u;
  for (int w = 0; w < kSelWaves; ++w) {
    total += wred[w];
    gmin = min(gmin, wmin[w]);
    gmax = max(gmax, wmax[w]);
  }
  const bool take_all = total <= s.budget;

  unsigned T = 0;
  long long R = s.budget;
  if (!take_all) {
    // digits start below the leading bits shared by every counted score
    const int lead = gmin == gmax ? 32 : __clz((int)(gmin ^ gmax));
    unsigned msk = lead == 0 ? 0u : (lead == 32 ? 0xffffffffu : ~0u << (32 - lead));
    unsigned pre = gmin & msk;
    for (int low = 32 - lead; low > 0;) {
      const int width = min(8, low);
      const int shift = low - width;
      const unsigned dmask = (1u << width) - 1u;
      low = shift;
      for (int i = lane; i < 256; i += 64) hist[wave][i] = 0;
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int r = 0; r < kSrRows; ++r)
#pragma unroll
        for (int c = 0; c < kSrCpl; ++c) {
          const long long w = cost(r, c);
          const bool in = w > 0 && (sb[r][c] & msk) == pre;
          const unsigned dig = (sb[r][c] >> shift) & dmask;
          const unsigned long long inb = __ballot(in);
          if (inb == 0) continue;
          const unsigned d0 = (unsigned)__shfl((int)dig, __ffsll((long long)inb) - 1, 64);
          if (__ballot(in && dig == d0) == inb) {
            const long long cw = wave_sum64(in ? w : 0);
            if (lane == 0) atomicAdd(&hist[wave][d0], (unsigned long long)cw);
          } else if (in) {
            atomicAdd(&hist[wave][dig], (unsigned long long)w);
          }
        }
      __syncthreads();
      if (tid < 256) {
        unsigned long long t = 0;
        for (int w = 0; w < kSelWaves; ++w) t += hist[w][tid];
        htot[tid] = t;
      }
      __syncthreads();
      if (wave == 0) {
        // lane l holds digits 4l .. 4l+3; the cut digit is the first from the
        // top whose own cost takes the cost above it past R (digit 0 if none)
        unsigned long long h[4], own = 0;
        for (int i = 0; i < 4; ++i) {
          h[i] = htot[4 * lane + i];
          own += h[i];
        }
        long long above = (long long)own;
        for (int off = 1; off < 64; off <<= 1) {
          const long long y = __shfl_down(above, off, 64);
          if (lane + off < 64) above += y;
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
    T = pre;
  }

  // cost of the ties at T held by each wave, for the index-order carry
  long long tc = 0;
  if (!take_all)
#pragma unroll
    for (int r = 0; r < kSrRows; ++r)
#pragma unroll
      for (int c = 0; c < kSrCpl; ++c) {
        const long long w = cost(r, c);
        if (w > 0 && sb[r][c] == T) tc += w;
      }
  tc = wave_sum64(tc);
  if (lane == 0) wred[wave] = tc;
  __syncthreads();
  long long carry = 0;
  for (int w = 0; w < wave; ++w) carry += wred[w];
  // keep decisions in index order (row, then column), packed one bit each
  unsigned long long keepm = 0;
  int wave_kept = 0;
#pragma unroll
  for (int r = 0; r < kSrRows; ++r)
#pragma unroll
    for (int c = 0; c < kSrCpl; ++c) {
      const long long w = cost(r, c);
      const bool tie = !take_all && w > 0 && sb[r][c] == T;
      long long incl = 0;
      if (__any(tie)) incl = wave_incl_scan64(tie ? w : 0, lane);
      const bool keep = take_all ? w > 0 : (w > 0 && (sb[r][c] > T || (tie && carry + incl <= R)));
      carry += __shfl(incl, 63, 64);
      if (keep) keepm |= 1ull << (r * kSrCpl + c);
      wave_kept += __popcll(__ballot(keep));
    }
  if (lane == 0) wcnt[wave] = wave_kept;
  __syncthreads();
  // CSR: wave w's rows start after the blocks kept by waves < w
  int start = 0;
  for (int w = 0; w < wave; ++w) start += wcnt[w];
  if (tid == 0) rr[0] = 0;
#pragma unroll
  for (int r = 0; r < kSrRows; ++r) {
    if (r >= nrow) break;
#pragma unroll
    for (int c = 0; c < kSrCpl; ++c) {
      const bool keep = (keepm >> (r * kSrCpl + c)) & 1ull;
      const unsigned long long bal = __ballot(keep);
      if (keep) rc[start + __popcll(bal & ((1ull << lane) - 1ull))] = 64 * c + lane;
      start += __popcll(bal);
    }
    if (lane == 0) rr[ra0 + r + 1] = start;
  }
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
};

// one wave per (head, cluster): E_a from the route row (indices clamped like the
// attention kernel clamps them)
__global__ void __launch_bounds__(256) comp_steps_kernel(CompOrderArgs o) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int bh = blockIdx.y, ca = blockIdx.x * 4 + wave;
  if (ca >= o.Cq) return;
  const int32_t* qo = o.q_off + (int64_t)bh * (o.Cq + 1);
  const int32_t* ko = o.k_off + (int64_t)bh * (o.Ck + 1);
  const int rb = max(0, min(o.rrow[(int64_t)bh * (o.Cq + 1) + ca], o.Cq * o.Ck));
  const int nk = max(0, min(o.rrow[(int64_t)bh * (o.Cq + 1) + ca + 1] - rb, min(o.Ck, o.Cq * o.Ck - rb)));
  const int32_t* cl = o.rcol + (int64_t)bh * o.Cq * o.Ck + rb;
  int e = 0;
  for (int i = lane; i < nk; i += 64) {
    const int b = max(0, min(cl[i], o.Ck - 1));
    e += ko[b + 1] - ko[b];
  }
  for (int off = 32; off > 0; off >>= 1) e += __shfl_xor(e, off, 64);
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
// the concatenated keys of the kept clusters of the row's query cluster (each
// staged row is gathered: slot -> kept cluster through a per-lane cursor over
// the kept-size prefix cum[], -> key row); sub-tiles u >= ne hold the virtual
// keys, one per key cluster b (bf16 centroid rows), whose logit gets the bias
// ln(n_b) / scale, or -inf when b is kept or empty.
constexpr int kCaMaxCk = 512;

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
comp_attn_d128_kernel(CompArgs p) {
  constexpr int D = 128, KT = 8, DT = 4, TILE = kCaBN * D;
  __shared__ __attribute__((aligned(1024))) uint16_t K0[TILE], K1[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t V0[TILE], V1[TILE];
  __shared__ int cum[kCaMaxCk + 1];    // prefix of kept cluster sizes
  __shared__ int kstart[kCaMaxCk];     // first key row of each kept cluster
  __shared__ float bias[kCaMaxCk];     // virtual-key logit bias (raw units) or -inf
  __shared__ int scan[256];

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
  for (int b = tid; b < a.Ck; b += 256) {
    const int n = ko[b + 1] - ko[b];
    bias[b] = n > 0 ? __logf((float)n) / p.scale : -__builtin_inff();
  }
  // prefix of kept sizes: thread t holds entries 2t, 2t + 1 (nk <= 512)
  int sz[2] = {0, 0};
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int i = 2 * tid + e;
    if (i < nk) {
      const int b = max(0, min(cl[i], a.Ck - 1));
      sz[e] = ko[b + 1] - ko[b];
      kstart[i] = ko[b];
    }
  }
  scan[tid] = sz[0] + sz[1];
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int add = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += add;
    __syncthreads();
  }
  {
    const int ex = scan[tid] - sz[0] - sz[1];
    if (2 * tid < nk) cum[2 * tid] = ex;
    if (2 * tid + 1 < nk) cum[2 * tid + 1] = ex + sz[0];
    if (tid == 255) cum[nk] = scan[255];
  }
  __syncthreads();
  for (int i = tid; i < nk; i += 256) bias[max(0, min(cl[i], a.Ck - 1))] = -__builtin_inff();
  const int E = __builtin_amdgcn_readfirstlane(cum[nk]);
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
  __syncthreads();  // cum, kstart and bias complete

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
  // a lane stages rows 16w + 4j + lane/16 (j = 0..3): increasing slots, so one
  // cursor (kept-list index of the cluster holding the slot) serves all four.
  // For those rows swz_k(row) = 4j + lane/16 and swz_v(row) = 4 (lane/16) + j,
  // so the swizzled chunk offsets are one per-lane base XOR an immediate.
  // The cursor's cluster bounds and first key row are kept in registers and
  // reloaded from LDS only when the cursor moves (about once per sub-tile),
  // so issuing a sub-tile's copies costs few LDS round trips.
  int cur = 0, c_lo = 0, c_hi = nk > 0 ? cum[1] : 0, k_lo = nk > 0 ? kstart[0] : 0;
  const uint32_t kbase = (uint32_t)(((lane & 15) ^ (lane >> 4)) * 16);
  const uint32_t vbase = (uint32_t)(((lane & 15) ^ (4 * (lane >> 4))) * 16);
  auto dma = [&](uint16_t* kst, uint16_t* vst, int u) {
    if (u < ne) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = 16 * wv + 4 * j + (lane >> 4);
        const int slot = min(u * kCaBN + row, E - 1);  // slots past E are masked below
        while (cur + 1 < nk && c_hi <= slot) {
          ++cur;
          c_lo = c_hi;
          c_hi = cum[cur + 1];
          k_lo = kstart[cur];
        }
        const uint32_t ro = (uint32_t)(k_lo + slot - c_lo) * row_bytes;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)&kst[(16 * wv + 4 * j) * D], 16,
                                                 ro + (kbase ^ (64u * j)), 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)&vst[(16 * wv + 4 * j) * D], 16,
                                                 ro + (vbase ^ (16u * j)), 0, 0, 0);
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
      const int bb = (u - ne) * kCaBN + 4 * hi;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int b = bb + kt * 32 + 8 * (r >> 2) + (r & 3);
          s[kt][r] = b < a.Ck ? s[kt][r] + bias[b] : -__builtin_inff();
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
    float psum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = fast_exp2(__builtin_fmaf(s[kt][r], c2, -mc));
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
                            hipStream_t stream) {
  SvgArgs a = svg_args(q, k, v, s, q_off, Cq, k_off, Ck);
  dim3 grid(Cq + Ck, s.B * s.H);
  if (s.D == 128) hipLaunchKernelGGL(centroid_kernel<128>, grid, dim3(256), 0, stream, a, qc, kc, vc);
  else if (s.D == 64) hipLaunchKernelGGL(centroid_kernel<64>, grid, dim3(256), 0, stream, a, qc, kc, vc);
  else return BSA_ERR_UNSUPPORTED;
  return launch_ok("cluster_centroids") ? BSA_OK : BSA_ERR_HIP;
}


static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

ProbePlan probe_plan(const bsa_shape& s, int Cq, int Ck) {
  ProbePlan p;
  const int bh = s.B * s.H;
  const int groups = (Cq + 127) / 128;
  // the head_dim-128 kernel addresses a head with 32-bit offsets
  p.d128 = s.D == 128 && ((int64_t)s.N + kPrBN) * s.stride_n * 2 < ((int64_t)1 << 31);
  int want = (512 + bh * groups - 1) / (bh * groups);
  if (want > Ck) want = Ck;
  if (want < 1) want = 1;
  p.cps = (Ck + want - 1) / want;
  if (p.d128 && p.cps > kPrMaxCps) p.cps = kPrMaxCps;
  p.splits = (Ck + p.cps - 1) / p.cps;
  const size_t blocks = (size_t)bh * Cq * Ck;
  p.off_e = 0;
  p.off_m = al256(p.off_e + blocks * 4);
  p.off_ms = al256(p.off_m + blocks * 4);
  p.off_zs = al256(p.off_ms + (size_t)bh * p.splits * Cq * 4);
  p.off_lc = al256(p.off_zs + (size_t)bh * p.splits * Cq * 4);
  p.total = al256(p.off_lc + (p.d128 ? blocks * 4 : 0));
  return p;
}

bsa_status launch_route_scores(const void* k, const void* v, const bsa_shape& s, const int32_t* q_off, int Cq,
                               const int32_t* k_off, int Ck, const float* qc, const float* kc, const float* vc,
                               float scale, float* score, void* ws, hipStream_t stream) {
  const ProbePlan pl = probe_plan(s, Cq, Ck);
  char* w = (char*)ws;
  ProbeArgs p;
  p.s = svg_args(nullptr, k, v, s, q_off, Cq, k_off, Ck);
  p.q_cent = qc; p.k_cent = kc; p.v_cent = vc;
  p.lc = pl.d128 ? (const float*)(w + pl.off_lc) : nullptr;
  p.e_buf = (float*)(w + pl.off_e); p.m_buf = (float*)(w + pl.off_m);
  p.m_split = (float*)(w + pl.off_ms); p.z_split = (float*)(w + pl.off_zs);
  p.splits = pl.splits; p.cps = pl.cps; p.c2 = scale * kLog2e;
  dim3 grid(pl.splits, s.B * s.H, (Cq + 127) / 128);
  if (pl.d128) {
    hipLaunchKernelGGL(proxy_logit_kernel<128>, dim3((Ck + 63) / 64, (Cq + 15) / 16, s.B * s.H), dim3(256), 0,
                       stream, qc, kc, (float*)(w + pl.off_lc), Cq, Ck, p.c2);
    hipLaunchKernelGGL(probe_d128_kernel, grid, dim3(256), 0, stream, p);
  } else if (s.D == 128) {
    hipLaunchKernelGGL(probe_kernel<128>, grid, dim3(256), 0, stream, p);
  } else if (s.D == 64) {
    hipLaunchKernelGGL(probe_kernel<64>, grid, dim3(256), 0, stream, p);
  } else {
    return BSA_ERR_UNSUPPORTED;
  }
  FinalizeArgs f{q_off, k_off, p.e_buf, p.m_buf, p.m_split, p.z_split, score, Cq, Ck, pl.splits};
  hipLaunchKernelGGL(probe_finalize_kernel, dim3(Cq, s.B * s.H), dim3(256), 0, stream, f);
  return launch_ok("route_scores") ? BSA_OK : BSA_ERR_HIP;
}

bsa_status launch_route_select(const float* score, const bsa_shape& s, const int32_t* q_off, int Cq,
                               const int32_t* k_off, int Ck, long long budget, int32_t* rrow, int32_t* rcol,
                               uint8_t* flags, hipStream_t stream) {
  SelectArgs a{score, q_off, k_off, rrow, rcol, flags, Cq, Ck, s.N, budget};
  if (Cq <= kSelWaves * kSrRows && Ck <= 64 * kSrCpl)
    hipLaunchKernelGGL(select_reg_kernel, dim3(s.B * s.H), dim3(kSelThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(select_kernel, dim3(s.B * s.H), dim3(kSelThreads), 0, stream, a);
  return launch_ok("route_select") ? BSA_OK : BSA_ERR_HIP;
}

static bool comp_d128(const bsa_shape& s) {
  return s.D == 128 && ((int64_t)s.N + kCaBN) * s.stride_n * 2 < ((int64_t)1 << 31);
}

// head_dim-128 workspace: bf16 k_cent, bf16 v_cent, per-cluster work and tile
// counts, the tile schedule (item, x) and its length
struct CompWs {
  size_t kb, vb, work, ntile, item, x, count, total;
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
  w.total = w.count + 256;
  return w;
}
size_t comp_attn_workspace(const bsa_shape& s, int Cq, int Ck) {
  if (!comp_d128(s)) return 0;
  return comp_ws(s, Cq, Ck).total;
}

bsa_status launch_comp_attn(const void* q, const void* k, const void* v, void* o, float* lse, const bsa_shape& s,
                            const int32_t* q_off, int Cq, const int32_t* k_off, int Ck, const int32_t* rrow,
                            const int32_t* rcol, const float* kc, const float* vc, float scale, void* ws,
                            hipStream_t stream) {
  CompArgs p;
  p.s = svg_args(q, k, v, s, q_off, Cq, k_off, Ck);
  p.o = (uint16_t*)o; p.lse = lse; p.rrow = rrow; p.rcol = rcol; p.k_cent = kc; p.v_cent = vc;
  p.scale = scale; p.c2 = scale * kLog2e;
  p.kc_bf = nullptr; p.vc_bf = nullptr;
  const int max_tiles = (s.N + 127) / 128 + Cq;
  dim3 grid(max_tiles, s.B * s.H);
  if (comp_d128(s)) {
    const CompWs w = comp_ws(s, Cq, Ck);
    char* base = (char*)ws;
    uint16_t* kb = (uint16_t*)(base + w.kb);
    uint16_t* vb = (uint16_t*)(base + w.vb);
    const int64_t n2 = (int64_t)s.B * s.H * Ck * s.D / 2;
    hipLaunchKernelGGL(centroid_bf16_kernel, dim3((unsigned)((n2 + 255) / 256)), dim3(256), 0, stream, kc, vc, kb,
                       vb, n2);
    CompOrderArgs oa{q_off, k_off, rrow, rcol, Cq, Ck, s.B * s.H, w.cap, (int32_t*)(base + w.work),
                     (int32_t*)(base + w.ntile), (int32_t*)(base + w.item), (int32_t*)(base + w.x),
                     (int32_t*)(base + w.count)};
    hipLaunchKernelGGL(comp_steps_kernel, dim3((Cq + 3) / 4, s.B * s.H), dim3(256), 0, stream, oa);
    hipLaunchKernelGGL(comp_order_kernel, dim3(1), dim3(1024), 0, stream, oa);
    p.kc_bf = kb; p.vc_bf = vb;
    p.tile_item = oa.tile_item; p.tile_x = oa.tile_x; p.tile_count = oa.tile_count;
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
