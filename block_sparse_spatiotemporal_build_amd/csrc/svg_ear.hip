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
  const int a = blockIdx.x, bh = blockIdx.y;
  __shared__ float mz[2];
  if (threadIdx.x == 0) {
    float m = -1e30f;
    for (int s = 0; s < f.splits; ++s) m = fmaxf(m, f.m_split[((int64_t)bh * f.splits + s) * f.Cq + a]);
    float z = 0.f;
    for (int s = 0; s < f.splits; ++s) {
      const int64_t o = ((int64_t)bh * f.splits + s) * f.Cq + a;
      z += f.z_split[o] * fast_exp2(f.m_split[o] - m);
    }
    mz[0] = m;
    mz[1] = z;
  }
  __syncthreads();
  const float m = mz[0], z = mz[1];
  const int32_t* qo = f.q_off + (int64_t)bh * (f.Cq + 1);
  const int32_t* ko = f.k_off + (int64_t)bh * (f.Ck + 1);
  const int na = qo[a + 1] - qo[a];
  const float inv_z2 = z > 0.f ? 1.f / (z * z) : 0.f;
  for (int b = threadIdx.x; b < f.Ck; b += 256) {
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

constexpr int kSelThreads = 1024;

// Inclusive scan of an int64 over the workgroup (wave shuffles + LDS).
__device__ long long block_scan_incl(long long x, long long* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int off = 1; off < 64; off <<= 1) {
    const long long y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  if (wave == 0) {
    long long t = lane < kSelThreads / 64 ? wsum[lane] : 0;
    for (int off = 1; off < 64; off <<= 1) {
      const long long y = __shfl_up(t, off, 64);
      if (lane >= off) t += y;
    }
    if (lane < kSelThreads / 64) wsum[lane] = t;
  }
  __syncthreads();
  const long long r = x + (wave > 0 ? wsum[wave - 1] : 0);
  __syncthreads();
  return r;
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

__global__ void __launch_bounds__(kSelThreads) select_kernel(SelectArgs s) {
  __shared__ unsigned long long hist[256];
  __shared__ long long wsum[64];
  __shared__ long long sh_R;
  __shared__ unsigned int sh_prefix, sh_mask;
  __shared__ int sh_all;
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int M = s.Cq * s.Ck;
  const float* sc = s.score + (int64_t)bh * M;
  const int32_t* qo = s.q_off + (int64_t)bh * (s.Cq + 1);
  const int32_t* ko = s.k_off + (int64_t)bh * (s.Ck + 1);
  uint8_t* fl = s.flags + (int64_t)bh * M;
  auto cost_of = [&](int e) -> long long {
    const int a = e / s.Ck, b = e % s.Ck;
    return (long long)(qo[a + 1] - qo[a]) * (long long)(ko[b + 1] - ko[b]);
  };

  // total cost of all non-empty blocks
  long long part = 0;
  for (int e = tid; e < M; e += kSelThreads) part += cost_of(e);
  const long long total = block_scan_incl(part, wsum);
  if (tid == kSelThreads - 1) {
    sh_all = total <= s.budget;
    sh_R = s.budget;
    sh_prefix = 0;
    sh_mask = 0;
  }
  __syncthreads();
  const bool take_all = sh_all;

  if (!take_all) {
    // radix select of the threshold bit pattern T, 8 bits at a time
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0;
      __syncthreads();
      const unsigned pre = sh_prefix, msk = sh_mask;
      for (int e = tid; e < M; e += kSelThreads) {
        const long long c = cost_of(e);
        const unsigned bits = __float_as_uint(sc[e]);
        if (c > 0 && (bits & msk) == pre) atomicAdd(&hist[(bits >> shift) & 255u], (unsigned long long)c);
      }
      __syncthreads();
      if (tid == 0) {
        long long acc = 0, R = sh_R;
        int d = 255;
        for (; d > 0; --d) {
          if (acc + (long long)hist[d] > R) break;
          acc += (long long)hist[d];
        }
        sh_R = R - acc;
        sh_prefix = pre | ((unsigned)d << shift);
        sh_mask = msk | (255u << shift);
      }
      __syncthreads();
    }
  }
  const unsigned T = sh_prefix;
  const long long R = sh_R;

  // flags: above the threshold, or in the tie group within the remaining budget (index order)
  long long carry = 0;
  for (int base = 0; base < M; base += kSelThreads) {
    const int e = base + tid;
    long long c = 0;
    unsigned bits = 0;
    if (e < M) {
      c = cost_of(e);
      bits = __float_as_uint(sc[e]);
    }
    const bool tie = !take_all && e < M && c > 0 && bits == T;
    const long long incl = block_scan_incl(tie ? c : 0, wsum);
    if (e < M) {
      bool keep;
      if (take_all) keep = c > 0;
      else keep = c > 0 && (bits > T || (tie && carry + incl <= R));
      fl[e] = keep ? 1 : 0;
    }
    if (tid == kSelThreads - 1) wsum[63] = incl;
    __syncthreads();
    carry += wsum[63];
    __syncthreads();
  }
  __syncthreads();

  // CSR of the kept blocks, columns ascending
  int32_t* rr = s.rrow + (int64_t)bh * (s.Cq + 1);
  int32_t* rc = s.rcol + (int64_t)bh * M;
  long long rowbase = 0;
  for (int a0 = 0; a0 < s.Cq; a0 += kSelThreads) {
    const int a = a0 + tid;
    int cnt = 0;
    if (a < s.Cq)
      for (int b = 0; b < s.Ck; ++b) cnt += fl[a * s.Ck + b];
    const long long incl = block_scan_incl(cnt, wsum);
    const long long start = rowbase + incl - cnt;
    if (a < s.Cq) {
      rr[a] = (int32_t)start;
      int w = (int)start;
      for (int b = 0; b < s.Ck; ++b)
        if (fl[a * s.Ck + b]) rc[w++] = b;
    }
    if (tid == kSelThreads - 1) wsum[63] = incl;
    __syncthreads();
    rowbase += wsum[63];
    __syncthreads();
  }
  if (tid == 0) rr[s.Cq] = (int32_t)rowbase;
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
  int want = (512 + bh * groups - 1) / (bh * groups);
  if (want > Ck) want = Ck;
  if (want < 1) want = 1;
  p.cps = (Ck + want - 1) / want;
  p.splits = (Ck + p.cps - 1) / p.cps;
  const size_t blocks = (size_t)bh * Cq * Ck;
  p.off_e = 0;
  p.off_m = al256(p.off_e + blocks * 4);
  p.off_ms = al256(p.off_m + blocks * 4);
  p.off_zs = al256(p.off_ms + (size_t)bh * p.splits * Cq * 4);
  p.total = al256(p.off_zs + (size_t)bh * p.splits * Cq * 4);
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
  p.e_buf = (float*)(w + pl.off_e); p.m_buf = (float*)(w + pl.off_m);
  p.m_split = (float*)(w + pl.off_ms); p.z_split = (float*)(w + pl.off_zs);
  p.splits = pl.splits; p.cps = pl.cps; p.c2 = scale * kLog2e;
  dim3 grid(pl.splits, s.B * s.H, (Cq + 127) / 128);
  if (s.D == 128) hipLaunchKernelGGL(probe_kernel<128>, grid, dim3(256), 0, stream, p);
  else if (s.D == 64) hipLaunchKernelGGL(probe_kernel<64>, grid, dim3(256), 0, stream, p);
  else return BSA_ERR_UNSUPPORTED;
  FinalizeArgs f{q_off, k_off, p.e_buf, p.m_buf, p.m_split, p.z_split, score, Cq, Ck, pl.splits};
  hipLaunchKernelGGL(probe_finalize_kernel, dim3(Cq, s.B * s.H), dim3(256), 0, stream, f);
  return launch_ok("route_scores") ? BSA_OK : BSA_ERR_HIP;
}

bsa_status launch_route_select(const float* score, const bsa_shape& s, const int32_t* q_off, int Cq,
                               const int32_t* k_off, int Ck, long long budget, int32_t* rrow, int32_t* rcol,
                               uint8_t* flags, hipStream_t stream) {
  SelectArgs a{score, q_off, k_off, rrow, rcol, flags, Cq, Ck, s.N, budget};
  hipLaunchKernelGGL(select_kernel, dim3(s.B * s.H), dim3(kSelThreads), 0, stream, a);
  return launch_ok("route_select") ? BSA_OK : BSA_ERR_HIP;
}

bsa_status launch_comp_attn(const void* q, const void* k, const void* v, void* o, float* lse, const bsa_shape& s,
                            const int32_t* q_off, int Cq, const int32_t* k_off, int Ck, const int32_t* rrow,
                            const int32_t* rcol, const float* kc, const float* vc, float scale,
                            hipStream_t stream) {
  CompArgs p;
  p.s = svg_args(q, k, v, s, q_off, Cq, k_off, Ck);
  p.o = (uint16_t*)o; p.lse = lse; p.rrow = rrow; p.rcol = rcol; p.k_cent = kc; p.v_cent = vc;
  p.scale = scale; p.c2 = scale * kLog2e;
  const int max_tiles = (s.N + 127) / 128 + Cq;
  dim3 grid(max_tiles, s.B * s.H);
  if (s.D == 128) hipLaunchKernelGGL(comp_attn_kernel<128>, grid, dim3(256), 0, stream, p);
  else if (s.D == 64) hipLaunchKernelGGL(comp_attn_kernel<64>, grid, dim3(256), 0, stream, p);
  else return BSA_ERR_UNSUPPORTED;
  return launch_ok("compensated_attn_fwd") ? BSA_OK : BSA_ERR_HIP;
}

}  // namespace bsa
