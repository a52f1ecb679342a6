// Token clustering for gfx950: k-means (Lloyd) of the token rows of every
// (batch, head), the stable cluster order, and row gather / scatter through it.
//
// Operation ("SVG-EAR: Parameter-Free Linear Compensation for Sparse Video
// Generation via Error-aware Routing", technical summary section 2 Method:
// query and key tokens are grouped into clusters by similarity before the
// cluster-block routing): from given centres, `iters` Lloyd steps (assign each
// token to the nearest centre, move each centre to the mean of its tokens; a
// centre without tokens stays), then a final assignment to the final centres.
// Ties go to the lowest centre index.  The assignment compares
// |c_b|^2 - 2 x . c_b with c_b the centre rounded to bf16: x . c_b is an fp32
// MFMA accumulation of exact bf16 products, |c_b|^2 is fp32.  The means are
// fp32 sums divided by the count (a fixed summation order: row group g sums
// rows g, g + 16, ... of the cluster in order, then the 16 group sums are added
// in group order).
//
// One Lloyd step is four launches, all deterministic:
//   assign : grid (256-token tiles, B*H).  Each wave holds 64 tokens as MFMA B
//            operands; the bf16 centres stream through LDS in 32-row chunks
//            (buffer loads one chunk ahead); S^T = C_chunk X^T with
//            32x32x16 MFMA, then a per-lane running (distance, index) minimum
//            over the lane's 16 centres per chunk (the chunk minimum first, the
//            index only where it improves), and one exchange between
//            the two lane halves at the end.  Labels go to global memory and a
//            per-tile label histogram (LDS integer atomics) to the workspace.
//   scan   : one workgroup per sequence: per cluster, the exclusive prefix of
//            the tile histograms in tile order, and the cluster offsets.
//   place  : one workgroup per tile: the stable rank of each token among the
//            equal labels of its tile (a 64-lane compare inside each wave and
//            per-wave label counts in LDS), giving its position in the cluster
//            order.
//   update : one workgroup per cluster: 16 row groups x 16 chunks of 8 dims
//            sum the cluster's rows (every 16th row in cluster order, fp32,
//            16-byte loads), the group sums are added in group order and
//            divided by the count; the
//            fp32 centre, its bf16 copy and |c_b|^2 go out for the next
//            assignment.

#include "launch.h"

namespace bsa {

constexpr int kKmTile = 256;  // tokens per assignment / placement tile

struct KmAssignArgs {
  const uint16_t* x;  // [B, H, N, D] with strides
  int64_t sb, sh, sn;
  int H, N, C, Cp, tiles;
  const uint16_t* cb;  // [BH][Cp][D] bf16 centres (rows >= C are zero)
  const float* cn;     // [BH][Cp] |c_b|^2 (+inf for rows >= C)
  int32_t* labels;     // [BH][N]
  int32_t* hist;       // [BH][tiles][C]
};

__device__ __forceinline__ const uint16_t* km_row(const uint16_t* x, int64_t sb, int64_t sh, int64_t sn, int H,
                                                  int bh, int n) {
  return x + (int64_t)(bh / H) * sb + (int64_t)(bh % H) * sh + (int64_t)n * sn;
}

__global__ void __launch_bounds__(256) km_assign_d128_kernel(KmAssignArgs a) {
  constexpr int D = 128, CH = 32 * D;  // one chunk: 32 centres
  __shared__ __attribute__((aligned(1024))) uint16_t S0[CH], S1[CH];
  __shared__ int hcnt[kMaxKmClusters];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hi = lane >> 5;
  const int tile = blockIdx.x, bh = blockIdx.y;
  const int nk = a.Cp / 32;
  const int wv = __builtin_amdgcn_readfirstlane(wave);

  for (int i = tid; i < a.C; i += 256) hcnt[i] = 0;

  // the wave's two 32-token B operands: token l32, head dims 16 t + 8 hi .. + 7
  bf16x8 xf[2][8];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int n = min(tile * kKmTile + 64 * wave + 32 * u + l32, a.N - 1);
    const uint16_t* src = km_row(a.x, a.sb, a.sh, a.sn, a.H, bh, n) + 8 * hi;
#pragma unroll
    for (int t = 0; t < 8; ++t) xf[u][t] = *(const bf16x8*)(src + 16 * t);
  }

  // chunk copies: wave w, instruction j stages centre rows 8 w + 4 j + lane / 16
  // of the chunk, 16-byte piece lane % 16 at its swizzled place
  const uint16_t* cbh = a.cb + (int64_t)bh * a.Cp * D;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)cbh, (short)0, a.Cp * D * 2, kBufferWord3);
  uint32_t off[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = 8 * wv + 4 * j + (lane >> 4);
    off[j] = (uint32_t)row * (D * 2) + (uint32_t)(((lane & 15) ^ swz_k(row)) * 16);
  }
  auto dma = [&](uint16_t* st, int k) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)&st[(8 * wv + 4 * j) * D], 16, off[j],
                                               (uint32_t)k * (32 * D * 2), 0, 0);
  };
  const float* cnh = a.cn + (int64_t)bh * a.Cp;

  float best[2] = {__builtin_inff(), __builtin_inff()};
  int bidx[2] = {0, 0};
  // one chunk: distances of the lane's 16 centres (32 k + 8 g + 4 hi + j) to its two tokens
  auto step = [&](const uint16_t* st, uint16_t* nxt, int k) {
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0): chunk k landed
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // the norms first: waiting for them then does not wait for the next chunk's copy
    f32x4 cq[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) cq[g] = *(const f32x4*)&cnh[32 * k + 8 * g + 4 * hi];
    if (k + 1 < nk) dma(nxt, k + 1);
    f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const bf16x8 cf = *(const bf16x8*)&st[l32 * D + (((2 * t + hi) ^ swz_k(l32)) << 3)];
#pragma unroll
      for (int u = 0; u < 2; ++u) s[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cf, xf[u][t], s[u], 0, 0, 0);
    }
    // the chunk's minimum first; only a lane that improves looks for its index
    // (the lowest of equal distances: the lane's centres rise with r)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float d[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) d[r] = __builtin_fmaf(-2.f, s[u][r], cq[r >> 2][r & 3]);
      float m = d[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) m = fminf(m, d[r]);
      if (m < best[u]) {
        int ix = 15;
#pragma unroll
        for (int r = 14; r >= 0; --r) ix = d[r] == m ? r : ix;
        best[u] = m;
        bidx[u] = 32 * k + 8 * (ix >> 2) + 4 * hi + (ix & 3);
      }
    }
  };
  dma(S0, 0);
  int k = 0;
  for (; k + 2 <= nk; k += 2) {
    step(S0, S1, k);
    step(S1, S0, k + 1);
  }
  if (k < nk) step(S0, S1, k);

  // the two halves of the wave saw different centres of the same tokens:
  // smaller distance wins, the lower index on equal distances
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const auto pb = __builtin_amdgcn_permlane32_swap(__float_as_uint(best[u]), __float_as_uint(best[u]), false, false);
    const auto pi = __builtin_amdgcn_permlane32_swap((uint32_t)bidx[u], (uint32_t)bidx[u], false, false);
    const float ob = __uint_as_float(hi ? pb[0] : pb[1]);
    const int oi = (int)(hi ? pi[0] : pi[1]);
    if (ob < best[u] || (ob == best[u] && oi < bidx[u])) bidx[u] = oi;
  }
  __syncthreads();  // hcnt zeroed
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int n = tile * kKmTile + 64 * wave + 32 * u + l32;
    if (hi == 0 && n < a.N) {
      a.labels[(int64_t)bh * a.N + n] = bidx[u];
      atomicAdd(&hcnt[bidx[u]], 1);
    }
  }
  __syncthreads();
  int32_t* hrow = a.hist + ((int64_t)bh * a.tiles + tile) * a.C;
  for (int i = tid; i < a.C; i += 256) hrow[i] = hcnt[i];
}

struct KmOrderArgs {
  const int32_t* labels;  // [BH][N]
  const int32_t* hist;    // [BH][tiles][C] label counts per tile
  int32_t* tbase;         // [BH][tiles][C] exclusive prefix over tiles, per cluster
  int32_t* off;           // [BH][C + 1]
  int32_t* perm;          // [BH][N]
  int N, C, tiles;
};

// one workgroup of kMaxKmClusters threads per sequence.  Thread (g, c), c < C,
// g < G (G = the largest power of two with G * C <= kMaxKmClusters) covers
// cluster c over the g-th of G contiguous tile ranges: it sums that range, the
// range sums give its start, and a second pass writes the running tile bases
// (eight loads in flight in both passes)
__device__ __forceinline__ int km_sum_tiles(const int32_t* __restrict__ h, int C, int t0, int t1) {
  int run = 0, t = t0;
  for (; t + 8 <= t1; t += 8) {
    int v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = h[(int64_t)(t + u) * C];
#pragma unroll
    for (int u = 0; u < 8; ++u) run += v[u];
  }
  for (; t < t1; ++t) run += h[(int64_t)t * C];
  return run;
}

__global__ void __launch_bounds__(kMaxKmClusters) km_scan_kernel(KmOrderArgs a) {
  __shared__ int sc[kMaxKmClusters];
  __shared__ int part[kMaxKmClusters];
  const int tid = threadIdx.x, bh = blockIdx.x;
  int G = 1;
  while (2 * G * a.C <= kMaxKmClusters) G *= 2;
  const int g = tid / a.C, c = tid - g * a.C;
  const bool act = g < G;
  const int t0 = act ? (int)((int64_t)a.tiles * g / G) : 0, t1 = act ? (int)((int64_t)a.tiles * (g + 1) / G) : 0;
  const int32_t* __restrict__ h = a.hist + (int64_t)bh * a.tiles * a.C + c;
  int32_t* __restrict__ tb = a.tbase + (int64_t)bh * a.tiles * a.C + c;
  if (act) part[tid] = km_sum_tiles(h, a.C, t0, t1);
  __syncthreads();
  int run = 0, total = 0;
  if (act) {
    for (int q = 0; q < G; ++q) {
      const int v = part[q * a.C + c];
      run += q < g ? v : 0;
      total += v;
    }
    int t = t0;
    for (; t + 8 <= t1; t += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = h[(int64_t)(t + u) * a.C];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        tb[(int64_t)(t + u) * a.C] = run;
        run += v[u];
      }
    }
    for (; t < t1; ++t) {
      const int v = h[(int64_t)t * a.C];
      tb[(int64_t)t * a.C] = run;
      run += v;
    }
  }
  // inclusive scan of the cluster counts (Hillis-Steele in LDS, thread c)
  const int cnt_c = tid < a.C ? total : 0;
  sc[tid] = cnt_c;
  __syncthreads();
  for (int d = 1; d < kMaxKmClusters; d <<= 1) {
    const int v = tid >= d ? sc[tid - d] : 0;
    __syncthreads();
    sc[tid] += v;
    __syncthreads();
  }
  int32_t* o = a.off + (int64_t)bh * (a.C + 1);
  if (tid < a.C) o[tid] = sc[tid] - cnt_c;
  if (tid == a.C - 1) o[a.C] = sc[tid];
}

// one workgroup per tile, wave b placing tokens 64 b .. 64 b + 63 of the tile:
// the tile's bases (cluster offset + earlier tiles) are staged in LDS, each
// wave counts its labels, and a token's position adds the counts of the
// earlier waves and its rank among the equal labels of its own wave
__global__ void __launch_bounds__(256) km_place_kernel(KmOrderArgs a) {
  __shared__ int base[kMaxKmClusters];
  __shared__ int cnt[4][kMaxKmClusters];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, tile = blockIdx.x, bh = blockIdx.y;
  const int32_t* tb = a.tbase + ((int64_t)bh * a.tiles + tile) * a.C;
  const int32_t* o = a.off + (int64_t)bh * (a.C + 1);
  for (int i = tid; i < a.C; i += 256) {
    base[i] = o[i] + tb[i];
    cnt[0][i] = cnt[1][i] = cnt[2][i] = cnt[3][i] = 0;
  }
  const int n = tile * kKmTile + 64 * wave + lane;
  const int l = n < a.N ? a.labels[(int64_t)bh * a.N + n] : -1;
  int rank = 0;
  for (int j = 0; j < 64; ++j) {
    const int lj = __builtin_amdgcn_readlane(l, j);
    rank += (j < lane && lj == l) ? 1 : 0;
  }
  __syncthreads();
  if (l >= 0) atomicAdd(&cnt[wave][l], 1);
  __syncthreads();
  if (l >= 0) {
    int pos = base[l] + rank;
    for (int w = 0; w < wave; ++w) pos += cnt[w][l];
    a.perm[(int64_t)bh * a.N + pos] = n;
  }
}

struct KmUpdateArgs {
  const uint16_t* x;
  int64_t sb, sh, sn;
  int H, N, C, Cp;
  const int32_t* perm;  // [BH][N]
  const int32_t* off;   // [BH][C + 1]
  float* cent;          // [BH][C][D] fp32 centres (in: current, out: updated)
  uint16_t* cb;         // [BH][Cp][D]
  float* cn;            // [BH][Cp]
};

__device__ __forceinline__ void km_store_centre(const KmUpdateArgs& a, int bh, int c, int lane, float m0, float m1) {
  constexpr int D = 128;
  *(f32x2*)&a.cent[((int64_t)bh * a.C + c) * D + 2 * lane] = f32x2{m0, m1};
  const uint32_t w = pack_bf16x2(m0, m1);
  *(uint32_t*)&a.cb[((int64_t)bh * a.Cp + c) * D + 2 * lane] = w;
  float q = bf16_lo(w) * bf16_lo(w) + bf16_hi(w) * bf16_hi(w);
  for (int s = 32; s > 0; s >>= 1) q += __shfl_xor(q, s, 64);
  if (lane == 0) a.cn[(int64_t)bh * a.Cp + c] = q;
}

// the bf16 copy and norm of given fp32 centres, one wave per centre (rows
// C..Cp-1 are padding: zero, and an infinite norm so they never win)
__global__ void __launch_bounds__(256) km_prepare_d128_kernel(KmUpdateArgs a) {
  constexpr int D = 128;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = blockIdx.x * 4 + wave, bh = blockIdx.y;
  if (c >= a.Cp) return;
  if (c >= a.C) {
    *(uint32_t*)&a.cb[((int64_t)bh * a.Cp + c) * D + 2 * lane] = 0u;
    if (lane == 0) a.cn[(int64_t)bh * a.Cp + c] = __builtin_inff();
    return;
  }
  const f32x2 old = *(const f32x2*)&a.cent[((int64_t)bh * a.C + c) * D + 2 * lane];
  km_store_centre(a, bh, c, lane, old[0], old[1]);
}

// one workgroup per cluster: thread (row group g = tid / 16, chunk cc =
// tid % 16) sums head dims 8 cc .. 8 cc + 7 of the cluster's rows g, g + 16,
// g + 32, ... in order (16-byte loads, four rows in flight); the 16 row-group
// sums are then added in group order and divided by the count
__global__ void __launch_bounds__(256) km_update_d128_kernel(KmUpdateArgs a) {
  constexpr int D = 128;
  __shared__ __attribute__((aligned(16))) float part[16][D];
  const int tid = threadIdx.x, cc = tid & 15, g = tid >> 4;
  const int c = blockIdx.x, bh = blockIdx.y;
  const int32_t* o = a.off + (int64_t)bh * (a.C + 1);
  const int i0 = o[c], i1 = o[c + 1];
  if (i1 == i0) {  // empty: the centre stays (its bf16 copy and norm are current)
    return;
  }
  const int32_t* perm = a.perm + (int64_t)bh * a.N;
  const uint16_t* xh = a.x + (int64_t)(bh / a.H) * a.sb + (int64_t)(bh % a.H) * a.sh + 8 * cc;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int i = i0 + g; i < i1; i += 64) {
    u32x4 w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      w[u] = i + 16 * u < i1 ? *(const u32x4*)(xh + (int64_t)perm[i + 16 * u] * a.sn) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += bf16_lo(w[u][e]);
        acc[2 * e + 1] += bf16_hi(w[u][e]);
      }
  }
  *(f32x4*)&part[g][8 * cc] = f32x4{acc[0], acc[1], acc[2], acc[3]};
  *(f32x4*)&part[g][8 * cc + 4] = f32x4{acc[4], acc[5], acc[6], acc[7]};
  __syncthreads();
  if (tid >= 64) return;
  float t0 = 0.f, t1 = 0.f;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    t0 += part[q][2 * tid];
    t1 += part[q][2 * tid + 1];
  }
  const float n = (float)(i1 - i0);
  km_store_centre(a, bh, c, tid, t0 / n, t1 / n);
}

// ---- row gather / scatter through a permutation ------------------------------

struct RowPermArgs {
  const uint8_t* src;
  uint8_t* dst;
  int64_t sb, sh, sn;  // bytes
  int H, N, chunks;    // 16-byte chunks per row
  const int32_t* perm; // [BH][N]
  int scatter;         // 0: dst[i] = src[perm[i]]; 1: dst[perm[i]] = src[i]
};

// one thread per 16-byte chunk of an output row (consecutive threads walk a
// row's chunks, then the next row); perm entries outside [0, N) are skipped
__global__ void __launch_bounds__(256) rows_permute_kernel(RowPermArgs a) {
  const int64_t item = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int bh = blockIdx.y;
  const int i = (int)(item / a.chunks), ch = (int)(item % a.chunks);
  if (i >= a.N) return;
  const int p = a.perm[(int64_t)bh * a.N + i];
  if (p < 0 || p >= a.N) return;
  const int64_t head = (int64_t)(bh / a.H) * a.sb + (int64_t)(bh % a.H) * a.sh;
  const int si = a.scatter ? i : p, di = a.scatter ? p : i;
  const u32x4 v = ((const u32x4*)(a.src + head + (int64_t)si * a.sn))[ch];
  ((u32x4*)(a.dst + head + (int64_t)di * a.sn))[ch] = v;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

static size_t km_align(size_t x) { return (x + 255) & ~(size_t)255; }

KmPlan kmeans_plan(const bsa_shape& s, int C) {
  KmPlan p;
  const size_t bh = (size_t)s.B * s.H;
  p.Cp = (C + 31) / 32 * 32;
  p.tiles = (s.N + kKmTile - 1) / kKmTile;
  p.off_cb = 0;
  p.off_cn = km_align(p.off_cb + bh * p.Cp * 128 * 2);
  p.off_hist = km_align(p.off_cn + bh * p.Cp * 4);
  p.off_tbase = km_align(p.off_hist + bh * p.tiles * C * 4);
  p.off_perm = km_align(p.off_tbase + bh * p.tiles * C * 4);
  p.off_off = km_align(p.off_perm + bh * s.N * 4);
  p.total = km_align(p.off_off + bh * (C + 1) * 4);
  return p;
}

bsa_status launch_kmeans(const void* x, const bsa_shape& s, int C, int iters, float* cent, int32_t* labels,
                         int32_t* perm, int32_t* offsets, void* ws, hipStream_t stream) {
  const KmPlan p = kmeans_plan(s, C);
  char* w = (char*)ws;
  const int bh = s.B * s.H;
  uint16_t* cb = (uint16_t*)(w + p.off_cb);
  float* cn = (float*)(w + p.off_cn);
  int32_t* hist = (int32_t*)(w + p.off_hist);
  int32_t* tbase = (int32_t*)(w + p.off_tbase);
  if (!perm) perm = (int32_t*)(w + p.off_perm);
  if (!offsets) offsets = (int32_t*)(w + p.off_off);
  KmAssignArgs aa{(const uint16_t*)x, s.stride_b, s.stride_h, s.stride_n, s.H, s.N, C, p.Cp, p.tiles,
                  cb, cn, labels, hist};
  KmOrderArgs oa{labels, hist, tbase, offsets, perm, s.N, C, p.tiles};
  KmUpdateArgs ua{(const uint16_t*)x, s.stride_b, s.stride_h, s.stride_n, s.H, s.N, C, p.Cp, perm, offsets,
                  cent, cb, cn};
  hipLaunchKernelGGL(km_prepare_d128_kernel, dim3((p.Cp + 3) / 4, bh), dim3(256), 0, stream, ua);
  for (int t = 0; t <= iters; ++t) {
    hipLaunchKernelGGL(km_assign_d128_kernel, dim3(p.tiles, bh), dim3(256), 0, stream, aa);
    hipLaunchKernelGGL(km_scan_kernel, dim3(bh), dim3(kMaxKmClusters), 0, stream, oa);
    hipLaunchKernelGGL(km_place_kernel, dim3(p.tiles, bh), dim3(256), 0, stream, oa);
    if (t < iters) hipLaunchKernelGGL(km_update_d128_kernel, dim3(C, bh), dim3(256), 0, stream, ua);
  }
  return launch_ok("kmeans") ? BSA_OK : BSA_ERR_HIP;
}

bsa_status launch_rows_permute(const void* src, const bsa_shape& s, int elem_bytes, const int32_t* perm, void* dst,
                               bool scatter, hipStream_t stream) {
  RowPermArgs a{(const uint8_t*)src, (uint8_t*)dst, s.stride_b * elem_bytes, s.stride_h * elem_bytes,
                s.stride_n * elem_bytes, s.H, s.N, s.D * elem_bytes / 16, perm, scatter ? 1 : 0};
  const int64_t items = (int64_t)s.N * a.chunks;
  hipLaunchKernelGGL(rows_permute_kernel, dim3((unsigned)((items + 255) / 256), s.B * s.H), dim3(256), 0, stream, a);
  return launch_ok(scatter ? "scatter_rows" : "gather_rows") ? BSA_OK : BSA_ERR_HIP;
}

}  // namespace bsa
