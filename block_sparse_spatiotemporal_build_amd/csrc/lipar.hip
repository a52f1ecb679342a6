// Latent inter-frame pruning and restoration for gfx950.
//
// Operation ("LIPAR: 비디오 생성 AI 를 위한 '스마트 스킵' 기술", section 2
// Methodology, B. LIPAR pipeline: latent inter-frame pruning and restoration):
// token n = f * P + p of a sequence is patch p of frame f.  A token of frame
// f >= 1 is kept iff sum_c |x[f, p, c] - x[f - 1, p, c]| > tau * D; frame 0 is
// always kept.  The pruned sequence holds the kept rows in token order.
// Restoration writes every token of the full sequence: a kept token from its
// pruned row, a pruned token from the restored row of (f - 1, p).
//
// The difference sum is taken in fp64 from the exact fp32 widening of the bf16
// values: for inputs within a normal exponent range it has no rounding at all,
// so the keep decision does not depend on the summation order.
//
// Launches:
//   flag    : one wave per patch walks its frames in order, holding the previous
//             frame's row in registers (each row is read once; the next two
//             frames' loads are in flight while a frame is reduced).
//   count   : kept tokens per 1024-token block.
//   scan    : one workgroup per sequence: block offsets and the kept count.
//   compact : per block, the position of every token among the kept ones
//             (ballots, in token order) and the kept-token list.
//   gather  : one wave per pruned row copies its token's row.
//   restore : one wave per output row finds its source frame (the latest kept
//             frame of its patch, from the flags) and copies that pruned row.

#include "launch.h"

namespace bsa {

constexpr int kLpBlock = 1024;      // tokens per count / compact block

struct LiparArgs {
  const uint16_t* x;   // [B, H, N, D] with strides
  int64_t sb, sh, sn;
  int H, N, D, F, P, nblk;
  double thr;          // tau * D
  uint8_t* keep;       // [BH][N]
  int32_t* cpos;       // [BH][N]: kept tokens before n
  int32_t* kidx;       // [BH][N]: token of pruned row j
  int32_t* nkept;      // [BH]
  uint16_t* xp;        // [BH][N][D] pruned rows (dense)
  int32_t* bcount;     // [BH][nblk] workspace
  int32_t* boff;       // [BH][nblk] workspace
};

__device__ __forceinline__ const uint16_t* lp_row(const LiparArgs& a, int bh, int n) {
  return a.x + (int64_t)(bh / a.H) * a.sb + (int64_t)(bh % a.H) * a.sh + (int64_t)n * a.sn;
}

// CPL = 16-byte chunks per lane (D <= 512 CPL); two frames in flight ahead of
// the one being reduced
template <int CPL>
__global__ void __launch_bounds__(256) lipar_flag_kernel(LiparArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int bh = blockIdx.y, p = blockIdx.x * 4 + wave;
  if (p >= a.P) return;
  const int nch = a.D / 8;  // 16-byte chunks per row
  auto load = [&](int f, u32x4 (&r)[CPL]) {
    const u32x4* src = (const u32x4*)lp_row(a, bh, min(f, a.F - 1) * a.P + p);
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = i * 64 + lane;
      r[i] = c < nch ? src[c] : u32x4{0, 0, 0, 0};
    }
  };
  uint8_t* keep = a.keep + (int64_t)bh * a.N;
  u32x4 prev[CPL], cur[CPL], n1[CPL], n2[CPL];
  load(0, prev);
  load(1, cur);
  load(2, n1);
  if (lane == 0) keep[p] = 1;
  for (int f = 1; f < a.F; ++f) {
    load(f + 2, n2);  // frames past the end re-read the last frame (unused)
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < CPL; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float d0 = bf16_lo(cur[i][e]) - bf16_lo(prev[i][e]);
        const float d1 = bf16_hi(cur[i][e]) - bf16_hi(prev[i][e]);
        s += (double)fabsf(d0) + (double)fabsf(d1);
      }
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    if (lane == 0) keep[f * a.P + p] = s > a.thr ? 1 : 0;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      prev[i] = cur[i];
      cur[i] = n1[i];
      n1[i] = n2[i];
    }
  }
}

__global__ void __launch_bounds__(256) lipar_count_kernel(LiparArgs a) {
  __shared__ int wsum[4];
  const int bh = blockIdx.y, blk = blockIdx.x, tid = threadIdx.x;
  const uint8_t* keep = a.keep + (int64_t)bh * a.N;
  int c = 0;
  for (int n = blk * kLpBlock + tid; n < min((blk + 1) * kLpBlock, a.N); n += 256) c += keep[n];
  for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off, 64);
  if ((tid & 63) == 0) wsum[tid >> 6] = c;
  __syncthreads();
  if (tid == 0) a.bcount[bh * a.nblk + blk] = wsum[0] + wsum[1] + wsum[2] + wsum[3];
}

// exclusive prefix of the block counts of one sequence (1024 threads, nblk <= 1024 * 64)
__global__ void __launch_bounds__(1024) lipar_scan_kernel(LiparArgs a) {
  __shared__ int part[1024];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int per = (a.nblk + 1023) / 1024;
  const int b0 = min(tid * per, a.nblk), b1 = min(b0 + per, a.nblk);
  const int32_t* cnt = a.bcount + (int64_t)bh * a.nblk;
  int s = 0;
  for (int b = b0; b < b1; ++b) s += cnt[b];
  part[tid] = s;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int add = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  int run = part[tid] - s;
  for (int b = b0; b < b1; ++b) {
    a.boff[(int64_t)bh * a.nblk + b] = run;
    run += cnt[b];
  }
  if (tid == 1023) a.nkept[bh] = part[1023];
}

// positions in token order and the copy of kept rows (4 waves; wave w takes the
// 64-token chunks w, w + 4, ... of the block, offsets from a per-chunk prefix)
__global__ void __launch_bounds__(256) lipar_compact_kernel(LiparArgs a) {
  __shared__ int chunk_cnt[kLpBlock / 64];
  const int bh = blockIdx.y, blk = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint8_t* keep = a.keep + (int64_t)bh * a.N;
  const int n0 = blk * kLpBlock;
  constexpr int NCH = kLpBlock / 64;
  bool kc[NCH / 4];
  unsigned long long bal[NCH / 4];
#pragma unroll
  for (int i = 0; i < NCH / 4; ++i) {
    const int n = n0 + (i * 4 + wave) * 64 + lane;
    kc[i] = n < a.N && keep[n] != 0;
    bal[i] = __ballot(kc[i]);
    if (lane == 0) chunk_cnt[i * 4 + wave] = __popcll(bal[i]);
  }
  __syncthreads();
  const int base = a.boff[(int64_t)bh * a.nblk + blk];
  int32_t* cpos = a.cpos + (int64_t)bh * a.N;
  int32_t* kidx = a.kidx + (int64_t)bh * a.N;
#pragma unroll
  for (int i = 0; i < NCH / 4; ++i) {
    const int ch = i * 4 + wave;
    int before = 0;
    for (int c = 0; c < ch; ++c) before += chunk_cnt[c];
    const int n = n0 + ch * 64 + lane;
    const int r = before + __popcll(bal[i] & ((1ull << lane) - 1ull));
    if (n < a.N) cpos[n] = base + r;
    if (kc[i]) kidx[base + r] = n;
  }
}

// the kept rows into the pruned sequence: one wave per pruned row slot
__global__ void __launch_bounds__(256) lipar_gather_kernel(LiparArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int bh = blockIdx.y, j = blockIdx.x * 4 + wave;
  if (j >= a.nkept[bh]) return;
  const int n = a.kidx[(int64_t)bh * a.N + j];
  const u32x4* src = (const u32x4*)lp_row(a, bh, n);
  u32x4* dst = (u32x4*)(a.xp + ((int64_t)bh * a.N + j) * a.D);
  const int nch = a.D / 8;
  for (int c = lane; c < nch; c += 64) dst[c] = src[c];
}

struct LiparRestoreArgs {
  const uint16_t* y;       // [BH][N][D] pruned rows (dense)
  const uint8_t* keep;     // [BH][N]
  const int32_t* cpos;     // [BH][N]
  uint16_t* o;             // [B, H, N, D] with strides
  int64_t sb, sh, sn;
  int H, N, D, F, P;
};

// one wave per output row (f, p): the source is the latest frame g <= f in which
// patch p was kept (frame 0 always is)
__global__ void __launch_bounds__(256) lipar_restore_kernel(LiparRestoreArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int bh = blockIdx.y, n = blockIdx.x * 4 + wave;
  if (n >= a.N) return;
  const uint8_t* keep = a.keep + (int64_t)bh * a.N;
  int g = n;
  while (g >= a.P && !keep[g]) g -= a.P;  // uniform over the wave
  const int j = a.cpos[(int64_t)bh * a.N + g];
  const u32x4* src = (const u32x4*)(a.y + ((int64_t)bh * a.N + j) * a.D);
  u32x4* dst = (u32x4*)(a.o + (int64_t)(bh / a.H) * a.sb + (int64_t)(bh % a.H) * a.sh + (int64_t)n * a.sn);
  const int nch = a.D / 8;
  for (int c = lane; c < nch; c += 64) dst[c] = src[c];
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

size_t lipar_workspace(const bsa_shape& s) {
  const size_t nblk = (size_t)(s.N + kLpBlock - 1) / kLpBlock;
  const size_t one = ((size_t)s.B * s.H * nblk * 4 + 255) / 256 * 256;  // block counts, then offsets
  return 2 * one;
}

bsa_status launch_lipar_prune(const void* x, const bsa_shape& s, int frames, float tau, uint8_t* keep,
                              int32_t* cpos, int32_t* kept_idx, int32_t* n_kept, void* x_pruned, void* ws,
                              hipStream_t stream) {
  LiparArgs a;
  a.x = (const uint16_t*)x; a.sb = s.stride_b; a.sh = s.stride_h; a.sn = s.stride_n;
  a.H = s.H; a.N = s.N; a.D = s.D; a.F = frames; a.P = s.N / frames;
  a.nblk = (s.N + kLpBlock - 1) / kLpBlock;
  a.thr = (double)tau * (double)s.D;
  a.keep = keep; a.cpos = cpos; a.kidx = kept_idx; a.nkept = n_kept; a.xp = (uint16_t*)x_pruned;
  const size_t half = lipar_workspace(s) / 2;
  a.bcount = (int32_t*)ws;
  a.boff = (int32_t*)((char*)ws + half);
  const int bh = s.B * s.H;
  const dim3 pg((a.P + 3) / 4, bh);
  const int cpl = (s.D / 8 + 63) / 64;
  if (cpl <= 1) hipLaunchKernelGGL(lipar_flag_kernel<1>, pg, dim3(256), 0, stream, a);
  else if (cpl <= 2) hipLaunchKernelGGL(lipar_flag_kernel<2>, pg, dim3(256), 0, stream, a);
  else if (cpl <= 4) hipLaunchKernelGGL(lipar_flag_kernel<4>, pg, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(lipar_flag_kernel<8>, pg, dim3(256), 0, stream, a);
  hipLaunchKernelGGL(lipar_count_kernel, dim3(a.nblk, bh), dim3(256), 0, stream, a);
  hipLaunchKernelGGL(lipar_scan_kernel, dim3(bh), dim3(1024), 0, stream, a);
  hipLaunchKernelGGL(lipar_compact_kernel, dim3(a.nblk, bh), dim3(256), 0, stream, a);
  hipLaunchKernelGGL(lipar_gather_kernel, dim3((s.N + 3) / 4, bh), dim3(256), 0, stream, a);
  return launch_ok("lipar_prune") ? BSA_OK : BSA_ERR_HIP;
}

bsa_status launch_lipar_restore(const void* y_pruned, const bsa_shape& s, int frames, const uint8_t* keep,
                                const int32_t* cpos, void* out, hipStream_t stream) {
  LiparRestoreArgs a;
  a.y = (const uint16_t*)y_pruned; a.keep = keep; a.cpos = cpos; a.o = (uint16_t*)out;
  a.sb = s.stride_b; a.sh = s.stride_h; a.sn = s.stride_n;
  a.H = s.H; a.N = s.N; a.D = s.D; a.F = frames; a.P = s.N / frames;
  hipLaunchKernelGGL(lipar_restore_kernel, dim3((s.N + 3) / 4, s.B * s.H), dim3(256), 0, stream, a);
  return launch_ok("lipar_restore") ? BSA_OK : BSA_ERR_HIP;
}

}  // namespace bsa
