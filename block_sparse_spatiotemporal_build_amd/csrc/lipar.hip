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
//   flag    : one wave per (patch, range of frames) walks its frames in order,
//             holding the previous frame's row in registers (each row is read
//             once, plus the row before the range; the next two frames' loads
//             are in flight while a frame is reduced).  The ranges give the
//             launch enough waves to keep HBM busy.
//   positions : one workgroup per frame: the position of every token among
//             the kept ones (in token order), the kept-token list and the
//             kept count.
//   gather  : one wave per pruned row copies its token's row.
//   restore : one wave per output row finds its source frame (the latest kept
//             frame of its patch: one flag per lane and a ballot) and copies
//             that pruned row.

#include "launch.h"

namespace bsa {


struct LiparArgs {
  const uint16_t* x;   // [B, H, N, D] with strides
  int64_t sb, sh, sn;
  int H, N, D, F, P;
  int R, FR;           // frame ranges per patch, frames per range (of frames 1 .. F - 1)
  double thr;          // tau * D
  uint8_t* keep;       // [BH][N]
  int32_t* cpos;       // [BH][N]: kept tokens before n
  int32_t* kidx;       // [BH][N]: token of pruned row j
  int32_t* nkept;      // [BH]
  uint16_t* xp;        // [BH][N][D] pruned rows (dense)
};

__device__ __forceinline__ const uint16_t* lp_row(const LiparArgs& a, int bh, int n) {
  return a.x + (int64_t)(bh / a.H) * a.sb + (int64_t)(bh % a.H) * a.sh + (int64_t)n * a.sn;
}

// CPL = 16-byte chunks per lane (D <= 512 CPL); two frames in flight ahead of
// the one being reduced.  Wave w of the launch takes patch w / R and frames
// [1 + r FR, 1 + (r + 1) FR) of it, r = w % R (the waves of one patch are
// neighbours, so the row read at a range boundary is still cached)
template <int CPL>
__global__ void __launch_bounds__(256) lipar_flag_kernel(LiparArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int bh = blockIdx.y, w = blockIdx.x * 4 + wave;
  const int p = w / a.R, r = w % a.R;
  if (p >= a.P) return;
  const int f_beg = 1 + r * a.FR, f_end = min(a.F, f_beg + a.FR);
  uint8_t* keep = a.keep + (int64_t)bh * a.N;
  if (r == 0 && lane == 0) keep[p] = 1;  // frame 0 is always kept
  if (f_beg >= f_end) return;
  const int nch = a.D / 8;  // 16-byte chunks per row
  auto load = [&](int f, u32x4 (&dst)[CPL]) {
    const u32x4* src = (const u32x4*)lp_row(a, bh, f * a.P + p);
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = i * 64 + lane;
      dst[i] = c < nch ? __builtin_nontemporal_load(src + c) : u32x4{0, 0, 0, 0};  // every row read once here
    }
  };
  u32x4 prev[CPL], cur[CPL], n1[CPL], n2[CPL];
  load(f_beg - 1, prev);
  load(f_beg, cur);
  if (f_beg + 1 < f_end) load(f_beg + 1, n1);
  for (int f = f_beg; f < f_end; ++f) {
    if (f + 2 < f_end) load(f + 2, n2);
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < CPL; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double d0 = (double)bf16_lo(cur[i][e]) - (double)bf16_lo(prev[i][e]);
        const double d1 = (double)bf16_hi(cur[i][e]) - (double)bf16_hi(prev[i][e]);
        s += fabs(d0) + fabs(d1);
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

// positions, one workgroup per (frame, sequence): the kept tokens of the
// earlier frames give the frame's first position (coalesced byte reads, summed
// over the workgroup), then the frame's P flags are scanned 1024 at a time in
// token order, writing cpos, the kept-token list and, for the last frame, the
// kept count
__global__ void __launch_bounds__(1024) lipar_positions_kernel(LiparArgs a) {
  __shared__ int wsum[16];
  const int f = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint8_t* keep = a.keep + (int64_t)bh * a.N;
  int32_t* cpos = a.cpos + (int64_t)bh * a.N;
  int32_t* kidx = a.kidx + (int64_t)bh * a.N;
  const int f0 = f * a.P;
  int c = 0;
  for (int n0 = 0; n0 < f0; n0 += 8 * 1024) {  // eight independent loads per round trip
    int v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int n = n0 + u * 1024 + tid;
      v[u] = n < f0 ? keep[n] : 0;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) c += v[u];
  }
  for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off, 64);
  if (lane == 0) wsum[wave] = c;
  __syncthreads();
  int run = 0;
  for (int w = 0; w < 16; ++w) run += wsum[w];
  __syncthreads();
  for (int p0 = 0; p0 < a.P; p0 += 1024) {
    const int n = f0 + p0 + tid;
    const bool k = p0 + tid < a.P && keep[n] != 0;
    const unsigned long long bal = __ballot(k);
    if (lane == 0) wsum[wave] = __popcll(bal);
    __syncthreads();
    int before = run;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    int total = 0;
    for (int w = 0; w < 16; ++w) total += wsum[w];
    const int r = before + __popcll(bal & ((1ull << lane) - 1ull));
    if (p0 + tid < a.P) cpos[n] = r;
    if (k) kidx[r] = n;
    run += total;
    __syncthreads();
  }
  if (f == a.F - 1 && tid == 0) a.nkept[bh] = run;
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
  const int f = n / a.P, p = n - f * a.P;
  // the latest frame g <= f that keeps patch p: lane l looks at frame f0 + l
  int g = 0;
  for (int f0 = 0; f0 <= f; f0 += 64) {
    const int ff = f0 + lane;
    const unsigned long long bal = __ballot(ff <= f && keep[ff * a.P + p] != 0);
    if (bal != 0ull) g = f0 + 63 - __builtin_clzll(bal);
  }
  const int j = a.cpos[(int64_t)bh * a.N + g * a.P + p];
  const u32x4* src = (const u32x4*)(a.y + ((int64_t)bh * a.N + j) * a.D);
  u32x4* dst = (u32x4*)(a.o + (int64_t)(bh / a.H) * a.sb + (int64_t)(bh % a.H) * a.sh + (int64_t)n * a.sn);
  const int nch = a.D / 8;
  // the full-length output is written once and not read back here: non-temporal
  for (int c = lane; c < nch; c += 64) __builtin_nontemporal_store(src[c], dst + c);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

bsa_status launch_lipar_prune(const void* x, const bsa_shape& s, int frames, float tau, uint8_t* keep,
                              int32_t* cpos, int32_t* kept_idx, int32_t* n_kept, void* x_pruned,
                              hipStream_t stream) {
  LiparArgs a;
  a.x = (const uint16_t*)x; a.sb = s.stride_b; a.sh = s.stride_h; a.sn = s.stride_n;
  a.H = s.H; a.N = s.N; a.D = s.D; a.F = frames; a.P = s.N / frames;
  a.thr = (double)tau * (double)s.D;
  a.keep = keep; a.cpos = cpos; a.kidx = kept_idx; a.nkept = n_kept; a.xp = (uint16_t*)x_pruned;
  const int bh = s.B * s.H;
  // frame ranges per patch: enough waves for about 4096 in the launch, each
  // range as long as possible (one extra row read per range)
  const int want = (4096 + a.P * bh - 1) / (a.P * bh);
  const int ranges = std::max(1, std::min(frames - 1, want));
  a.FR = std::max(1, (frames - 1 + ranges - 1) / ranges);
  a.R = std::max(1, (frames - 1 + a.FR - 1) / a.FR);
  const dim3 pg((unsigned)(((int64_t)a.P * a.R + 3) / 4), bh);
  const int cpl = (s.D / 8 + 63) / 64;
  if (cpl <= 1) hipLaunchKernelGGL(lipar_flag_kernel<1>, pg, dim3(256), 0, stream, a);
  else if (cpl <= 2) hipLaunchKernelGGL(lipar_flag_kernel<2>, pg, dim3(256), 0, stream, a);
  else if (cpl <= 4) hipLaunchKernelGGL(lipar_flag_kernel<4>, pg, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(lipar_flag_kernel<8>, pg, dim3(256), 0, stream, a);
  hipLaunchKernelGGL(lipar_positions_kernel, dim3(frames, bh), dim3(1024), 0, stream, a);
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
