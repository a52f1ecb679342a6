// Block-mask builder: spatiotemporal keep rule -> CSR of int32 block indices.
//
// Rules: "[논문리뷰] LVSA: Training-Free Sparse Attention for Long Video Diffusion",
// section 3 Method & Key Results with Figures 1-2 (local frame window plus
// periodic global anchor frames that rotate with the denoising step), and the
// Radial Attention headline page (static mask whose spatial window shrinks
// exponentially with temporal distance).  A block pair is kept when any real
// token pair in it is kept.
//
// Launches, all integer and deterministic:
//   count: one workgroup per block row, row_ptr[i + 1] = number of kept columns
//   scan : one workgroup, inclusive prefix sum of row_ptr[1..nb]
//   fill : one workgroup per block row, kept columns written in ascending order
//          using wave ballots for the in-row prefix
//   order: (optional) the row schedule for the attention launch (long rows
//          first, see mask_order_kernel).

#include "launch.h"

namespace bsa {

struct MaskArgs {
  int kind, F, P, block, window, period, step, rows, radial_w;
  int N, nb;
};

// Smallest anchor frame >= f0, or a huge value when there are none.
__device__ __forceinline__ int next_anchor(const MaskArgs& m, int f0) {
  if (m.period <= 0) return 0x7fffffff;
  int s = m.step % m.period;
  int r = ((s - f0) % m.period + m.period) % m.period;
  return f0 + r;
}

// Window/anchor test on whole frame ranges [q0, q1] x [k0, k1] (O(1)).
__device__ __forceinline__ bool window_anchor_keep(const MaskArgs& m, int q0, int q1, int k0, int k1) {
  int gap = max(0, max(k0 - q1, q0 - k1));  // smallest |fq - fk| over the two ranges
  if (gap <= m.window) return true;
  if (next_anchor(m, k0) <= k1) return true;
  if (m.rows && next_anchor(m, q0) <= q1) return true;
  return false;
}

// Radial test over the per-frame pieces of two blocks.
__device__ bool radial_keep(const MaskArgs& m, int t0, int t1, int u0, int u1) {
  const int P = m.P;
  for (int fq = t0 / P; fq <= (t1 - 1) / P; ++fq) {
    int qlo = max(t0, fq * P) - fq * P, qhi = min(t1, (fq + 1) * P) - 1 - fq * P;
    for (int fk = u0 / P; fk <= (u1 - 1) / P; ++fk) {
      int dt = fq > fk ? fq - fk : fk - fq;
      if (dt == 0) return true;
      int klo = max(u0, fk * P) - fk * P, khi = min(u1, (fk + 1) * P) - 1 - fk * P;
      int dist = max(0, max(klo - qhi, qlo - khi));
      int r = 31 - __clz(dt);
      if (((long long)dist << r) <= (long long)m.radial_w) return true;
    }
  }
  return false;
}

__device__ __forceinline__ bool block_keep(const MaskArgs& m, int i, int j) {
  if (m.kind == BSA_MASK_ALL) return true;
  int t0 = i * m.block, t1 = min(t0 + m.block, m.N);
  int u0 = j * m.block, u1 = min(u0 + m.block, m.N);
  if (m.kind == BSA_MASK_WINDOW_ANCHOR)
    return window_anchor_keep(m, t0 / m.P, (t1 - 1) / m.P, u0 / m.P, (u1 - 1) / m.P);
  return radial_keep(m, t0, t1, u0, u1);
}

constexpr int kMaskThreads = 256;

__global__ void __launch_bounds__(kMaskThreads) mask_count_kernel(MaskArgs m, int32_t* row_ptr) {
  __shared__ int wave_sum[kMaskThreads / 64];
  const int i = blockIdx.x;
  int cnt = 0;
  for (int j = threadIdx.x; j < m.nb; j += kMaskThreads) cnt += block_keep(m, i, j) ? 1 : 0;
  for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off, 64);
  if ((threadIdx.x & 63) == 0) wave_sum[threadIdx.x >> 6] = cnt;
  __syncthreads();
  if (threadIdx.x == 0) {
    int t = 0;
    for (int w = 0; w < kMaskThreads / 64; ++w) t += wave_sum[w];
    row_ptr[i + 1] = t;
    if (i == 0) row_ptr[0] = 0;
  }
}

constexpr int kScanThreads = 1024;

// In-place inclusive scan of row_ptr[1..nb] (row_ptr[0] == 0 already).
__global__ void __launch_bounds__(kScanThreads) mask_scan_kernel(int32_t* row_ptr, int nb) {
  __shared__ int part[kScanThreads];
  const int per = (nb + kScanThreads - 1) / kScanThreads;
  const int b0 = 1 + threadIdx.x * per, b1 = min(b0 + per, nb + 1);
  int s = 0;
  for (int x = b0; x < b1; ++x) s += row_ptr[x];
  part[threadIdx.x] = s;
  __syncthreads();
  // Hillis-Steele inclusive scan over the per-thread sums
  for (int off = 1; off < kScanThreads; off <<= 1) {
    int add = threadIdx.x >= off ? part[threadIdx.x - off] : 0;
    __syncthreads();
    part[threadIdx.x] += add;
    __syncthreads();
  }
  int run = part[threadIdx.x] - s;  // exclusive prefix of this thread's chunk
  for (int x = b0; x < b1; ++x) {
    run += row_ptr[x];
    row_ptr[x] = run;
  }
}

__global__ void __launch_bounds__(kMaskThreads) mask_fill_kernel(MaskArgs m, const int32_t* row_ptr,
                                                                 int32_t* col_idx) {
  __shared__ int wave_cnt[kMaskThreads / 64];
  const int i = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int base = row_ptr[i];
  for (int j0 = 0; j0 < m.nb; j0 += kMaskThreads) {
    const int j = j0 + threadIdx.x;
    const bool keep = j < m.nb && block_keep(m, i, j);
    const unsigned long long bal = __ballot(keep);
    const int before = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wave_cnt[wave] = __popcll(bal);
    __syncthreads();
    int off = base;
    for (int w = 0; w < wave; ++w) off += wave_cnt[w];
    if (keep) col_idx[off + before] = j;
    int total = 0;
    for (int w = 0; w < kMaskThreads / 64; ++w) total += wave_cnt[w];
    base += total;
    __syncthreads();
  }
}

// Row schedule for the attention launch, int32[nb + 1].  Rows with at least 1.5x
// the mean kept-block count are "long": they come first, by descending count
// (ties by ascending index), and their number nh goes to row_order[nb]; the
// other rows follow in ascending index order.  Every row of length >= a long
// row's length is long too, so a long row's rank is #rows longer + #rows of
// equal length before it; a short row's rank is nh + #short rows before it.
// One wave per row: its lanes read 64 row lengths at a time and the counts
// are ballots (integer, so the schedule does not depend on any order).
__device__ __forceinline__ bool long_row(int len, int nb, int total) {
  return 2 * (int64_t)len * nb >= 3 * (int64_t)total && len > 0;
}

constexpr int kOrderRowsPerBlock = 4;  // waves (rows) per workgroup

__global__ void __launch_bounds__(64 * kOrderRowsPerBlock) mask_order_kernel(const int32_t* row_ptr, int nb,
                                                                               int32_t* row_order) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * kOrderRowsPerBlock + (threadIdx.x >> 6);
  if (i >= nb) return;  // wave-uniform; the kernel has no barrier
  const int total = row_ptr[nb];
  const int li = row_ptr[i + 1] - row_ptr[i];
  const bool li_long = long_row(li, nb, total);
  int longer = 0, equal_before = 0, n_long = 0, short_before = 0;
  for (int j0 = 0; j0 < nb; j0 += 64) {
    const int j = j0 + lane;
    const bool valid = j < nb;
    const int lj = valid ? row_ptr[j + 1] - row_ptr[j] : -1;
    const bool jl = valid && long_row(lj, nb, total);
    longer += __popcll(__ballot(valid && lj > li));
    equal_before += __popcll(__ballot(valid && lj == li && j < i));
    n_long += __popcll(__ballot(jl));
    short_before += __popcll(__ballot(valid && !jl && j < i));
  }
  if (lane == 0) {
    row_order[li_long ? longer + equal_before : n_long + short_before] = i;
    if (i == 0) row_order[nb] = n_long;
  }
}

bsa_status launch_build_block_mask(const bsa_mask_desc& d, int32_t* row_ptr, int32_t* col_idx,
                                   int32_t* row_order, hipStream_t stream) {
  MaskArgs m;
  m.kind = d.kind; m.F = d.frames; m.P = d.frame_tokens; m.block = d.block;
  m.window = d.window; m.period = d.anchor_period; m.step = d.anchor_step;
  m.rows = d.anchor_rows; m.radial_w = d.radial_w;
  m.N = d.frames * d.frame_tokens;
  m.nb = (m.N + m.block - 1) / m.block;
  hipLaunchKernelGGL(mask_count_kernel, dim3(m.nb), dim3(kMaskThreads), 0, stream, m, row_ptr);
  hipLaunchKernelGGL(mask_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, row_ptr, m.nb);
  hipLaunchKernelGGL(mask_fill_kernel, dim3(m.nb), dim3(kMaskThreads), 0, stream, m, row_ptr, col_idx);
  if (row_order != nullptr)
    hipLaunchKernelGGL(mask_order_kernel, dim3((m.nb + kOrderRowsPerBlock - 1) / kOrderRowsPerBlock),
                       dim3(64 * kOrderRowsPerBlock), 0, stream, row_ptr, m.nb, row_order);
  return launch_ok("build_block_mask") ? BSA_OK : BSA_ERR_HIP;
}

void launch_block_order(const int32_t* ptr, int nb, int32_t* order, hipStream_t stream) {
  hipLaunchKernelGGL(mask_order_kernel, dim3((nb + kOrderRowsPerBlock - 1) / kOrderRowsPerBlock),
                     dim3(64 * kOrderRowsPerBlock), 0, stream, ptr, nb, order);
}

void launch_inclusive_scan(int32_t* a, int n, hipStream_t stream) {
  hipLaunchKernelGGL(mask_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, a, n);
}

}  // namespace bsa
