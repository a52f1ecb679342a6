// Block-sparse softmax attention forward for gfx950.
//
// Operation: for each real query row, softmax(scale * q K^T) V over the keys of
// the kept key blocks of its block row, plus the natural-log LSE ("[논문리뷰]
// LVSA: Training-Free Sparse Attention for Long Video Diffusion", section 1 Key
// Terms and section 3: block-sparse attention over a frame window and anchor
// frames; SVG-EAR page, technical summary section 1: sparse attention computes
// the kept blocks and skips the rest).  Skipped key blocks are never read.
//
// bf16 path (attn_bf16_kernel).  One workgroup per (query block, head, batch);
// BM = block query rows, 32 rows per wave.  The loop walks the row's kept key
// blocks in 64-key sub-tiles:
//   * K (64 x D) and V (64 x D) are fetched with 16-byte coalesced loads into
//     registers one sub-tile ahead and written to a double-buffered LDS stage;
//     K is stored row-major, V is stored transposed (d-major) so that the second
//     product reads 8 consecutive keys per lane.
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: Q stays in registers as the B
//     operand for the whole kernel.  In the transposed product each lane owns
//     one query column, so the online softmax is lane-local except for one
//     exchange with the lane 32 apart.
//   * O^T += V^T P^T, again 32x32x16 MFMA; P^T comes straight from the S^T
//     accumulator registers (fp32 -> bf16), V^T from LDS.  The key order inside
//     each 16-key group of the V^T stage is permuted to match the accumulator
//     layout, so no data moves between lanes.
//   * exp2 with scale*log2(e) folded in; fp32 running max / sum per lane.
//
// fp32 path (attn_f32_kernel).  Straightforward: one thread per query row,
// 32-key tiles of K and V staged in LDS, fp32 FMA dot products, expf.

#include "common.h"

namespace bsa {

// ---------------------------------------------------------------------------
// bf16 MFMA kernel
// ---------------------------------------------------------------------------

constexpr int kBN = 64;  // keys per sub-tile

template <int D>
struct AttnCfg {
  // K stage: row stride D + 8 elements (row step = 4 banks mod 64), so the 16 rows
  // read by 16 consecutive lanes cover all 64 banks.
  static constexpr int KST = D + 8;
  // V stage: row-major, stride D + 32 elements (row step = 16 banks mod 64), so the
  // 4-row x 64-byte footprint of a 32-lane transpose read covers all 64 banks.
  static constexpr int VST = D + 32;
  static constexpr int K_ELEMS = kBN * KST;
  static constexpr int V_ELEMS = kBN * VST;
  static constexpr int KT = D / 16;     // k-steps of the first product
  static constexpr int DT = D / 32;     // 32-wide d tiles of the output
  static constexpr int CH = D / 8;      // 16-byte chunks per row
};

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  int64_t sb, sh, sn;
  int B, H, N, block, nb;
  float scale_log2;  // scale * log2(e)
};

template <int D, int BM>
__global__ void __launch_bounds__(BM * 2) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bf16_kernel(AttnArgs a) {
  using C = AttnCfg<D>;
  constexpr int NT = BM * 2;                 // BM / 32 waves of 64 lanes
  constexpr int LCH = kBN * C::CH / NT;      // 16-byte chunks per thread per tile (K and V each)
  static_assert(LCH >= 1 && LCH * NT == kBN * C::CH, "tile/thread mismatch");

  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][C::K_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][C::V_ELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int N = a.N;

  // Work item.  The hardware deals workgroups round-robin to the 8 XCDs; give
  // each XCD a contiguous range of (batch, head, query block) so that the
  // workgroups sharing one L2 walk neighbouring query blocks of one head.
  int wid = blockIdx.x;
  const int total = gridDim.x;
  if ((total & 7) == 0) wid = (wid & 7) * (total >> 3) + (wid >> 3);
  const int qblk = wid % a.nb;
  const int h = (wid / a.nb) % a.H;
  const int b = wid / (a.nb * a.H);

  const int64_t head_off = (int64_t)b * a.sb + (int64_t)h * a.sh;
  const uint16_t* __restrict__ Qh = a.q + head_off;
  const uint16_t* __restrict__ Kh = a.k + head_off;
  const uint16_t* __restrict__ Vh = a.v + head_off;

  // ---- Q fragment (B operand of S^T = K Q^T): query column l32, 8 d per k-step
  const int qrow = qblk * a.block + wave * 32 + l32;
  bf16x8 qf[C::KT];
  {
    const uint16_t* src = Qh + (int64_t)min(qrow, N - 1) * a.sn + hi * 8;
#pragma unroll
    for (int t = 0; t < C::KT; ++t) qf[t] = __builtin_bit_cast(bf16x8, *(const u32x4*)(src + t * 16));
  }

  const int rbeg = a.row_ptr[qblk], rend = a.row_ptr[qblk + 1];
  const int spb = a.block / kBN;  // sub-tiles per key block
  int nsub = (rend - rbeg) * spb;
  if (nsub > 0 && a.col_idx[rend - 1] == a.nb - 1) {
    // drop trailing sub-tiles of the last key block that hold no real key
    const int last_real = N - (a.nb - 1) * a.block;
    nsub -= spb - (last_real + kBN - 1) / kBN;
  }
  auto sub_key0 = [&](int u) -> int { return a.col_idx[rbeg + u / spb] * a.block + (u % spb) * kBN; };

  // ---- global -> registers (one sub-tile ahead) -> LDS.  Rows past N are
  // clamped to row N - 1: their logits are masked to -inf below, so they carry
  // weight 0.
  u32x4 kreg[LCH], vreg[LCH];
  auto fetch = [&](int key0) {
#pragma unroll
    for (int i = 0; i < LCH; ++i) {
      const int c = tid + NT * i;
      const int row = c / C::CH, col = (c % C::CH) * 8;
      const int64_t off = (int64_t)min(key0 + row, N - 1) * a.sn + col;
      kreg[i] = *(const u32x4*)(Kh + off);
      vreg[i] = *(const u32x4*)(Vh + off);
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LCH; ++i) {
      const int c = tid + NT * i;
      const int row = c / C::CH, col = (c % C::CH) * 8;
      *(u32x4*)&Ks[buf][row * C::KST + col] = kreg[i];
      *(u32x4*)&Vs[buf][row * C::VST + col] = vreg[i];
    }
  };

  // ---- running state: lane owns query column l32 (shared with lane l32 + 32)
  f32x16 o[C::DT];
#pragma unroll
  for (int i = 0; i < C::DT; ++i) o[i] = f32x16{};
  float m_run = -1e30f;  // finite start: exp2(m_old - m_new) never sees inf - inf
  float l_run = 0.f;
  const float c2 = a.scale_log2;

  // per-lane constants of the V^T operand reads (see lds_tr16)
  const int g16 = lane >> 4, j16 = lane & 15;
  const int v_row = 4 * hi + (j16 >> 2);
  const int v_col = 16 * (g16 & 1) + 4 * (j16 & 3);

  if (nsub > 0) {
    fetch(sub_key0(0));
    stage(0);
  }
  __syncthreads();

  for (int u = 0; u < nsub; ++u) {
    const int buf = u & 1;
    const int key0 = sub_key0(u);
    if (u + 1 < nsub) fetch(sub_key0(u + 1));

    // S^T tile: 64 keys x 32 queries per wave as two 32x32 accumulators.
    // Accumulator layout: s[kt][r] = S^T[key kt*32 + 8*(r/4) + 4*hi + r%4][query l32].
    f32x16 s[2];
    s[0] = f32x16{};
    s[1] = f32x16{};
    const uint16_t* Kb = Ks[buf];
#pragma unroll
    for (int t = 0; t < C::KT; ++t) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const bf16x8 kf = *(const bf16x8*)&Kb[(kt * 32 + l32) * C::KST + t * 16 + hi * 8];
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[t], s[kt], 0, 0, 0);
      }
    }

    if (key0 + kBN > N) {  // tail: keys past N do not exist
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + kt * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (key >= N) s[kt][r] = -__builtin_inff();
        }
    }

    // online softmax in the log2 domain; O and l are rescaled only when the
    // running max of some lane moved
    float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int r = 2; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
    const float m_new = fmaxf(m_run, pair_max(mx));
    if (__any(m_new > m_run)) {
      const float alpha = fast_exp2((m_run - m_new) * c2);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < C::DT; ++i) o[i] *= alpha;
      m_run = m_new;
    }
    const float mc = m_run * c2;
    float psum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(__builtin_fmaf(s[kt][r], c2, -mc));
        s[kt][r] = p;
        psum += p;
      }
    l_run += psum;

    // P^T operands: k-step ks covers S^T registers 8*(ks%2) .. +8 of tile ks/2,
    // i.e. keys 16ks + 8*(e/4) + 4*hi + e%4 for element e.
    bf16x8 pf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kt = ks >> 1, r0 = (ks & 1) * 8;
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(s[kt][r0 + 2 * e], s[kt][r0 + 2 * e + 1]);
      pf[ks] = __builtin_bit_cast(bf16x8, w);
    }

    // O^T += V^T P^T.  The A operand (row d = dt*32 + l32, the same 8 keys as
    // P^T) is two transpose reads of 4 keys each from the row-major V stage.
    const uint16_t* Vb = Vs[buf];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
        const uint16_t* p0 = &Vb[(ks * 16 + v_row) * C::VST + dt * 32 + v_col];
        const u32x2 lo = lds_tr16(p0);
        const u32x2 hi2 = lds_tr16(p0 + 8 * C::VST);
        const u32x4 w = {lo[0], lo[1], hi2[0], hi2[1]};
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w), pf[ks], o[dt], 0, 0, 0);
      }
    }

    if (u + 1 < nsub) stage(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: normalise and store. o[dt][r] = O^T[d dt*32 + 8*(r/4) + 4*hi + r%4][query l32]
  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qrow < N) {
    uint16_t* dst = a.o + head_off + (int64_t)qrow * a.sn;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = dt * 32 + 8 * g + 4 * hi;
        u32x2 w = {pack_bf16x2(o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv),
                   pack_bf16x2(o[dt][4 * g + 2] * inv, o[dt][4 * g + 3] * inv)};
        *(u32x2*)(dst + d0) = w;
      }
    if (a.lse != nullptr && hi == 0) {
      const float v = l_tot > 0.f ? (m_run * c2 + __builtin_log2f(l_tot)) * kLn2 : -__builtin_inff();
      a.lse[((int64_t)b * a.H + h) * N + qrow] = v;
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 kernel
// ---------------------------------------------------------------------------

constexpr int kF32Keys = 32;

struct AttnF32Args {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  int64_t sb, sh, sn;
  int H, N, block, nb;
  float scale;
};

template <int D>
__global__ void __launch_bounds__(128) attn_f32_kernel(AttnF32Args a) {
  __shared__ float Qs[128][D + 1];
  __shared__ float Ks[kF32Keys][D + 1];
  __shared__ float Vs[kF32Keys][D];
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;  // == block
  const int qblk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int N = a.N;
  const int64_t head_off = (int64_t)b * a.sb + (int64_t)h * a.sh;
  const int q0 = qblk * a.block;
  for (int x = tid; x < a.block * D; x += nthr) {
    const int r = x / D, d = x % D;
    Qs[r][d] = (q0 + r < N) ? a.q[head_off + (int64_t)(q0 + r) * a.sn + d] : 0.f;
  }
  float acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const int rbeg = a.row_ptr[qblk], rend = a.row_ptr[qblk + 1];
  for (int e = rbeg; e < rend; ++e) {
    const int kb0 = a.col_idx[e] * a.block;
    const int kend = min(kb0 + a.block, N);
    for (int t0 = kb0; t0 < kend; t0 += kF32Keys) {
      const int nk = min(kF32Keys, kend - t0);
      __syncthreads();
      for (int x = tid; x < kF32Keys * D; x += nthr) {
        const int r = x / D, d = x % D;
        const bool ok = r < nk;
        Ks[r][d] = ok ? a.k[head_off + (int64_t)(t0 + r) * a.sn + d] : 0.f;
        Vs[r][d] = ok ? a.v[head_off + (int64_t)(t0 + r) * a.sn + d] : 0.f;
      }
      __syncthreads();
      float s[kF32Keys];
      float mx = m_run;
#pragma unroll
      for (int j = 0; j < kF32Keys; ++j) {
        float dot = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) dot = __builtin_fmaf(Qs[tid][d], Ks[j][d], dot);
        s[j] = j < nk ? dot * a.scale : -INFINITY;
        mx = fmaxf(mx, s[j]);
      }
      const float corr = (m_run == -INFINITY) ? 0.f : expf(m_run - mx);
      l_run *= corr;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] *= corr;
#pragma unroll
      for (int j = 0; j < kF32Keys; ++j) {
        const float p = j < nk ? expf(s[j] - mx) : 0.f;
        l_run += p;
#pragma unroll
        for (int d = 0; d < D; ++d) acc[d] = __builtin_fmaf(p, Vs[j][d], acc[d]);
      }
      m_run = mx;
    }
  }
  const int qrow = q0 + tid;
  if (tid < a.block && qrow < N) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    float* dst = a.o + head_off + (int64_t)qrow * a.sn;
#pragma unroll
    for (int d = 0; d < D; ++d) dst[d] = acc[d] * inv;
    if (a.lse != nullptr) a.lse[((int64_t)b * a.H + h) * N + qrow] = l_run > 0.f ? m_run + logf(l_run) : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

bsa_status launch_attn_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                            const bsa_shape& s, const int32_t* row_ptr, const int32_t* col_idx,
                            int block, float scale, hipStream_t stream) {
  AttnArgs a;
  a.q = (const uint16_t*)q; a.k = (const uint16_t*)k; a.v = (const uint16_t*)v; a.o = (uint16_t*)o;
  a.lse = lse; a.row_ptr = row_ptr; a.col_idx = col_idx;
  a.sb = s.stride_b; a.sh = s.stride_h; a.sn = s.stride_n;
  a.B = s.B; a.H = s.H; a.N = s.N; a.block = block; a.nb = (s.N + block - 1) / block;
  a.scale_log2 = scale * kLog2e;
  dim3 grid((unsigned)((int64_t)a.nb * s.H * s.B));
  if (s.D == 128 && block == 128)
    hipLaunchKernelGGL((attn_bf16_kernel<128, 128>), grid, dim3(256), 0, stream, a);
  else if (s.D == 128 && block == 64)
    hipLaunchKernelGGL((attn_bf16_kernel<128, 64>), grid, dim3(128), 0, stream, a);
  else if (s.D == 64 && block == 128)
    hipLaunchKernelGGL((attn_bf16_kernel<64, 128>), grid, dim3(256), 0, stream, a);
  else if (s.D == 64 && block == 64)
    hipLaunchKernelGGL((attn_bf16_kernel<64, 64>), grid, dim3(128), 0, stream, a);
  else
    return BSA_ERR_UNSUPPORTED;
  return launch_ok("block_sparse_attn_fwd(bf16)") ? BSA_OK : BSA_ERR_HIP;
}

bsa_status launch_attn_f32(const void* q, const void* k, const void* v, void* o, float* lse,
                           const bsa_shape& s, const int32_t* row_ptr, const int32_t* col_idx,
                           int block, float scale, hipStream_t stream) {
  AttnF32Args a;
  a.q = (const float*)q; a.k = (const float*)k; a.v = (const float*)v; a.o = (float*)o;
  a.lse = lse; a.row_ptr = row_ptr; a.col_idx = col_idx;
  a.sb = s.stride_b; a.sh = s.stride_h; a.sn = s.stride_n;
  a.H = s.H; a.N = s.N; a.block = block; a.nb = (s.N + block - 1) / block;
  a.scale = scale;
  dim3 grid(a.nb, s.H, s.B);
  if (s.D == 128)
    hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(block), 0, stream, a);
  else if (s.D == 64)
    hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(block), 0, stream, a);
  else if (s.D == 32)
    hipLaunchKernelGGL(attn_f32_kernel<32>, grid, dim3(block), 0, stream, a);
  else
    return BSA_ERR_UNSUPPORTED;
  return launch_ok("block_sparse_attn_fwd(f32)") ? BSA_OK : BSA_ERR_HIP;
}

}  // namespace bsa
