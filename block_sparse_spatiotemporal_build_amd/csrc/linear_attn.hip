// Non-causal elu+1 linear attention for gfx950.
//
// Operation (LinVideo page, technical summary sections 1-2: O(n) linear
// attention in place of quadratic softmax attention; feature map
// phi(x) = elu(x) + 1):
//   S = sum_n phi(k_n) v_n^T (D x D),  z = sum_n phi(k_n),
//   out_n = phi(q_n)^T S / (phi(q_n)^T z).
//
// Three launches, all deterministic:
//   state  : grid (splits, B*H).  Each workgroup streams a fixed chunk of
//            tokens: K and V tiles of 64 tokens are loaded with 16-byte
//            coalesced loads one tile ahead, phi is applied to K in fp32 while
//            staging (z partials accumulate in fp32 from the same values),
//            phi(K) is rounded to bf16 and both tiles are stored row-major in
//            LDS.  S_part^T-free form: S = phi(K)^T V with 32x32x16 bf16 MFMA,
//            both operands read with the transpose read (token-contiguous per
//            lane).  Each split writes an fp32 partial.
//   reduce : sums the partials of a head in split order; writes S (fp32, the
//            caller's optional output), S^T rounded to bf16 and z (workspace).
//   apply  : grid (row groups, B*H).  S^T (bf16) and z are staged in LDS once
//            per workgroup; for each 128-query tile, O^T = S^T phi(Q)^T with Q
//            as the B operand straight from global memory (phi in fp32, then
//            bf16), and the denominator phi(q).z in fp32 per lane.

#include "common.h"

namespace bsa {

__device__ __forceinline__ float phi(float x) { return x > 0.f ? x + 1.f : __expf(x); }

constexpr int kLinTok = 64;      // tokens per state tile
constexpr int kLinThreads = 256;

template <int D>
struct LinCfg {
  static constexpr int ST = D + 32;          // LDS row stride (elements) for transpose reads
  static constexpr int CH = D / 8;           // 16-byte chunks per row
  static constexpr int LCH = kLinTok * CH / kLinThreads;  // chunks per thread per tensor
  static constexpr int NT32 = D / 32;        // 32-wide tiles per dimension
  static constexpr int TPW = NT32 * NT32 / 4;  // S tiles per wave
};

struct LinStateArgs {
  const uint16_t* k;
  const uint16_t* v;
  float* part_s;   // [BH][splits][D][D]
  float* part_z;   // [BH][splits][D]
  int64_t sb, sh, sn;
  int H, N, splits, chunk;
};

template <int D>
__global__ void __launch_bounds__(kLinThreads) lin_state_kernel(LinStateArgs a) {
  using C = LinCfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kLinTok * C::ST];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][kLinTok * C::ST];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hi = lane >> 5;
  const int split = blockIdx.x, bh = blockIdx.y;
  const int b = bh / a.H, h = bh % a.H;
  const int64_t head_off = (int64_t)b * a.sb + (int64_t)h * a.sh;
  const uint16_t* __restrict__ Kh = a.k + head_off;
  const uint16_t* __restrict__ Vh = a.v + head_off;
  const int n0 = split * a.chunk;
  const int n1 = min(n0 + a.chunk, a.N);
  const int ntile = (n1 - n0 + kLinTok - 1) / kLinTok;

  // staging: thread handles chunk column cc (8 consecutive d) of rows rr, rr + RS, ...
  const int cc = tid % C::CH;
  constexpr int RS = kLinThreads / C::CH;
  const int rr = tid / C::CH;
  float zacc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) zacc[e] = 0.f;

  u32x4 kreg[C::LCH], vreg[C::LCH];
  auto fetch = [&](int t0) {
#pragma unroll
    for (int i = 0; i < C::LCH; ++i) {
      const int row = rr + RS * i;
      const int64_t off = (int64_t)min(t0 + row, a.N - 1) * a.sn + cc * 8;
      kreg[i] = *(const u32x4*)(Kh + off);
      vreg[i] = *(const u32x4*)(Vh + off);
    }
  };
  auto stage = [&](int buf, int t0) {
#pragma unroll
    for (int i = 0; i < C::LCH; ++i) {
      const int row = rr + RS * i;
      const bool ok = t0 + row < n1;
      u32x4 pk, pv = ok ? vreg[i] : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f0 = ok ? phi(bf16_lo(kreg[i][w])) : 0.f;
        const float f1 = ok ? phi(bf16_hi(kreg[i][w])) : 0.f;
        zacc[2 * w] += f0;
        zacc[2 * w + 1] += f1;
        pk[w] = pack_bf16x2(f0, f1);
      }
      *(u32x4*)&Ks[buf][row * C::ST + cc * 8] = pk;
      *(u32x4*)&Vs[buf][row * C::ST + cc * 8] = pv;
    }
  };

  f32x16 acc[C::TPW];
#pragma unroll
  for (int i = 0; i < C::TPW; ++i) acc[i] = f32x16{};
  const int g16 = lane >> 4, j16 = lane & 15;
  const int tr_row = 4 * hi + (j16 >> 2);
  const int tr_col = 16 * (g16 & 1) + 4 * (j16 & 3);

  if (ntile > 0) {
    fetch(n0);
    stage(0, n0);
  }
  __syncthreads();
  for (int t = 0; t < ntile; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntile) fetch(n0 + (t + 1) * kLinTok);
#pragma unroll
    for (int ks = 0; ks < kLinTok / 16; ++ks) {
#pragma unroll
      for (int i = 0; i < C::TPW; ++i) {
        const int tile = wave * C::TPW + i;
        const int d1t = tile / C::NT32, d2t = tile % C::NT32;
        const uint16_t* pa = &Ks[buf][(ks * 16 + tr_row) * C::ST + d1t * 32 + tr_col];
        const uint16_t* pb = &Vs[buf][(ks * 16 + tr_row) * C::ST + d2t * 32 + tr_col];
        const u32x2 a0 = lds_tr16(pa), a1 = lds_tr16(pa + 8 * C::ST);
        const u32x2 b0 = lds_tr16(pb), b1 = lds_tr16(pb + 8 * C::ST);
        const u32x4 av = {a0[0], a0[1], a1[0], a1[1]};
        const u32x4 bv = {b0[0], b0[1], b1[0], b1[1]};
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                         __builtin_bit_cast(bf16x8, bv), acc[i], 0, 0, 0);
      }
    }
    if (t + 1 < ntile) stage(buf ^ 1, n0 + (t + 1) * kLinTok);
    __syncthreads();
  }

  // partial S: acc[i][r] = S[d1t*32 + 8*(r/4) + 4*hi + r%4][d2t*32 + l32]
  float* ps = a.part_s + ((int64_t)bh * a.splits + split) * D * D;
  const int l32 = lane & 31;
#pragma unroll
  for (int i = 0; i < C::TPW; ++i) {
    const int tile = wave * C::TPW + i;
    const int d1t = tile / C::NT32, d2t = tile % C::NT32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int d1 = d1t * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
      ps[d1 * D + d2t * 32 + l32] = acc[i][r];
    }
  }
  // partial z: reduce the per-thread column sums over the RS row groups, in the
  // K stage (free after the loop's last barrier)
  static_assert(RS * D * 4 <= kLinTok * C::ST * 2, "z scratch does not fit the stage");
  float(*zred)[D] = reinterpret_cast<float(*)[D]>(&Ks[0][0]);
#pragma unroll
  for (int e = 0; e < 8; ++e) zred[rr][cc * 8 + e] = zacc[e];
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
    for (int g = 0; g < RS; ++g) s += zred[g][tid];
    a.part_z[((int64_t)bh * a.splits + split) * D + tid] = s;
  }
}

struct LinReduceArgs {
  const float* part_s;
  const float* part_z;
  float* S;          // nullable [BH][D][D]
  float* z;          // nullable [BH][D]
  uint16_t* st_bf;   // [BH][D][D] = S^T in bf16
  float* z_ws;       // [BH][D]
  int splits;
};

template <int D>
__global__ void __launch_bounds__(256) lin_reduce_kernel(LinReduceArgs a) {
  const int bh = blockIdx.y;
  const int idx = blockIdx.x * 256 + threadIdx.x;  // element of S (row-major d1, d2)
  const float* ps = a.part_s + (int64_t)bh * a.splits * D * D;
  if (idx < D * D) {
    float s = 0.f;
    for (int p = 0; p < a.splits; ++p) s += ps[(int64_t)p * D * D + idx];
    const int d1 = idx / D, d2 = idx % D;
    if (a.S) a.S[(int64_t)bh * D * D + idx] = s;
    a.st_bf[(int64_t)bh * D * D + d2 * D + d1] = (uint16_t)f2bf(s);
  }
  if (blockIdx.x == 0 && threadIdx.x < D) {
    const float* pz = a.part_z + (int64_t)bh * a.splits * D;
    float s = 0.f;
    for (int p = 0; p < a.splits; ++p) s += pz[p * D + threadIdx.x];
    a.z_ws[bh * D + threadIdx.x] = s;
    if (a.z) a.z[bh * D + threadIdx.x] = s;
  }
}

constexpr int kApplyRows = 128;      // queries per tile (4 waves x 32)
constexpr int kApplyTiles = 4;       // tiles per workgroup

struct LinApplyArgs {
  const uint16_t* q;
  uint16_t* o;
  const uint16_t* st_bf;
  const float* z_ws;
  int64_t sb, sh, sn;
  int H, N;
};

template <int D>
__global__ void __launch_bounds__(256) lin_apply_kernel(LinApplyArgs a) {
  constexpr int SST = D + 8;       // S^T stage stride (16 rows per 16 lanes cover all banks)
  constexpr int KT = D / 16, DT = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t Ss[D * SST];
  __shared__ float zs[D];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int bh = blockIdx.y;
  const int b = bh / a.H, h = bh % a.H;
  const int64_t head_off = (int64_t)b * a.sb + (int64_t)h * a.sh;

  const uint16_t* st = a.st_bf + (int64_t)bh * D * D;
  for (int c = tid; c < D * D / 8; c += 256) {
    const int row = c / (D / 8), col = (c % (D / 8)) * 8;
    *(u32x4*)&Ss[row * SST + col] = *(const u32x4*)(st + row * D + col);
  }
  if (tid < D) zs[tid] = a.z_ws[bh * D + tid];
  __syncthreads();

  for (int tile = 0; tile < kApplyTiles; ++tile) {
    const int q0 = (blockIdx.x * kApplyTiles + tile) * kApplyRows;
    if (q0 >= a.N) break;
    const int qrow = q0 + wave * 32 + l32;
    const uint16_t* src = a.q + head_off + (int64_t)min(qrow, a.N - 1) * a.sn + hi * 8;
    u32x4 qr[KT];
#pragma unroll
    for (int t = 0; t < KT; ++t) qr[t] = *(const u32x4*)(src + t * 16);
    bf16x8 qf[KT];
    float den = 0.f;
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = t * 16 + hi * 8 + 2 * e;
        const float f0 = phi(bf16_lo(qr[t][e])), f1 = phi(bf16_hi(qr[t][e]));
        den = __builtin_fmaf(f0, zs[d], den);
        den = __builtin_fmaf(f1, zs[d + 1], den);
        w[e] = pack_bf16x2(f0, f1);
      }
      qf[t] = __builtin_bit_cast(bf16x8, w);
    }
    {
      den = pair_sum(den);
    }
    f32x16 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      o[dt] = f32x16{};
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        const bf16x8 sf = *(const bf16x8*)&Ss[(dt * 32 + l32) * SST + t * 16 + hi * 8];
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sf, qf[t], o[dt], 0, 0, 0);
      }
    }
    if (qrow < a.N) {
      const float inv = 1.f / den;
      uint16_t* dst = a.o + head_off + (int64_t)qrow * a.sn;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = dt * 32 + 8 * g + 4 * hi;
          u32x2 w = {pack_bf16x2(o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv),
                     pack_bf16x2(o[dt][4 * g + 2] * inv, o[dt][4 * g + 3] * inv)};
          *(u32x2*)(dst + d0) = w;
        }
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

struct LinPlan {
  int splits, chunk;
  size_t off_part_s, off_part_z, off_st, off_z, total;
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

LinPlan linear_plan(const bsa_shape& s) {
  LinPlan p;
  const int64_t bh = (int64_t)s.B * s.H;
  // about two workgroups per CU in total, at least one 64-token tile each
  int64_t want = (512 + bh - 1) / bh;
  const int64_t tiles = (s.N + kLinTok - 1) / kLinTok;
  if (want > tiles) want = tiles;
  if (want < 1) want = 1;
  const int64_t per = (tiles + want - 1) / want;
  p.chunk = (int)(per * kLinTok);
  p.splits = (int)((s.N + p.chunk - 1) / p.chunk);
  const size_t D = s.D;
  p.off_part_s = 0;
  p.off_part_z = align256(p.off_part_s + (size_t)bh * p.splits * D * D * 4);
  p.off_st = align256(p.off_part_z + (size_t)bh * p.splits * D * 4);
  p.off_z = align256(p.off_st + (size_t)bh * D * D * 2);
  p.total = align256(p.off_z + (size_t)bh * D * 4);
  return p;
}

bsa_status launch_linear_attn(const void* q, const void* k, const void* v, void* o, const bsa_shape& s,
                              float* S, float* z, void* ws, hipStream_t stream) {
  const LinPlan p = linear_plan(s);
  char* w = (char*)ws;
  const int bh = s.B * s.H;
  LinStateArgs sa{(const uint16_t*)k, (const uint16_t*)v, (float*)(w + p.off_part_s),
                  (float*)(w + p.off_part_z), s.stride_b, s.stride_h, s.stride_n, s.H, s.N, p.splits, p.chunk};
  LinReduceArgs ra{(const float*)(w + p.off_part_s), (const float*)(w + p.off_part_z), S, z,
                   (uint16_t*)(w + p.off_st), (float*)(w + p.off_z), p.splits};
  LinApplyArgs aa{(const uint16_t*)q, (uint16_t*)o, (const uint16_t*)(w + p.off_st),
                  (const float*)(w + p.off_z), s.stride_b, s.stride_h, s.stride_n, s.H, s.N};
  const int row_groups = (s.N + kApplyRows * kApplyTiles - 1) / (kApplyRows * kApplyTiles);
  if (s.D == 128) {
    hipLaunchKernelGGL(lin_state_kernel<128>, dim3(p.splits, bh), dim3(kLinThreads), 0, stream, sa);
    hipLaunchKernelGGL(lin_reduce_kernel<128>, dim3(128 * 128 / 256, bh), dim3(256), 0, stream, ra);
    hipLaunchKernelGGL(lin_apply_kernel<128>, dim3(row_groups, bh), dim3(256), 0, stream, aa);
  } else if (s.D == 64) {
    hipLaunchKernelGGL(lin_state_kernel<64>, dim3(p.splits, bh), dim3(kLinThreads), 0, stream, sa);
    hipLaunchKernelGGL(lin_reduce_kernel<64>, dim3(64 * 64 / 256, bh), dim3(256), 0, stream, ra);
    hipLaunchKernelGGL(lin_apply_kernel<64>, dim3(row_groups, bh), dim3(256), 0, stream, aa);
  } else {
    return BSA_ERR_UNSUPPORTED;
  }
  return launch_ok("linear_attn_fwd") ? BSA_OK : BSA_ERR_HIP;
}

}  // namespace bsa
