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

#include <mutex>

#include "launch.h"

namespace bsa {

// elu(x) + 1 = max(1 + x, min(e^x, 1)): for x > 0 the clamped exponential is 1
// and 1 + x wins; for x <= 0, e^x >= 1 + x (convexity) and the exponential
// wins.  The clamp is the exp instruction's output modifier, so this is a
// multiply, the exp, an add and a max (no compare / select); it can differ from
// the branch form only where e^x and 1 + x agree to about an fp32 ulp (|x| < 5e-4)
__device__ __forceinline__ float phi(float x) {
  return fmaxf(x + 1.f, __builtin_amdgcn_fmed3f(__builtin_amdgcn_exp2f(x * kLog2e), 0.f, 1.f));
}

// In the non-causal call Q, K, V are read once and O written once: their
// loads, LDS copies and stores carry the non-temporal cache policy, so the
// stream does not evict lines that others reuse (a plain copy streams read +
// write about 9 % faster with it on this memory system; the call at 32K took
// 0.106 ms instead of 0.124 ms).  Cache-policy operand of the buffer copies:
// bit 1 = nt.
constexpr int kNt = 2;
// The causal path reads K and V twice (state pass, then the walk), so those
// copies keep the default policy; only the walk's Q copies are non-temporal
// (0.180 -> 0.173 ms at 32K).  Its O stores stay default as well: they are
// 8-byte pieces of rows, and non-temporal partial-line stores made the call
// take 0.29 ms.

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

// head_dim 128 state kernel.  K and V tiles of 32 tokens go straight from
// global memory to LDS with buffer loads into a ring of five stages (ten
// distinct LDS objects, 80 KiB, the loop unrolled by five so no LDS read ever
// waits for a copy in flight): four tiles are in flight while one is computed,
// 128 KiB per CU at two workgroups per CU, to cover the memory latency.  Rows
// are swizzled for the transpose read.  Wave w owns S rows d1 in
// [32w, 32w + 32) and all four 32-column blocks of d2: its phi(K)^T fragment
// (A operand) is read once per 16 tokens, phi is applied in fp32 (rows past
// the split's end set to 0), the values are summed into the lane's z partial
// for d1 = 32w + lane % 32 and rounded to bf16; the V fragments (B operand)
// come from the same transpose read.  Element e of a fragment read for token
// group ks is token 16 ks + 8 (e / 4) + 4 (lane / 32) + e % 4 of the tile.
constexpr int kLinTok2 = 32;  // tokens per tile of the head_dim-128 state kernel

// CP: cache policy of the K and V copies (kNt when nothing reads K and V
// again in the call, 0 when the causal walk does)
template <int CP>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
lin_state_d128_kernel(LinStateArgs a) {
  constexpr int D = 128, TILE = kLinTok2 * D;
  __shared__ __attribute__((aligned(1024))) uint16_t K0[TILE], K1[TILE], K2[TILE], K3[TILE], K4[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t V0[TILE], V1[TILE], V2[TILE], V3[TILE], V4[TILE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hi = lane >> 5;
  const int g16 = lane >> 4, j16 = lane & 15;
  const int split = blockIdx.x, bh = blockIdx.y;
  const int b = bh / a.H, h = bh % a.H;
  const int64_t head_off = (int64_t)b * a.sb + (int64_t)h * a.sh;
  const int n0 = split * a.chunk, n1 = min(n0 + a.chunk, a.N);
  const int ntile = (n1 - n0 + kLinTok2 - 1) / kLinTok2;

  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t row_bytes = (uint32_t)a.sn * 2u;
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.k + head_off), (short)0, 0x7fffffff, kBufferWord3);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.v + head_off), (short)0, 0x7fffffff, kBufferWord3);
  // copy roles: wave w, instruction j covers tile rows 8w + 4j + lane/16
  uint32_t off[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = 8 * wv + 4 * j + (lane >> 4);
    off[j] = (uint32_t)row * row_bytes + (uint32_t)(((lane & 15) ^ swz_v(row)) * 16);
  }
  // each wave issues 4 copy instructions per tile
  auto dma = [&](uint16_t* kst, uint16_t* vst, int t0) {
    if (t0 + kLinTok2 <= a.N) {
      const uint32_t so = (uint32_t)t0 * row_bytes;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)&kst[(8 * wv + 4 * j) * D], 16, off[j], so, 0, CP);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)&vst[(8 * wv + 4 * j) * D], 16, off[j], so, 0, CP);
      }
    } else {  // last tile of the sequence: rows past N are clamped to row N - 1 (masked below)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = 8 * wv + 4 * j + (lane >> 4);
        const uint32_t o = (uint32_t)min(t0 + row, a.N - 1) * row_bytes +
                           (uint32_t)(((lane & 15) ^ swz_v(row)) * 16);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)&kst[(8 * wv + 4 * j) * D], 16, o, 0, 0, CP);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)&vst[(8 * wv + 4 * j) * D], 16, o, 0, 0, CP);
      }
    }
  };

  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
  float zl = 0.f;
  // transpose reads (token group ks, 32-column block dt of the tile; rows +8
  // for the second half of the fragment) as byte offsets base ^ immediate:
  //   va2 ^ (4096 ks + 64 dt)  and  va2 ^ (4096 ks + 64 dt + 2080)
  // (the K and V stages are both swizzled with swz_v; the identities are
  // checked for every lane on the host)
  const int q4 = j16 >> 2, c0 = 2 * (g16 & 1) + ((j16 >> 1) & 1), half4 = (j16 & 1) * 4;
  const uint32_t va2 = 2 * ((4 * hi + q4) * D + 32 * q4 + 8 * (c0 ^ hi) + half4);
  const uint32_t kw2 = va2 ^ (64 * wave);  // this wave's K rows d1 = 32 w + ...
  auto tr_frag = [&](const uint16_t* st, uint32_t base, uint32_t imm) -> u32x4 {
    const u32x2 x0 = lds_tr16(lds_byte(st, base ^ imm)), x1 = lds_tr16(lds_byte(st, base ^ (imm + 2080)));
    return u32x4{x0[0], x0[1], x1[0], x1[1]};
  };

  // tile t sits in stage t % 5; at its step the copies of tiles t + 1 .. t + 3
  // may still be in flight (4 instructions each per wave), and the copy of
  // tile t + 4 is issued into the stage that tile t - 1 used
  auto step = [&](const uint16_t* Kb, const uint16_t* Vb, uint16_t* Kn, uint16_t* Vn, int t) {
    const int t0 = n0 + t * kLinTok2;
    const int ahead = ntile - 1 - t;  // tiles after t already issued: min(ahead, 3)
    if (ahead >= 3) __builtin_amdgcn_s_waitcnt(0x007C);       // vmcnt(12) lgkmcnt(0)
    else if (ahead == 2) __builtin_amdgcn_s_waitcnt(0x0078);  // vmcnt(8) lgkmcnt(0)
    else if (ahead == 1) __builtin_amdgcn_s_waitcnt(0x0074);  // vmcnt(4) lgkmcnt(0)
    else __builtin_amdgcn_s_waitcnt(0x0070);                  // vmcnt(0) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    if (t + 4 < ntile) dma(Kn, Vn, t0 + 4 * kLinTok2);
    uint32_t kw = kw2, va = va2;
    asm volatile("" : "+v"(kw), "+v"(va));
    const int lim = n1 - t0 - 4 * hi;  // element e is a real token iff 16 ks + 8 (e / 4) + e % 4 < lim
    const bool full = n1 - t0 >= kLinTok2;  // uniform: no token of the tile is past the split's end
#pragma unroll
    for (int ks = 0; ks < kLinTok2 / 16; ++ks) {
      const u32x4 kr = tr_frag(Kb, kw, 4096 * ks);
      u32x4 vr[4];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) vr[dt] = tr_frag(Vb, va, 4096 * ks + 64 * dt);
      u32x4 kp;
      if (full) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float f0 = phi(bf16_lo(kr[w])), f1 = phi(bf16_hi(kr[w]));
          zl += f0 + f1;
          kp[w] = pack_bf16x2(f0, f1);
        }
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int e0 = 2 * w, e1 = 2 * w + 1;
          float f0 = phi(bf16_lo(kr[w])), f1 = phi(bf16_hi(kr[w]));
          if (16 * ks + 8 * (e0 >> 2) + (e0 & 3) >= lim) f0 = 0.f;
          if (16 * ks + 8 * (e1 >> 2) + (e1 & 3) >= lim) f1 = 0.f;
          zl += f0 + f1;
          kp[w] = pack_bf16x2(f0, f1);
        }
      }
      const bf16x8 af = __builtin_bit_cast(bf16x8, kp);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, __builtin_bit_cast(bf16x8, vr[dt]), acc[dt], 0, 0, 0);
    }
  };

  if (ntile > 0) dma(K0, V0, n0);
  if (ntile > 1) dma(K1, V1, n0 + kLinTok2);
  if (ntile > 2) dma(K2, V2, n0 + 2 * kLinTok2);
  if (ntile > 3) dma(K3, V3, n0 + 3 * kLinTok2);
  int t = 0;
  for (; t + 5 <= ntile; t += 5) {
    step(K0, V0, K4, V4, t);
    step(K1, V1, K0, V0, t + 1);
    step(K2, V2, K1, V1, t + 2);
    step(K3, V3, K2, V2, t + 3);
    step(K4, V4, K3, V3, t + 4);
  }
  if (t < ntile) step(K0, V0, K4, V4, t);
  if (t + 1 < ntile) step(K1, V1, K0, V0, t + 1);
  if (t + 2 < ntile) step(K2, V2, K1, V1, t + 2);
  if (t + 3 < ntile) step(K3, V3, K2, V2, t + 3);

  // partial S: acc[dt][r] = S[32 w + 8 (r / 4) + 4 hi + r % 4][32 dt + lane % 32]
  float* ps = a.part_s + ((int64_t)bh * a.splits + split) * D * D;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int d1 = 32 * wave + 8 * (r >> 2) + 4 * hi + (r & 3);
      ps[d1 * D + 32 * dt + l32] = acc[dt][r];
    }
  const float z = pair_sum(zl);
  if (hi == 0) a.part_z[((int64_t)bh * a.splits + split) * D + 32 * wave + l32] = z;
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

// 256 threads = 32 float4 columns of S x 8 groups of splits; each thread sums
// its group's splits in order, then the 8 group sums are added in group order
// (a fixed order: deterministic).  One workgroup per 128 elements of S.
constexpr int kRedGroups = 8, kRedCols = 256 / kRedGroups;

template <int D>
__global__ void __launch_bounds__(256) lin_reduce_kernel(LinReduceArgs a) {
  __shared__ float4 part[kRedGroups][kRedCols];
  const int bh = blockIdx.y, tid = threadIdx.x;
  const int c4 = tid % kRedCols, g = tid / kRedCols;
  const int idx4 = blockIdx.x * kRedCols + c4;  // float4 index into S (row-major d1, d2)
  const float4* ps = reinterpret_cast<const float4*>(a.part_s + (int64_t)bh * a.splits * D * D);
  const int per = (a.splits + kRedGroups - 1) / kRedGroups;
  const int p0 = g * per, p1 = min(p0 + per, a.splits);
  float4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (int p = p0; p < p1; ++p) {
    const float4 x = ps[(int64_t)p * (D * D / 4) + idx4];
    acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
  }
  part[g][c4] = acc;
  __syncthreads();
  if (g == 0) {
    float4 t = part[0][c4];
#pragma unroll
    for (int q = 1; q < kRedGroups; ++q) {
      const float4 x = part[q][c4];
      t.x += x.x; t.y += x.y; t.z += x.z; t.w += x.w;
    }
    const int e = idx4 * 4, d1 = e / D, d2 = e % D;
    if (a.S) reinterpret_cast<float4*>(a.S + (int64_t)bh * D * D)[idx4] = t;
    uint16_t* st = a.st_bf + (int64_t)bh * D * D;
    st[(d2 + 0) * D + d1] = (uint16_t)f2bf(t.x);
    st[(d2 + 1) * D + d1] = (uint16_t)f2bf(t.y);
    st[(d2 + 2) * D + d1] = (uint16_t)f2bf(t.z);
    st[(d2 + 3) * D + d1] = (uint16_t)f2bf(t.w);
  }
  if (blockIdx.x == 0 && tid < D) {
    const float* pz = a.part_z + (int64_t)bh * a.splits * D;
    float z = 0.f;
#pragma unroll 8
    for (int p = 0; p < a.splits; ++p) z += pz[p * D + tid];
    a.z_ws[bh * D + tid] = z;
    if (a.z) a.z[bh * D + tid] = z;
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
  int tph, total, tpw;  // head_dim 128 kernel: tiles per head, all tiles, tiles per workgroup
  float mix_r;          // head_dim 128 kernel: < 0 plain; else o = mix_r * o + (1 - mix_r) * linear
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

// head_dim 128 apply.  The (batch, head, 128-query tile) items are dealt to
// workgroups in equal contiguous runs of tpw items (one round of workgroups
// covers the whole job).  S^T (bf16, rows d2 swizzled) and z are staged in
// LDS with buffer loads whenever the run enters a new head.  Global traffic is
// row-contiguous: a wave loads its 32 Q rows of the next tile with 16-byte
// loads that cover 4 whole rows per instruction (issued before the current
// tile's compute, so one tile is always in flight), writes them into its own
// 8 KiB LDS region (rows swizzled like the K stages), reads the MFMA operand
// fragments back from there, and sends O the same way in reverse: the
// accumulators go to the region, whole rows come back and are stored with
// 16-byte stores.  The region is private to the wave, so no barrier is needed.
__global__ void __launch_bounds__(256) lin_apply_d128_kernel(LinApplyArgs a) {
  constexpr int D = 128, KT = 8, DT = 4, RW = 32;  // rows per wave
  __shared__ __attribute__((aligned(1024))) uint16_t Ss[D * D];
  __shared__ __attribute__((aligned(1024))) uint16_t Xs[4 * RW * D];
  __shared__ float zs[D];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int it0 = blockIdx.x * a.tpw, it1 = min(it0 + a.tpw, a.total);
  if (it0 >= it1) return;
  uint16_t* X = Xs + wv * RW * D;
  // element offset of 16-byte chunk c of wave row r in the region
  auto xoff = [](int r, int c) { return r * D + 8 * (c ^ (r & 15)); };

  auto stage_head = [&](int bh) {
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.st_bf + (int64_t)bh * D * D), (short)0, D * D * 2, kBufferWord3);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = 32 * wv + 4 * j + (lane >> 4);
      const uint32_t o = (uint32_t)row * (D * 2) + (uint32_t)(((lane & 15) ^ swz_k(row)) * 16);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, (lds_void*)&Ss[(32 * wv + 4 * j) * D], 16, o, 0, 0, 0);
    }
    if (tid < D) zs[tid] = a.z_ws[bh * D + tid];
  };
  auto head_off = [&](int bh) { return (int64_t)(bh / a.H) * a.sb + (int64_t)(bh % a.H) * a.sh; };
  // instruction i covers wave rows 4 i + lane / 16, chunk lane % 16
  auto q_load = [&](int item, u32x4 (&buf)[8]) {
    const int bh = item / a.tph, tile = item % a.tph;
    const uint16_t* base = a.q + head_off(bh) + 8 * (lane & 15);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = min(tile * kApplyRows + RW * wv + 4 * i + (lane >> 4), a.N - 1);
      buf[i] = __builtin_nontemporal_load((const u32x4*)(base + (int64_t)row * a.sn));
    }
  };

  u32x4 qb[8];
  q_load(it0, qb);
  int cur_bh = -1;
  for (int it = it0; it < it1; ++it) {
    const int bh = it / a.tph, tile = it % a.tph;
    if (bh != cur_bh) {
      __syncthreads();  // every wave is done with the previous head's S^T
      stage_head(bh);
      __builtin_amdgcn_s_waitcnt(0x0070);
      __syncthreads();
      cur_bh = bh;
    }
    // this tile's Q rows into the region, then the next tile's loads
#pragma unroll
    for (int i = 0; i < 8; ++i) *(u32x4*)&X[xoff(4 * i + (lane >> 4), lane & 15)] = qb[i];
    if (it + 1 < it1) q_load(it + 1, qb);
    // B operand: lane (l32, hi) takes row l32, head dims 16 t + 8 hi .. + 7
    bf16x8 qf[KT];
    float den = 0.f;
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      const u32x4 raw = *(const u32x4*)&X[xoff(l32, 2 * t + hi)];
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = t * 16 + hi * 8 + 2 * e;
        const float f0 = phi(bf16_lo(raw[e])), f1 = phi(bf16_hi(raw[e]));
        den = __builtin_fmaf(f0, zs[d], den);
        den = __builtin_fmaf(f1, zs[d + 1], den);
        w[e] = pack_bf16x2(f0, f1);
      }
      qf[t] = __builtin_bit_cast(bf16x8, w);
    }
    den = pair_sum(den);
    f32x16 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      o[dt] = f32x16{};
      const int row = dt * 32 + l32;
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        const bf16x8 sf = *(const bf16x8*)&Ss[row * D + (((2 * t + hi) ^ swz_k(row)) << 3)];
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sf, qf[t], o[dt], 0, 0, 0);
      }
    }
    // O^T accumulators -> region (row l32, head dims 32 dt + 8 g + 4 hi .. + 3)
    const float inv = 1.f / den;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w = {pack_bf16x2(o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv),
                   pack_bf16x2(o[dt][4 * g + 2] * inv, o[dt][4 * g + 3] * inv)};
        *(u32x2*)&X[xoff(l32, 4 * dt + g) + 4 * hi] = w;
      }
    // whole rows back out, 16-byte stores (rows past N are not stored); in the
    // mixed form each row is first blended with the row already in o
    uint16_t* obase = a.o + head_off(bh) + 8 * (lane & 15);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 4 * i + (lane >> 4);
      u32x4 v = *(const u32x4*)&X[xoff(r, lane & 15)];
      const int row = tile * kApplyRows + RW * wv + r;
      if (row < a.N) {
        if (a.mix_r >= 0.f) {
          const u32x4 sft = __builtin_nontemporal_load((const u32x4*)(obase + (int64_t)row * a.sn));
          const float wl = 1.f - a.mix_r;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            v[e] = pack_bf16x2(__builtin_fmaf(a.mix_r, bf16_lo(sft[e]), wl * bf16_lo(v[e])),
                               __builtin_fmaf(a.mix_r, bf16_hi(sft[e]), wl * bf16_hi(v[e])));
        }
        __builtin_nontemporal_store(v, (u32x4*)(obase + (int64_t)row * a.sn));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Causal (chunked) linear attention, head_dim 128.
//
//   out_n = phi(q_n)^T S_n / phi(q_n)^T z_n,  S_n = S0 + sum_{m <= n} phi(k_m) v_m^T,
//   z_n = z0 + sum_{m <= n} phi(k_m),
// with (S0, z0) the state carried in from earlier tokens (zero if none).
//
// Three launches:
//   state  : lin_state_d128_kernel over token splits of chunk_s tokens.
//   prefix : per head, the split partials are summed in order; every f-th split
//            is overwritten with the state before it (exclusive prefix, starting
//            from the carried state), and the state after the last token is the
//            optional output.
//   causal : grid (apply splits, B*H), an apply split being f state splits.  A
//            workgroup walks its split in steps of 32 tokens, holding the running
//            state in MFMA accumulators (wave w owns S columns d2 in
//            [32w, 32w+32)) and z in LDS.  Per step:
//              - Q, K, V tiles arrive by buffer loads into a ring of three stages
//                (rows swizzled for the transpose read), two steps ahead;
//              - phi is applied in place to the K and Q tiles (fp32, rounded to
//                bf16; K rows past the split are zeroed), the fp32 phi(k) column
//                sums go to z and phi(q_n) . z_prev to a per-row LDS slot;
//              - every wave computes the 32 x 32 score tile A^T = phi(K) phi(Q)^T
//                of the step (keys x queries) and masks keys after the query;
//              - wave w produces output columns d2 in [32w, 32w+32):
//                O^T = S_prev^T phi(Q)^T + V^T A^T (the P operand of the second
//                product is the masked score accumulator, as in the softmax
//                kernel's O^T += V^T P^T);
//              - the denominator is phi(q_n) . z_prev plus the masked score row
//                sum;
//              - the state takes the step: S += phi(K)^T V (its bf16 rounding
//                for the inter-step product is taken from the accumulators
//                before the update).
// ---------------------------------------------------------------------------

struct LinPrefixArgs {
  float* part_s;       // [BH][splits][D][D]: partials in; exclusive prefix at every f-th split out
  float* part_z;       // [BH][splits][D]
  const float* s_in;   // nullable [BH][D][D] carried state
  const float* z_in;   // nullable [BH][D]
  float* s_out;        // nullable [BH][D][D] state after the sequence (may alias s_in)
  float* z_out;        // nullable [BH][D]
  int splits, f;
};

// one thread per float4 column of a head's S (or z); reads every partial once,
// in split order (deterministic).  The partials are loaded 16 splits at a time
// (one memory round trip per 16 splits, not per split).
template <int C4>
__device__ __forceinline__ void prefix_column(float4* __restrict__ p, const float4* in, float4* out, int idx,
                                              int splits, int f) {
  constexpr int U = 16;
  float4 run = in ? in[idx] : float4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < splits; s0 += U) {
    float4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      x[u] = s0 + u < splits ? p[(int64_t)(s0 + u) * C4 + idx] : float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + u;
      if (s < splits && s % f == 0) p[(int64_t)s * C4 + idx] = run;
      run.x += x[u].x; run.y += x[u].y; run.z += x[u].z; run.w += x[u].w;
    }
  }
  if (out) out[idx] = run;
}

// grid (17, BH): blocks 0..15 scan S (4096 float4 columns), block 16 scans z
__global__ void __launch_bounds__(256) lin_prefix_d128_kernel(LinPrefixArgs a) {
  constexpr int D = 128;
  const int bh = blockIdx.y, tid = threadIdx.x;
  if (blockIdx.x < 16) {
    const int64_t h = (int64_t)bh * D * D;
    prefix_column<D * D / 4>((float4*)(a.part_s + h * a.splits), a.s_in ? (const float4*)(a.s_in + h) : nullptr,
                             a.s_out ? (float4*)(a.s_out + h) : nullptr, blockIdx.x * 256 + tid, a.splits, a.f);
  } else if (tid < D / 4) {
    const int64_t h = (int64_t)bh * D;
    prefix_column<D / 4>((float4*)(a.part_z + h * a.splits), a.z_in ? (const float4*)(a.z_in + h) : nullptr,
                         a.z_out ? (float4*)(a.z_out + h) : nullptr, tid, a.splits, a.f);
  }
}

struct CausalArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  const float* pre_s;  // [BH][splits_s][D][D]: state before state split j (j a multiple of f)
  const float* pre_z;  // [BH][splits_s][D]
  int64_t sb, sh, sn;
  int H, N, chunk, splits_s, f;
};

constexpr int kCT = 32;  // tokens per step of the causal kernel

// compiler-only ordering point next to a hardware barrier (emits nothing)
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};

// sum over the 16 lanes of a DPP row (every lane gets the sum)
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp_f<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp_f<0x141>(x);  // row_half_mirror
  x += dpp_f<0x140>(x);  // row_mirror
  return x;
}

// x + x of lane ^ 16
__device__ __forceinline__ float xor16_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Wave w owns the state columns d2 in [32w, 32w + 32): acc[t][r] =
// S[32 t + 8 (r / 4) + 4 hi + r % 4][32 w + l32].  That block, rounded to bf16,
// is the A operand of the inter-step product O^T[d2 in the wave's block] =
// S^T phi(Q)^T: for k-step f (d1 in [16 f, 16 f + 16)) the two halves of the
// wave swap the 4-value groups they do not hold, after which lane (l32, hi)
// has d1 = 16 f + 8 hi .. + 7 like the phi(Q) row fragment (one 16-byte read).
// No copy of S goes through LDS; LDS holds the tile ring (72 KiB) and z, so
// two workgroups fit a CU.
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
causal_lin_d128_kernel(CausalArgs a) {
  constexpr int D = 128, TILE = kCT * D;
  // ring stage s: Q and K tiles in QKs (Q first), V in Vs.  Six objects: the
  // compiler tells the copies into one stage from the reads of another only
  // for a few distinct LDS objects (with nine it made the tile reads wait for
  // the copies of the next tiles)
  __shared__ __attribute__((aligned(1024))) uint16_t QK0[2 * TILE], QK1[2 * TILE], QK2[2 * TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t V0[TILE], V1[TILE], V2[TILE];
  uint16_t *const Q0 = QK0, *const Q1 = QK1, *const Q2 = QK2;
  uint16_t *const K0 = QK0 + TILE, *const K1 = QK1 + TILE, *const K2 = QK2 + TILE;
  __shared__ __attribute__((aligned(16))) float zs[2][D];
  __shared__ __attribute__((aligned(16))) float zred[4][D];
  __shared__ float dq[kCT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hi = lane >> 5;
  const int g16 = lane >> 4, j16 = lane & 15;
  const int split = blockIdx.x, bh = blockIdx.y;
  const int64_t head_off = (int64_t)(bh / a.H) * a.sb + (int64_t)(bh % a.H) * a.sh;
  const int n0 = split * a.chunk, n1 = min(n0 + a.chunk, a.N);
  const int nch = (n1 - n0 + kCT - 1) / kCT;

  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t row_bytes = (uint32_t)a.sn * 2u;
  const __amdgpu_buffer_rsrc_t qrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.q + head_off), (short)0, 0x7fffffff, kBufferWord3);
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.k + head_off), (short)0, 0x7fffffff, kBufferWord3);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.v + head_off), (short)0, 0x7fffffff, kBufferWord3);
  // copy roles: wave w, instruction j covers tile rows 8w + 4j + lane/16
  uint32_t off[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = 8 * wv + 4 * j + (lane >> 4);
    off[j] = (uint32_t)row * row_bytes + (uint32_t)(((lane & 15) ^ swz_v(row)) * 16);
  }
  // six copy instructions per wave and step
  auto dma = [&](uint16_t* qs, uint16_t* ks, uint16_t* vs, int t0) {
    if (t0 + kCT <= a.N) {
      const uint32_t so = (uint32_t)t0 * row_bytes;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = (8 * wv + 4 * j) * D;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(qrs, (lds_void*)&qs[r], 16, off[j], so, 0, kNt);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)&ks[r], 16, off[j], so, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)&vs[r], 16, off[j], so, 0, 0);
      }
    } else {  // the sequence's last tile: rows past N repeat row N - 1 (zeroed or not stored)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = 8 * wv + 4 * j + (lane >> 4);
        const uint32_t o = (uint32_t)min(t0 + row, a.N - 1) * row_bytes +
                           (uint32_t)(((lane & 15) ^ swz_v(row)) * 16);
        const int r = (8 * wv + 4 * j) * D;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(qrs, (lds_void*)&qs[r], 16, o, 0, 0, kNt);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)&ks[r], 16, o, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)&vs[r], 16, o, 0, 0, 0);
      }
    }
  };
  // transpose read: lane (l32, hi) gets column 32 dt + l32 at the tile rows
  // 16 ks + 8 (e / 4) + 4 hi + e % 4, e = 0..7 (the accumulator row order)
  auto tr_frag = [&](const uint16_t* st, int ks, int dt) -> bf16x8 {
    const int r0 = ks * 16 + 4 * hi + (j16 >> 2), r1 = r0 + 8;
    const int lc = 4 * dt + 2 * (g16 & 1) + ((j16 & 3) >> 1);
    const int half = (j16 & 1) * 4;
    const u32x2 x0 = lds_tr16(&st[r0 * D + ((lc ^ swz_v(r0)) << 3) + half]);
    const u32x2 x1 = lds_tr16(&st[r1 * D + ((lc ^ swz_v(r1)) << 3) + half]);
    return __builtin_bit_cast(bf16x8, u32x4{x0[0], x0[1], x1[0], x1[1]});
  };
  // row fragment f of tile row r: head dims 16 f + 8 hi .. + 7 (one 16-byte chunk)
  auto row_frag = [&](const uint16_t* st, int r, int f) -> bf16x8 {
    return *(const bf16x8*)&st[r * D + (((2 * f + hi) ^ swz_v(r)) << 3)];
  };

  // state at the split's first token
  f32x16 acc[4];
  {
    const int64_t j = (int64_t)bh * a.splits_s + (int64_t)split * a.f;
    const float* ps = a.pre_s + j * D * D + 32 * wave + l32;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[t][r] = ps[(32 * t + 8 * (r >> 2) + 4 * hi + (r & 3)) * D];
    if (tid < D) zs[0][tid] = a.pre_z[j * D + tid];
  }
  // the state loads retire here, before any tile copy: the step waits count
  // the copies and stores only (and the compiler then adds no wait for them
  // inside the loop)
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
  if (nch > 0) dma(Q0, K0, V0, n0);
  if (nch > 1) dma(Q1, K1, V1, n0 + kCT);

  const int cc = tid & 15;            // phi pass: logical 16-byte chunk
  const int prow = tid >> 4;          // phi pass: tile rows prow and prow + 16
  uint16_t* obase = a.o + head_off + 32 * wave + 4 * hi;

  auto step = [&](uint16_t* Qb, uint16_t* Kb, uint16_t* Vb, uint16_t* Qn, uint16_t* Kn, uint16_t* Vn, int c) {
    const int t0 = n0 + c * kCT;
    const float* zp = zs[c & 1];
    // Wait for this step's tile.  The copies (loads) retire in issue order;
    // the output stores in between may retire in any order relative to them,
    // so the count allows only the loads issued after tile c's: the 6 copies
    // of tile c + 1 (issued at the top of step c - 1, or before the loop), if
    // there is such a tile.  (lgkmcnt(0) as well.)
    if (c + 1 < nch) __builtin_amdgcn_s_waitcnt(0x0076);  // vmcnt(6)
    else __builtin_amdgcn_s_waitcnt(0x0070);              // vmcnt(0)
    lds_barrier();
    // the tile two steps ahead goes into the stage of step c - 1: every wave
    // has passed this barrier, so none still reads it
    if (c + 2 < nch) dma(Qn, Kn, Vn, t0 + 2 * kCT);

    // phi in place on the K and Q tiles; z and phi(q) . z_prev partials in fp32
    // (K rows past the split are zeroed; only a sequence's last tile has any)
    auto convert = [&](auto full) {
      float zk[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) zk[e] = 0.f;
      const f32x4 z0 = *(const f32x4*)&zp[8 * cc], z1 = *(const f32x4*)&zp[8 * cc + 4];
      const float zz[8] = {z0[0], z0[1], z0[2], z0[3], z1[0], z1[1], z1[2], z1[3]};
      // both rows' chunks are read before either is written back
      u32x4 krr[2], qrr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = prow + 16 * i;
        const int po = row * D + ((cc ^ swz_v(row)) << 3);
        krr[i] = *(const u32x4*)&Kb[po];
        qrr[i] = *(const u32x4*)&Qb[po];
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = prow + 16 * i;
        const int po = row * D + ((cc ^ swz_v(row)) << 3);
        const bool live = decltype(full)::value || t0 + row < n1;
        const u32x4 kr = krr[i], qr = qrr[i];
        u32x4 kp, qp;
        float d = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float k0 = live ? phi(bf16_lo(kr[w])) : 0.f, k1 = live ? phi(bf16_hi(kr[w])) : 0.f;
          zk[2 * w] += k0;
          zk[2 * w + 1] += k1;
          kp[w] = pack_bf16x2(k0, k1);
          const float q0 = phi(bf16_lo(qr[w])), q1 = phi(bf16_hi(qr[w]));
          d = __builtin_fmaf(q0, zz[2 * w], d);
          d = __builtin_fmaf(q1, zz[2 * w + 1], d);
          qp[w] = pack_bf16x2(q0, q1);
        }
        *(u32x4*)&Kb[po] = kp;
        *(u32x4*)&Qb[po] = qp;
        d = row16_sum(d);  // the 16 lanes of this row hold its 16 chunks
        if (cc == 0) dq[row] = d;
      }
      // lanes l, l ^ 16, l ^ 32, l ^ 48 hold the same chunk
#pragma unroll
      for (int e = 0; e < 8; ++e) zk[e] = pair_sum(xor16_sum(zk[e]));
      if (lane < 16) {
        *(f32x4*)&zred[wave][8 * cc] = f32x4{zk[0], zk[1], zk[2], zk[3]};
        *(f32x4*)&zred[wave][8 * cc + 4] = f32x4{zk[4], zk[5], zk[6], zk[7]};
      }
    };
    if (t0 + kCT <= n1) convert(BoolTag<true>{});
    else convert(BoolTag<false>{});
    // S_prev^T for the inter-step product, rounded before this step's update.
    // k-step f = 2 t + ks covers d1 = 16 f + 8 hi + e: the lane of half hi
    // holds d1 = 32 t + 8 g + 4 hi + 0..3 (g = 2 ks, 2 ks + 1), so the halves
    // trade the 4-value groups they lack (one swap of lanes l and l + 32)
    bf16x8 sf[8];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int g0 = 2 * ks, g1 = g0 + 1;
        const uint32_t x0 = pack_bf16x2(acc[t][4 * g0], acc[t][4 * g0 + 1]);
        const uint32_t x1 = pack_bf16x2(acc[t][4 * g0 + 2], acc[t][4 * g0 + 3]);
        const uint32_t y0 = pack_bf16x2(acc[t][4 * g1], acc[t][4 * g1 + 1]);
        const uint32_t y1 = pack_bf16x2(acc[t][4 * g1 + 2], acc[t][4 * g1 + 3]);
        // lanes < 32 keep x and take the upper lanes' x; lanes >= 32 take the
        // lower lanes' y and keep y
        const auto p0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
        const auto p1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
        sf[2 * t + ks] = __builtin_bit_cast(bf16x8, u32x4{p0[0], p1[0], p0[1], p1[1]});
      }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    lds_barrier();
    if (tid < D) zs[(c + 1) & 1][tid] = zp[tid] + zred[0][tid] + zred[1][tid] + zred[2][tid] + zred[3][tid];

    // scores A^T = phi(K) phi(Q)^T (keys x queries) and O^T = S_prev^T phi(Q)^T
    f32x16 s = f32x16{}, o = f32x16{};
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      const bf16x8 qf = row_frag(Qb, l32, f);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag(Kb, l32, f), qf, s, 0, 0, 0);
      o = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sf[f], qf, o, 0, 0, 0);
    }
    // the step's state: S[d1, d2 = 32 w + ..] += phi(K)^T V
    bf16x8 vf[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      vf[ks] = tr_frag(Vb, ks, wave);
#pragma unroll
      for (int t = 0; t < 4; ++t)
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag(Kb, ks, t), vf[ks], acc[t], 0, 0, 0);
    }
    // causal mask: s[r] is key 8 (r / 4) + 4 hi + r % 4 of the step, query l32
    float rs = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (8 * (r >> 2) + 4 * hi + (r & 3) > l32) s[r] = 0.f;
      rs += s[r];
    }
    const float den = pair_sum(rs) + dq[l32];
    // intra-step term O^T += V^T A^T over the step's keys
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const u32x4 pw = {pack_bf16x2(s[8 * ks], s[8 * ks + 1]), pack_bf16x2(s[8 * ks + 2], s[8 * ks + 3]),
                        pack_bf16x2(s[8 * ks + 4], s[8 * ks + 5]), pack_bf16x2(s[8 * ks + 6], s[8 * ks + 7])};
      o = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[ks], __builtin_bit_cast(bf16x8, pw), o, 0, 0, 0);
    }
    // o[r] = O^T[32 w + 8 (r / 4) + 4 hi + r % 4][query l32]
    const int row = t0 + l32;
    if (row < n1) {
      const float inv = 1.f / den;
      uint16_t* dst = obase + (int64_t)row * a.sn;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x2 w = {pack_bf16x2(o[4 * g] * inv, o[4 * g + 1] * inv),
                         pack_bf16x2(o[4 * g + 2] * inv, o[4 * g + 3] * inv)};
        *(u32x2*)(dst + 8 * g) = w;
      }
    }
  };

  int c = 0;
  for (; c + 3 <= nch; c += 3) {
    step(Q0, K0, V0, Q2, K2, V2, c);
    step(Q1, K1, V1, Q0, K0, V0, c + 1);
    step(Q2, K2, V2, Q1, K1, V1, c + 2);
  }
  if (c < nch) step(Q0, K0, V0, Q2, K2, V2, c);
  if (c + 1 < nch) step(Q1, K1, V1, Q0, K0, V0, c + 1);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------


static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

LinPlan linear_plan(const bsa_shape& s) {
  LinPlan p;
  const int64_t bh = (int64_t)s.B * s.H;
  // the head_dim-128 kernels address a head with 32-bit offsets
  p.d128 = s.D == 128 && ((int64_t)s.N + kLinTok) * s.stride_n * 2 < ((int64_t)1 << 31);
  // state: at most two workgroups per CU in total, so the whole launch is one
  // round (a few workgroups past 2 per CU would double the time)
  const int tok = p.d128 ? kLinTok2 : kLinTok;
  int64_t want = 512 / bh;
  const int64_t tiles = (s.N + tok - 1) / tok;
  if (want > tiles) want = tiles;
  if (want < 1) want = 1;
  const int64_t per = (tiles + want - 1) / want;
  p.chunk = (int)(per * tok);
  p.splits = (int)((s.N + p.chunk - 1) / p.chunk);
  // apply (head_dim 128): (head, tile) items in equal runs over <= 512 workgroups
  p.tph = (s.N + kApplyRows - 1) / kApplyRows;
  const int64_t items = bh * p.tph;
  p.tpw = (int)((items + 511) / 512);
  p.apply_wgs = (int)((items + p.tpw - 1) / p.tpw);
  const size_t D = s.D;
  p.off_part_s = 0;
  p.off_part_z = align256(p.off_part_s + (size_t)bh * p.splits * D * D * 4);
  p.off_st = align256(p.off_part_z + (size_t)bh * p.splits * D * 4);
  p.off_z = align256(p.off_st + (size_t)bh * D * D * 2);
  p.total = align256(p.off_z + (size_t)bh * D * 4);
  return p;
}

bsa_status launch_linear_attn(const void* q, const void* k, const void* v, void* o, const bsa_shape& s,
                              float* S, float* z, void* ws, hipStream_t stream, float mix_r) {
  const LinPlan p = linear_plan(s);
  char* w = (char*)ws;
  const int bh = s.B * s.H;
  LinStateArgs sa{(const uint16_t*)k, (const uint16_t*)v, (float*)(w + p.off_part_s),
                  (float*)(w + p.off_part_z), s.stride_b, s.stride_h, s.stride_n, s.H, s.N, p.splits, p.chunk};
  LinReduceArgs ra{(const float*)(w + p.off_part_s), (const float*)(w + p.off_part_z), S, z,
                   (uint16_t*)(w + p.off_st), (float*)(w + p.off_z), p.splits};
  LinApplyArgs aa{(const uint16_t*)q, (uint16_t*)o, (const uint16_t*)(w + p.off_st),
                  (const float*)(w + p.off_z), s.stride_b, s.stride_h, s.stride_n, s.H, s.N,
                  p.tph, bh * p.tph, p.tpw, mix_r};
  const int row_groups = (s.N + kApplyRows * kApplyTiles - 1) / (kApplyRows * kApplyTiles);
  if (s.D == 128 && p.d128) {
    hipLaunchKernelGGL(lin_state_d128_kernel<kNt>, dim3(p.splits, bh), dim3(kLinThreads), 0, stream, sa);
    hipLaunchKernelGGL(lin_reduce_kernel<128>, dim3(128 * 128 / (4 * kRedCols), bh), dim3(256), 0, stream, ra);
    hipLaunchKernelGGL(lin_apply_d128_kernel, dim3(p.apply_wgs), dim3(256), 0, stream, aa);
  } else if (s.D == 128) {
    hipLaunchKernelGGL(lin_state_kernel<128>, dim3(p.splits, bh), dim3(kLinThreads), 0, stream, sa);
    hipLaunchKernelGGL(lin_reduce_kernel<128>, dim3(128 * 128 / (4 * kRedCols), bh), dim3(256), 0, stream, ra);
    hipLaunchKernelGGL(lin_apply_kernel<128>, dim3(row_groups, bh), dim3(256), 0, stream, aa);
  } else if (s.D == 64) {
    hipLaunchKernelGGL(lin_state_kernel<64>, dim3(p.splits, bh), dim3(kLinThreads), 0, stream, sa);
    hipLaunchKernelGGL(lin_reduce_kernel<64>, dim3(64 * 64 / (4 * kRedCols), bh), dim3(256), 0, stream, ra);
    hipLaunchKernelGGL(lin_apply_kernel<64>, dim3(row_groups, bh), dim3(256), 0, stream, aa);
  } else {
    return BSA_ERR_UNSUPPORTED;
  }
  return launch_ok("linear_attn_fwd") ? BSA_OK : BSA_ERR_HIP;
}

// ---- the no-allocation variant ---------------------------------------------
// Workspace of bsa_linear_attn_fwd_noalloc (the linear_plan layout), held in a
// file-scope device array: each GPU the library runs on holds its own copy
// until the process ends, and every call on that GPU shares it.  Nothing in it
// has to start at zero (every partial is written before it is read).  In host
// code `scratch` names a host-side stand-in, not device memory: the device
// address is looked up with hipGetSymbolAddress, once per device, with that
// device current, and only that address is passed to the kernels.
static __device__ __align__(256) unsigned char scratch[kLinNoAllocBytes];

static constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

bsa_status linear_noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_error("bsa_linear_attn_fwd_noalloc: hipGetDevice failed: %s", hipGetErrorString(e));
    return BSA_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    set_error("bsa_linear_attn_fwd_noalloc: device %d beyond the supported %d", dev, kMaxDevices);
    return BSA_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      set_error("bsa_linear_attn_fwd_noalloc: hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                hipGetErrorString(e));
      return BSA_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return BSA_OK;
}

CausalPlan causal_plan(const bsa_shape& s) {
  CausalPlan p;
  const int64_t bh = (int64_t)s.B * s.H;
  // two workgroups per CU for both the state and the causal kernel (at most
  // 512 in all, one round); the prefix starts every state split (f = 1)
  const int64_t tiles = (s.N + kCT - 1) / kCT;
  int64_t want = 512 / bh;
  if (want > tiles) want = tiles;
  if (want < 1) want = 1;
  const int64_t per = (tiles + want - 1) / want;
  p.f = 1;
  p.chunk_a = (int)(per * kCT);
  p.chunk_s = p.chunk_a / p.f;
  p.splits_a = (int)((s.N + p.chunk_a - 1) / p.chunk_a);
  p.splits_s = (int)((s.N + p.chunk_s - 1) / p.chunk_s);
  const size_t D = s.D;
  p.off_part_s = 0;
  p.off_part_z = align256((size_t)bh * p.splits_s * D * D * 4);
  p.total = align256(p.off_part_z + (size_t)bh * p.splits_s * D * 4);
  return p;
}

bsa_status launch_causal_linear_attn(const void* q, const void* k, const void* v, void* o, const bsa_shape& s,
                                     const float* s_in, const float* z_in, float* s_out, float* z_out, void* ws,
                                     hipStream_t stream) {
  const CausalPlan p = causal_plan(s);
  char* w = (char*)ws;
  const int bh = s.B * s.H;
  float* part_s = (float*)(w + p.off_part_s);
  float* part_z = (float*)(w + p.off_part_z);
  LinStateArgs sa{(const uint16_t*)k, (const uint16_t*)v, part_s, part_z, s.stride_b, s.stride_h, s.stride_n,
                  s.H, s.N, p.splits_s, p.chunk_s};
  LinPrefixArgs pa{part_s, part_z, s_in, z_in, s_out, z_out, p.splits_s, p.f};
  CausalArgs ca{(const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, part_s, part_z,
                s.stride_b, s.stride_h, s.stride_n, s.H, s.N, p.chunk_a, p.splits_s, p.f};
  hipLaunchKernelGGL(lin_state_d128_kernel<0>, dim3(p.splits_s, bh), dim3(kLinThreads), 0, stream, sa);
  hipLaunchKernelGGL(lin_prefix_d128_kernel, dim3(17, bh), dim3(256), 0, stream, pa);
  hipLaunchKernelGGL(causal_lin_d128_kernel, dim3(p.splits_a, bh), dim3(256), 0, stream, ca);
  return launch_ok("causal_linear_attn_fwd") ? BSA_OK : BSA_ERR_HIP;
}

}  // namespace bsa
