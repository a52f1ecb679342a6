// Backward pass of block-sparse softmax attention, bf16, head_dim 128, blocks
// of 128 tokens, for gfx950.
//
// Operation: the gradients of the block-sparse attention of attn_fwd.hip
// (LVSA review page, section 1 Key Terms: block-sparse attention; needed by the
// training uses on the Radial Attention headline (LoRA fine-tuning for longer
// videos) and the LinVideo page (post-training)).  For query block i with kept
// key set K(i), P = softmax(scale * Q_i K^T) is recomputed from the forward's
// log-sum-exp, and
//   dV_K += P^T dO_i,  dP = dO_i V_K^T,  Delta = rowsum(dO_i * O_i),
//   dS = P * (dP - Delta),  dQ_i = scale * dS K_K,  dK_K += scale * dS^T Q_i.
//
// Two launches, no atomics (deterministic):
//   dq   : a workgroup per (query block, sequence), dealt to XCDs in
//          contiguous ranges; 4 waves x 32 query rows.  Q and dO of the
//          wave's rows are register-resident B operands; Delta comes from dO
//          and O of the same rows (fp32) and is stored for the second launch.
//          The row's kept key blocks stream through LDS in 64-key sub-tiles
//          (K and V by buffer loads, one sub-tile ahead, rows swizzled for the
//          transpose read).  Per sub-tile: S^T = K Q^T and dP^T = V dO^T
//          (32x32x16 MFMA, keys x queries: each lane owns one query column),
//          P^T = exp2(S^T scale log2e - lse log2e), dS^T = P^T (dP^T - Delta),
//          and dQ^T += K^T dS^T with K^T from the transpose read and dS^T taken
//          straight from the accumulators (the softmax kernel's P^T trick).
//   dkdv : a workgroup per (key block, sequence), 4 waves x 32 key rows,
//          walking the query blocks that keep the key block (the transposed
//          CSR) in 32-query sub-tiles.  K of the block's keys is staged once in
//          LDS, V of the wave's keys is register-resident.  S = Q K^T and
//          dP = dO V^T with queries x keys, so each lane owns one key column;
//          P and dS from the staged lse and Delta of the sub-tile; then
//          dV^T += dO^T P and dK^T += Q^T dS with the transpose reads of the
//          staged dO and Q.  S and dP are formed once for both gradients.
// Accumulation is fp32; P and dS enter the MFMA as bf16; the gradients are
// stored as bf16.

#include "launch.h"

namespace bsa {

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dO;
  const float* lse;       // [BH][N] natural log
  float* delta;           // [BH][N] workspace
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const int32_t* col_ptr;  // transposed CSR
  const int32_t* row_idx;
  int64_t sb, sh, sn;
  int H, N, nb;
  float scale, c2;         // softmax scale, scale * log2(e)
  int head_major;          // 1: XCD ranges within windows of launch order; 0: over the whole list
  const int32_t* order;    // block schedule [nb + 1]: long blocks first, their count last
};

// (block, sequence) of this workgroup.  The long blocks of the schedule (rows
// or columns with many kept blocks, e.g. anchor frames) run first, for every
// sequence; the rest are dealt so that the workgroups the hardware sends to one
// XCD take one contiguous range of (sequence, block), and blocks that share
// key (or query) tiles share that XCD's L2; when eight sequences' tensors
// would not fit the last-level cache, the same within consecutive windows of
// launch order (one sequence at a time).
__device__ __forceinline__ int2 bwd_item(const BwdArgs& a) {
  const int pid = blockIdx.x, total = gridDim.x, hb = total / a.nb;
  const int nh = a.order[a.nb], S = nh * hb;
  if (pid < S) return int2{a.order[pid / hb], pid % hb};
  const int rest = a.nb - nh;
  const int item = a.head_major ? xcd_windowed(pid - S, S, total - S, kXcdWindow)
                                : xcd_contiguous(pid - S, S, total - S);
  return int2{a.order[nh + item % rest], item / rest};
}

constexpr int kBwdBlock = 128;

__device__ __forceinline__ void bwd_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// dQ (and Delta)
// ---------------------------------------------------------------------------

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bwd_dq_d128_kernel(BwdArgs a) {
  constexpr int D = 128, KT = 8, DT = 4, SUB = 64, TILE = SUB * D;
  __shared__ __attribute__((aligned(1024))) uint16_t K0[TILE], K1[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t V0[TILE], V1[TILE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hi = lane >> 5;
  const int2 it = bwd_item(a);
  const int qblk = it.x, bh = it.y;
  const int N = a.N;
  const int64_t head_off = (int64_t)(bh / a.H) * a.sb + (int64_t)(bh % a.H) * a.sh;
  const int qrow = qblk * kBwdBlock + 32 * wave + l32;
  const int qr = min(qrow, N - 1);

  // B operands: query l32, head dims 16 t + 8 hi .. + 7; Delta from dO and O
  bf16x8 qf[KT], gf[KT];
  float dl = 0.f;
  {
    const int64_t ro = head_off + (int64_t)qr * a.sn + 8 * hi;
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      qf[t] = *(const bf16x8*)(a.q + ro + 16 * t);
      const u32x4 g = *(const u32x4*)(a.dO + ro + 16 * t);
      const u32x4 ov = *(const u32x4*)(a.o + ro + 16 * t);
      gf[t] = __builtin_bit_cast(bf16x8, g);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dl = __builtin_fmaf(bf16_lo(g[e]), bf16_lo(ov[e]), dl);
        dl = __builtin_fmaf(bf16_hi(g[e]), bf16_hi(ov[e]), dl);
      }
    }
  }
  dl = pair_sum(dl);
  if (hi == 0 && qrow < N) a.delta[(int64_t)bh * N + qrow] = dl;
  const float lse2 = a.lse[(int64_t)bh * N + qr] * kLog2e;

  const int rbeg = a.row_ptr[qblk], rend = a.row_ptr[qblk + 1];
  int nsub = (rend - rbeg) * 2;
  if (nsub > 0 && a.col_idx[rend - 1] == a.nb - 1) {
    const int last_real = N - (a.nb - 1) * kBwdBlock;
    nsub -= 2 - (last_real + SUB - 1) / SUB;
  }
  const cint_ptr cols = (cint_ptr)a.col_idx;
  auto key0_of = [&](int u) -> int { return cols[rbeg + (u >> 1)] * kBwdBlock + (u & 1) * SUB; };

  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t row_bytes = (uint32_t)a.sn * 2u;
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.k + head_off), (short)0, 0x7fffffff, kBufferWord3);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.v + head_off), (short)0, 0x7fffffff, kBufferWord3);
  // copy roles: wave w, instruction j stages rows 16 w + 4 j + lane / 16, whose
  // swz_v is 4 (lane / 16) + j: the chunk offset is one per-lane base XOR 16 j and
  // the row offset a per-lane base plus a uniform multiple of 4 rows
  const uint32_t rbase = (uint32_t)(16 * wv + (lane >> 4)) * row_bytes;
  const uint32_t cbase = (uint32_t)(((lane & 15) ^ (4 * (lane >> 4))) * 16);
  auto dma = [&](uint16_t* kst, uint16_t* vst, int key0) {
    if (key0 + SUB <= N) {
      const uint32_t so = (uint32_t)key0 * row_bytes;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t o = rbase + (uint32_t)(4 * j) * row_bytes + (cbase ^ (16u * j));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)&kst[(16 * wv + 4 * j) * D], 16, o, so, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)&vst[(16 * wv + 4 * j) * D], 16, o, so, 0, 0);
      }
    } else {  // tail sub-tile: rows past N repeat row N - 1 (their scores are masked)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = 16 * wv + 4 * j + (lane >> 4);
        const uint32_t o = (uint32_t)min(key0 + row, N - 1) * row_bytes + (cbase ^ (16u * j));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)&kst[(16 * wv + 4 * j) * D], 16, o, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)&vst[(16 * wv + 4 * j) * D], 16, o, 0, 0, 0);
      }
    }
  };

  // LDS byte offsets of the stage reads, one per-lane base XOR an immediate:
  //   row fragment (row 32 kt + l32, head dims 16 t + 8 hi ..): 8192 kt + (rb ^ 32 t)
  //   transpose read (rows 16 ks + 4 hi + (lane % 16) / 4, column block dt):
  //   4096 ks + (tb ^ 64 dt), and 8 rows on 4096 ks + 2048 + (tb ^ 32 ^ 64 dt)
  const int j16 = lane & 15, a4 = j16 >> 2, c4 = 2 * ((lane >> 4) & 1) + ((j16 & 3) >> 1);
  const uint32_t rb = (uint32_t)(l32 * 256 + ((hi ^ swz_v(l32)) << 4));
  const uint32_t tb = (uint32_t)((4 * hi + a4) * 256 + 64 * a4 + 16 * (c4 ^ hi) + 8 * (j16 & 1));
  auto row_frag = [&](const uint16_t* st, int kt, int t) -> bf16x8 {
    return *(const bf16x8*)((const char*)st + 8192 * kt + (rb ^ (32u * t)));
  };
  auto tr_frag = [&](const uint16_t* st, int ks, int dt) -> bf16x8 {
    const char* b = (const char*)st + 4096 * ks;
    const u32x2 x0 = lds_tr16((const uint16_t*)(b + (tb ^ (64u * dt))));
    const u32x2 x1 = lds_tr16((const uint16_t*)(b + 2048 + (tb ^ 32u ^ (64u * dt))));
    return __builtin_bit_cast(bf16x8, u32x4{x0[0], x0[1], x1[0], x1[1]});
  };

  f32x16 dq[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) dq[i] = f32x16{};

  auto step = [&](const uint16_t* Kb, const uint16_t* Vb, uint16_t* Kn, uint16_t* Vn, int u) {
    const int key0 = key0_of(u);
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0): sub-tile u landed
    bwd_barrier();
    if (u + 1 < nsub) dma(Kn, Vn, key0_of(u + 1));
    // the two 32-key halves one after the other (fewer live accumulators)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      f32x16 s = f32x16{}, dp = f32x16{};
      bf16x8 kf[KT], vf[KT];
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        kf[t] = row_frag(Kb, kt, t);
        vf[t] = row_frag(Vb, kt, t);
      }
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[t], qf[t], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[t], gf[t], dp, 0, 0, 0);
      }
      // reads run four ahead of the MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < 12; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      // s[r] is key key0 + 32 kt + 8 (r / 4) + 4 hi + r % 4 of query l32
      float ds[16];
      if (key0 + 32 * kt + 32 <= N) {
#pragma unroll
        for (int r = 0; r < 16; ++r) ds[r] = fast_exp2(__builtin_fmaf(s[r], a.c2, -lse2)) * (dp[r] - dl);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const bool live = key0 + 32 * kt + 8 * (r >> 2) + 4 * hi + (r & 3) < N;
          const float p = live ? fast_exp2(__builtin_fmaf(s[r], a.c2, -lse2)) : 0.f;
          ds[r] = p * (dp[r] - dl);
        }
      }
      // dQ^T += K^T dS^T over the half's 32 keys (k-steps 2 kt, 2 kt + 1), at
      // raised wave priority as in the dK / dV kernel
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const u32x4 w = {pack_bf16x2(ds[8 * h2], ds[8 * h2 + 1]), pack_bf16x2(ds[8 * h2 + 2], ds[8 * h2 + 3]),
                         pack_bf16x2(ds[8 * h2 + 4], ds[8 * h2 + 5]), pack_bf16x2(ds[8 * h2 + 6], ds[8 * h2 + 7])};
        const bf16x8 df = __builtin_bit_cast(bf16x8, w);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          dq[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag(Kb, 2 * kt + h2, dt), df, dq[dt], 0, 0, 0);
      }
      __builtin_amdgcn_s_setprio(0);
    }
  };

  if (nsub > 0) dma(K0, V0, key0_of(0));
  int u = 0;
  for (; u + 2 <= nsub; u += 2) {
    step(K0, V0, K1, V1, u);
    step(K1, V1, K0, V0, u + 1);
  }
  if (u < nsub) step(K0, V0, K1, V1, u);

  // dq[dt][r] = dQ^T[32 dt + 8 (r / 4) + 4 hi + r % 4][query l32] / scale
  if (qrow < N) {
    uint16_t* dst = a.dq + head_off + (int64_t)qrow * a.sn;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x2 w = {pack_bf16x2(dq[dt][4 * g] * a.scale, dq[dt][4 * g + 1] * a.scale),
                         pack_bf16x2(dq[dt][4 * g + 2] * a.scale, dq[dt][4 * g + 3] * a.scale)};
        *(u32x2*)(dst + 32 * dt + 8 * g + 4 * hi) = w;
      }
  }
}

// ---------------------------------------------------------------------------
// dK and dV in one launch: S and dP are formed once per query tile and feed
// both accumulators.  Two waves per SIMD still fit because K of the
// workgroup's 128 keys is staged once in LDS (32 KB, read back as the B
// operand of S) instead of being held in registers; V of the wave's keys stays
// register-resident, and Q and dO stream through two 32-query stages (8 KB
// each), so one workgroup needs about 65 KB of LDS and two share a CU.
// ---------------------------------------------------------------------------

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bwd_dkdv_d128_kernel(BwdArgs a) {
  constexpr int D = 128, KT = 8, DT = 4, SUB = 32, TILE = SUB * D;
  __shared__ __attribute__((aligned(1024))) uint16_t Ks[kBwdBlock * D];
  __shared__ __attribute__((aligned(1024))) uint16_t Q0[TILE], Q1[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t G0[TILE], G1[TILE];
  __shared__ __attribute__((aligned(16))) float L[2][SUB], E[2][SUB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hi = lane >> 5;
  const int2 it = bwd_item(a);
  const int kblk = it.x, bh = it.y;
  const int N = a.N;
  const int64_t head_off = (int64_t)(bh / a.H) * a.sb + (int64_t)(bh % a.H) * a.sh;
  const int krow = kblk * kBwdBlock + 32 * wave + l32;

  // B operand of dP = dO V^T: key l32, head dims 16 t + 8 hi .. + 7
  bf16x8 vf[KT];
  {
    const int64_t ro = head_off + (int64_t)min(krow, N - 1) * a.sn + 8 * hi;
#pragma unroll
    for (int t = 0; t < KT; ++t) vf[t] = *(const bf16x8*)(a.v + ro + 16 * t);
  }

  const int cbeg = a.col_ptr[kblk], cend = a.col_ptr[kblk + 1];
  constexpr int PER = kBwdBlock / SUB;  // sub-tiles per query block
  int nsub = (cend - cbeg) * PER;
  if (nsub > 0 && a.row_idx[cend - 1] == a.nb - 1) {
    const int last_real = N - (a.nb - 1) * kBwdBlock;
    nsub -= PER - (last_real + SUB - 1) / SUB;
  }
  const cint_ptr ridx = (cint_ptr)a.row_idx;
  auto q0_of = [&](int u) -> int { return ridx[cbeg + u / PER] * kBwdBlock + (u % PER) * SUB; };

  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t row_bytes = (uint32_t)a.sn * 2u;
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.k + head_off), (short)0, 0x7fffffff, kBufferWord3);
  const __amdgpu_buffer_rsrc_t qrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.q + head_off), (short)0, 0x7fffffff, kBufferWord3);
  const __amdgpu_buffer_rsrc_t grs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.dO + head_off), (short)0, 0x7fffffff, kBufferWord3);
  // copy roles: each instruction moves 4 rows (16 lanes per row, one 16-byte
  // chunk each, at physical chunk lane % 16 of a swz_v-swizzled row); rows past
  // N repeat row N - 1 (their columns or rows are masked or never stored);
  // r0 is the (wave-uniform) first of the 4 rows
  auto dma_rows = [&](__amdgpu_buffer_rsrc_t rs, uint16_t* st, int r0, int g0) {
    const int row = r0 + (lane >> 4);
    const uint32_t o = (uint32_t)min(g0 + row, N - 1) * row_bytes + (uint32_t)(((lane & 15) ^ swz_v(row)) * 16);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)&st[r0 * D], 16, o, 0, 0, 0);
  };
  // Q and dO of a 32-query sub-tile: wave w, instruction j stages rows 8 w + 4 j + lane / 16
  auto dma = [&](uint16_t* qst, uint16_t* gst, int q0) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      dma_rows(qrs, qst, 8 * wv + 4 * j, q0);
      dma_rows(grs, gst, 8 * wv + 4 * j, q0);
    }
  };
  const float* lse_h = a.lse + (int64_t)bh * N;
  const float* del_h = a.delta + (int64_t)bh * N;
  float nl = 0.f, ne = 0.f;
  // (the raw values are kept until the store at the end of the step, so the
  // loads' latency is waited for there, not before the copies are issued)
  auto side_load = [&](int q0) {
    if (wave == 0 && lane < SUB) {
      const int qq = q0 + lane;
      nl = qq < N ? lse_h[qq] : __builtin_inff();
      ne = qq < N ? del_h[qq] : 0.f;
    }
  };
  auto side_store = [&](int buf) {
    if (wave == 0 && lane < SUB) {
      L[buf][lane] = nl * kLog2e;
      E[buf][lane] = ne;
    }
  };

  f32x16 dk[DT], dv[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) dk[i] = dv[i] = f32x16{};

  // Per-lane LDS byte offsets as one base XOR / plus immediates, so few
  // registers stay live (stages are swz_v-swizzled [rows][128] bf16):
  //   Q or dO row fragment (query l32, head dims 16 t + 8 hi ..):  rq ^ 32 t
  //   K row fragment (key 32 w + l32, same dims):   rk ^ 32 t,  rk = rq + 8192 w
  //   transpose read (rows 16 ks + 4 hi + (lane % 16) / 4 and 8 more, columns
  //   32 dt + 16 ((lane / 16) % 2) + 4 (lane % 4) ..): 4096 ks + (tq ^ 64 dt)
  //   and 4096 ks + 2048 + (tq ^ 32 ^ 64 dt)
  const int j16 = lane & 15, g16 = lane >> 4;
  int rq = 2 * (l32 * D + 8 * (hi ^ swz_v(l32)));
  int rk = rq + 64 * D * wv;
  const int tc1 = 2 * (g16 & 1) + ((j16 & 3) >> 1);
  int tq = 2 * ((4 * hi + (j16 >> 2)) * D + ((tc1 ^ (4 * (j16 >> 2) + hi)) << 3) + (j16 & 1) * 4);
  auto row_frag = [&](const uint16_t* st, int off) { return *(const bf16x8*)((const char*)st + off); };
  auto tr_frag = [&](const uint16_t* st, int ks, int dt) {
    const char* b = (const char*)st + 4096 * ks;
    const u32x2 x0 = lds_tr16((const uint16_t*)(b + (tq ^ (64 * dt))));
    const u32x2 x1 = lds_tr16((const uint16_t*)(b + 2048 + (tq ^ 32 ^ (64 * dt))));
    return __builtin_bit_cast(bf16x8, u32x4{x0[0], x0[1], x1[0], x1[1]});
  };

  auto step = [&](const uint16_t* Qb, const uint16_t* Gb, uint16_t* Qn, uint16_t* Gn, int u) {
    const int buf = u & 1;
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0): sub-tile u (and K) landed
    bwd_barrier();
    if (u + 1 < nsub) {  // lse / Delta loads first: their use then waits for them only
      side_load(q0_of(u + 1));
      dma(Qn, Gn, q0_of(u + 1));
    }
    // the bases are opaque here, so the 24 XORed offsets are formed next to
    // their reads instead of being hoisted out of the loop (and spilled)
    asm volatile("" : "+v"(rq), "+v"(rk), "+v"(tq));
    // S = Q K^T and dP = dO V^T, queries x keys: s[r] is query 8 (r / 4) + 4 hi + r % 4 of the sub-tile, key l32
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag(Qb, rq ^ (32 * t)), row_frag(Ks, rk ^ (32 * t)), s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag(Gb, rq ^ (32 * t)), vf[t], dp, 0, 0, 0);
    }
    // reads run two k-steps ahead of the MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    float pw[16], dw[16];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 lg = *(const f32x4*)&L[buf][8 * g + 4 * hi];
      const f32x4 eg = *(const f32x4*)&E[buf][8 * g + 4 * hi];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 4 * g + j;
        const float p = fast_exp2(__builtin_fmaf(s[r], a.c2, -lg[j]));
        pw[r] = p;
        dw[r] = p * (dp[r] - eg[j]);
      }
    }
    // dV^T += dO^T P and dK^T += Q^T dS over the sub-tile's two 16-query k-steps,
    // at raised wave priority (co-resident waves drift out of phase, one's
    // exponentials under the other's matrix work)
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const u32x4 pp = {pack_bf16x2(pw[8 * ks], pw[8 * ks + 1]), pack_bf16x2(pw[8 * ks + 2], pw[8 * ks + 3]),
                        pack_bf16x2(pw[8 * ks + 4], pw[8 * ks + 5]), pack_bf16x2(pw[8 * ks + 6], pw[8 * ks + 7])};
      const u32x4 dd = {pack_bf16x2(dw[8 * ks], dw[8 * ks + 1]), pack_bf16x2(dw[8 * ks + 2], dw[8 * ks + 3]),
                        pack_bf16x2(dw[8 * ks + 4], dw[8 * ks + 5]), pack_bf16x2(dw[8 * ks + 6], dw[8 * ks + 7])};
      const bf16x8 pf = __builtin_bit_cast(bf16x8, pp), df = __builtin_bit_cast(bf16x8, dd);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag(Gb, ks, dt), pf, dv[dt], 0, 0, 0);
        dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag(Qb, ks, dt), df, dk[dt], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    if (u + 1 < nsub) side_store(buf ^ 1);
  };

  if (nsub > 0) {
    // K of the block's 128 keys: wave w, instruction j stages rows 32 w + 4 j + lane / 16
    side_load(q0_of(0));
#pragma unroll
    for (int j = 0; j < 8; ++j) dma_rows(krs, Ks, 32 * wv + 4 * j, kblk * kBwdBlock);
    dma(Q0, G0, q0_of(0));
    side_store(0);
  }
  int u = 0;
  for (; u + 2 <= nsub; u += 2) {
    step(Q0, G0, Q1, G1, u);
    step(Q1, G1, Q0, G0, u + 1);
  }
  if (u < nsub) step(Q0, G0, Q1, G1, u);

  // dk / dv[dt][r] = dK^T / scale and dV^T at [32 dt + 8 (r / 4) + 4 hi + r % 4][key l32]
  if (krow < N) {
    const int64_t ro = head_off + (int64_t)krow * a.sn;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * dt + 8 * g + 4 * hi;
        const u32x2 wk = {pack_bf16x2(dk[dt][4 * g] * a.scale, dk[dt][4 * g + 1] * a.scale),
                          pack_bf16x2(dk[dt][4 * g + 2] * a.scale, dk[dt][4 * g + 3] * a.scale)};
        const u32x2 wvv = {pack_bf16x2(dv[dt][4 * g], dv[dt][4 * g + 1]),
                           pack_bf16x2(dv[dt][4 * g + 2], dv[dt][4 * g + 3])};
        *(u32x2*)(a.dk + ro + d0) = wk;
        *(u32x2*)(a.dv + ro + d0) = wvv;
      }
  }
}

// ---------------------------------------------------------------------------
// transposed block CSR
// ---------------------------------------------------------------------------

__device__ __forceinline__ bool csr_has(const int32_t* cols, int b, int e, int j) {
  while (b < e) {  // columns ascending
    const int m = (b + e) >> 1;
    const int c = cols[m];
    if (c == j) return true;
    if (c < j) b = m + 1;
    else e = m;
  }
  return false;
}

// one wave per key block j: the lanes test 64 query blocks at a time (binary
// search of j in the block's ascending columns) and a ballot keeps them in order
template <bool FILL>
__global__ void __launch_bounds__(256) mask_transpose_kernel(const int32_t* row_ptr, const int32_t* col_idx, int nb,
                                                             int32_t* col_ptr, int32_t* row_idx) {
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (!FILL && j == 0 && lane == 0) col_ptr[0] = 0;
  if (j >= nb) return;
  int pos = FILL ? col_ptr[j] : 0;
  for (int i0 = 0; i0 < nb; i0 += 64) {
    const int i = i0 + lane;
    const bool has = i < nb && csr_has(col_idx, row_ptr[i], row_ptr[i + 1], j);
    const unsigned long long bal = __ballot(has);
    if (FILL && has) row_idx[pos + __popcll(bal & ((1ull << lane) - 1ull))] = i;
    pos += __popcll(bal);
  }
  if (!FILL && lane == 0) col_ptr[j + 1] = pos;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

bsa_status launch_transpose_block_mask(const int32_t* row_ptr, const int32_t* col_idx, int nb, int32_t* col_ptr,
                                       int32_t* row_idx, hipStream_t stream) {
  const dim3 g((nb + 3) / 4);
  hipLaunchKernelGGL(mask_transpose_kernel<false>, g, dim3(256), 0, stream, row_ptr, col_idx, nb, col_ptr, row_idx);
  launch_inclusive_scan(col_ptr, nb, stream);  // counts in col_ptr[1..nb] -> offsets
  hipLaunchKernelGGL(mask_transpose_kernel<true>, g, dim3(256), 0, stream, row_ptr, col_idx, nb, col_ptr, row_idx);
  return launch_ok("transpose_block_mask") ? BSA_OK : BSA_ERR_HIP;
}

size_t attn_bwd_workspace(const bsa_shape& s) {
  const size_t nb = (s.N + kBwdBlock - 1) / kBwdBlock;
  return ((size_t)s.B * s.H * s.N * 4 + 2 * (nb + 1) * 4 + 255) & ~(size_t)255;
}

bsa_status launch_attn_bwd_bf16(const void* q, const void* k, const void* v, const void* o, const void* dO,
                                const float* lse, const bsa_shape& s, const int32_t* row_ptr, const int32_t* col_idx,
                                const int32_t* col_ptr, const int32_t* row_idx, float scale, void* dq, void* dk,
                                void* dv, void* ws, hipStream_t stream) {
  BwdArgs a;
  a.q = (const uint16_t*)q; a.k = (const uint16_t*)k; a.v = (const uint16_t*)v;
  a.o = (const uint16_t*)o; a.dO = (const uint16_t*)dO; a.lse = lse; a.delta = (float*)ws;
  a.dq = (uint16_t*)dq; a.dk = (uint16_t*)dk; a.dv = (uint16_t*)dv;
  a.row_ptr = row_ptr; a.col_idx = col_idx; a.col_ptr = col_ptr; a.row_idx = row_idx;
  a.sb = s.stride_b; a.sh = s.stride_h; a.sn = s.stride_n;
  a.H = s.H; a.N = s.N; a.nb = (s.N + kBwdBlock - 1) / kBwdBlock;
  a.scale = scale; a.c2 = scale * kLog2e;
  // eight sequences' K and V (or Q and dO) against the 256 MiB last-level cache
  a.head_major = 8 * (2 * (int64_t)s.N * s.D * 2) > (256ll << 20) ? 1 : 0;
  const dim3 grid(a.nb * s.B * s.H);
  // block schedules: rows of the mask for dQ, columns for dK / dV
  int32_t* row_order = (int32_t*)((char*)ws + (size_t)s.B * s.H * s.N * 4);
  int32_t* col_order = row_order + a.nb + 1;
  launch_block_order(row_ptr, a.nb, row_order, stream);
  launch_block_order(col_ptr, a.nb, col_order, stream);
  a.order = row_order;
  hipLaunchKernelGGL(attn_bwd_dq_d128_kernel, grid, dim3(256), 0, stream, a);
  a.order = col_order;
  hipLaunchKernelGGL(attn_bwd_dkdv_d128_kernel, grid, dim3(256), 0, stream, a);
  return launch_ok("block_sparse_attn_bwd") ? BSA_OK : BSA_ERR_HIP;
}

}  // namespace bsa
