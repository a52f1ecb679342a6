// Block-sparse softmax attention forward for gfx950.
//
// Operation: for each real query row, softmax(scale * q K^T) V over the keys of
// the kept key blocks of its block row, plus the natural-log LSE ("[논문리뷰]
// LVSA: Training-Free Sparse Attention for Long Video Diffusion", section 1 Key
// Terms and section 3: block-sparse attention over a frame window and anchor
// frames; SVG-EAR page, technical summary section 1: sparse attention computes
// the kept blocks and skips the rest).  Skipped key blocks are never read.
//
// bf16 path (attn_bf16_kernel; attn_bf16_d128_kernel for head_dim 128 with
// 128-token blocks, the same math with direct global->LDS staging, see below).
// One workgroup per (query block, head, batch);
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

#include "launch.h"

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
  const int32_t* row_order;  // nullable: schedule of query-block rows, int32[nb + 1]
  int64_t sb, sh, sn;
  int B, H, N, block, nb;
  int head_major;    // 1: rows taken head by head, in windows split over the XCDs (see map_work)
  float scale_log2;  // scale * log2(e)
};

// Work item (query block, head, batch) of workgroup `pid`.
//  * Rows not singled out below, default: each XCD gets a contiguous range of
//    the (batch, head, query block) list, so the workgroups sharing an L2 walk
//    neighbouring query blocks of one head and reuse their key blocks.  The
//    eight XCDs then work on eight different heads at a time.
//  * head_major: the list is taken in windows of kXcdWindow items in launch
//    order, and inside a window each XCD takes a contiguous run, so at any time
//    all XCDs work on neighbouring query blocks of the same head and each
//    XCD's L2 holds the key band its run of query blocks shares.  The launcher
//    picks this when eight heads of K and V would not fit the last-level
//    cache: the key blocks that miss in one XCD's L2 are then found in that
//    cache.
//  * With a row order whose first nh = row_order[nb] rows are long ones (LVSA
//    anchor rows are about twice the mean length): those rows, for every head,
//    take the first nh * H * B workgroups, so they start in the first wave and
//    do not stretch the tail of the launch; the other rows follow as above, in
//    the order row_order lists them.
struct WorkItem {
  int qblk, h, b;
};
__device__ __forceinline__ WorkItem map_work(const AttnArgs& a) {
  const int pid = blockIdx.x, total = gridDim.x, hb = a.H * a.B;
  if (a.row_order != nullptr) {
    const cint_ptr ord = (cint_ptr)a.row_order;
    const int nh = ord[a.nb];
    const int S = nh * hb;
    if (pid < S) {
      const int r = pid % hb;
      return WorkItem{ord[pid / hb], r % a.H, r / a.H};
    }
    const int rest = a.nb - nh;
    const int item = a.head_major ? xcd_windowed(pid - S, S, total - S, kXcdWindow)
                                  : xcd_contiguous(pid - S, S, total - S);
    const int r = item / rest;
    return WorkItem{ord[nh + item % rest], r % a.H, r / a.H};
  }
  const int item = a.head_major ? xcd_windowed(pid, 0, total, kXcdWindow) : xcd_contiguous(pid, 0, total);
  return WorkItem{item % a.nb, (item / a.nb) % a.H, item / (a.nb * a.H)};
}

// Last-level cache (Infinity Cache) capacity used by the mapping choice above.
constexpr int64_t kLastLevelCacheBytes = 256ll << 20;
// Eight heads of K and V in flight (one per XCD) would not fit that cache.
inline int choose_head_major(const bsa_shape& s, int elem_bytes) {
  const int64_t kv_per_head = 2 * (int64_t)s.N * s.D * elem_bytes;
  return 8 * kv_per_head > kLastLevelCacheBytes ? 1 : 0;
}

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

  const WorkItem wi = map_work(a);
  const int qblk = wi.qblk, h = wi.h, b = wi.b;

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
  retire_loads();

  // The CSR is read-only for the whole kernel: read it through the constant
  // address space so that the uniform index loads are scalar (s_load).
  const cint_ptr rowp = (cint_ptr)a.row_ptr;
  const cint_ptr cols = (cint_ptr)a.col_idx;
  const int rbeg = rowp[qblk], rend = rowp[qblk + 1];
  constexpr int spb = BM / kBN;  // sub-tiles per key block (block == BM)
  int nsub = (rend - rbeg) * spb;
  if (nsub > 0 && cols[rend - 1] == a.nb - 1) {
    // drop trailing sub-tiles of the last key block that hold no real key
    const int last_real = N - (a.nb - 1) * BM;
    nsub -= spb - (last_real + kBN - 1) / kBN;
  }
  auto sub_key0 = [&](int u) -> int { return cols[rbeg + u / spb] * BM + (u % spb) * kBN; };

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

  // key offsets run two sub-tiles ahead of their use (scalar loads in flight)
  int key_cur = nsub > 0 ? sub_key0(0) : 0;
  int key_nxt = nsub > 1 ? sub_key0(1) : 0;
  if (nsub > 0) {
    fetch(key_cur);
    stage(0);
  }
  __syncthreads();

  for (int u = 0; u < nsub; ++u) {
    const int buf = u & 1;
    const int key0 = key_cur;
    const int key_nn = u + 2 < nsub ? sub_key0(u + 2) : 0;
    if (u + 1 < nsub) fetch(key_nxt);

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
    if (__any((m_new - m_run) * c2 > kLazyRescaleLog2)) {
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
    key_cur = key_nxt;
    key_nxt = key_nn;
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
// bf16 MFMA kernel, head_dim 128 and 128-token blocks: direct global->LDS loads
// ---------------------------------------------------------------------------
//
// Same math and register layouts as attn_bf16_kernel, with the K/V staging done
// by buffer_load_dwordx4 ... lds: each lane's 16 bytes land at (LDS base + 16 *
// lane), so the tile layout is chosen by which global chunk each lane loads.
// Rows are 256 bytes with an XOR swizzle of their 16 chunks instead of padding:
//   K: physical chunk = logical ^ (row & 15): the 16 rows read by 16 lanes for
//      one MFMA A operand hit 16 different chunks (all 64 banks);
//   V: physical chunk = logical ^ (4 (row & 3) + ((row >> 2) & 3)): the 4 rows x
//      4 chunks that 32 lanes touch in one ds_read_b64_tr_b16 are all distinct.
// Two 32 KB stages; the loads for sub-tile u+1 are issued right after the
// barrier that opens sub-tile u and overlap its compute; their completion is
// waited for with an explicit vmcnt before the next barrier.  The stages are
// separate LDS objects and the loop is unrolled by two, so that every LDS read
// provably misses the stage being filled (otherwise the compiler makes the
// first read wait for the copy in flight, which serialises copy and compute).


__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bf16_d128_kernel(AttnArgs a) {
  constexpr int D = 128, BM = 128, KT = 8, DT = 4, TILE = kBN * D;
  // two stages as four distinct LDS objects: the compiler can then tell that
  // the copy into one stage never overlaps the reads of the other and does not
  // make those reads wait for the copy
  __shared__ __attribute__((aligned(1024))) uint16_t K0[TILE], K1[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t V0[TILE], V1[TILE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hi = lane >> 5;
  const int N = a.N;
  const WorkItem wi = map_work(a);
  const int qblk = wi.qblk, h = wi.h, b = wi.b;
  const int64_t head_off = (int64_t)b * a.sb + (int64_t)h * a.sh;
  const uint16_t* __restrict__ Qh = a.q + head_off;
  const uint16_t* __restrict__ Kh = a.k + head_off;
  const uint16_t* __restrict__ Vh = a.v + head_off;

  const int qrow = qblk * BM + wave * 32 + l32;
  bf16x8 qf[KT];
  {
    const uint16_t* src = Qh + (int64_t)min(qrow, N - 1) * a.sn + hi * 8;
#pragma unroll
    for (int t = 0; t < KT; ++t) qf[t] = __builtin_bit_cast(bf16x8, *(const u32x4*)(src + t * 16));
  }
  retire_loads();

  const cint_ptr rowp = (cint_ptr)a.row_ptr;
  const cint_ptr cols = (cint_ptr)a.col_idx;
  const int rbeg = rowp[qblk], rend = rowp[qblk + 1];
  int nsub = (rend - rbeg) * 2;
  if (nsub > 0 && cols[rend - 1] == a.nb - 1) {
    const int last_real = N - (a.nb - 1) * BM;
    nsub -= 2 - (last_real + kBN - 1) / kBN;
  }
  // key blocks of the row: the current one (sub-tiles 2 i, 2 i + 1) and the
  // next, held in scalar registers; the one after is loaded a step before it
  // is needed
  const int nblk = rend - rbeg;
  int blk_cur = nblk > 0 ? cols[rbeg] : 0, blk_nxt = nblk > 1 ? cols[rbeg + 1] : 0;

  // Copy roles: wave w, instruction j covers tile rows 16w + 4j + lane/16 at
  // physical chunk lane%16 (i.e. logical chunk (lane%16) ^ swizzle(row)).  The
  // copies are buffer loads straight to LDS: one descriptor per tensor and head,
  // a 32-bit per-lane offset (row * row_bytes + 16 * chunk) and the sub-tile
  // start in the scalar offset.  The host keeps (N + 64) * row_bytes < 2^31.
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t row_bytes = (uint32_t)a.sn * 2u;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)Kh, (short)0, 0x7fffffff, kBufferWord3);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)Vh, (short)0, 0x7fffffff, kBufferWord3);
  // For rows 16w + 4j + lane/16: swz_k(row) = 4j + lane/16 and swz_v(row) =
  // 4 (lane/16) + j, so the swizzled 16-byte chunk offsets are one per-lane
  // base XOR an immediate, and the row offsets one per-lane base plus a
  // uniform multiple of 4 rows (few registers live across the loop).
  const uint32_t rbase = (uint32_t)(16 * wv + (lane >> 4)) * row_bytes;
  const uint32_t kbase = (uint32_t)(((lane & 15) ^ (lane >> 4)) * 16);
  const uint32_t vbase = (uint32_t)(((lane & 15) ^ (4 * (lane >> 4))) * 16);
  auto dma = [&](uint16_t* kst, uint16_t* vst, int key0) {
    if (key0 + kBN <= N) {
      const uint32_t so = (uint32_t)key0 * row_bytes;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t ro = rbase + (uint32_t)(4 * j) * row_bytes;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)&kst[(16 * wv + 4 * j) * D], 16,
                                                 ro + (kbase ^ (64u * j)), so, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)&vst[(16 * wv + 4 * j) * D], 16,
                                                 ro + (vbase ^ (16u * j)), so, 0, 0);
      }
    } else {  // tail sub-tile: rows past N are clamped to row N - 1 (masked below)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = 16 * wv + 4 * j + (lane >> 4);
        const uint32_t ro = (uint32_t)min(key0 + row, N - 1) * row_bytes;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)&kst[(16 * wv + 4 * j) * D], 16,
                                                 ro + (kbase ^ (64u * j)), 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)&vst[(16 * wv + 4 * j) * D], 16,
                                                 ro + (vbase ^ (16u * j)), 0, 0, 0);
      }
    }
  };

  f32x16 o[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) o[i] = f32x16{};
  float m_run = -1e30f, l_run = 0.f;
  const float c2 = a.scale_log2;
  const int g16 = lane >> 4, j16 = lane & 15;
  // LDS element offsets of the swizzled stage reads, as one per-lane base and
  // an XOR / add of immediates:
  //   K fragment (kt, t):        4096 kt + (kaddr ^ 16 t)
  //   V transpose read (ks, dt): 2048 ks + (vaddr ^ 32 dt)  (+ vdelta for rows + 8)
  const int kaddr = l32 * 128 + 16 * ((l32 & 15) >> 1) + 8 * (hi ^ (l32 & 1));
  const int vq = j16 >> 2, vc1 = (2 * (g16 & 1) + ((j16 >> 1) & 1)) ^ hi;
  const int vaddr = (4 * hi + vq) * 128 + 32 * vq + 8 * vc1 + (j16 & 1) * 4;
  const int vdelta = 1024 + 8 * ((vc1 ^ 2) - vc1);

  // One 64-key sub-tile u held in (Kb, Vb); the copy of sub-tile u + 1 goes to
  // (Kn, Vn) as soon as every wave has passed the barrier (they have all
  // finished reading that stage in step u - 1).
  // k = u % 2: sub-tile u is half k of block blk_cur; sub-tile u + 1 is half 1
  // of it (k = 0) or half 0 of the next block (k = 1)
  auto step = [&](const uint16_t* Kb, const uint16_t* Vb, uint16_t* Kn, uint16_t* Vn, int u, int k) {
    const int key0 = blk_cur * BM + k * kBN;
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0): sub-tile u landed, other stage drained
    __builtin_amdgcn_s_barrier();
    if (u + 1 < nsub) dma(Kn, Vn, k == 0 ? blk_cur * BM + kBN : blk_nxt * BM);

    // S^T = K Q^T: read the 16 K fragments, then the MFMAs (reads run four ahead)
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

    if (key0 + kBN > N) {  // key row of s[kt][r]: key0 + 32 kt + 8 (r / 4) + 4 hi + r % 4
      const uint32_t vm = tile_row_mask(N - key0, hi);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (!((vm >> (16 * kt + r)) & 1u)) s[kt][r] = -__builtin_inff();
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
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kt][r] = fast_exp2(__builtin_fmaf(s[kt][r], c2, -mc));
    // P as bf16 (the operand of the value product); the row sum is taken over
    // the same rounded values with v_dot2 against bf16 ones
    bf16x8 pf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kt = ks >> 1, r0 = (ks & 1) * 8;
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w[e] = pack_bf16x2(s[kt][r0 + 2 * e], s[kt][r0 + 2 * e + 1]);
        l_run = dot2_bf16(w[e], 0x3f803f80u, l_run);
      }
      pf[ks] = __builtin_bit_cast(bf16x8, w);
    }

    // O^T += V^T P^T with the transpose reads of the swizzled V stage.  The
    // wave raises its issue priority for this block: the two waves sharing a
    // SIMD (from different workgroups) then drift out of phase, one wave's
    // softmax running under the other's matrix work.
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
    if (k == 1) {  // the next step opens the next block
      const int i = u >> 1;
      blk_cur = blk_nxt;
      blk_nxt = i + 2 < nblk ? cols[rbeg + i + 2] : 0;
    }
  };

  if (nsub > 0) dma(K0, V0, blk_cur * BM);
  int u = 0;
  for (; u + 2 <= nsub; u += 2) {
    step(K0, V0, K1, V1, u, 0);
    step(K1, V1, K0, V0, u + 1, 1);
  }
  if (u < nsub) step(K0, V0, K1, V1, u, 0);

  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qrow < N) {
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
                            const int32_t* row_order, int block, float scale, hipStream_t stream) {
  AttnArgs a;
  a.q = (const uint16_t*)q; a.k = (const uint16_t*)k; a.v = (const uint16_t*)v; a.o = (uint16_t*)o;
  a.lse = lse; a.row_ptr = row_ptr; a.col_idx = col_idx; a.row_order = row_order;
  a.sb = s.stride_b; a.sh = s.stride_h; a.sn = s.stride_n;
  a.B = s.B; a.H = s.H; a.N = s.N; a.block = block; a.nb = (s.N + block - 1) / block;
  a.head_major = choose_head_major(s, 2);
  a.scale_log2 = scale * kLog2e;
  dim3 grid((unsigned)((int64_t)a.nb * s.H * s.B));
  // the buffer-load kernel addresses a head with 32-bit offsets
  const bool offsets_fit = ((int64_t)s.N + 64) * a.sn * 2 < ((int64_t)1 << 31);
  if (s.D == 128 && block == 128 && offsets_fit)
    hipLaunchKernelGGL(attn_bf16_d128_kernel, grid, dim3(256), 0, stream, a);
  else if (s.D == 128 && block == 128)
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
