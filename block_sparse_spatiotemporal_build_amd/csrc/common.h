// Internal helpers shared by the gfx950 kernels of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bsa.h"

namespace bsa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;   // MFMA A/B operand (8 x bf16)
typedef __attribute__((ext_vector_type(16))) float f32x16;   // 32x32 MFMA accumulator
typedef __attribute__((ext_vector_type(4))) float f32x4;     // 16x16 MFMA accumulator
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;  // 16-byte load unit
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 bits -> float (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f2bf(float x) {
  __bf16 b = (__bf16)x;
  return (uint32_t)__builtin_bit_cast(uint16_t, b);
}
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
// two floats -> packed bf16 pair (RNE), one v_cvt_pk_bf16_f32 on gfx950
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// acc + a.lo * b.lo + a.hi * b.hi for packed bf16 pairs (v_dot2_f32_bf16).
// Written as inline asm because the compiler builtin, fed 32-bit elements of a
// vector register tuple, read the tuple's first element for every element.
// The hardware does not interlock a dot result: another VALU instruction that
// reads it (other than as the accumulator of the next v_dot2) must come at least
// three instructions later, and the compiler cannot see this inside inline asm
// (a v_add one instruction after the last dot of a chain read the value from
// before the chain).  So the results here only feed the next dot of a chain or
// are read much later; a CPU test scans the compiled kernels for reads that
// come too soon.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  float d;
  asm volatile("v_dot2_f32_bf16 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(acc));
  return d;
}

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// 4 bf16 of one column from 4 consecutive rows of a row-major LDS tile.
// ds_read_b64_tr_b16: within each 16-lane group, lane j supplies the address of
// 4 consecutive elements M[j][0..3]; lane i receives M[4e + i/4][i%4], e = 0..3.
// With lane j pointing at row j/4, column 4*(j%4), lane i gets column i of rows 0..3.
__device__ __forceinline__ u32x2 lds_tr16(const uint16_t* p) {
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(u32x2, r);
}

// Combine a value of lane l with that of lane l ^ 32 (v_permlane32_swap).
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Wait for every outstanding vector-memory load of this wave (s_waitcnt vmcnt(0)).
// Used after loading registers that a loop then reuses: the loop's own prefetch
// loads share the in-order vmcnt counter, so without a retire point before the
// loop the compiler's waits for those registers would also wait for the
// prefetch issued in each iteration.
// Staging of 256-byte rows (head_dim 128, bf16) straight from global memory to
// LDS with buffer_load ... lds: lane i of one instruction writes 16 bytes at
// (LDS base + 16 i), so a tile's layout is chosen by which 16-byte chunk each
// lane loads.  Rows keep their 16 chunks XOR-swizzled instead of padded:
//   swz_k: chunk ^ (row & 15) -- the 16 rows that 16 lanes read for one MFMA A
//          operand hit 16 different chunks (all 64 banks);
//   swz_v: chunk ^ (4 (row & 3) + ((row >> 2) & 3)) -- the 4 rows x 4 chunks
//          touched by one ds_read_b64_tr_b16 over 32 lanes are distinct.
typedef __attribute__((address_space(3))) void lds_void;
// int32 index arrays read through the constant address space: uniform indices
// become scalar loads (counted by lgkmcnt), so fetching the next block index
// never makes a wave wait on its own vector-memory copies in flight
typedef const __attribute__((address_space(4))) int32_t* cint_ptr;
typedef const __attribute__((address_space(4))) int64_t* cint64_ptr;
constexpr int kBufferWord3 = 0x00020000;  // raw (untyped, stride 0) buffer loads, gfx9 family
// Raw buffer descriptor as four scalar words (base, stride 0, size, format),
// for copies issued from inline assembly.
typedef __attribute__((ext_vector_type(4))) int32_t i32x4;
__device__ __forceinline__ i32x4 raw_buffer_desc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)base;
  return i32x4{(int32_t)(uint32_t)b, (int32_t)((b >> 32) & 0xffffu), (int32_t)bytes, kBufferWord3};
}
// buffer_load_dwordx4 ... lds: lane i copies 16 bytes at byte offset voff of
// the buffer to LDS byte address lds + 16 i (lds is wave-uniform).  Issued from
// assembly so the compiler's wait insertion does not see it: it cannot tell
// which LDS stage such a copy writes and would otherwise wait for copies still
// in flight before reading any stage.  The caller orders every read of the
// destination after an explicit vmcnt wait (which counts these copies) and a
// barrier; the copy writes no register.
// The copy writes M0, which the compiler treats as reserved: a kernel that
// uses it must not also use the compiler's LDS-copy builtins (which keep their
// LDS address in M0) or anything else that holds a value in M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_copy16(i32x4 rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(lds)
               : "memory", "m0");
}
// The same with a uniform byte offset soff added to every lane's voff.
__device__ __forceinline__ void lds_copy16_so(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(lds), "s"(soff)
               : "memory", "m0");
}
#pragma clang diagnostic pop
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_void*)p;
}
// LDS element at a byte offset from a stage base
__device__ __forceinline__ const uint16_t* lds_byte(const uint16_t* base, uint32_t off) {
  return (const uint16_t*)((const char*)base + off);
}
__device__ __forceinline__ int swz_k(int row) { return row & 15; }
__device__ __forceinline__ int swz_v(int row) { return 4 * (row & 3) + ((row >> 2) & 3); }

// Valid-row mask of the S^T accumulators of a 64-key sub-tile when only its
// first n rows are real keys: bit 16 kt + r covers s[kt][r], whose key row is
// 32 kt + 8 (r / 4) + 4 hi + r % 4 (hi = lane / 32).  Built from n with
// immediates only, so that the per-element tests need no per-element registers.
__device__ __forceinline__ uint32_t tile_row_mask(int n, int hi) {
  uint32_t m = 0;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = min(max(n - (32 * kt + 8 * g + 4 * hi), 0), 4);
      m |= ((1u << c) - 1u) << (16 * kt + 4 * g);
    }
  return m;
}

// Online softmax with a lazily moved reference: the running maximum used as
// the exponent reference is replaced only when a new score exceeds it by more
// than this many powers of two, so weights stay below 2^8 and the O/l rescale
// is skipped on most tiles.  O and l always share one reference, so the
// normalised output and the LSE are unchanged up to rounding.
constexpr float kLazyRescaleLog2 = 8.f;

__device__ __forceinline__ void retire_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Launch-error check used by every entry point after enqueueing kernels.
bool launch_ok(const char* what);

// Records a failure message for bsa_last_error() (host, thread-local).
void set_error(const char* fmt, ...);

// Index, in a list of R items, of the item that workgroup S + j runs, chosen so
// that the workgroups the hardware deals round-robin to one XCD (those with the
// same pid mod 8) take one contiguous range of the list, in order.
__device__ __forceinline__ int xcd_contiguous(int j, int S, int R) {
  const int x = (S + j) & 7, off = S & 7;
  int base = 0;
  for (int y = 0; y < x; ++y) {
    const int j0 = (y - off) & 7;
    base += j0 < R ? (R - 1 - j0) / 8 + 1 : 0;
  }
  return base + (j - ((x - off) & 7)) / 8;
}

// The same over consecutive windows of W items (W a multiple of 8, one
// workgroup per CU): item order is kept from window to window, and inside a
// window each XCD takes one contiguous run.  So the XCDs work on
// neighbouring items (one head at a time in head-major order) while the
// workgroups sharing an L2 still share their neighbours' tiles.
__device__ __forceinline__ int xcd_windowed(int j, int S, int R, int W) {
  const int base = (j / W) * W;
  return base + xcd_contiguous(j - base, S + base, min(W, R - base));
}
constexpr int kXcdWindow = 256;

}  // namespace bsa
