// C-ABI entry points: argument validation, dispatch, status and error text.
//
// Validation runs entirely on the host before any HIP call, so a rejected
// call launches nothing and touches no output.

#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "launch.h"

namespace bsa {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

bool launch_ok(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("%s: kernel launch failed: %s", what, hipGetErrorString(e));
    return false;
  }
  return true;
}

static bsa_status fail(bsa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Block CSR invariants on host arrays (the checker behind bsa_check_csr).
static bsa_status check_csr_host(const int32_t* rp, const int32_t* ci, int32_t nrows, int32_t ncols, int64_t cap,
                                 const char* fn) {
  if (rp == nullptr || (ci == nullptr && nrows > 0)) return fail(BSA_ERR_ARG, "%s: NULL pointer", fn);
  if (nrows < 0 || ncols < 0) return fail(BSA_ERR_ARG, "%s: negative size", fn);
  if (rp[0] != 0) return fail(BSA_ERR_ARG, "%s: row_ptr[0] = %d, not 0", fn, rp[0]);
  for (int32_t r = 0; r < nrows; ++r)
    if (rp[r + 1] < rp[r])
      return fail(BSA_ERR_ARG, "%s: row_ptr decreases at row %d (%d -> %d)", fn, r, rp[r], rp[r + 1]);
  if ((int64_t)rp[nrows] > cap)
    return fail(BSA_ERR_CAPACITY, "%s: %d entries exceed the capacity %lld", fn, rp[nrows], (long long)cap);
  for (int32_t r = 0; r < nrows; ++r)
    for (int32_t e = rp[r]; e < rp[r + 1]; ++e) {
      if (ci[e] < 0 || ci[e] >= ncols)
        return fail(BSA_ERR_ARG, "%s: row %d has column %d outside [0, %d)", fn, r, ci[e], ncols);
      if (e > rp[r] && ci[e] <= ci[e - 1])
        return fail(BSA_ERR_ARG, "%s: row %d columns not strictly ascending (%d then %d)", fn, r, ci[e - 1], ci[e]);
    }
  return BSA_OK;
}

// BSA_DEBUG, read at every call that can check its output
static bool debug_mode() {
  const char* e = getenv("BSA_DEBUG");
  return e != nullptr && e[0] != 0 && strcmp(e, "0") != 0;
}

// Debug check of a device CSR just written on `stream`: synchronise, copy it
// back and run the host checker; BSA_ERR_CHECK on a violation.
static bsa_status debug_check_device_csr(const int32_t* rp_dev, const int32_t* ci_dev, int32_t nrows, int32_t ncols,
                                         int64_t cap, hipStream_t stream, const char* fn) {
  if (hipStreamSynchronize(stream) != hipSuccess) return fail(BSA_ERR_HIP, "%s: debug check: synchronise failed", fn);
  int32_t* rp = (int32_t*)malloc(sizeof(int32_t) * ((size_t)nrows + 1));
  if (rp == nullptr) return fail(BSA_ERR_CHECK, "%s: debug check: out of host memory", fn);
  if (hipMemcpy(rp, rp_dev, sizeof(int32_t) * ((size_t)nrows + 1), hipMemcpyDeviceToHost) != hipSuccess) {
    free(rp);
    return fail(BSA_ERR_HIP, "%s: debug check: copy of row_ptr failed", fn);
  }
  const int64_t n = rp[nrows] < 0 ? 0 : (rp[nrows] > cap ? cap : rp[nrows]);
  int32_t* ci = (int32_t*)malloc(sizeof(int32_t) * ((size_t)n + 1));
  if (ci == nullptr) {
    free(rp);
    return fail(BSA_ERR_CHECK, "%s: debug check: out of host memory", fn);
  }
  if (n > 0 && hipMemcpy(ci, ci_dev, sizeof(int32_t) * (size_t)n, hipMemcpyDeviceToHost) != hipSuccess) {
    free(rp);
    free(ci);
    return fail(BSA_ERR_HIP, "%s: debug check: copy of col_idx failed", fn);
  }
  bsa_status st = check_csr_host(rp, ci, nrows, ncols, cap, fn);
  free(rp);
  free(ci);
  if (st != BSA_OK) {
    char msg[512];
    snprintf(msg, sizeof msg, "%s", g_err);
    return fail(BSA_ERR_CHECK, "BSA_DEBUG: %s", msg);
  }
  return BSA_OK;
}

// Shape checks shared by the tensor calls: sizes positive, strides that keep
// each row inside its own head, D contiguous, 16-byte aligned rows.
static bsa_status check_shape(const bsa_shape* s, int elem_bytes, const char* fn) {
  if (s == nullptr) return fail(BSA_ERR_ARG, "%s: shape is NULL", fn);
  if (s->B <= 0 || s->H <= 0 || s->N <= 0 || s->D <= 0)
    return fail(BSA_ERR_ARG, "%s: B, H, N, D must be positive (got %d, %d, %d, %d)", fn, s->B, s->H,
                s->N, s->D);
  if (s->stride_n < s->D || s->stride_h < 0 || s->stride_b < 0)
    return fail(BSA_ERR_ARG, "%s: stride_n must be >= D and strides non-negative", fn);
  if (((int64_t)s->stride_n * elem_bytes) % 16 != 0 || ((int64_t)s->stride_h * elem_bytes) % 16 != 0 ||
      ((int64_t)s->stride_b * elem_bytes) % 16 != 0)
    return fail(BSA_ERR_ARG, "%s: strides must be multiples of 16 bytes", fn);
  return BSA_OK;
}

static bsa_status check_desc(const bsa_mask_desc* d, const char* fn) {
  if (d == nullptr) return fail(BSA_ERR_ARG, "%s: desc is NULL", fn);
  if (d->kind < BSA_MASK_ALL || d->kind > BSA_MASK_RADIAL)
    return fail(BSA_ERR_ARG, "%s: unknown mask kind %d", fn, d->kind);
  if (d->frames < 1 || d->frame_tokens < 1 || d->block < 1 || d->block > 4096)
    return fail(BSA_ERR_ARG, "%s: frames, frame_tokens >= 1 and 1 <= block <= 4096 required", fn);
  if (d->window < 0 || d->anchor_period < 0 || d->anchor_step < 0 || d->radial_w < 0)
    return fail(BSA_ERR_ARG, "%s: window, anchor_period, anchor_step, radial_w must be >= 0", fn);
  const int64_t N = (int64_t)d->frames * d->frame_tokens;
  if (N > 0x7fffffffLL - 4096) return fail(BSA_ERR_ARG, "%s: frames * frame_tokens too large", fn);
  const int64_t nb = (N + d->block - 1) / d->block;
  if (nb > 46340) return fail(BSA_ERR_ARG, "%s: %lld blocks exceed the limit of 46340", fn, (long long)nb);
  return BSA_OK;
}

}  // namespace bsa

using namespace bsa;

extern "C" {

int32_t bsa_mask_num_blocks(const bsa_mask_desc* desc) {
  if (check_desc(desc, "bsa_mask_num_blocks") != BSA_OK) return -1;
  const int64_t N = (int64_t)desc->frames * desc->frame_tokens;
  return (int32_t)((N + desc->block - 1) / desc->block);
}

bsa_status bsa_build_block_mask(const bsa_mask_desc* desc, int32_t* row_ptr, int32_t* col_idx,
                                int64_t col_capacity, int32_t* row_order, void* stream) {
  const char* fn = "bsa_build_block_mask";
  bsa_status st = check_desc(desc, fn);
  if (st != BSA_OK) return st;
  if (row_ptr == nullptr || col_idx == nullptr) return fail(BSA_ERR_ARG, "%s: NULL output pointer", fn);
  const int64_t nb = bsa_mask_num_blocks(desc);
  if (col_capacity < nb * nb)
    return fail(BSA_ERR_CAPACITY, "%s: col_capacity %lld < nb*nb = %lld", fn, (long long)col_capacity,
                (long long)(nb * nb));
  g_err[0] = 0;
  st = launch_build_block_mask(*desc, row_ptr, col_idx, row_order, (hipStream_t)stream);
  if (st == BSA_OK && debug_mode())
    st = debug_check_device_csr(row_ptr, col_idx, (int32_t)nb, (int32_t)nb, col_capacity, (hipStream_t)stream, fn);
  return st;
}

bsa_status bsa_block_sparse_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                                     bsa_dtype dtype, const bsa_shape* shape, const int32_t* row_ptr,
                                     const int32_t* col_idx, const int32_t* row_order, int32_t block,
                                     float scale, void* stream) {
  const char* fn = "bsa_block_sparse_attn_fwd";
  if (dtype != BSA_DT_BF16 && dtype != BSA_DT_F32) return fail(BSA_ERR_ARG, "%s: unknown dtype %d", fn, dtype);
  const int eb = dtype == BSA_DT_BF16 ? 2 : 4;
  bsa_status st = check_shape(shape, eb, fn);
  if (st != BSA_OK) return st;
  if (!q || !k || !v || !o || !row_ptr || !col_idx) return fail(BSA_ERR_ARG, "%s: NULL tensor pointer", fn);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(BSA_ERR_ARG, "%s: q, k, v, o must be 16-byte aligned", fn);
  if (!__builtin_isfinite(scale) || scale <= 0.f) return fail(BSA_ERR_ARG, "%s: scale must be finite and > 0", fn);
  if (block < 1) return fail(BSA_ERR_ARG, "%s: block must be >= 1", fn);
  if (dtype == BSA_DT_BF16) {
    if (shape->D != 64 && shape->D != 128)
      return fail(BSA_ERR_UNSUPPORTED, "%s: bf16 supports D in {64, 128} (got %d)", fn, shape->D);
    if (block != 64 && block != 128)
      return fail(BSA_ERR_UNSUPPORTED, "%s: bf16 supports block in {64, 128} (got %d)", fn, block);
  } else {
    if (shape->D != 32 && shape->D != 64 && shape->D != 128)
      return fail(BSA_ERR_UNSUPPORTED, "%s: f32 supports D in {32, 64, 128} (got %d)", fn, shape->D);
    if (block != 16 && block != 32 && block != 64 && block != 128)
      return fail(BSA_ERR_UNSUPPORTED, "%s: f32 supports block in {16, 32, 64, 128} (got %d)", fn, block);
  }
  if ((int64_t)shape->B * shape->H > 65535 * 65535LL || shape->H > 65535 || shape->B > 65535)
    return fail(BSA_ERR_ARG, "%s: B and H must be <= 65535", fn);
  g_err[0] = 0;
  if (dtype == BSA_DT_BF16)
    return launch_attn_bf16(q, k, v, o, lse, *shape, row_ptr, col_idx, row_order, block, scale,
                            (hipStream_t)stream);
  return launch_attn_f32(q, k, v, o, lse, *shape, row_ptr, col_idx, block, scale, (hipStream_t)stream);
}

bsa_status bsa_transpose_block_mask(const int32_t* row_ptr, const int32_t* col_idx, int32_t nb, int32_t* col_ptr,
                                    int32_t* row_idx, int64_t capacity, void* stream) {
  const char* fn = "bsa_transpose_block_mask";
  if (nb < 1 || nb > 46340) return fail(BSA_ERR_ARG, "%s: nb must be in [1, 46340]", fn);
  if (!row_ptr || !col_idx || !col_ptr || !row_idx) return fail(BSA_ERR_ARG, "%s: NULL pointer", fn);
  if (capacity < (int64_t)nb * nb)
    return fail(BSA_ERR_CAPACITY, "%s: capacity %lld < nb*nb = %lld", fn, (long long)capacity,
                (long long)nb * nb);
  g_err[0] = 0;
  return launch_transpose_block_mask(row_ptr, col_idx, nb, col_ptr, row_idx, (hipStream_t)stream);
}

size_t bsa_block_sparse_attn_bwd_workspace(const bsa_shape* shape) {
  if (check_shape(shape, 2, "bsa_block_sparse_attn_bwd_workspace") != BSA_OK) return 0;
  return attn_bwd_workspace(*shape);
}

bsa_status bsa_block_sparse_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
                                     const float* lse, bsa_dtype dtype, const bsa_shape* shape,
                                     const int32_t* row_ptr, const int32_t* col_idx, const int32_t* col_ptr,
                                     const int32_t* row_idx, int32_t block, float scale, void* dq, void* dk,
                                     void* dv, void* workspace, size_t ws_bytes, void* stream) {
  const char* fn = "bsa_block_sparse_attn_bwd";
  if (dtype != BSA_DT_BF16) return fail(BSA_ERR_UNSUPPORTED, "%s: only bf16 is implemented", fn);
  bsa_status st = check_shape(shape, 2, fn);
  if (st != BSA_OK) return st;
  if (shape->D != 128) return fail(BSA_ERR_UNSUPPORTED, "%s: D must be 128 (got %d)", fn, shape->D);
  if (block != 128) return fail(BSA_ERR_UNSUPPORTED, "%s: block must be 128 (got %d)", fn, block);
  if (!q || !k || !v || !o || !dO || !lse || !row_ptr || !col_idx || !col_ptr || !row_idx || !dq || !dk || !dv)
    return fail(BSA_ERR_ARG, "%s: NULL pointer", fn);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dO) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv))
    return fail(BSA_ERR_ARG, "%s: tensors must be 16-byte aligned", fn);
  if (!__builtin_isfinite(scale) || scale <= 0.f) return fail(BSA_ERR_ARG, "%s: scale must be finite and > 0", fn);
  if ((int64_t)shape->B * shape->H * ((shape->N + 127) / 128) > 0x7fffffffLL)
    return fail(BSA_ERR_ARG, "%s: too many (block, sequence) pairs", fn);
  if (((int64_t)shape->N + 128) * shape->stride_n * 2 >= ((int64_t)1 << 31))
    return fail(BSA_ERR_UNSUPPORTED, "%s: a head must fit 32-bit byte offsets", fn);
  const size_t need = bsa_block_sparse_attn_bwd_workspace(shape);
  if (workspace == nullptr || ws_bytes < need || ((uintptr_t)workspace & 255u) != 0)
    return fail(BSA_ERR_WORKSPACE, "%s: workspace of %zu bytes (256-byte aligned) required, got %zu", fn, need,
                workspace ? ws_bytes : (size_t)0);
  g_err[0] = 0;
  return launch_attn_bwd_bf16(q, k, v, o, dO, lse, *shape, row_ptr, col_idx, col_ptr, row_idx, scale, dq, dk, dv,
                              workspace, (hipStream_t)stream);
}

size_t bsa_linear_attn_workspace(const bsa_shape* shape) {
  if (check_shape(shape, 2, "bsa_linear_attn_workspace") != BSA_OK) return 0;
  return linear_plan(*shape).total;
}

static bsa_status check_linear(const void* q, const void* k, const void* v, void* o, bsa_dtype dtype,
                               const bsa_shape* shape, const char* fn) {
  if (dtype != BSA_DT_BF16) return fail(BSA_ERR_UNSUPPORTED, "%s: only bf16 is implemented", fn);
  bsa_status st = check_shape(shape, 2, fn);
  if (st != BSA_OK) return st;
  if (shape->D != 64 && shape->D != 128)
    return fail(BSA_ERR_UNSUPPORTED, "%s: D must be 64 or 128 (got %d)", fn, shape->D);
  if (!q || !k || !v || !o) return fail(BSA_ERR_ARG, "%s: NULL tensor pointer", fn);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(BSA_ERR_ARG, "%s: q, k, v, o must be 16-byte aligned", fn);
  if ((int64_t)shape->B * shape->H > 65535) return fail(BSA_ERR_ARG, "%s: B * H must be <= 65535", fn);
  return BSA_OK;
}

bsa_status bsa_linear_attn_fwd(const void* q, const void* k, const void* v, void* o, bsa_dtype dtype,
                               const bsa_shape* shape, float* S, float* z, void* workspace, size_t ws_bytes,
                               void* stream) {
  const char* fn = "bsa_linear_attn_fwd";
  bsa_status st = check_linear(q, k, v, o, dtype, shape, fn);
  if (st != BSA_OK) return st;
  const size_t need = linear_plan(*shape).total;
  if (workspace == nullptr || ws_bytes < need || ((uintptr_t)workspace & 255u) != 0)
    return fail(BSA_ERR_WORKSPACE, "%s: workspace of %zu bytes (256-byte aligned) required, got %zu", fn, need,
                workspace ? ws_bytes : (size_t)0);
  g_err[0] = 0;
  return launch_linear_attn(q, k, v, o, *shape, S, z, workspace, (hipStream_t)stream);
}

size_t bsa_linear_attn_noalloc_max_scratch(void) { return kLinNoAllocBytes; }

bsa_status bsa_linear_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, bsa_dtype dtype,
                                       const bsa_shape* shape, float* S, float* z, void* stream) {
  const char* fn = "bsa_linear_attn_fwd_noalloc";
  bsa_status st = check_linear(q, k, v, o, dtype, shape, fn);
  if (st != BSA_OK) return st;
  const size_t need = linear_plan(*shape).total;
  if (need > kLinNoAllocBytes)
    return fail(BSA_ERR_UNSUPPORTED,
                "%s: this shape needs %zu bytes of scratch, more than the %zu of the no-allocation call "
                "(use bsa_linear_attn_fwd with a workspace)", fn, need, kLinNoAllocBytes);
  void* ws = nullptr;
  st = linear_noalloc_scratch(&ws);
  if (st != BSA_OK) return st;
  g_err[0] = 0;
  return launch_linear_attn(q, k, v, o, *shape, S, z, ws, (hipStream_t)stream);
}

size_t bsa_causal_linear_attn_workspace(const bsa_shape* shape) {
  if (check_shape(shape, 2, "bsa_causal_linear_attn_workspace") != BSA_OK) return 0;
  if (shape->D != 128 || !linear_plan(*shape).d128) return 0;
  return causal_plan(*shape).total;
}

bsa_status bsa_causal_linear_attn_fwd(const void* q, const void* k, const void* v, void* o, bsa_dtype dtype,
                                      const bsa_shape* shape, const float* S_in, const float* z_in,
                                      float* S_out, float* z_out, void* workspace, size_t ws_bytes,
                                      void* stream) {
  const char* fn = "bsa_causal_linear_attn_fwd";
  if (dtype != BSA_DT_BF16) return fail(BSA_ERR_UNSUPPORTED, "%s: only bf16 is implemented", fn);
  bsa_status st = check_shape(shape, 2, fn);
  if (st != BSA_OK) return st;
  if (shape->D != 128 || !linear_plan(*shape).d128)
    return fail(BSA_ERR_UNSUPPORTED, "%s: D must be 128 (and a head within 32-bit offsets)", fn);
  if (!q || !k || !v || !o) return fail(BSA_ERR_ARG, "%s: NULL tensor pointer", fn);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(BSA_ERR_ARG, "%s: q, k, v, o must be 16-byte aligned", fn);
  if ((S_in == nullptr) != (z_in == nullptr)) return fail(BSA_ERR_ARG, "%s: give both S_in and z_in or neither", fn);
  if (!aligned16(S_in) || !aligned16(z_in) || !aligned16(S_out) || !aligned16(z_out))
    return fail(BSA_ERR_ARG, "%s: S_in, z_in, S_out, z_out must be 16-byte aligned", fn);
  if ((int64_t)shape->B * shape->H > 65535) return fail(BSA_ERR_ARG, "%s: B * H must be <= 65535", fn);
  const size_t need = causal_plan(*shape).total;
  if (workspace == nullptr || ws_bytes < need || ((uintptr_t)workspace & 255u) != 0)
    return fail(BSA_ERR_WORKSPACE, "%s: workspace of %zu bytes (256-byte aligned) required, got %zu", fn, need,
                workspace ? ws_bytes : (size_t)0);
  g_err[0] = 0;
  return launch_causal_linear_attn(q, k, v, o, *shape, S_in, z_in, S_out, z_out, workspace, (hipStream_t)stream);
}

bsa_status bsa_mixed_attn_fwd(const void* q, const void* k, const void* v, void* o, bsa_dtype dtype,
                              const bsa_shape* shape, const int32_t* row_ptr, const int32_t* col_idx,
                              const int32_t* row_order, int32_t block, float scale, float r, void* workspace,
                              size_t ws_bytes, void* stream) {
  const char* fn = "bsa_mixed_attn_fwd";
  if (dtype != BSA_DT_BF16) return fail(BSA_ERR_UNSUPPORTED, "%s: only bf16 is implemented", fn);
  bsa_status st = check_shape(shape, 2, fn);
  if (st != BSA_OK) return st;
  if (!(r >= 0.f && r <= 1.f)) return fail(BSA_ERR_ARG, "%s: r must be in [0, 1]", fn);
  if (shape->D != 128 || !linear_plan(*shape).d128)
    return fail(BSA_ERR_UNSUPPORTED, "%s: D must be 128 (and a head within 32-bit offsets)", fn);
  if (!q || !k || !v || !o || (r > 0.f && (!row_ptr || !col_idx)))
    return fail(BSA_ERR_ARG, "%s: NULL pointer", fn);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(BSA_ERR_ARG, "%s: q, k, v, o must be 16-byte aligned", fn);
  if (r > 0.f) {
    if (!__builtin_isfinite(scale) || scale <= 0.f) return fail(BSA_ERR_ARG, "%s: scale must be finite and > 0", fn);
    if (block != 64 && block != 128) return fail(BSA_ERR_UNSUPPORTED, "%s: block must be 64 or 128", fn);
  }
  if ((int64_t)shape->B * shape->H > 65535) return fail(BSA_ERR_ARG, "%s: B * H must be <= 65535", fn);
  const size_t need = linear_plan(*shape).total;
  if (r < 1.f && (workspace == nullptr || ws_bytes < need || ((uintptr_t)workspace & 255u) != 0))
    return fail(BSA_ERR_WORKSPACE, "%s: workspace of %zu bytes (256-byte aligned) required", fn, need);
  g_err[0] = 0;
  hipStream_t sm = (hipStream_t)stream;
  if (r > 0.f) {
    st = launch_attn_bf16(q, k, v, o, nullptr, *shape, row_ptr, col_idx, row_order, block, scale, sm);
    if (st != BSA_OK || r == 1.f) return st;
  }
  return launch_linear_attn(q, k, v, o, *shape, nullptr, nullptr, workspace, sm, r > 0.f ? r : -1.f);
}

// ---- token clustering --------------------------------------------------------

size_t bsa_kmeans_workspace(const bsa_shape* shape, int32_t C) {
  if (check_shape(shape, 2, "bsa_kmeans_workspace") != BSA_OK) return 0;
  if (shape->D != 128 || C < 1 || C > kMaxKmClusters) return 0;
  return kmeans_plan(*shape, C).total;
}

bsa_status bsa_kmeans(const void* x, bsa_dtype dtype, const bsa_shape* shape, int32_t C, int32_t iters,
                      float* centroids, int32_t* labels, int32_t* perm, int32_t* offsets, void* workspace,
                      size_t ws_bytes, void* stream) {
  const char* fn = "bsa_kmeans";
  if (dtype != BSA_DT_BF16) return fail(BSA_ERR_UNSUPPORTED, "%s: only bf16 is implemented", fn);
  bsa_status st = check_shape(shape, 2, fn);
  if (st != BSA_OK) return st;
  if (shape->D != 128) return fail(BSA_ERR_UNSUPPORTED, "%s: D must be 128 (got %d)", fn, shape->D);
  if (C < 1 || C > kMaxKmClusters) return fail(BSA_ERR_ARG, "%s: C must be in [1, %d]", fn, kMaxKmClusters);
  if (iters < 0 || iters > 100000) return fail(BSA_ERR_ARG, "%s: iters must be in [0, 100000]", fn);
  if (!x || !centroids || !labels) return fail(BSA_ERR_ARG, "%s: NULL pointer", fn);
  if (!aligned16(x) || !aligned16(centroids) || !aligned16(labels) || !aligned16(perm) || !aligned16(offsets))
    return fail(BSA_ERR_ARG, "%s: x, centroids, labels, perm, offsets must be 16-byte aligned", fn);
  if ((int64_t)shape->B * shape->H > 65535) return fail(BSA_ERR_ARG, "%s: B * H must be <= 65535", fn);
  if ((int64_t)(shape->N + 255) / 256 > 65535) return fail(BSA_ERR_ARG, "%s: N too large", fn);
  const size_t need = kmeans_plan(*shape, C).total;
  if (workspace == nullptr || ws_bytes < need || ((uintptr_t)workspace & 255u) != 0)
    return fail(BSA_ERR_WORKSPACE, "%s: workspace of %zu bytes (256-byte aligned) required, got %zu", fn, need,
                workspace ? ws_bytes : (size_t)0);
  g_err[0] = 0;
  return launch_kmeans(x, *shape, C, iters, centroids, labels, perm, offsets, workspace, (hipStream_t)stream);
}

static bsa_status rows_permute(const void* src, bsa_dtype dtype, const bsa_shape* shape, const int32_t* perm,
                               void* dst, void* stream, bool scatter) {
  const char* fn = scatter ? "bsa_scatter_rows" : "bsa_gather_rows";
  if (dtype != BSA_DT_BF16 && dtype != BSA_DT_F32) return fail(BSA_ERR_ARG, "%s: unknown dtype %d", fn, dtype);
  const int eb = dtype == BSA_DT_BF16 ? 2 : 4;
  bsa_status st = check_shape(shape, eb, fn);
  if (st != BSA_OK) return st;
  if ((shape->D * eb) % 16 != 0) return fail(BSA_ERR_ARG, "%s: rows must be a multiple of 16 bytes", fn);
  if (shape->D * eb > 16 * 1024) return fail(BSA_ERR_UNSUPPORTED, "%s: rows above 16 KiB", fn);
  if (!src || !dst || !perm) return fail(BSA_ERR_ARG, "%s: NULL pointer", fn);
  if (src == dst) return fail(BSA_ERR_ARG, "%s: in place is not supported", fn);
  if (!aligned16(src) || !aligned16(dst)) return fail(BSA_ERR_ARG, "%s: tensors must be 16-byte aligned", fn);
  if ((int64_t)shape->B * shape->H > 65535) return fail(BSA_ERR_ARG, "%s: B * H must be <= 65535", fn);
  if ((int64_t)(shape->N + 3) / 4 > 0x7fffffffLL) return fail(BSA_ERR_ARG, "%s: N too large", fn);
  g_err[0] = 0;
  return launch_rows_permute(src, *shape, eb, perm, dst, scatter, (hipStream_t)stream);
}

bsa_status bsa_gather_rows(const void* x, bsa_dtype dtype, const bsa_shape* shape, const int32_t* perm, void* out,
                           void* stream) {
  return rows_permute(x, dtype, shape, perm, out, stream, false);
}

bsa_status bsa_scatter_rows(const void* y, bsa_dtype dtype, const bsa_shape* shape, const int32_t* perm, void* out,
                            void* stream) {
  return rows_permute(y, dtype, shape, perm, out, stream, true);
}

// ---- clustered compensation (SVG-EAR) -------------------------------------

static constexpr int kMaxKeyClusters = 512;

static size_t align256h(size_t x) { return (x + 255) & ~(size_t)255; }

static bsa_status check_clusters(const bsa_shape* shape, const int32_t* q_off, int32_t Cq, const int32_t* k_off,
                                 int32_t Ck, const char* fn) {
  bsa_status st = check_shape(shape, 2, fn);
  if (st != BSA_OK) return st;
  if (shape->D != 64 && shape->D != 128)
    return fail(BSA_ERR_UNSUPPORTED, "%s: D must be 64 or 128 (got %d)", fn, shape->D);
  if (Cq < 1 || Ck < 1) return fail(BSA_ERR_ARG, "%s: Cq and Ck must be >= 1", fn);
  if (Cq > 65535 || (int64_t)Cq * Ck > (1LL << 30))
    return fail(BSA_ERR_ARG, "%s: Cq <= 65535 and Cq * Ck <= 2^30 required", fn);
  if ((int64_t)shape->B * shape->H > 65535) return fail(BSA_ERR_ARG, "%s: B * H must be <= 65535", fn);
  if (!q_off || !k_off) return fail(BSA_ERR_ARG, "%s: NULL offsets", fn);
  return BSA_OK;
}

// floor(N * N * ppm / 10^6) in 128-bit integers: N * N * ppm needs up to 82
// bits; the result is at most N * N < 2^62
static long long budget_of(int N, int32_t density_ppm) {
  return (long long)((__int128)N * N * density_ppm / 1000000);
}

bsa_status bsa_cluster_centroids(const void* q, const void* k, const void* v, bsa_dtype dtype, const bsa_shape* shape,
                                 const int32_t* q_off, int32_t Cq, const int32_t* k_off, int32_t Ck, float* q_cent,
                                 float* k_cent, float* v_cent, void* stream) {
  const char* fn = "bsa_cluster_centroids";
  if (dtype != BSA_DT_BF16) return fail(BSA_ERR_UNSUPPORTED, "%s: only bf16 is implemented", fn);
  bsa_status st = check_clusters(shape, q_off, Cq, k_off, Ck, fn);
  if (st != BSA_OK) return st;
  const bool want_q = q_cent != nullptr, want_k = k_cent != nullptr || v_cent != nullptr;
  if (!want_q && !want_k) return fail(BSA_ERR_ARG, "%s: no output requested", fn);
  if (want_k && (!k_cent || !v_cent)) return fail(BSA_ERR_ARG, "%s: give both k_cent and v_cent or neither", fn);
  if ((want_q && !q) || (want_k && (!k || !v))) return fail(BSA_ERR_ARG, "%s: NULL input", fn);
  if ((want_q && !aligned16(q)) || (want_k && (!aligned16(k) || !aligned16(v))))
    return fail(BSA_ERR_ARG, "%s: q, k, v must be 16-byte aligned", fn);
  g_err[0] = 0;
  const CentroidSet which = want_q && want_k ? kCentAll : (want_q ? kCentQuery : kCentKey);
  return launch_centroids(q, k, v, *shape, q_off, Cq, k_off, Ck, q_cent, k_cent, v_cent, (hipStream_t)stream, which);
}

size_t bsa_route_scores_workspace(const bsa_shape* shape, int32_t Cq, int32_t Ck) {
  if (check_shape(shape, 2, "bsa_route_scores_workspace") != BSA_OK || Cq < 1 || Ck < 1) return 0;
  return probe_plan(*shape, Cq, Ck).total;
}

bsa_status bsa_route_scores(const void* k, const void* v, bsa_dtype dtype, const bsa_shape* shape,
                            const int32_t* q_off, int32_t Cq, const int32_t* k_off, int32_t Ck, const float* q_cent,
                            float* k_cent, float* v_cent, float scale, float* score, void* workspace,
                            size_t ws_bytes, void* stream) {
  const char* fn = "bsa_route_scores";
  if (dtype != BSA_DT_BF16) return fail(BSA_ERR_UNSUPPORTED, "%s: only bf16 is implemented", fn);
  bsa_status st = check_clusters(shape, q_off, Cq, k_off, Ck, fn);
  if (st != BSA_OK) return st;
  if (!k || !v || !q_cent || !k_cent || !v_cent || !score) return fail(BSA_ERR_ARG, "%s: NULL pointer", fn);
  if (!aligned16(k) || !aligned16(v) || !aligned16(q_cent) || !aligned16(k_cent) || !aligned16(v_cent))
    return fail(BSA_ERR_ARG, "%s: misaligned pointer", fn);
  if (!__builtin_isfinite(scale) || scale <= 0.f) return fail(BSA_ERR_ARG, "%s: scale must be finite and > 0", fn);
  const size_t need = probe_plan(*shape, Cq, Ck).total;
  if (!workspace || ws_bytes < need || ((uintptr_t)workspace & 255u))
    return fail(BSA_ERR_WORKSPACE, "%s: workspace of %zu bytes (256-byte aligned) required", fn, need);
  g_err[0] = 0;
  return launch_route_scores(k, v, *shape, q_off, Cq, k_off, Ck, q_cent, k_cent, v_cent, scale, score, workspace,
                             (hipStream_t)stream);
}

// debug check of every head's route CSR: rows [BH][Cq + 1], columns
// [BH][Cq * Ck] (each head's columns start at its own r * Cq * Ck)
static bsa_status debug_check_route(const bsa_shape* shape, const int32_t* rrow, const int32_t* rcol, int32_t Cq,
                                    int32_t Ck, void* stream, const char* fn) {
  const int64_t bh = (int64_t)shape->B * shape->H;
  for (int64_t r = 0; r < bh; ++r) {
    bsa_status st = debug_check_device_csr(rrow + r * (Cq + 1), rcol + r * (int64_t)Cq * Ck, Cq, Ck,
                                           (int64_t)Cq * Ck, (hipStream_t)stream, fn);
    if (st != BSA_OK) return st;
  }
  return BSA_OK;
}

// selection workspace: the cost histograms of the scores
size_t bsa_route_select_workspace(const bsa_shape* shape, int32_t Cq, int32_t Ck) {
  if (check_shape(shape, 2, "bsa_route_select_workspace") != BSA_OK || Cq < 1 || Ck < 1) return 0;
  return route_hist_bytes(*shape, Cq);
}

bsa_status bsa_route_select(const float* score, const bsa_shape* shape, const int32_t* q_off, int32_t Cq,
                            const int32_t* k_off, int32_t Ck, int32_t density_ppm, int32_t* route_row_ptr,
                            int32_t* route_col, void* workspace, size_t ws_bytes, void* stream) {
  const char* fn = "bsa_route_select";
  bsa_status st = check_clusters(shape, q_off, Cq, k_off, Ck, fn);
  if (st != BSA_OK) return st;
  if (!score || !route_row_ptr || !route_col) return fail(BSA_ERR_ARG, "%s: NULL pointer", fn);
  if (density_ppm < 0 || density_ppm > 1000000) return fail(BSA_ERR_ARG, "%s: density_ppm must be in [0, 1e6]", fn);
  const size_t need = bsa_route_select_workspace(shape, Cq, Ck);
  if (!workspace || ws_bytes < need || ((uintptr_t)workspace & 255u))
    return fail(BSA_ERR_WORKSPACE, "%s: workspace of %zu bytes (256-byte aligned) required", fn, need);
  g_err[0] = 0;
  st = launch_route_select(score, *shape, q_off, Cq, k_off, Ck, budget_of(shape->N, density_ppm), route_row_ptr,
                           route_col, workspace, false, (hipStream_t)stream);
  if (st == BSA_OK && debug_mode()) st = debug_check_route(shape, route_row_ptr, route_col, Cq, Ck, stream, fn);
  return st;
}

size_t bsa_compensated_attn_workspace(const bsa_shape* shape, int32_t Cq, int32_t Ck) {
  if (check_shape(shape, 2, "bsa_compensated_attn_workspace") != BSA_OK || Cq < 1 || Ck < 1) return 0;
  return comp_attn_workspace(*shape, Cq, Ck);
}

bsa_status bsa_compensated_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, bsa_dtype dtype,
                                    const bsa_shape* shape, const int32_t* q_off, int32_t Cq, const int32_t* k_off,
                                    int32_t Ck, const int32_t* route_row_ptr, const int32_t* route_col,
                                    const float* k_cent, const float* v_cent, float scale, void* workspace,
                                    size_t ws_bytes, void* stream) {
  const char* fn = "bsa_compensated_attn_fwd";
  if (dtype != BSA_DT_BF16) return fail(BSA_ERR_UNSUPPORTED, "%s: only bf16 is implemented", fn);
  bsa_status st = check_clusters(shape, q_off, Cq, k_off, Ck, fn);
  if (st != BSA_OK) return st;
  if (Ck > kMaxKeyClusters) return fail(BSA_ERR_UNSUPPORTED, "%s: Ck must be <= %d", fn, kMaxKeyClusters);
  if (!q || !k || !v || !o || !route_row_ptr || !route_col || !k_cent || !v_cent)
    return fail(BSA_ERR_ARG, "%s: NULL pointer", fn);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(k_cent) || !aligned16(v_cent))
    return fail(BSA_ERR_ARG, "%s: misaligned pointer", fn);
  if (!__builtin_isfinite(scale) || scale <= 0.f) return fail(BSA_ERR_ARG, "%s: scale must be finite and > 0", fn);
  const size_t need = comp_attn_workspace(*shape, Cq, Ck);
  if (need > 0 && (!workspace || ws_bytes < need || ((uintptr_t)workspace & 255u)))
    return fail(BSA_ERR_WORKSPACE, "%s: workspace of %zu bytes (256-byte aligned) required", fn, need);
  g_err[0] = 0;
  return launch_comp_attn(q, k, v, o, lse, *shape, q_off, Cq, k_off, Ck, route_row_ptr, route_col, k_cent, v_cent,
                          scale, workspace, (hipStream_t)stream);
}

// fused call: workspace = centroids | scores | probe scratch (with the cost
// histograms) | compensated-attention workspace
struct CompPlan {
  size_t qc, kc, vc, sc, probe, attn, total;
};
static CompPlan comp_plan(const bsa_shape& s, int Cq, int Ck) {
  CompPlan p;
  const size_t bh = (size_t)s.B * s.H, D = s.D;
  p.qc = 0;
  p.kc = align256h(p.qc + bh * Cq * D * 4);
  p.vc = align256h(p.kc + bh * Ck * D * 4);
  p.sc = align256h(p.vc + bh * Ck * D * 4);
  p.probe = align256h(p.sc + bh * Cq * Ck * 4);
  p.attn = align256h(p.probe + probe_plan(s, Cq, Ck).total);
  p.total = align256h(p.attn + comp_attn_workspace(s, Cq, Ck));
  return p;
}

size_t bsa_centroid_compensate_workspace(const bsa_shape* shape, int32_t Cq, int32_t Ck) {
  if (check_shape(shape, 2, "bsa_centroid_compensate_workspace") != BSA_OK || Cq < 1 || Ck < 1) return 0;
  return comp_plan(*shape, Cq, Ck).total;
}

bsa_status bsa_centroid_compensate(const void* q, const void* k, const void* v, void* o, float* lse, bsa_dtype dtype,
                                   const bsa_shape* shape, const int32_t* q_off, int32_t Cq, const int32_t* k_off,
                                   int32_t Ck, int32_t density_ppm, int32_t use_given_route, float scale,
                                   int32_t* route_row_ptr, int32_t* route_col, float* score, void* workspace,
                                   size_t ws_bytes, void* stream) {
  const char* fn = "bsa_centroid_compensate";
  if (dtype != BSA_DT_BF16) return fail(BSA_ERR_UNSUPPORTED, "%s: only bf16 is implemented", fn);
  bsa_status st = check_clusters(shape, q_off, Cq, k_off, Ck, fn);
  if (st != BSA_OK) return st;
  if (Ck > kMaxKeyClusters) return fail(BSA_ERR_UNSUPPORTED, "%s: Ck must be <= %d", fn, kMaxKeyClusters);
  if (!q || !k || !v || !o || !route_row_ptr || !route_col) return fail(BSA_ERR_ARG, "%s: NULL pointer", fn);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(BSA_ERR_ARG, "%s: q, k, v, o must be 16-byte aligned", fn);
  if (use_given_route != 0 && use_given_route != 1) return fail(BSA_ERR_ARG, "%s: use_given_route must be 0 or 1", fn);
  if (!use_given_route && (density_ppm < 0 || density_ppm > 1000000))
    return fail(BSA_ERR_ARG, "%s: density_ppm must be in [0, 1e6]", fn);
  if (!__builtin_isfinite(scale) || scale <= 0.f) return fail(BSA_ERR_ARG, "%s: scale must be finite and > 0", fn);
  const CompPlan pl = comp_plan(*shape, Cq, Ck);
  if (!workspace || ws_bytes < pl.total || ((uintptr_t)workspace & 255u))
    return fail(BSA_ERR_WORKSPACE, "%s: workspace of %zu bytes (256-byte aligned) required", fn, pl.total);
  g_err[0] = 0;
  char* w = (char*)workspace;
  float* qc = (float*)(w + pl.qc);
  float* kc = (float*)(w + pl.kc);
  float* vc = (float*)(w + pl.vc);
  hipStream_t sm = (hipStream_t)stream;
  if (use_given_route) {
    // the route is an input: centroids, then the compensated attention
    st = launch_centroids(q, k, v, *shape, q_off, Cq, k_off, Ck, qc, kc, vc, sm, kCentAll);
    if (st != BSA_OK) return st;
    return launch_comp_attn(q, k, v, o, lse, *shape, q_off, Cq, k_off, Ck, route_row_ptr, route_col, kc, vc, scale,
                            w + pl.attn, sm);
  }
  float* sc = score ? score : (float*)(w + pl.sc);
  uint16_t *kb = nullptr, *vb = nullptr;
  comp_attn_bf16_slots(*shape, Cq, Ck, w + pl.attn, &kb, &vb);
  const ProbePlan pp = probe_plan(*shape, Cq, Ck);
  const bool bf16_ready = pp.fused && kb != nullptr;
  // query centroids, then one pass over K and V for the key centroids and the scores
  st = launch_centroids(q, k, v, *shape, q_off, Cq, k_off, Ck, qc, nullptr, nullptr, sm, kCentQuery);
  if (st != BSA_OK) return st;
  st = launch_route_scores(k, v, *shape, q_off, Cq, k_off, Ck, qc, kc, vc, scale, sc, w + pl.probe, sm,
                           bf16_ready ? kb : nullptr, bf16_ready ? vb : nullptr);
  if (st != BSA_OK) return st;
  st = launch_route_select(sc, *shape, q_off, Cq, k_off, Ck, budget_of(shape->N, density_ppm), route_row_ptr,
                           route_col, w + pl.probe + pp.off_hist, true, sm);
  if (st == BSA_OK && debug_mode()) st = debug_check_route(shape, route_row_ptr, route_col, Cq, Ck, stream, fn);
  if (st != BSA_OK) return st;
  return launch_comp_attn(q, k, v, o, lse, *shape, q_off, Cq, k_off, Ck, route_row_ptr, route_col, kc, vc, scale,
                          w + pl.attn, sm, bf16_ready);
}

// ---- latent inter-frame pruning (LIPAR) ----------------------------------

static bsa_status check_lipar(const bsa_shape* shape, int32_t frames, const char* fn) {
  bsa_status st = check_shape(shape, 2, fn);
  if (st != BSA_OK) return st;
  if (shape->D % 8 != 0 || shape->D > 4096)
    return fail(BSA_ERR_UNSUPPORTED, "%s: D must be a multiple of 8 and <= 4096 (got %d)", fn, shape->D);
  if (frames < 1 || shape->N % frames != 0)
    return fail(BSA_ERR_ARG, "%s: frames must be >= 1 and divide N (got %d, N = %d)", fn, frames, shape->N);
  if ((int64_t)shape->B * shape->H > 65535) return fail(BSA_ERR_ARG, "%s: B * H must be <= 65535", fn);
  return BSA_OK;
}

bsa_status bsa_lipar_prune(const void* x, bsa_dtype dtype, const bsa_shape* shape, int32_t frames, float tau,
                           uint8_t* keep, int32_t* cpos, int32_t* kept_idx, int32_t* n_kept, void* x_pruned,
                           void* stream) {
  const char* fn = "bsa_lipar_prune";
  if (dtype != BSA_DT_BF16) return fail(BSA_ERR_UNSUPPORTED, "%s: only bf16 is implemented", fn);
  bsa_status st = check_lipar(shape, frames, fn);
  if (st != BSA_OK) return st;
  if (!x || !keep || !cpos || !kept_idx || !n_kept || !x_pruned) return fail(BSA_ERR_ARG, "%s: NULL pointer", fn);
  if (!aligned16(x) || !aligned16(x_pruned)) return fail(BSA_ERR_ARG, "%s: x, x_pruned must be 16-byte aligned", fn);
  if (__builtin_isnan(tau)) return fail(BSA_ERR_ARG, "%s: tau is NaN", fn);
  g_err[0] = 0;
  return launch_lipar_prune(x, *shape, frames, tau, keep, cpos, kept_idx, n_kept, x_pruned, (hipStream_t)stream);
}

bsa_status bsa_lipar_restore(const void* y_pruned, bsa_dtype dtype, const bsa_shape* shape, int32_t frames,
                             const uint8_t* keep, const int32_t* cpos, void* out, void* stream) {
  const char* fn = "bsa_lipar_restore";
  if (dtype != BSA_DT_BF16) return fail(BSA_ERR_UNSUPPORTED, "%s: only bf16 is implemented", fn);
  bsa_status st = check_lipar(shape, frames, fn);
  if (st != BSA_OK) return st;
  if (!y_pruned || !keep || !cpos || !out) return fail(BSA_ERR_ARG, "%s: NULL pointer", fn);
  if (!aligned16(y_pruned) || !aligned16(out)) return fail(BSA_ERR_ARG, "%s: y_pruned, out must be 16-byte aligned", fn);
  g_err[0] = 0;
  return launch_lipar_restore(y_pruned, *shape, frames, keep, cpos, out, (hipStream_t)stream);
}

bsa_status bsa_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  const char* fn = "bsa_hbm_read_probe";
  if (!buf || !sink) return fail(BSA_ERR_ARG, "%s: NULL pointer", fn);
  if (!aligned16(buf) || bytes % 16 != 0) return fail(BSA_ERR_ARG, "%s: buf and bytes must be 16-byte aligned", fn);
  g_err[0] = 0;
  return launch_hbm_read(buf, bytes, sink, (hipStream_t)stream);
}

bsa_status bsa_check_csr(const int32_t* row_ptr, const int32_t* col_idx, int32_t nrows, int32_t ncols,
                         int64_t capacity) {
  return check_csr_host(row_ptr, col_idx, nrows, ncols, capacity, "bsa_check_csr");
}

int64_t bsa_route_budget(int32_t N, int32_t density_ppm) {
  if (N < 0 || density_ppm < 0 || density_ppm > 1000000) return -1;
  return budget_of(N, density_ppm);
}

const char* bsa_status_string(bsa_status s) {
  switch (s) {
    case BSA_OK: return "ok";
    case BSA_ERR_ARG: return "invalid argument";
    case BSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case BSA_ERR_CAPACITY: return "output capacity too small";
    case BSA_ERR_WORKSPACE: return "workspace missing or too small";
    case BSA_ERR_HIP: return "HIP runtime error";
    case BSA_ERR_CHECK: return "debug invariant check failed";
  }
  return "unknown status";
}

const char* bsa_last_error(void) { return g_err; }

}  // extern "C"
