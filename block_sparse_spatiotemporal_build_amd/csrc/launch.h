// Host-side launchers and workspace plans shared between the C-ABI layer
// (api.hip) and the kernel files.  Every plan struct is defined here once: a
// second copy with a stale layout in another translation unit would make the
// C-ABI layer read the wrong fields (and overrun the returned struct).
#pragma once

#include "common.h"

namespace bsa {

// ---- block mask and block-sparse attention ---------------------------------
bsa_status launch_build_block_mask(const bsa_mask_desc& d, int32_t* row_ptr, int32_t* col_idx,
                                   int32_t* row_order, hipStream_t stream);
bsa_status launch_attn_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                            const bsa_shape& s, const int32_t* row_ptr, const int32_t* col_idx,
                            const int32_t* row_order, int block, float scale, hipStream_t stream);
bsa_status launch_attn_f32(const void* q, const void* k, const void* v, void* o, float* lse,
                           const bsa_shape& s, const int32_t* row_ptr, const int32_t* col_idx,
                           int block, float scale, hipStream_t stream);

// in-place inclusive scan of a[1..n] (one workgroup; a[0] untouched)
void launch_inclusive_scan(int32_t* a, int n, hipStream_t stream);
// block schedule of a CSR pointer array (long rows first; see mask.hip)
void launch_block_order(const int32_t* ptr, int nb, int32_t* order, hipStream_t stream);

// ---- block-sparse attention backward (bf16, head_dim 128, block 128) ----------
bsa_status launch_transpose_block_mask(const int32_t* row_ptr, const int32_t* col_idx, int nb, int32_t* col_ptr,
                                       int32_t* row_idx, hipStream_t stream);
size_t attn_bwd_workspace(const bsa_shape& s);  // Delta [BH][N] + row and column schedules
bsa_status launch_attn_bwd_bf16(const void* q, const void* k, const void* v, const void* o, const void* dO,
                                const float* lse, const bsa_shape& s, const int32_t* row_ptr, const int32_t* col_idx,
                                const int32_t* col_ptr, const int32_t* row_idx, float scale, void* dq, void* dk,
                                void* dv, void* ws, hipStream_t stream);

// ---- linear attention ------------------------------------------------------
struct LinPlan {
  int splits, chunk;  // state: token splits per head and tokens per split
  bool d128;          // head_dim 128 kernels (buffer-load staging, 32-bit offsets within a head)
  int tph, tpw, apply_wgs;  // apply (head_dim 128): tiles per head, tiles per workgroup, workgroups
  size_t off_part_s, off_part_z, off_st, off_z, total;  // workspace layout (bytes)
};
LinPlan linear_plan(const bsa_shape& s);
// mix_r >= 0 (head_dim-128 plan only): o = mix_r * o + (1 - mix_r) * linear attention
bsa_status launch_linear_attn(const void* q, const void* k, const void* v, void* o, const bsa_shape& s,
                              float* S, float* z, void* ws, hipStream_t stream, float mix_r = -1.f);

// The scratch behind bsa_linear_attn_fwd_noalloc: a file-scope device array of
// this many bytes in linear_attn.hip holding the workspace of linear_plan.
constexpr size_t kLinNoAllocBytes = (size_t)40 << 20;
// This device's address of that array (looked up once per device with
// hipGetSymbolAddress; the array's name is not a device address in host code).
bsa_status linear_noalloc_scratch(void** ptr);

// causal (chunked) linear attention, head_dim 128: state partials over splits
// of chunk_s tokens, an exclusive prefix at every f-th split, and the causal
// walk over apply splits of chunk_a = f * chunk_s tokens
struct CausalPlan {
  int chunk_s, splits_s, chunk_a, splits_a, f;
  size_t off_part_s, off_part_z, total;  // workspace layout (bytes)
};
CausalPlan causal_plan(const bsa_shape& s);
bsa_status launch_causal_linear_attn(const void* q, const void* k, const void* v, void* o, const bsa_shape& s,
                                     const float* s_in, const float* z_in, float* s_out, float* z_out, void* ws,
                                     hipStream_t stream);

// ---- token clustering (k-means, cluster order, row permutation) -------------
constexpr int kMaxKmClusters = 1024;
struct KmPlan {
  int Cp, tiles;  // centres padded to a multiple of 32; 256-token tiles per sequence
  size_t off_cb, off_cn, off_hist, off_tbase, off_perm, off_off, total;  // workspace layout (bytes)
};
KmPlan kmeans_plan(const bsa_shape& s, int C);
bsa_status launch_kmeans(const void* x, const bsa_shape& s, int C, int iters, float* cent, int32_t* labels,
                         int32_t* perm, int32_t* offsets, void* ws, hipStream_t stream);
bsa_status launch_rows_permute(const void* src, const bsa_shape& s, int elem_bytes, const int32_t* perm, void* dst,
                               bool scatter, hipStream_t stream);

// ---- centroid compensation with error-aware routing ------------------------
struct ProbePlan {
  int splits, cps;  // key-cluster splits per head and clusters per split
  bool fused;       // head_dim 128: key centroids, logits and errors in one pass over K and V
  size_t off_e, off_m, off_ms, off_zs, off_hist, total;  // workspace layout (bytes)
};
ProbePlan probe_plan(const bsa_shape& s, int Cq, int Ck);
// which clusters launch_centroids averages: all, the query clusters, the key clusters
enum CentroidSet { kCentAll = 0, kCentQuery = 1, kCentKey = 2 };
bsa_status launch_centroids(const void* q, const void* k, const void* v, const bsa_shape& s, const int32_t* q_off,
                            int Cq, const int32_t* k_off, int Ck, float* qc, float* kc, float* vc,
                            hipStream_t stream, CentroidSet which = kCentAll);
// scores from the query centroids qc; writes the key / value centroids kc, vc
// (and their bf16 copies when kc_bf, vc_bf are given, fused path only) and
// the scores' cost histograms (at off_hist of the workspace, the start of the
// selection scratch)
bsa_status launch_route_scores(const void* k, const void* v, const bsa_shape& s, const int32_t* q_off, int Cq,
                               const int32_t* k_off, int Ck, const float* qc, float* kc, float* vc, float scale,
                               float* score, void* ws, hipStream_t stream, uint16_t* kc_bf = nullptr,
                               uint16_t* vc_bf = nullptr);
// bytes of the selection scratch (the scores' cost histograms first, then the
// per-head selection state, the cut-bin keys and the per-row kept counts)
size_t route_hist_bytes(const bsa_shape& s, int Cq);
// hist_ready: the histograms of `score` are already at the start of
// `scratch` (launch_route_scores writes them there)
bsa_status launch_route_select(const float* score, const bsa_shape& s, const int32_t* q_off, int Cq,
                               const int32_t* k_off, int Ck, long long budget, int32_t* rrow, int32_t* rcol,
                               void* scratch, bool hist_ready, hipStream_t stream);
// compensated attention workspace: bf16 copies of the key / value centroids
// and the tile schedule of the head_dim-128 kernel (0 bytes otherwise)
size_t comp_attn_workspace(const bsa_shape& s, int Cq, int Ck);
// the bf16 centroid slots in that workspace (null when it has none)
void comp_attn_bf16_slots(const bsa_shape& s, int Cq, int Ck, void* ws, uint16_t** kb, uint16_t** vb);
// bf16_ready: the bf16 centroid copies are already in the workspace
bsa_status launch_comp_attn(const void* q, const void* k, const void* v, void* o, float* lse, const bsa_shape& s,
                            const int32_t* q_off, int Cq, const int32_t* k_off, int Ck, const int32_t* rrow,
                            const int32_t* rcol, const float* kc, const float* vc, float scale, void* ws,
                            hipStream_t stream, bool bf16_ready = false);

bsa_status launch_lipar_prune(const void* x, const bsa_shape& s, int frames, float tau, uint8_t* keep,
                              int32_t* cpos, int32_t* kept_idx, int32_t* n_kept, void* x_pruned,
                              hipStream_t stream);
bsa_status launch_lipar_restore(const void* y_pruned, const bsa_shape& s, int frames, const uint8_t* keep,
                                const int32_t* cpos, void* out, hipStream_t stream);

// read-only HBM probe (measurement reference)
bsa_status launch_hbm_read(const void* p, size_t bytes, uint32_t* sink, hipStream_t stream);

}  // namespace bsa
