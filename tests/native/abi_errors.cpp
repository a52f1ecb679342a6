// Drives every argument check of the C-ABI entry points (include/bsa.h) with
// arguments each check must reject, and verifies the status and the error
// text.  Built host-only with AddressSanitizer and UndefinedBehaviorSanitizer
// by tests/test_native_sanitized.py; a rejected call must touch neither the
// GPU nor any output, so the program runs without a GPU.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/bsa.h"

static int g_cases = 0, g_fail = 0;

static void expect(bsa_status got, bsa_status want, const char* what) {
  ++g_cases;
  const char* msg = bsa_last_error();
  if (got != want || msg == nullptr || msg[0] == 0) {
    ++g_fail;
    printf("FAIL %s: status %d (want %d), error '%s'\n", what, (int)got, (int)want, msg ? msg : "(null)");
  }
}

static void expect_i(long long got, long long want, const char* what) {
  ++g_cases;
  if (got != want) {
    ++g_fail;
    printf("FAIL %s: got %lld want %lld\n", what, got, want);
  }
}

// fake device pointers: 256-byte aligned host memory, never dereferenced by a
// rejected call (a dereference would be caught by the sanitizer)
alignas(256) static unsigned char g_buf[8][4096];
static void* P(int i) { return g_buf[i]; }
static void* MIS(int i) { return g_buf[i] + 2; }  // misaligned

int main() {
  const bsa_shape good = {1, 2, 256, 128, 2 * 256 * 128, 256 * 128, 128};
  bsa_shape s;
  float* f = (float*)P(5);
  int32_t* ip = (int32_t*)P(6);

  // ---- shapes (check_shape, through several calls)
  expect(bsa_block_sparse_attn_fwd(P(0), P(1), P(2), P(3), f, BSA_DT_BF16, nullptr, ip, ip, nullptr, 128, 0.1f, nullptr),
         BSA_ERR_ARG, "fwd: NULL shape");
  s = good; s.N = 0;
  expect(bsa_block_sparse_attn_fwd(P(0), P(1), P(2), P(3), f, BSA_DT_BF16, &s, ip, ip, nullptr, 128, 0.1f, nullptr),
         BSA_ERR_ARG, "fwd: N = 0");
  s = good; s.B = -1;
  expect(bsa_block_sparse_attn_fwd(P(0), P(1), P(2), P(3), f, BSA_DT_BF16, &s, ip, ip, nullptr, 128, 0.1f, nullptr),
         BSA_ERR_ARG, "fwd: B < 0");
  s = good; s.stride_n = 64;
  expect(bsa_block_sparse_attn_fwd(P(0), P(1), P(2), P(3), f, BSA_DT_BF16, &s, ip, ip, nullptr, 128, 0.1f, nullptr),
         BSA_ERR_ARG, "fwd: stride_n < D");
  s = good; s.stride_h = -8;
  expect(bsa_block_sparse_attn_fwd(P(0), P(1), P(2), P(3), f, BSA_DT_BF16, &s, ip, ip, nullptr, 128, 0.1f, nullptr),
         BSA_ERR_ARG, "fwd: negative stride");
  s = good; s.stride_n = 132;
  expect(bsa_block_sparse_attn_fwd(P(0), P(1), P(2), P(3), f, BSA_DT_BF16, &s, ip, ip, nullptr, 128, 0.1f, nullptr),
         BSA_ERR_ARG, "fwd: stride not a multiple of 16 bytes");

  // ---- mask descriptor
  bsa_mask_desc d;
  memset(&d, 0, sizeof d);
  d.kind = BSA_MASK_WINDOW_ANCHOR; d.frames = 4; d.frame_tokens = 64; d.block = 64; d.window = 1;
  bsa_mask_desc bad = d; bad.kind = 99;
  expect(bsa_build_block_mask(&bad, ip, ip, 1 << 20, nullptr, nullptr), BSA_ERR_ARG, "mask: unknown kind");
  expect(bsa_build_block_mask(nullptr, ip, ip, 1 << 20, nullptr, nullptr), BSA_ERR_ARG, "mask: NULL desc");
  bad = d; bad.block = 0;
  expect(bsa_build_block_mask(&bad, ip, ip, 1 << 20, nullptr, nullptr), BSA_ERR_ARG, "mask: block 0");
  bad = d; bad.window = -1;
  expect(bsa_build_block_mask(&bad, ip, ip, 1 << 20, nullptr, nullptr), BSA_ERR_ARG, "mask: negative window");
  bad = d; bad.frames = 1 << 20; bad.frame_tokens = 1 << 20;
  expect(bsa_build_block_mask(&bad, ip, ip, 1 << 20, nullptr, nullptr), BSA_ERR_ARG, "mask: too many tokens");
  bad = d; bad.frames = 100000; bad.frame_tokens = 1000; bad.block = 1;
  expect(bsa_build_block_mask(&bad, ip, ip, 1 << 20, nullptr, nullptr), BSA_ERR_ARG, "mask: too many blocks");
  expect(bsa_build_block_mask(&d, nullptr, ip, 1 << 20, nullptr, nullptr), BSA_ERR_ARG, "mask: NULL row_ptr");
  expect(bsa_build_block_mask(&d, ip, ip, 15, nullptr, nullptr), BSA_ERR_CAPACITY, "mask: capacity < nb^2");
  expect_i(bsa_mask_num_blocks(&bad), -1, "num_blocks of a bad desc");
  expect_i(bsa_mask_num_blocks(&d), 4, "num_blocks");

  // ---- forward attention
  expect(bsa_block_sparse_attn_fwd(P(0), P(1), P(2), P(3), f, (bsa_dtype)7, &good, ip, ip, nullptr, 128, 0.1f, nullptr),
         BSA_ERR_ARG, "fwd: unknown dtype");
  expect(bsa_block_sparse_attn_fwd(nullptr, P(1), P(2), P(3), f, BSA_DT_BF16, &good, ip, ip, nullptr, 128, 0.1f, nullptr),
         BSA_ERR_ARG, "fwd: NULL q");
  expect(bsa_block_sparse_attn_fwd(MIS(0), P(1), P(2), P(3), f, BSA_DT_BF16, &good, ip, ip, nullptr, 128, 0.1f, nullptr),
         BSA_ERR_ARG, "fwd: misaligned q");
  expect(bsa_block_sparse_attn_fwd(P(0), P(1), P(2), P(3), f, BSA_DT_BF16, &good, ip, ip, nullptr, 128, 0.f, nullptr),
         BSA_ERR_ARG, "fwd: scale 0");
  expect(bsa_block_sparse_attn_fwd(P(0), P(1), P(2), P(3), f, BSA_DT_BF16, &good, ip, ip, nullptr, 128, -1.f, nullptr),
         BSA_ERR_ARG, "fwd: negative scale");
  expect(bsa_block_sparse_attn_fwd(P(0), P(1), P(2), P(3), f, BSA_DT_BF16, &good, ip, ip, nullptr, 0, 0.1f, nullptr),
         BSA_ERR_ARG, "fwd: block 0");
  expect(bsa_block_sparse_attn_fwd(P(0), P(1), P(2), P(3), f, BSA_DT_BF16, &good, ip, ip, nullptr, 32, 0.1f, nullptr),
         BSA_ERR_UNSUPPORTED, "fwd: bf16 block 32");
  s = good; s.D = 96; s.stride_n = 96; s.stride_h = 96 * 256; s.stride_b = 2 * 96 * 256;
  expect(bsa_block_sparse_attn_fwd(P(0), P(1), P(2), P(3), f, BSA_DT_BF16, &s, ip, ip, nullptr, 128, 0.1f, nullptr),
         BSA_ERR_UNSUPPORTED, "fwd: bf16 D 96");
  expect(bsa_block_sparse_attn_fwd(P(0), P(1), P(2), P(3), f, BSA_DT_F32, &good, ip, ip, nullptr, 256, 0.1f, nullptr),
         BSA_ERR_UNSUPPORTED, "fwd: f32 block 256");

  // ---- mask transpose and backward
  expect(bsa_transpose_block_mask(ip, ip, 0, ip, ip, 16, nullptr), BSA_ERR_ARG, "transpose: nb 0");
  expect(bsa_transpose_block_mask(ip, nullptr, 4, ip, ip, 16, nullptr), BSA_ERR_ARG, "transpose: NULL");
  expect(bsa_transpose_block_mask(ip, ip, 4, ip, ip, 15, nullptr), BSA_ERR_CAPACITY, "transpose: capacity");
  expect_i((long long)bsa_block_sparse_attn_bwd_workspace(nullptr), 0, "bwd workspace of NULL shape");
  expect(bsa_block_sparse_attn_bwd(P(0), P(1), P(2), P(3), P(4), f, BSA_DT_F32, &good, ip, ip, ip, ip, 128, 0.1f, P(0),
                                   P(1), P(2), P(7), 1 << 30, nullptr),
         BSA_ERR_UNSUPPORTED, "bwd: f32");
  expect(bsa_block_sparse_attn_bwd(P(0), P(1), P(2), P(3), P(4), f, BSA_DT_BF16, &good, ip, ip, ip, ip, 64, 0.1f, P(0),
                                   P(1), P(2), P(7), 1 << 30, nullptr),
         BSA_ERR_UNSUPPORTED, "bwd: block 64");
  expect(bsa_block_sparse_attn_bwd(P(0), P(1), P(2), P(3), nullptr, f, BSA_DT_BF16, &good, ip, ip, ip, ip, 128, 0.1f,
                                   P(0), P(1), P(2), P(7), 1 << 30, nullptr),
         BSA_ERR_ARG, "bwd: NULL dO");
  expect(bsa_block_sparse_attn_bwd(P(0), P(1), P(2), P(3), P(4), f, BSA_DT_BF16, &good, ip, ip, ip, ip, 128, 0.1f, P(0),
                                   P(1), P(2), P(7), 16, nullptr),
         BSA_ERR_WORKSPACE, "bwd: small workspace");

  // ---- linear attention (workspace and no-allocation forms)
  expect(bsa_linear_attn_fwd(P(0), P(1), P(2), P(3), BSA_DT_F32, &good, nullptr, nullptr, P(7), 1 << 30, nullptr),
         BSA_ERR_UNSUPPORTED, "linear: f32");
  expect(bsa_linear_attn_fwd(P(0), P(1), nullptr, P(3), BSA_DT_BF16, &good, nullptr, nullptr, P(7), 1 << 30, nullptr),
         BSA_ERR_ARG, "linear: NULL v");
  expect(bsa_linear_attn_fwd(P(0), P(1), P(2), P(3), BSA_DT_BF16, &good, nullptr, nullptr, MIS(7), 1 << 30, nullptr),
         BSA_ERR_WORKSPACE, "linear: misaligned workspace");
  expect(bsa_linear_attn_fwd(P(0), P(1), P(2), P(3), BSA_DT_BF16, &good, nullptr, nullptr, P(7), 100, nullptr),
         BSA_ERR_WORKSPACE, "linear: small workspace");
  // 1024 heads: one split each, 64 KiB of partial state per head
  s = good; s.H = 1024; s.stride_b = s.stride_h * 1024;
  expect(bsa_linear_attn_fwd_noalloc(P(0), P(1), P(2), P(3), BSA_DT_BF16, &s, nullptr, nullptr, nullptr),
         BSA_ERR_UNSUPPORTED, "linear no-alloc: beyond its scratch");
  expect(bsa_causal_linear_attn_fwd(P(0), P(1), P(2), P(3), BSA_DT_BF16, &good, f, nullptr, nullptr, nullptr, P(7),
                                    1 << 30, nullptr),
         BSA_ERR_ARG, "causal: S_in without z_in");
  expect(bsa_causal_linear_attn_fwd(P(0), P(1), P(2), P(3), BSA_DT_BF16, &good, nullptr, nullptr, (float*)MIS(5),
                                    nullptr, P(7), 1 << 30, nullptr),
         BSA_ERR_ARG, "causal: misaligned S_out");
  expect(bsa_mixed_attn_fwd(P(0), P(1), P(2), P(3), BSA_DT_BF16, &good, ip, ip, nullptr, 128, 0.1f, 1.5f, P(7), 1 << 30,
                            nullptr),
         BSA_ERR_ARG, "mixed: r > 1");
  expect(bsa_mixed_attn_fwd(P(0), P(1), P(2), P(3), BSA_DT_BF16, &good, nullptr, ip, nullptr, 128, 0.1f, 0.5f, P(7),
                            1 << 30, nullptr),
         BSA_ERR_ARG, "mixed: NULL row_ptr with r > 0");
  expect(bsa_mixed_attn_fwd(P(0), P(1), P(2), P(3), BSA_DT_BF16, &good, ip, ip, nullptr, 32, 0.1f, 0.5f, P(7), 1 << 30,
                            nullptr),
         BSA_ERR_UNSUPPORTED, "mixed: block 32");
  expect(bsa_mixed_attn_fwd(P(0), P(1), P(2), P(3), BSA_DT_BF16, &good, ip, ip, nullptr, 128, 0.1f, 0.5f, nullptr, 0,
                            nullptr),
         BSA_ERR_WORKSPACE, "mixed: no workspace");

  // ---- clustering and row permutations
  expect(bsa_kmeans(P(0), BSA_DT_BF16, &good, 0, 10, f, ip, ip, ip, P(7), 1 << 30, nullptr), BSA_ERR_ARG,
         "kmeans: C 0");
  expect(bsa_kmeans(P(0), BSA_DT_BF16, &good, 4, -1, f, ip, ip, ip, P(7), 1 << 30, nullptr), BSA_ERR_ARG,
         "kmeans: iters < 0");
  expect(bsa_kmeans(P(0), BSA_DT_BF16, &good, 4, 10, nullptr, ip, ip, ip, P(7), 1 << 30, nullptr), BSA_ERR_ARG,
         "kmeans: NULL centroids");
  expect(bsa_kmeans(P(0), BSA_DT_BF16, &good, 4, 10, f, ip, ip, ip, P(7), 8, nullptr), BSA_ERR_WORKSPACE,
         "kmeans: small workspace");
  expect(bsa_gather_rows(P(0), BSA_DT_BF16, &good, ip, P(0), nullptr), BSA_ERR_ARG, "gather: in place");
  expect(bsa_scatter_rows(P(0), BSA_DT_BF16, &good, nullptr, P(1), nullptr), BSA_ERR_ARG, "scatter: NULL perm");
  expect(bsa_gather_rows(P(0), (bsa_dtype)5, &good, ip, P(1), nullptr), BSA_ERR_ARG, "gather: unknown dtype");

  // ---- clustered compensation
  const int32_t* qo = ip;
  expect(bsa_cluster_centroids(P(0), P(1), P(2), BSA_DT_BF16, &good, qo, 0, qo, 4, f, f, f, nullptr), BSA_ERR_ARG,
         "centroids: Cq 0");
  expect(bsa_cluster_centroids(P(0), P(1), P(2), BSA_DT_BF16, &good, qo, 4, qo, 4, nullptr, nullptr, nullptr, nullptr),
         BSA_ERR_ARG, "centroids: no output");
  expect(bsa_cluster_centroids(P(0), P(1), P(2), BSA_DT_BF16, &good, qo, 4, qo, 4, nullptr, f, nullptr, nullptr),
         BSA_ERR_ARG, "centroids: k_cent without v_cent");
  expect(bsa_cluster_centroids(P(0), P(1), P(2), BSA_DT_BF16, &good, nullptr, 4, qo, 4, f, f, f, nullptr), BSA_ERR_ARG,
         "centroids: NULL offsets");
  expect(bsa_route_scores(P(1), P(2), BSA_DT_BF16, &good, qo, 4, qo, 4, f, f, f, 0.f, f, P(7), 1 << 30, nullptr),
         BSA_ERR_ARG, "scores: scale 0");
  expect(bsa_route_scores(P(1), P(2), BSA_DT_BF16, &good, qo, 4, qo, 4, f, f, f, 0.1f, f, P(7), 0, nullptr),
         BSA_ERR_WORKSPACE, "scores: no workspace");
  expect(bsa_route_select(f, &good, qo, 4, qo, 4, 2000000, ip, ip, P(7), 1 << 30, nullptr), BSA_ERR_ARG,
         "select: density above 1e6");
  expect(bsa_route_select(f, &good, qo, 4, qo, 4, 1000, ip, ip, P(7), 0, nullptr), BSA_ERR_WORKSPACE,
         "select: no workspace");
  expect(bsa_compensated_attn_fwd(P(0), P(1), P(2), P(3), f, BSA_DT_BF16, &good, qo, 4, qo, 600, ip, ip, f, f, 0.1f,
                                  P(7), 1 << 30, nullptr),
         BSA_ERR_UNSUPPORTED, "compensated: Ck above 512");
  expect(bsa_centroid_compensate(P(0), P(1), P(2), P(3), f, BSA_DT_BF16, &good, qo, 4, qo, 4, 1000, 2, 0.1f, ip, ip,
                                 nullptr, P(7), 1 << 30, nullptr),
         BSA_ERR_ARG, "fused: use_given_route 2");
  expect(bsa_centroid_compensate(P(0), P(1), P(2), P(3), f, BSA_DT_BF16, &good, qo, 4, qo, 4, -5, 0, 0.1f, ip, ip,
                                 nullptr, P(7), 1 << 30, nullptr),
         BSA_ERR_ARG, "fused: negative density");
  expect(bsa_centroid_compensate(P(0), P(1), P(2), P(3), f, BSA_DT_BF16, &good, qo, 4, qo, 4, 1000, 0, 0.1f, ip, ip,
                                 nullptr, P(7), 64, nullptr),
         BSA_ERR_WORKSPACE, "fused: small workspace");
  expect_i(bsa_route_budget(32760, 150000), 160982640LL, "route budget");
  expect_i(bsa_route_budget(10, -1), -1, "route budget of a negative density");

  // ---- latent pruning
  expect(bsa_lipar_prune(P(0), BSA_DT_BF16, &good, 3, 0.1f, (uint8_t*)P(1), ip, ip, ip, P(2), nullptr), BSA_ERR_ARG,
         "lipar: frames do not divide N");
  expect(bsa_lipar_prune(P(0), BSA_DT_BF16, &good, 4, __builtin_nanf(""), (uint8_t*)P(1), ip, ip, ip, P(2), nullptr),
         BSA_ERR_ARG, "lipar: tau NaN");
  expect(bsa_lipar_restore(P(0), BSA_DT_BF16, &good, 4, nullptr, ip, P(2), nullptr), BSA_ERR_ARG,
         "lipar restore: NULL keep");

  // ---- measurement probe
  expect(bsa_hbm_read_probe(nullptr, 1024, (uint32_t*)P(1), nullptr), BSA_ERR_ARG, "read probe: NULL buffer");
  expect(bsa_hbm_read_probe(P(0), 1000, (uint32_t*)P(1), nullptr), BSA_ERR_ARG, "read probe: bytes not a multiple of 16");

  // ---- block CSR checker (host arrays)
  {
    const int32_t rp_ok[4] = {0, 2, 3, 5}, ci_ok[5] = {0, 2, 1, 0, 2};
    expect_i(bsa_check_csr(rp_ok, ci_ok, 3, 3, 5), BSA_OK, "csr: valid");
    const int32_t rp_bad[4] = {0, 3, 2, 5};
    expect(bsa_check_csr(rp_bad, ci_ok, 3, 3, 5), BSA_ERR_ARG, "csr: row_ptr not monotone");
    const int32_t ci_desc[5] = {2, 0, 1, 0, 2};
    expect(bsa_check_csr(rp_ok, ci_desc, 3, 3, 5), BSA_ERR_ARG, "csr: columns not ascending");
    const int32_t ci_oob[5] = {0, 3, 1, 0, 2};
    expect(bsa_check_csr(rp_ok, ci_oob, 3, 3, 5), BSA_ERR_ARG, "csr: column out of range");
    expect(bsa_check_csr(rp_ok, ci_ok, 3, 3, 4), BSA_ERR_CAPACITY, "csr: entries beyond capacity");
    const int32_t rp_start[4] = {1, 2, 3, 5};
    expect(bsa_check_csr(rp_start, ci_ok, 3, 3, 5), BSA_ERR_ARG, "csr: row_ptr[0] != 0");
    expect(bsa_check_csr(nullptr, ci_ok, 3, 3, 5), BSA_ERR_ARG, "csr: NULL row_ptr");
  }

  printf("%d cases, %d failures\n", g_cases, g_fail);
  return g_fail == 0 ? 0 : 1;
}
