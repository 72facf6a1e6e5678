// moe_internal.h -- host-side launchers of the gfx950 kernels.  Each returns
// hipSuccess or the launch error.  Shapes have been validated by the caller.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// ---- router ---------------------------------------------------------------
// logits = x[T,H] . w_router[E,H]^T (bf16 inputs, fp32 accumulate) as
// router_splits(T, H) partial sums over K: logits [nsplit][T][E] fp32
int router_splits(int64_t T, int H);
hipError_t launch_router_logits(const void* x, const void* w_router, float* logits,
                                int T, int E, int H, hipStream_t s);
// per-token sigmoid + bias + top-k + weights (partial logits summed in order)
hipError_t launch_topk(const float* logits, int nsplit, const float* bias, int T, int E, int k, float scale,
                       int norm, int32_t* ids, float* w, hipStream_t s, float* s_out = nullptr);
// weights of caller-supplied expert ids from the same partial logits
hipError_t launch_replay_weights(const float* logits, int nsplit, const int32_t* ids, int T, int E, int k,
                                 float scale, int norm, float* w, hipStream_t s, int32_t* ids_out = nullptr,
                                 float* s_out = nullptr);
// ids[p] = p mod E for the P = T*k pairs
hipError_t launch_balanced_ids(int32_t* ids, int64_t P, int E, hipStream_t s);

// ---- permutation ----------------------------------------------------------
size_t permute_scratch_bytes(int64_t P, int E);   // P = T * k pairs
hipError_t launch_permute(const int32_t* ids, int T, int k, int E, int32_t* counts, int32_t* offsets,
                          int32_t* row_to_pair, int32_t* pair_to_row, void* scratch, hipStream_t s);
// the permutation and, when tile_start != nullptr, the bm-row tile plan
// (with an extra group of extra_rows rows) in as few launches as the size allows
hipError_t launch_permute_plan(const int32_t* ids, int T, int k, int E, int32_t* counts, int32_t* offsets,
                               int32_t* row_to_pair, int32_t* pair_to_row, void* scratch, int bm, int extra_rows,
                               int32_t* tile_start, hipStream_t s);

// ---- grouped / dense GEMMs ------------------------------------------------
// Tile plan for a grouped GEMM with bm-row tiles: tile_start[E+1] (E+2 with
// an extra group of extra_rows rows after the E groups).
hipError_t launch_tile_plan(const int32_t* offsets, int E, int bm, int extra_rows, int32_t* tile_start,
                            hipStream_t s);

// Weight-streaming bf16 GEMMs (direct-to-LDS DMA ring).
// Up: h[rows, N] bf16 = act(A[rows] . W13^T) with A rows gathered through
// a_rows / a_div (clamped to a_nrows) or dense; W13 [2N, K] per group.
// Down: C[rows, N] = A[rows, K] . W^T, C scaled fp16 rows (expert_row_bytes(N) each) or fp32.
// Grouped when offsets != nullptr (groups, tile_start from the plan with the
// same bm, max_tiles bounds the plan); otherwise dense with M rows.  An extra
// group (extra_rows > 0, grouped only) follows the groups: rows
// offsets[groups] .. + extra_rows, A row = row - offsets[groups], weights
// W_extra, limit limit_extra.  K % 64 == 0; N % 64 == 0 (up).
struct GroupedArgs {
    const void* A = nullptr;
    const int32_t* a_rows = nullptr;
    int a_div = 1, a_nrows = 0;
    const void* W = nullptr;
    int64_t w_group_stride = 0;
    void* C = nullptr;
    int M = 0, N = 0, K = 0;
    float limit = 0.f;
    const int32_t* offsets = nullptr;
    const int32_t* tile_start = nullptr;
    int groups = 1, max_tiles = 0, bm = 256;
    int extra_rows = 0;
    const void* W_extra = nullptr;
    float limit_extra = 0.f;
    void* gu_out = nullptr;          // first projection: also keep the pre-activations (bf16 [rows][2N])
    int rot_group = -1;              // dense launch: add over K in the order group rot_group's grouped launch uses
    void* items = nullptr;           // grouped 256-row launches (optional): scratch for the work-item
                                     // table, grouped_item_bytes(max_tiles, N, K-side) bytes
};
// bytes of the work-item table of a grouped 256-row launch with max_tiles
// tiles over n_tiles column tiles
size_t grouped_item_bytes(int64_t max_tiles, int n_tiles);
// the work-item table of a grouped launch ({group, first row, rows, n-tile}
// per item after a 64-byte header of 9 XCD range starts), from the tile plan;
// `balance` deals the routed groups to the XCDs by cost
hipError_t launch_item_table(const int32_t* offsets, const int32_t* tile_start, int groups, int extra_rows,
                             int n_tiles, bool balance, void* buf, hipStream_t s);
// bytes of one expert output row of H columns: H fp16 values, then one int8
// exponent per 128 columns (padded to 16 bytes); value = fp16 * 2^exponent
int64_t expert_row_bytes(int H);
int grouped_tile_m(int64_t rows, int groups);
hipError_t launch_grouped_up(const GroupedArgs& a, hipStream_t s);
hipError_t launch_grouped_down(const GroupedArgs& a, bool c_fp32, hipStream_t s);

// FP8 E4M3 routed experts (128 x 128 block-scaled weights, activations
// quantised per (row, 128 columns), 128-row tiles).
// quant: xq[rows, H] E4M3 codes, xs[H/128][ld] fp32 scales (amax / 448).
// up: hq[rows, N] codes + hs[N/128][hs_ld] scales of act(A . W13^T), A rows
// gathered through a_rows / a_div; W13 [groups][2N, K] codes, w13s
// [groups][2N/128][K/128].  down: y = hq . W2^T as scaled fp16 rows (expert_row_bytes(N) each).
// K % 128 == 0, N % 128 == 0.
int fp8_tile_m();
hipError_t launch_quant_rows(const void* x, int rows, int H, void* xq, float* xs, int ld, hipStream_t s);
// items (required; hipErrorInvalidValue when null): grouped_item_bytes(max_tiles, n-tiles) of
// scratch for the work-item table, which the persistent grid walks
hipError_t launch_fp8_up(const void* xq, const float* xs, int xs_ld, const int32_t* a_rows, int a_div,
                         int a_nrows, const void* w13, const float* w13s, void* hq, float* hs, int hs_ld, int N,
                         int K, float limit, const int32_t* offsets, const int32_t* tile_start, int groups,
                         int max_tiles, void* items, hipStream_t s);
hipError_t launch_fp8_down(const void* hq, const float* hs, int hs_ld, int rows, const void* w2, const float* w2s,
                           void* y, int N, int K, const int32_t* offsets, const int32_t* tile_start, int groups,
                           int max_tiles, void* items, hipStream_t s);

// ---- combine --------------------------------------------------------------
// shared expert output: y_shared fp32 [T, H], or shared_rows (scaled fp16 rows), or neither
// zero-centred RMSNorm of fp32 rows -> bf16 rows (H % 4 == 0)
hipError_t launch_rmsnorm(const float* resid, const float* norm_weight, float eps, void* x, int T, int H,
                          hipStream_t s);
// the same RMSNorm fused with the router logits (logits [T][E] fp32, the same
// bits as launch_router_logits on the normalised rows); for T >= 512, H <= 4096,
// H % 256 == 0, E <= 384 (rmsnorm_router_fusable)
bool rmsnorm_router_fusable(int64_t T, int H, int E);
hipError_t launch_rmsnorm_router(const float* resid, const float* norm_weight, float eps, const void* w_router,
                                 void* x, float* logits, int T, int E, int H, hipStream_t s);
// resid (optional, fp32 [T,H]) is added last; out may be the same buffer
hipError_t launch_combine(const void* y_rows, const int32_t* pair_to_row, const float* topk_w,
                          const float* y_shared, const void* shared_rows, const float* resid, void* out,
                          bool out_bf16, int T, int H, int k, hipStream_t s);

// ---- backward ------------------------------------------------------------

// grouped GEMMs of the backward (bwd_gemm.hip); see Params there
struct BwdArgs {
    const void* A = nullptr;
    int64_t lda = 0;
    const void* B = nullptr;
    int64_t ldb = 0;
    int64_t b_group_stride = 0;
    const void* B_extra = nullptr;
    const void* zero_row = nullptr;
    void* C = nullptr;
    int64_t ldc = 0;
    int64_t c_group_stride = 0;
    void* C_extra = nullptr;
    const void* gu = nullptr;
    float limit = 0.f, limit_extra = 0.f;
    int M = 0, N = 0, K = 0;
    const int32_t* offsets = nullptr;
    const int32_t* tile_start = nullptr;
    int groups = 0;
    int extra_rows = 0;
    int max_tiles = 0;
};
// DGRAD: rows grouped, B = the group's weight [K][N]; act: the SwiGLU
// backward epilogue writing dgu [rows][2N] bf16, else fp32 rows
hipError_t launch_bwd_dgrad(const BwdArgs& a, bool act, hipStream_t s);
// WGRAD: the contraction runs over each group's rows; fp32 [M][N] per group
hipError_t launch_bwd_wgrad(const BwdArgs& a, hipStream_t s);
// per token: dw_j = dout . y_j, dy rows (w_j dout; the shared rows dout) in
// bf16, and the router's da_j from the saved raw scores (bwd.hip)
hipError_t launch_bwd_prep(const float* dout, const void* y_rows, const int32_t* p2r, const float* w,
                           const float* s_raw, float scale, int norm, bool shared, void* dy, float* da, int T,
                           int H, int k, hipStream_t s);
// dx[t] = sum_j dxr[p2r[t,j]] + dxr[P + t] (shared) + sum_j da[t,j] Wg[ids[t,j]]
hipError_t launch_bwd_dx(const float* dxr, const int32_t* p2r, const float* da, const int32_t* ids,
                         const void* w_router, bool shared, float* dx, int T, int H, int k, hipStream_t s);
// dWg[e] = sum over e's rows r of da[pair r] x[token r]
hipError_t launch_bwd_router_wgrad(const float* da, const int32_t* offsets, const int32_t* r2p, const void* x,
                                   float* dwg, int E, int H, int k, hipStream_t s);
hipError_t launch_zero_u32(void* p, int64_t words, hipStream_t s);
// x rows in the permuted row order: row r < P is x[r2p[r] / k], row P + t is
// x[t] when shared (bf16, H % 8 == 0)
hipError_t launch_gather_rows(const void* x, const int32_t* r2p, bool shared, void* out, int T, int H, int k,
                              hipStream_t s);

}  // namespace moe
