// gemm.hip -- bf16 MFMA GEMMs of the MoE layer on gfx950.
//
//   C[r, n] = sum_k A[src(r), k] * W_g[n, k]        (both operands K-contiguous)
//
// used for the routed experts' first
// projection with the clipped SwiGLU fused into the epilogue (bf16 h out),
// their second projection (fp16 rows out), and the shared expert.
//
// Grouped mode: rows are the expert-major permuted rows; the tile plan maps
// blockIdx.x to (expert g, first row of the tile); W_g = W + g * stride.  The
// A rows of the routed first projection are gathered straight from x via
// row_to_pair / k, so no permuted copy of x is ever written.
//
// Tiling: BM x BN block tile, BK = 64, waves of WM x WN built from
// v_mfma_f32_16x16x32_bf16; operands staged through LDS (row stride padded
// by 16 bytes so the 16-byte fragment reads of 16 rows hit distinct banks),
// double-buffered with register prefetch of the next K slice.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

enum { MODE_SWIGLU = 0, MODE_OUT_F16 = 1, MODE_OUT_F32 = 2 };

struct GemmParams {
    const uint16_t* A;
    const int32_t* a_rows;   // gather: source row = a_rows[r] / a_div (nullptr: r)
    int a_div;
    const uint16_t* W;
    int64_t w_group_stride;  // elements between groups' weights
    void* C;
    int M;                   // dense: rows; gathered: number of source rows of A
    int N;                   // output columns (SwiGLU: h width; W has 2N rows)
    int K;
    float limit;
    const int32_t* offsets;  // grouped: row offsets [groups+1]
    const int32_t* tile_start;  // grouped: tile plan [groups+1]
    int groups;
};

constexpr int BK = 64;
constexpr int LDS_STRIDE = BK + 8;  // bf16 elements per LDS row

template <int BM, int BN, int WM, int WN, int MODE>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * kWave) void gemm_kernel(GemmParams p) {
    constexpr int WAVES_N = BN / WN;
    constexpr int NT = (BM / WM) * WAVES_N * kWave;
    constexpr int TM = WM / 16, TN = WN / 16;
    constexpr int A_CHUNKS = BM * BK / 8 / NT;   // 16-byte chunks per thread
    constexpr int B_CHUNKS = BN * BK / 8 / NT;
    static_assert(A_CHUNKS >= 1 && B_CHUNKS >= 1, "tile too small for the block");
    static_assert(MODE != MODE_SWIGLU || (WN % 32) == 0, "SwiGLU needs gate and up tiles per wave");

    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDS_STRIDE];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LDS_STRIDE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    // ---- which rows / weights this block works on
    int row0, row_end, g = 0;
    if (p.tile_start) {
        const int ntiles = p.tile_start[p.groups];
        const int bx = blockIdx.x;
        if (bx >= ntiles) return;
        int lo = 0, hi = p.groups - 1;       // largest g with tile_start[g] <= bx
        while (lo < hi) {
            int mid = (lo + hi + 1) >> 1;
            if (p.tile_start[mid] <= bx) lo = mid; else hi = mid - 1;
        }
        g = lo;
        row0 = p.offsets[g] + (bx - p.tile_start[g]) * BM;
        row_end = p.offsets[g + 1];
    } else {
        row0 = blockIdx.x * BM;
        row_end = p.M;
    }
    if (row0 >= row_end) return;
    const uint16_t* Wg = p.W + (int64_t)g * p.w_group_stride;
    const int K = p.K;

    // ---- per-thread global source pointers for the tile loads
    const uint16_t* a_src[A_CHUNKS];
    int a_dst[A_CHUNKS];
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
        int c = tid + i * NT;
        int r = c / (BK / 8), c8 = c % (BK / 8);
        int grow = min(row0 + r, row_end - 1);
        // gathered rows are clamped to the M source rows, so a corrupt row
        // map can never read outside A
        int src = p.a_rows ? min(max(p.a_rows[grow] / p.a_div, 0), p.M - 1) : grow;
        a_src[i] = p.A + (int64_t)src * K + c8 * 8;
        a_dst[i] = r * LDS_STRIDE + c8 * 8;
    }
    const uint16_t* b_src[B_CHUNKS];
    int b_dst[B_CHUNKS];
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i) {
        int c = tid + i * NT;
        int r = c / (BK / 8), c8 = c % (BK / 8);
        int wrow;
        if (MODE == MODE_SWIGLU) {
            // tile column r -> (wave column, n-subtile, lane) -> gate or up row
            constexpr int HALF = WN / 32;
            int wcol = r / WN, rr = r % WN, j = rr / 16, i16 = rr % 16;
            int hcol = blockIdx.y * (BN / 2) + wcol * (WN / 2) + (j % HALF) * 16 + i16;
            hcol = min(hcol, p.N - 1);
            wrow = (j < HALF) ? hcol : p.N + hcol;
        } else {
            wrow = min(blockIdx.y * BN + r, p.N - 1);
        }
        b_src[i] = Wg + (int64_t)wrow * K + c8 * 8;
        b_dst[i] = r * LDS_STRIDE + c8 * 8;
    }

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint4 ra[A_CHUNKS], rb[B_CHUNKS];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) ra[i] = *(const uint4*)(a_src[i] + k0);
#pragma unroll
        for (int i = 0; i < B_CHUNKS; ++i) rb[i] = *(const uint4*)(b_src[i] + k0);
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) *(uint4*)(&As[buf][a_dst[i]]) = ra[i];
#pragma unroll
        for (int i = 0; i < B_CHUNKS; ++i) *(uint4*)(&Bs[buf][b_dst[i]]) = rb[i];
    };

    const int nk = K / BK;
    gload(0);
    lstore(0);
    __syncthreads();
    const int frag_row = lane & 15, frag_k = (lane >> 4) * 8;
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
        for (int ks = 0; ks < BK; ks += 32) {
            bf16x8 af[TM], bfr[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                af[i] = *(const bf16x8*)(&As[buf][(wm * WM + i * 16 + frag_row) * LDS_STRIDE + ks + frag_k]);
#pragma unroll
            for (int j = 0; j < TN; ++j)
                bfr[j] = *(const bf16x8*)(&Bs[buf][(wn * WN + j * 16 + frag_row) * LDS_STRIDE + ks + frag_k]);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) {
            lstore(buf ^ 1);
            __syncthreads();
        }
    }

    // ---- epilogue: lane holds column (lane & 15), rows 4*(lane >> 4) + v
    const int ccol = lane & 15, crow = (lane >> 4) * 4;
    if (MODE == MODE_SWIGLU) {
        constexpr int HALF = WN / 32;
        uint16_t* H = (uint16_t*)p.C;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int jj = 0; jj < HALF; ++jj) {
                int hcol = blockIdx.y * (BN / 2) + wn * (WN / 2) + jj * 16 + ccol;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    int row = row0 + wm * WM + i * 16 + crow + v;
                    if (row < row_end && hcol < p.N)
                        H[(int64_t)row * p.N + hcol] =
                            f32_to_bf16(swiglu_clip(acc[i][jj][v], acc[i][jj + HALF][v], p.limit));
                }
            }
    } else {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                int col = blockIdx.y * BN + wn * WN + j * 16 + ccol;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    int row = row0 + wm * WM + i * 16 + crow + v;
                    if (row < row_end && col < p.N) {
                        if (MODE == MODE_OUT_F32)
                            ((float*)p.C)[(int64_t)row * p.N + col] = acc[i][j][v];
                        else
                            ((_Float16*)p.C)[(int64_t)row * p.N + col] = f32_to_f16_sat(acc[i][j][v]);
                    }
                }
            }
    }
}

// tile_start[g] = sum over groups before g of ceil(count / bm); one block
__global__ void tile_plan_kernel(const int32_t* offsets, int groups, int bm, int32_t* tile_start) {
    __shared__ int32_t part[1024];
    const int t = threadIdx.x;
    int mine = 0;
    if (t < groups) mine = (offsets[t + 1] - offsets[t] + bm - 1) / bm;
    part[t] = mine;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {      // inclusive Hillis-Steele scan
        int v = t >= o ? part[t - o] : 0;
        __syncthreads();
        part[t] += v;
        __syncthreads();
    }
    if (t < groups) tile_start[t + 1] = part[t];
    if (t == 0) tile_start[0] = 0;
}

constexpr int BIG_BM = 128, BIG_BN = 128;

int gemm_tile_m() { return BIG_BM; }

hipError_t launch_tile_plan(const int32_t* offsets, int E, int bm, int32_t* tile_start, hipStream_t s) {
    tile_plan_kernel<<<1, 1024, 0, s>>>(offsets, E, bm, tile_start);
    return hipGetLastError();
}

static GemmParams make_params(const void* A, const int32_t* a_rows, int a_div, const void* W,
                              int64_t stride, void* C, int M, int N, int K, float limit,
                              const int32_t* offsets, const int32_t* tile_start, int groups) {
    GemmParams p;
    p.A = (const uint16_t*)A;
    p.a_rows = a_rows;
    p.a_div = a_div > 0 ? a_div : 1;
    p.W = (const uint16_t*)W;
    p.w_group_stride = stride;
    p.C = C;
    p.M = M;
    p.N = N;
    p.K = K;
    p.limit = limit;
    p.offsets = offsets;
    p.tile_start = tile_start;
    p.groups = groups;
    return p;
}

hipError_t launch_gemm_swiglu(const void* A, const int32_t* a_rows, int a_div, const void* W13,
                              int64_t w_group_stride, void* h, int M, int N, int K, float limit,
                              const int32_t* offsets, const int32_t* tile_start, int groups,
                              int max_tiles, hipStream_t s) {
    GemmParams p = make_params(A, a_rows, a_div, W13, w_group_stride, h, M, N, K, limit, offsets,
                               tile_start, groups);
    const int gx = tile_start ? max_tiles : (M + BIG_BM - 1) / BIG_BM;
    if (gx <= 0) return hipSuccess;
    dim3 grid(gx, (N + BIG_BN / 2 - 1) / (BIG_BN / 2));
    gemm_kernel<BIG_BM, BIG_BN, 64, 64, MODE_SWIGLU><<<grid, 256, 0, s>>>(p);
    return hipGetLastError();
}

hipError_t launch_gemm_out(const void* A, const void* W, int64_t w_group_stride, void* C, bool c_fp32,
                           int M, int N, int K, const int32_t* offsets, const int32_t* tile_start,
                           int groups, int max_tiles, hipStream_t s) {
    // c_fp32 == false: fp16 output (the routed experts' rows)
    GemmParams p = make_params(A, nullptr, 1, W, w_group_stride, C, M, N, K, 0.f, offsets,
                               tile_start, groups);
    const int gx = tile_start ? max_tiles : (M + BIG_BM - 1) / BIG_BM;
    if (gx <= 0) return hipSuccess;
    dim3 grid(gx, (N + BIG_BN - 1) / BIG_BN);
    if (c_fp32)
        gemm_kernel<BIG_BM, BIG_BN, 64, 64, MODE_OUT_F32><<<grid, 256, 0, s>>>(p);
    else
        gemm_kernel<BIG_BM, BIG_BN, 64, 64, MODE_OUT_F16><<<grid, 256, 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace moe
