// grouped_gemm.hip -- the routed experts' weight-streaming GEMMs on gfx950.
//
//   C[r, n] = sum_k A[src(r), k] * W_e[n, k]      for every row r of expert e
//
// Mode SWIGLU (first projection): the block's 128 weight rows are 64 gate
// rows and the matching 64 up rows, and the epilogue writes
// h = act(gate, up, L) in bf16 (clipped SwiGLU).  Mode F16 / F32 (second
// projection, shared expert): plain output.
//
// Shape of the work.  At the shapes of the layer the expert weights are
// streamed from HBM once per M tile, so the M tile is 256 rows: with top-8
// of 288-352 experts almost every expert fits one tile.  A block computes
// 256 rows x 128 weight rows with 4 waves stacked along M (64 rows each);
// MFMA 16-row sub-tiles past the expert's last row are skipped.
//
//   * B (weights): a ring of STAGES K-slices (64 wide) in LDS, filled by
//     direct global->LDS loads (global_load_lds_dwordx4, one 1 KiB row group
//     per wave instruction).  Each 128-byte row is stored with its eight
//     16-byte chunks XOR-swizzled by (row & 7) so the fragment reads of 8
//     consecutive rows hit 8 different bank groups.
//   * A (activation rows): only the wave that owns a row uses it, so A goes
//     straight from global memory (the gathered x row, or h) to registers in
//     MFMA layout, prefetched one K-slice ahead.  No permuted copy of x is
//     ever written.
//   * K order inside a 64-wide slice: lane group g (lane >> 4) of MFMA step s
//     takes chunk 2g+s, for A and B alike (a dot product does not care about
//     the order of its terms), so each lane's A data for a slice are 32
//     contiguous bytes.
//   * Work order: (expert, n-tile, m-tile) with m fastest, so the m-tiles of
//     one expert's weight panel run together and share it in L2; each XCD
//     (blocks b with b % 8 == x) takes a contiguous range of that list.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace gg {

constexpr int BM = 256, BN = 128, BK = 64;
constexpr int TM = 4;    // 16-row MFMA tiles per wave (64 rows)
constexpr int TN = 8;    // 16-col MFMA tiles per wave (128 cols)
constexpr int NXCD = 8;

enum { SWIGLU = 0, OUT_F16 = 1, OUT_F32 = 2 };

struct Params {
    const uint16_t* A;          // bf16 activations
    const int32_t* a_rows;      // gather: A row = a_rows[r] / a_div; nullptr: row r
    int a_div;
    int a_nrows;                // rows of A (gather clamp)
    const uint16_t* W;          // bf16 weights [groups][Nw][K]
    int64_t w_group_stride;
    void* C;
    int N;                      // output columns (SWIGLU: h width, W has 2N rows)
    int K;
    float limit;
    const int32_t* offsets;     // [groups+1] row offsets; nullptr: dense with M rows
    const int32_t* tile_start;  // [groups+1] BM-tile plan (grouped)
    int groups;
    int M;                      // dense rows
    int n_tiles;                // BN tiles along N (SWIGLU: of 2N weight rows)
};

// Register rings: B slices are loaded RING-1 ahead into registers and
// written to the LDS double buffer one slice ahead of use; A slices are
// loaded RING-1 ahead.  The K loop is unrolled by RING so every ring slot
// is a compile-time register set.
constexpr int RING = 3;
constexpr int B_CHUNKS = BN * BK / 8 / 256;   // 16-byte chunks per thread per slice (4)

template <int MODE>
__global__ __launch_bounds__(256, 1) void kernel(Params p) {
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * BK];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    // ---- decode the work item ------------------------------------------
    int g = 0, m_tile, n_tile, row0, row_end;
    {
        const int b = blockIdx.x;
        const int xcd = b % NXCD, slot = b / NXCD;
        if (p.offsets) {
            const int ntiles = p.tile_start[p.groups];
            const int total = ntiles * p.n_tiles;
            const int per = (total + NXCD - 1) / NXCD;
            if (slot >= per) return;
            const int w = xcd * per + slot;
            if (w >= total) return;
            // expert owning work item w: largest g with tile_start[g]*n_tiles <= w
            int lo = 0, hi = p.groups - 1;
            while (lo < hi) {
                int mid = (lo + hi + 1) >> 1;
                if (p.tile_start[mid] * p.n_tiles <= w) lo = mid; else hi = mid - 1;
            }
            g = lo;
            const int mt = p.tile_start[g + 1] - p.tile_start[g];
            const int local = w - p.tile_start[g] * p.n_tiles;
            n_tile = local / mt;
            m_tile = local % mt;
            row0 = p.offsets[g] + m_tile * BM;
            row_end = p.offsets[g + 1];
        } else {
            const int mt = (p.M + BM - 1) / BM;
            const int total = mt * p.n_tiles;
            const int per = (total + NXCD - 1) / NXCD;
            if (slot >= per) return;
            const int w = xcd * per + slot;
            if (w >= total) return;
            n_tile = w / mt;
            m_tile = w % mt;
            row0 = m_tile * BM;
            row_end = p.M;
        }
    }
    const int valid = min(row_end - row0, BM);
    const int K = p.K;
    const uint16_t* Wg = p.W + (int64_t)g * p.w_group_stride;

    // ---- B: this thread's 4 chunks of each 128 x 64 slice ------------------
    const uint16_t* bsrc[B_CHUNKS];
    int bdst[B_CHUNKS];
#pragma unroll
    for (int q = 0; q < B_CHUNKS; ++q) {
        const int c = tid + 256 * q;
        const int r = c >> 3, kc = c & 7;             // tile row, k-chunk
        int wrow;
        if (MODE == SWIGLU) {
            const int hcol = min(n_tile * (BN / 2) + (r & 63), p.N - 1);
            wrow = (r < 64) ? hcol : p.N + hcol;
        } else {
            wrow = min(n_tile * BN + r, p.N - 1);
        }
        bsrc[q] = Wg + (int64_t)wrow * K + kc * 8;
        bdst[q] = r * BK + ((kc ^ (r & 7)) << 3);     // swizzled slot
    }

    // ---- A: per-lane row pointers (rows of this wave) ---------------------
    const int g4 = lane >> 4;                         // lane group: chunks 2*g4, 2*g4+1
    int n_i = (valid - 64 * wave + 15) >> 4;          // valid 16-row tiles of this wave
    n_i = n_i < 0 ? 0 : (n_i > TM ? TM : n_i);
    n_i = __builtin_amdgcn_readfirstlane(n_i);        // wave-uniform: scalar branches
    const uint16_t* asrc[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        int r = row0 + min(64 * wave + 16 * i + (lane & 15), valid - 1);
        int src = r;
        if (p.a_rows) src = min(max(p.a_rows[r] / p.a_div, 0), p.a_nrows - 1);
        asrc[i] = p.A + (int64_t)src * K + g4 * 16;
    }

    u32x4 breg[RING][B_CHUNKS];
    bf16x8 areg[RING][TM][2];
    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = K / BK;
    const int frow = lane & 15;

#define GG_LOAD(J, KT)                                                              \
    do {                                                                            \
        const int k0_ = (KT) * BK;                                                  \
        _Pragma("unroll") for (int q = 0; q < B_CHUNKS; ++q)                        \
            breg[J][q] = *(const u32x4*)(bsrc[q] + k0_);                            \
        _Pragma("unroll") for (int i = 0; i < TM; ++i) {                            \
            areg[J][i][0] = *(const bf16x8*)(asrc[i] + k0_);                        \
            areg[J][i][1] = *(const bf16x8*)(asrc[i] + k0_ + 8);                    \
        }                                                                           \
    } while (0)

#define GG_STORE_B(J, BUF)                                                          \
    do {                                                                            \
        _Pragma("unroll") for (int q = 0; q < B_CHUNKS; ++q)                        \
            *(u32x4*)(&Bs[BUF][bdst[q]]) = breg[J][q];                              \
    } while (0)

#define GG_COMPUTE(J, BUF)                                                          \
    do {                                                                            \
        const uint16_t* bs_ = Bs[BUF];                                              \
        _Pragma("unroll") for (int s = 0; s < 2; ++s) {                             \
            bf16x8 bfr[TN];                                                         \
            _Pragma("unroll") for (int j = 0; j < TN; ++j) {                        \
                const int r = 16 * j + frow;                                        \
                const int c = 2 * g4 + s;                                           \
                bfr[j] = *(const bf16x8*)(bs_ + r * BK + ((c ^ (r & 7)) << 3));     \
            }                                                                       \
            _Pragma("unroll") for (int i = 0; i < TM; ++i) {                        \
                if (i < n_i) {                                                      \
                    _Pragma("unroll") for (int j = 0; j < TN; ++j)                  \
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(        \
                            areg[J][i][s], bfr[j], acc[i][j], 0, 0, 0);             \
                }                                                                   \
            }                                                                       \
        }                                                                           \
    } while (0)

    // One K step: slice KT+RING-1 starts loading into the register slot that
    // slice KT-1 used; slice KT (slot J = KT % RING) is computed from LDS
    // buffer KT % 2; then slice KT+1 moves registers -> LDS buffer (KT+1) % 2
    // (read in the previous step, which every wave has left), so the B loads
    // of a slice have two steps to arrive.  Loads past the last slice re-read
    // the last slice, so every step issues the same loads and the compiler's
    // wait counts stay exact.
#define GG_STEP(J, KT)                                                              \
    do {                                                                            \
        GG_LOAD(((J) + RING - 1) % RING, min((KT) + RING - 1, nk - 1));             \
        GG_COMPUTE(J, (KT) & 1);                                                    \
        GG_STORE_B(((J) + 1) % RING, ((KT) + 1) & 1);                               \
        __syncthreads();                                                            \
    } while (0)

    // prologue: slices 0 .. RING-2 loading, slice 0 staged in LDS
#pragma unroll
    for (int j = 0; j < RING - 1; ++j) GG_LOAD(j, min(j, nk - 1));
    GG_STORE_B(0, 0);
    __syncthreads();

    int kt = 0;
    for (; kt + RING <= nk; kt += RING) {
        GG_STEP(0, kt);
        GG_STEP(1, kt + 1);
        GG_STEP(2, kt + 2);
    }
    if (kt < nk) GG_STEP(0, kt);
    if (kt + 1 < nk) GG_STEP(1, kt + 1);
#undef GG_STEP
#undef GG_COMPUTE
#undef GG_STORE_B
#undef GG_LOAD

    // ---- epilogue: lane holds column (lane & 15), rows 4*(lane >> 4) + v ---
    const int ccol = lane & 15, crow = (lane >> 4) * 4;
    if (MODE == SWIGLU) {
        uint16_t* H = (uint16_t*)p.C;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            if (i >= n_i) continue;
#pragma unroll
            for (int j = 0; j < TN / 2; ++j) {
                const int hcol = n_tile * (BN / 2) + 16 * j + ccol;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int lr = 64 * wave + 16 * i + crow + v;
                    if (lr < valid && hcol < p.N)
                        H[(int64_t)(row0 + lr) * p.N + hcol] =
                            f32_to_bf16(swiglu_clip(acc[i][j][v], acc[i][j + TN / 2][v], p.limit));
                }
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            if (i >= n_i) continue;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int col = n_tile * BN + 16 * j + ccol;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int lr = 64 * wave + 16 * i + crow + v;
                    if (lr < valid && col < p.N) {
                        if (MODE == OUT_F32)
                            ((float*)p.C)[(int64_t)(row0 + lr) * p.N + col] = acc[i][j][v];
                        else
                            ((_Float16*)p.C)[(int64_t)(row0 + lr) * p.N + col] = f32_to_f16_sat(acc[i][j][v]);
                    }
                }
            }
        }
    }
}

static int grid_blocks(int64_t work) {
    const int64_t per = (work + NXCD - 1) / NXCD;
    return (int)(per * NXCD);
}

}  // namespace gg

int grouped_tile_m() { return gg::BM; }

hipError_t launch_grouped_up(const void* A, const int32_t* a_rows, int a_div, int a_nrows, const void* W13,
                             int64_t w_group_stride, void* h, int M, int N, int K, float limit,
                             const int32_t* offsets, const int32_t* tile_start, int groups, int max_tiles,
                             hipStream_t s) {
    gg::Params p{};
    p.A = (const uint16_t*)A;
    p.a_rows = a_rows;
    p.a_div = a_div > 0 ? a_div : 1;
    p.a_nrows = a_nrows;
    p.W = (const uint16_t*)W13;
    p.w_group_stride = w_group_stride;
    p.C = h;
    p.N = N;
    p.K = K;
    p.limit = limit;
    p.offsets = offsets;
    p.tile_start = tile_start;
    p.groups = groups;
    p.M = M;
    p.n_tiles = (2 * N) / gg::BN;
    const int64_t tiles = offsets ? max_tiles : (M + gg::BM - 1) / gg::BM;
    if (tiles <= 0) return hipSuccess;
    gg::kernel<gg::SWIGLU><<<gg::grid_blocks(tiles * p.n_tiles), 256, 0, s>>>(p);
    return hipGetLastError();
}

hipError_t launch_grouped_down(const void* A, const void* W, int64_t w_group_stride, void* C, bool c_fp32,
                               int M, int N, int K, const int32_t* offsets, const int32_t* tile_start,
                               int groups, int max_tiles, hipStream_t s) {
    gg::Params p{};
    p.A = (const uint16_t*)A;
    p.a_rows = nullptr;
    p.a_div = 1;
    p.a_nrows = M;
    p.W = (const uint16_t*)W;
    p.w_group_stride = w_group_stride;
    p.C = C;
    p.N = N;
    p.K = K;
    p.offsets = offsets;
    p.tile_start = tile_start;
    p.groups = groups;
    p.M = M;
    p.n_tiles = (N + gg::BN - 1) / gg::BN;
    const int64_t tiles = offsets ? max_tiles : (M + gg::BM - 1) / gg::BM;
    if (tiles <= 0) return hipSuccess;
    if (c_fp32)
        gg::kernel<gg::OUT_F32><<<gg::grid_blocks(tiles * p.n_tiles), 256, 0, s>>>(p);
    else
        gg::kernel<gg::OUT_F16><<<gg::grid_blocks(tiles * p.n_tiles), 256, 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace moe
