// permute.hip -- stable grouping of the T*k (token, slot) pairs by expert.
//
// The rows the grouped experts run on are expert-major and, inside an
// expert, in ascending pair order p = t*k + j (so ascending in token).  The
// rank of pair p inside expert e is the number of earlier pairs routed to
// e.  It is computed without sorting and without any order-dependent
// atomics, so the result is deterministic:
//   1. one bitmap per expert over the pairs: bit p of bitmap[e] is set when
//      pair p goes to e (atomicOr; the bits commute);
//   2. one block per expert: popcount of every 32-bit word, exclusive scan
//      over the words -> word_prefix[e][w], and counts[e];
//   3. one block: exclusive scan of counts -> offsets;
//   4. one thread per pair: row = offsets[e] + word_prefix[e][p/32]
//      + popcount(bitmap[e][p/32] & bits below p).
// Scratch: 2 * E * ceil(P/32) words.
// Small batches (all bitmaps fit in 64 KiB: decode) take one launch instead:
// one block builds the bitmaps in LDS and does steps 2-4 there (same stable
// order), and also writes the grouped GEMMs' tile plan when asked.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

static inline int64_t words_for(int64_t P) { return (P + 31) / 32; }

size_t permute_scratch_bytes(int64_t P, int E) {
    return (size_t)2 * (size_t)E * (size_t)words_for(P) * 4;
}

__global__ void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (; i < n; i += stride) p[i] = v;
}

__global__ void set_bits_kernel(const int32_t* __restrict__ ids, int64_t P, int E, int64_t W,
                                uint32_t* __restrict__ bm) {
    int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= P) return;
    int e = min(max(ids[p], 0), E - 1);
    atomicOr(&bm[(int64_t)e * W + (p >> 5)], 1u << (p & 31));
}

// block-wide exclusive scan of one int per thread (256 threads); returns the
// exclusive prefix and writes the block total to *total
__device__ int block_exclusive_scan_256(int v, int* total) {
    __shared__ int wsum[4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int u = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += u;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        if (w < wave) base += wsum[w];
        tot += wsum[w];
    }
    __syncthreads();
    *total = tot;
    return base + incl - v;
}

__global__ __launch_bounds__(256) void expert_scan_kernel(const uint32_t* __restrict__ bm, int64_t W,
                                                          int32_t* __restrict__ word_prefix,
                                                          int32_t* __restrict__ counts) {
    const int e = blockIdx.x;
    const uint32_t* b = bm + (int64_t)e * W;
    int32_t* wp = word_prefix + (int64_t)e * W;
    // each thread owns a contiguous run of words per pass
    const int64_t per = (W + 255) / 256;
    const int64_t w0 = (int64_t)threadIdx.x * per;
    int mine = 0;
    for (int64_t w = w0; w < w0 + per && w < W; ++w) mine += __popc(b[w]);
    int total;
    int run = block_exclusive_scan_256(mine, &total);
    for (int64_t w = w0; w < w0 + per && w < W; ++w) {
        wp[w] = run;
        run += __popc(b[w]);
    }
    if (threadIdx.x == 0) counts[e] = total;
}

__global__ __launch_bounds__(1024) void offsets_kernel(const int32_t* __restrict__ counts, int E,
                                                       int32_t* __restrict__ offsets) {
    __shared__ int part[1024];
    const int t = threadIdx.x;
    part[t] = t < E ? counts[t] : 0;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {
        int v = t >= o ? part[t - o] : 0;
        __syncthreads();
        part[t] += v;
        __syncthreads();
    }
    if (t < E) offsets[t + 1] = part[t];
    if (t == 0) offsets[0] = 0;
}

__global__ void scatter_kernel(const int32_t* __restrict__ ids, int64_t P, int E, int64_t W,
                               const uint32_t* __restrict__ bm, const int32_t* __restrict__ word_prefix,
                               const int32_t* __restrict__ offsets, int32_t* __restrict__ row_to_pair,
                               int32_t* __restrict__ pair_to_row) {
    int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= P) return;
    int e = min(max(ids[p], 0), E - 1);
    int64_t w = p >> 5;
    uint32_t below = bm[(int64_t)e * W + w] & ((1u << (p & 31)) - 1u);
    int row = offsets[e] + word_prefix[(int64_t)e * W + w] + __popc(below);
    row_to_pair[row] = (int32_t)p;
    pair_to_row[p] = row;
}

// One-block path: bitmaps of all experts in LDS (E * ceil(P/32) words).
constexpr int SMALL_WORDS = 16384;                // 64 KiB of LDS

static bool small_path(int64_t P, int E) { return P > 0 && (int64_t)E * words_for(P) <= SMALL_WORDS; }

__global__ __launch_bounds__(1024) void permute_small_kernel(const int32_t* __restrict__ ids, int P, int E,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ row_to_pair,
                                                             int32_t* __restrict__ pair_to_row, int bm,
                                                             int extra_rows, int32_t* __restrict__ tile_start) {
    __shared__ uint32_t bits[SMALL_WORDS];
    __shared__ int32_t part[1024];
    const int t = threadIdx.x;
    const int W = (P + 31) >> 5;
    for (int i = t; i < E * W; i += 1024) bits[i] = 0u;
    __syncthreads();
    for (int p = t; p < P; p += 1024) {
        const int e = min(max(ids[p], 0), E - 1);
        atomicOr(&bits[e * W + (p >> 5)], 1u << (p & 31));   // bits commute: order-free
    }
    __syncthreads();
    int cnt = 0;
    if (t < E)
        for (int w = 0; w < W; ++w) cnt += __popc(bits[t * W + w]);
    // inclusive scan of the counts
    part[t] = cnt;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {
        const int v = t >= o ? part[t - o] : 0;
        __syncthreads();
        part[t] += v;
        __syncthreads();
    }
    if (t < E) {
        const int off = part[t] - cnt;
        counts[t] = cnt;
        offsets[t] = off;
        if (t == E - 1) offsets[E] = off + cnt;
    }
    __syncthreads();
    // rank of pair p inside its expert = set bits of the expert's bitmap below p
    for (int p = t; p < P; p += 1024) {
        const int e = min(max(ids[p], 0), E - 1);
        const int wp = p >> 5;
        int below = __popc(bits[e * W + wp] & ((1u << (p & 31)) - 1u));
        for (int w = 0; w < wp; ++w) below += __popc(bits[e * W + w]);
        const int row = (e > 0 ? part[e - 1] : 0) + below;    // exclusive offset of e + rank
        row_to_pair[row] = p;
        pair_to_row[p] = row;
    }
    if (!tile_start) return;                      // uniform over the block
    const int tiles = t < E ? (cnt + bm - 1) / bm : 0;
    __syncthreads();
    part[t] = tiles;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {
        const int v = t >= o ? part[t - o] : 0;
        __syncthreads();
        part[t] += v;
        __syncthreads();
    }
    if (t < E) tile_start[t + 1] = part[t];
    if (t == 0) tile_start[0] = 0;
    if (t == E - 1 && extra_rows > 0) tile_start[E + 1] = part[t] + (extra_rows + bm - 1) / bm;
}

hipError_t launch_permute_plan(const int32_t* ids, int T, int k, int E, int32_t* counts, int32_t* offsets,
                               int32_t* row_to_pair, int32_t* pair_to_row, void* scratch, int bm, int extra_rows,
                               int32_t* tile_start, hipStream_t s) {
    const int64_t P = (int64_t)T * k;
    if (small_path(P, E)) {
        permute_small_kernel<<<1, 1024, 0, s>>>(ids, (int)P, E, counts, offsets, row_to_pair, pair_to_row, bm,
                                                extra_rows, tile_start);
        return hipGetLastError();
    }
    hipError_t e = launch_permute(ids, T, k, E, counts, offsets, row_to_pair, pair_to_row, scratch, s);
    if (e != hipSuccess || !tile_start) return e;
    return launch_tile_plan(offsets, E, bm, extra_rows, tile_start, s);
}

hipError_t launch_permute(const int32_t* ids, int T, int k, int E, int32_t* counts, int32_t* offsets,
                          int32_t* row_to_pair, int32_t* pair_to_row, void* scratch, hipStream_t s) {
    const int64_t P = (int64_t)T * k;
    if (small_path(P, E)) {
        permute_small_kernel<<<1, 1024, 0, s>>>(ids, (int)P, E, counts, offsets, row_to_pair, pair_to_row, 1, 0,
                                                nullptr);
        return hipGetLastError();
    }
    const int64_t W = words_for(P);
    uint32_t* bm = (uint32_t*)scratch;
    int32_t* wp = (int32_t*)(bm + (int64_t)E * W);
    if (P > 0) {
        int64_t n = (int64_t)E * W;
        int blocks = (int)std::min<int64_t>((n + 255) / 256, 4096);
        fill_u32_kernel<<<blocks, 256, 0, s>>>(bm, n, 0u);
        set_bits_kernel<<<(unsigned)((P + 255) / 256), 256, 0, s>>>(ids, P, E, W, bm);
    }
    expert_scan_kernel<<<E, 256, 0, s>>>(bm, P > 0 ? W : 0, wp, counts);
    offsets_kernel<<<1, 1024, 0, s>>>(counts, E, offsets);
    if (P > 0)
        scatter_kernel<<<(unsigned)((P + 255) / 256), 256, 0, s>>>(ids, P, E, W, bm, wp, offsets,
                                                                    row_to_pair, pair_to_row);
    return hipGetLastError();
}

}  // namespace moe
