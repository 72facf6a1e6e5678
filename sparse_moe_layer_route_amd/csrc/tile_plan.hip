// tile_plan.hip -- the tile plan of the grouped expert GEMMs: for expert
// groups with row offsets[E+1] and bm-row tiles,
//   tile_start[g] = sum over groups before g of ceil(rows_g / bm),
// so a grouped launch maps its work item to (expert, tile) without the host
// ever reading the routing.  An optional extra group of extra_rows rows
// (index E) gets its tiles after the experts'.  One block of 1024 threads
// (E <= 1024).
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

__global__ __launch_bounds__(1024) void tile_plan_kernel(const int32_t* __restrict__ offsets, int groups, int bm,
                                                         int extra_rows, int32_t* __restrict__ tile_start) {
    __shared__ int32_t part[1024];
    const int t = threadIdx.x;
    part[t] = t < groups ? (offsets[t + 1] - offsets[t] + bm - 1) / bm : 0;
    const int extra_tiles = (extra_rows + bm - 1) / bm;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {      // inclusive Hillis-Steele scan
        const int v = t >= o ? part[t - o] : 0;
        __syncthreads();
        part[t] += v;
        __syncthreads();
    }
    if (t < groups) tile_start[t + 1] = part[t];
    if (t == 0) tile_start[0] = 0;
    if (t == groups - 1 && extra_rows > 0) tile_start[groups + 1] = part[t] + extra_tiles;
}

hipError_t launch_tile_plan(const int32_t* offsets, int E, int bm, int extra_rows, int32_t* tile_start,
                            hipStream_t s) {
    tile_plan_kernel<<<1, 1024, 0, s>>>(offsets, E, bm, extra_rows, tile_start);
    return hipGetLastError();
}

}  // namespace moe
