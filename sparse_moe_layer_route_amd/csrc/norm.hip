// norm.hip -- the zero-centred RMSNorm in front of the MoE layer (page
// "MAX 中 Step-3.5-Flash 架构解析…": the block's norms are zero-centred
// RMSNorms with weight_offset 1, so a stored weight g scales by 1 + g; the
// AutoModel page's benchmark keeps norms and the residual stream in FP32):
//   x[t, h] = bf16( r[t, h] / sqrt(mean_h r[t, :]^2 + eps) * (1 + g[h]) )
// from the fp32 residual r [T,H], in fp32, rounded to nearest even.
//
// HBM-bound: one read of the fp32 row, one write of the bf16 row.  One
// wavefront per row (4 rows per 256-thread block).  Rows of up to 64*4*NV
// values are held in registers: all 16-byte loads of the row are issued at
// once, a wave sum gives the mean square, and the scaled bf16 values go out
// 8 bytes per lane.  Longer rows take two passes, the second reading the row
// again (from the cache).
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

template <int NV>
__global__ __launch_bounds__(256) void rmsnorm_regs_kernel(const float* __restrict__ r, const float* __restrict__ g,
                                                           float eps, uint16_t* __restrict__ x, int T, int H) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const float4* row = (const float4*)(r + (int64_t)t * H);
    const float4* g4 = (const float4*)g;
    const int n4 = H / 4;
    float4 v[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j)
        if (lane + 64 * j < n4) v[j] = row[lane + 64 * j];
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j)
        if (lane + 64 * j < n4) ss += v[j].x * v[j].x + v[j].y * v[j].y + v[j].z * v[j].z + v[j].w * v[j].w;
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)H + eps);
    uint2* out = (uint2*)(x + (int64_t)t * H);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int i = lane + 64 * j;
        if (i < n4) {
            const float4 w = g4[i];
            uint2 o;
            o.x = pack_bf16x2(v[j].x * inv * (1.0f + w.x), v[j].y * inv * (1.0f + w.y));
            o.y = pack_bf16x2(v[j].z * inv * (1.0f + w.z), v[j].w * inv * (1.0f + w.w));
            out[i] = o;
        }
    }
}

__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ r, const float* __restrict__ g,
                                                      float eps, uint16_t* __restrict__ x, int T, int H) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const float4* row = (const float4*)(r + (int64_t)t * H);
    const float4* g4 = (const float4*)g;
    const int n4 = H / 4;
    float ss = 0.f;
    for (int i = lane; i < n4; i += 64) {
        const float4 v = row[i];
        ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)H + eps);
    uint2* out = (uint2*)(x + (int64_t)t * H);
    for (int i = lane; i < n4; i += 64) {
        const float4 v = row[i];
        const float4 w = g4[i];
        uint2 o;
        o.x = pack_bf16x2(v.x * inv * (1.0f + w.x), v.y * inv * (1.0f + w.y));
        o.y = pack_bf16x2(v.z * inv * (1.0f + w.z), v.w * inv * (1.0f + w.w));
        out[i] = o;
    }
}

hipError_t launch_rmsnorm(const float* resid, const float* norm_weight, float eps, void* x, int T, int H,
                          hipStream_t s) {
    if (T <= 0) return hipSuccess;
    const unsigned blocks = (unsigned)((T + 3) / 4);
    if (H <= 64 * 4 * 16)
        rmsnorm_regs_kernel<16><<<blocks, 256, 0, s>>>(resid, norm_weight, eps, (uint16_t*)x, T, H);
    else
        rmsnorm_kernel<<<blocks, 256, 0, s>>>(resid, norm_weight, eps, (uint16_t*)x, T, H);
    return hipGetLastError();
}

}  // namespace moe
