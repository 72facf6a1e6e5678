// bwd.hip -- the layer backward's row kernels (the GEMMs are in bwd_gemm.hip).
//
// With dout = dL/dout [T,H] fp32, the saved forward (expert choice, weights
// w_j, raw scores s_j, expert output rows y_j) and the loss sum(out * dout):
//   dw_j = dout . y_j                     (the weight's gradient)
//   dy_j = w_j dout                       (the expert output's gradient)
//   ds_j = scale/S (dw_j - sum_j' dw_j' s_j'/S), S = sum_j s_j  (scale dw_j
//          without normalisation);  da_j = ds_j s_j (1 - s_j)   (the logit's)
//   dx   = sum_j dxr_j + dxr_shared + sum_j da_j W_router[e_j]
//   dW_router[e] = sum over the rows of e of da x
// The choice itself passes no gradient and the routing bias gets none.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// One block (256 threads) per token: the k dot products dout . y_j (block
// sums in slot order), the bf16 dy rows, and da.
__global__ __launch_bounds__(256) void bwd_prep_kernel(const float* __restrict__ dout,
                                                       const char* __restrict__ y_rows,
                                                       const int32_t* __restrict__ p2r, const float* __restrict__ w,
                                                       const float* __restrict__ s_raw, float scale, int norm,
                                                       int shared, uint16_t* __restrict__ dy, float* __restrict__ da,
                                                       int T, int H, int k) {
    __shared__ float red[4];
    __shared__ float dws[32];
    const int t = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float* d = dout + (int64_t)t * H;
    const int64_t P = (int64_t)T * k;
    for (int j = 0; j < k; ++j) {
        const int64_t r = p2r[(int64_t)t * k + j];
        const float wj = w[(int64_t)t * k + j];
        const char* y = y_rows + r * yrow_bytes(H);
        uint16_t* o = dy + r * H;
        float acc = 0.f;
        for (int h = tid * 4; h < H; h += 256 * 4) {
            const float4 dv = *(const float4*)(d + h);
            typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
            const f16x4 yv = *(const f16x4*)(y + 2 * h);
            const float sc = exp2_int((signed char)y[2 * H + (h >> 7)]);
            acc += (dv.x * (float)yv[0] + dv.y * (float)yv[1] + dv.z * (float)yv[2] + dv.w * (float)yv[3]) * sc;
            uint2 q;
            q.x = pack_bf16x2(wj * dv.x, wj * dv.y);
            q.y = pack_bf16x2(wj * dv.z, wj * dv.w);
            *(uint2*)(o + h) = q;
        }
        acc = wave_sum(acc);
        if (lane == 0) red[wave] = acc;
        __syncthreads();
        if (tid == 0) dws[j] = (red[0] + red[1]) + (red[2] + red[3]);
        __syncthreads();
    }
    if (shared) {
        uint16_t* o = dy + (P + t) * H;
        for (int h = tid * 4; h < H; h += 256 * 4) {
            const float4 dv = *(const float4*)(d + h);
            uint2 q;
            q.x = pack_bf16x2(dv.x, dv.y);
            q.y = pack_bf16x2(dv.z, dv.w);
            *(uint2*)(o + h) = q;
        }
    }
    if (tid < 64) {
        const float sj = lane < k ? s_raw[(int64_t)t * k + lane] : 0.f;
        const float dwj = lane < k ? dws[lane] : 0.f;
        const float S = norm ? wave_sum(sj) : 1.0f;
        const float sdw = wave_sum(dwj * sj) / S;
        const float ds = norm ? scale / S * (dwj - sdw) : scale * dwj;
        if (lane < k) da[(int64_t)t * k + lane] = ds * sj * (1.0f - sj);
    }
}

// One block per (token, 2048 columns): 8 columns per thread.
__global__ __launch_bounds__(256) void bwd_dx_kernel(const float* __restrict__ dxr, const int32_t* __restrict__ p2r,
                                                     const float* __restrict__ da, const int32_t* __restrict__ ids,
                                                     const uint16_t* __restrict__ wr, int shared,
                                                     float* __restrict__ dx, int T, int H, int k) {
    const int t = blockIdx.x;
    const int col = (blockIdx.y * 256 + threadIdx.x) * 8;
    if (col >= H) return;
    const int64_t P = (int64_t)T * k;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    auto add_row = [&](const float* src) {
        const float4 a = *(const float4*)src, b = *(const float4*)(src + 4);
        acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
        acc[4] += b.x; acc[5] += b.y; acc[6] += b.z; acc[7] += b.w;
    };
    for (int j = 0; j < k; ++j) add_row(dxr + (int64_t)p2r[(int64_t)t * k + j] * H + col);
    if (shared) add_row(dxr + (P + t) * H + col);
    for (int j = 0; j < k; ++j) {
        const float a = da[(int64_t)t * k + j];
        const uint4 wv = *(const uint4*)(wr + (int64_t)ids[(int64_t)t * k + j] * H + col);
        const uint32_t u[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            acc[2 * q] += a * bf16_to_f32((uint16_t)(u[q] & 0xffff));
            acc[2 * q + 1] += a * bf16_to_f32((uint16_t)(u[q] >> 16));
        }
    }
    float4* o = (float4*)(dx + (int64_t)t * H + col);
    o[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    o[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

// One block per (expert, 2048 columns): the expert's rows in order.
__global__ __launch_bounds__(256) void bwd_router_wgrad_kernel(const float* __restrict__ da,
                                                               const int32_t* __restrict__ offsets,
                                                               const int32_t* __restrict__ r2p,
                                                               const uint16_t* __restrict__ x, float* __restrict__ dwg,
                                                               int H, int k) {
    const int e = blockIdx.x;
    const int col = (blockIdx.y * 256 + threadIdx.x) * 8;
    if (col >= H) return;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    for (int r = offsets[e]; r < offsets[e + 1]; ++r) {
        const int p = r2p[r];
        const float a = da[p];
        const uint4 xv = *(const uint4*)(x + (int64_t)(p / k) * H + col);
        const uint32_t u[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            acc[2 * q] += a * bf16_to_f32((uint16_t)(u[q] & 0xffff));
            acc[2 * q + 1] += a * bf16_to_f32((uint16_t)(u[q] >> 16));
        }
    }
    float4* o = (float4*)(dwg + (int64_t)e * H + col);
    o[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    o[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

// one block per row: 16 bytes per thread and step
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t* __restrict__ x,
                                                          const int32_t* __restrict__ r2p, uint16_t* __restrict__ out,
                                                          int64_t P, int H, int k) {
    const int64_t r = blockIdx.x;
    const int64_t src = r < P ? r2p[r] / k : r - P;
    const uint4* from = (const uint4*)(x + src * H);
    uint4* to = (uint4*)(out + r * H);
    for (int i = threadIdx.x; i < H / 8; i += 256) to[i] = from[i];
}

__global__ __launch_bounds__(256) void zero_u32_kernel(uint32_t* __restrict__ p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0u;
}

hipError_t launch_bwd_prep(const float* dout, const void* y_rows, const int32_t* p2r, const float* w,
                           const float* s_raw, float scale, int norm, bool shared, void* dy, float* da, int T,
                           int H, int k, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    bwd_prep_kernel<<<T, 256, 0, s>>>(dout, (const char*)y_rows, p2r, w, s_raw, scale, norm, shared ? 1 : 0,
                                      (uint16_t*)dy, da, T, H, k);
    return hipGetLastError();
}

hipError_t launch_bwd_dx(const float* dxr, const int32_t* p2r, const float* da, const int32_t* ids,
                         const void* w_router, bool shared, float* dx, int T, int H, int k, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    bwd_dx_kernel<<<dim3(T, (H + 2047) / 2048), 256, 0, s>>>(dxr, p2r, da, ids, (const uint16_t*)w_router,
                                                             shared ? 1 : 0, dx, T, H, k);
    return hipGetLastError();
}

hipError_t launch_bwd_router_wgrad(const float* da, const int32_t* offsets, const int32_t* r2p, const void* x,
                                   float* dwg, int E, int H, int k, hipStream_t s) {
    bwd_router_wgrad_kernel<<<dim3(E, (H + 2047) / 2048), 256, 0, s>>>(da, offsets, r2p, (const uint16_t*)x, dwg,
                                                                       H, k);
    return hipGetLastError();
}

hipError_t launch_gather_rows(const void* x, const int32_t* r2p, bool shared, void* out, int T, int H, int k,
                              hipStream_t s) {
    const int64_t P = (int64_t)T * k;
    const int64_t rows = P + (shared ? T : 0);
    if (rows <= 0) return hipSuccess;
    gather_rows_kernel<<<(unsigned)rows, 256, 0, s>>>((const uint16_t*)x, r2p, (uint16_t*)out, P, H, k);
    return hipGetLastError();
}

hipError_t launch_zero_u32(void* p, int64_t words, hipStream_t s) {
    if (words <= 0) return hipSuccess;
    const int64_t need = (words + 255) / 256;
    zero_u32_kernel<<<(unsigned)(need < 1024 ? need : 1024), 256, 0, s>>>((uint32_t*)p, words);
    return hipGetLastError();
}

}  // namespace moe
