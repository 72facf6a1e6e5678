// combine.hip -- weighted un-permute of the routed experts' rows plus the
// shared expert (page "MAX 中 Step-3.5-Flash 架构解析…", section
// "MoE：共享专家、sigmoid 路由与激活裁剪": the layer output is the routed
// mixture plus the shared expert's output):
//   out[t, :] = sum_j w[t, j] * y_rows[pair_to_row[t*k + j], :] + y_shared[t, :]
// fp32 accumulation, in slot order j = 0..k-1, so results are deterministic.
// With a residual (the block's fp32 residual stream, AutoModel page benchmark
// table) the layer output is added to it last: out = resid + (the sum above);
// out may be the residual buffer itself (each thread reads its 8 values
// before it writes them).
// The expert rows are scaled fp16 rows (fp16 values and one power-of-two
// exponent per 128 columns).  The shared expert's output comes as fp32 rows
// (y_shared) or, when it ran inside the grouped expert launches, as rows of
// the same scaled format (shared_rows).
// One block of 256 threads per (token, 2048-column slice); each thread moves
// 8 contiguous columns (16-byte loads of each of the k rows, one exponent byte).
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void combine_kernel(const char* __restrict__ y_rows,
                                                      const int32_t* __restrict__ pair_to_row,
                                                      const float* __restrict__ topk_w,
                                                      const float* __restrict__ y_shared,
                                                      const char* __restrict__ shared_rows,
                                                      const float* resid, void* out, int H, int k) {
    typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
    const int t = blockIdx.x;
    const int col = (blockIdx.y * 256 + threadIdx.x) * 8;
    if (col >= H) return;
    const int64_t rb = yrow_bytes(H);
    const int eoff = 2 * H + (col >> 7);            // this thread's exponent byte in a row
    float acc[8];
    if (y_shared) {
        const float4* ys = (const float4*)(y_shared + (int64_t)t * H + col);
        float4 a = ys[0], b = ys[1];
        acc[0] = a.x; acc[1] = a.y; acc[2] = a.z; acc[3] = a.w;
        acc[4] = b.x; acc[5] = b.y; acc[6] = b.z; acc[7] = b.w;
    } else if (shared_rows) {
        const char* row = shared_rows + (int64_t)t * rb;
        const f16x8 v = *(const f16x8*)(row + 2 * col);
        const float sc = exp2_int((signed char)row[eoff]);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = (float)v[i] * sc;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    }
    // all k rows in flight at once: indices and weights first, then the
    // rows (8 at a time), then the sums in slot order; a row's power-of-two
    // scale is exact, so it goes into the value before the weight
    const int32_t* pr = pair_to_row + (int64_t)t * k;
    const float* pw = topk_w + (int64_t)t * k;
    for (int j0 = 0; j0 < k; j0 += 8) {
        const int nj = min(8, k - j0);
        f16x8 v[8];
        float wj[8], sj[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (j < nj) {
                const char* row = y_rows + (int64_t)pr[j0 + j] * rb;
                v[j] = *(const f16x8*)(row + 2 * col);
                sj[j] = exp2_int((signed char)row[eoff]);
                wj[j] = pw[j0 + j];
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (j < nj) {
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] += wj[j] * ((float)v[j][i] * sj[j]);
            }
    }
    if (resid) {
        const float4* rs = (const float4*)(resid + (int64_t)t * H + col);
        const float4 a = rs[0], b = rs[1];
        acc[0] = a.x + acc[0]; acc[1] = a.y + acc[1]; acc[2] = a.z + acc[2]; acc[3] = a.w + acc[3];
        acc[4] = b.x + acc[4]; acc[5] = b.y + acc[5]; acc[6] = b.z + acc[6]; acc[7] = b.w + acc[7];
    }
    if (OUT_BF16) {
        uint4 o;
        o.x = pack_bf16x2(acc[0], acc[1]);
        o.y = pack_bf16x2(acc[2], acc[3]);
        o.z = pack_bf16x2(acc[4], acc[5]);
        o.w = pack_bf16x2(acc[6], acc[7]);
        *(uint4*)((uint16_t*)out + (int64_t)t * H + col) = o;
    } else {
        float4* o = (float4*)((float*)out + (int64_t)t * H + col);
        o[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        o[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
}

hipError_t launch_combine(const void* y_rows, const int32_t* pair_to_row, const float* topk_w,
                          const float* y_shared, const void* shared_rows, const float* resid, void* out,
                          bool out_bf16, int T, int H, int k, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    dim3 grid(T, (H + 2047) / 2048);
    if (out_bf16)
        combine_kernel<true><<<grid, 256, 0, s>>>((const char*)y_rows, pair_to_row, topk_w, y_shared,
                                                  (const char*)shared_rows, resid, out, H, k);
    else
        combine_kernel<false><<<grid, 256, 0, s>>>((const char*)y_rows, pair_to_row, topk_w, y_shared,
                                                   (const char*)shared_rows, resid, out, H, k);
    return hipGetLastError();
}

}  // namespace moe
