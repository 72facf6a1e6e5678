// route.hip -- the router's selection step on gfx950: one wavefront per token.
//
// From the fp32 router logits (page "MAX 中 Step-3.5-Flash 架构解析…", section
// "MoE：共享专家、sigmoid 路由与激活裁剪", Step3p5MoEGate paragraph):
//   s = sigmoid(logit), c = s + bias            (fp32)
//   ids = the k largest c, descending, ties to the lower index, NaN last
//   w_j = s[ids_j]; if norm: w_j /= sum_j w_j; w_j *= scale
//
// Each lane holds up to 16 of the E <= 1024 scores in registers.  The order
// is encoded in one 64-bit key per expert: the high word is the fp32 bit
// pattern of c mapped to an unsigned order (negative values flipped, -0
// folded into +0, NaN mapped to 0 so it ranks below every number), the low
// word is ~index so that equal scores prefer the lower index.  Each of the k
// rounds is a lane-local max followed by a 6-step xor-shuffle max across
// the wave; the winner's owner lane retires it (key 0, below every live key).
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int TOPK_MAX_PER_LANE = 16;   // E <= 1024

__device__ __forceinline__ uint64_t order_key(float c, int e) {
    uint32_t hi;
    if (c != c) {
        hi = 0u;                                   // NaN: lowest of all numbers
    } else {
        uint32_t u = __float_as_uint(c == 0.0f ? 0.0f : c);
        hi = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    }
    return ((uint64_t)hi << 32) | (uint64_t)(~(uint32_t)e);
}

__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits,
                                                   const float* __restrict__ bias, int T, int E, int k,
                                                   float scale, int norm, int32_t* __restrict__ ids,
                                                   float* __restrict__ wout) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;                            // whole wave leaves together
    const float* lg = logits + (int64_t)t * E;

    uint64_t key[TOPK_MAX_PER_LANE];
    float sc[TOPK_MAX_PER_LANE];
#pragma unroll
    for (int i = 0; i < TOPK_MAX_PER_LANE; ++i) {
        int e = lane + 64 * i;
        key[i] = 0;
        sc[i] = 0.f;
        if (e < E) {
            float a = lg[e];
            float s = 1.0f / (1.0f + expf(-a));
            sc[i] = s;
            key[i] = order_key(s + bias[e], e);
        }
    }

    float my_w = 0.f;   // lane j < k keeps the raw score of the j-th choice
    for (int j = 0; j < k; ++j) {
        uint64_t best = 0;
        float best_s = 0.f;
#pragma unroll
        for (int i = 0; i < TOPK_MAX_PER_LANE; ++i)
            if (key[i] > best) { best = key[i]; best_s = sc[i]; }
        uint64_t win = wave_max_u64(best);
        int e = (int)(~(uint32_t)(win & 0xffffffffu));
        e = min(max(e, 0), E - 1);                 // index guard
        int owner = e & 63;
        float s_win = __shfl(best_s, owner, kWave);
        if (lane == owner) {
#pragma unroll
            for (int i = 0; i < TOPK_MAX_PER_LANE; ++i)
                if (lane + 64 * i == e) key[i] = 0;
        }
        if (lane == j) my_w = s_win;
        if (lane == 0) ids[(int64_t)t * k + j] = e;
    }
    float sum = wave_sum(lane < k ? my_w : 0.f);
    float w = norm ? my_w / sum : my_w;
    if (lane < k) wout[(int64_t)t * k + lane] = w * scale;
}

hipError_t launch_topk(const float* logits, const float* bias, int T, int E, int k, float scale, int norm,
                       int32_t* ids, float* w, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    topk_kernel<<<(T + 3) / 4, 256, 0, s>>>(logits, bias, T, E, k, scale, norm, ids, w);
    return hipGetLastError();
}

}  // namespace moe
