// route.hip -- the router's selection step on gfx950: one wavefront per token.
//
// From the fp32 router logits (page "MAX 中 Step-3.5-Flash 架构解析…", section
// "MoE：共享专家、sigmoid 路由与激活裁剪", Step3p5MoEGate paragraph), given
// as nsplit partial sums over K that are added in split order:
//   s = sigmoid(logit), c = s + bias            (fp32)
//   ids = the k largest c, descending, ties to the lower index, NaN last
//   w_j = s[ids_j]; if norm: w_j /= sum_j w_j; w_j *= scale
//
// Each lane holds up to 16 of the E <= 1024 scores in registers as 32-bit
// order keys: the fp32 bit pattern of c mapped to an unsigned order
// (negative values flipped, -0 folded into +0); NaN gets key 1, below every
// number, and a retired expert key 0.  Each of the k rounds takes a
// lane-local maximum (lowest index first among equal keys), a wave maximum
// of the keys and then a wave minimum of the indices holding that key (the
// lower-index tie-break), both as DPP reductions; the owner lane retires the
// winner.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int TOPK_MAX_PER_LANE = 16;   // E <= 1024

__device__ __forceinline__ uint32_t order_key(float c) {
    if (c != c) return 1u;                                   // NaN: below every number
    uint32_t u = __float_as_uint(c == 0.0f ? 0.0f : c);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);      // >= 0x007fffff for numbers
}

// BATCH: splits loaded at once (1 when the logits come whole); NPL: scores
// per lane (E <= 64 * NPL), so the lane-local scans cover only real experts
template <int BATCH, int NPL>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int nsplit,
                                                   const float* __restrict__ bias, int T, int E, int k,
                                                   float scale, int norm, int32_t* __restrict__ ids,
                                                   float* __restrict__ wout, float* __restrict__ s_out) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;                            // whole wave leaves together
    const float* lg = logits + (int64_t)t * E;

    uint32_t key[NPL];
    float sc[NPL];
    float a[NPL];
    // partial logits, added in split order.  They were just written by other
    // XCDs, so every read misses this XCD's L2: BATCH splits are loaded at
    // once, then added, so the latency is paid once per BATCH splits.
#pragma unroll
    for (int i = 0; i < NPL; ++i) a[i] = 0.f;
    for (int z0 = 0; z0 < nsplit; z0 += BATCH) {
        float part[BATCH][NPL];
#pragma unroll
        for (int z = 0; z < BATCH; ++z)
#pragma unroll
            for (int i = 0; i < NPL; ++i)
                part[z][i] = (z0 + z < nsplit && lane + 64 * i < E)
                                 ? lg[(int64_t)(z0 + z) * T * E + lane + 64 * i] : 0.f;
#pragma unroll
        for (int z = 0; z < BATCH; ++z)
#pragma unroll
            for (int i = 0; i < NPL; ++i)
                if (z0 + z < nsplit) a[i] += part[z][i];
    }
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int e = lane + 64 * i;
        key[i] = 0u;
        sc[i] = 0.f;
        if (e < E) {
            const float s = 1.0f / (1.0f + expf(-a[i]));
            sc[i] = s;
            key[i] = order_key(s + bias[e]);
        }
    }

    float my_w = 0.f;   // lane j < k keeps the raw score of the j-th choice
    for (int j = 0; j < k; ++j) {
        uint32_t bk = 0u;
        int bi = 0;
        float bs = 0.f;
#pragma unroll
        for (int i = 0; i < NPL; ++i)
            if (key[i] > bk) { bk = key[i]; bi = i; bs = sc[i]; }
        const uint32_t wmax = wave_max_u32(bk);
        const uint32_t cand = (bk == wmax) ? (uint32_t)(lane + 64 * bi) : 0xFFFFFFFFu;
        int e = (int)wave_min_u32(cand);
        e = min(max(e, 0), E - 1);                 // index guard
        const int owner = e & 63;
        const float s_win = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(bs), owner));
        if (lane == owner) {
#pragma unroll
            for (int i = 0; i < NPL; ++i)
                if (64 * i + lane == e) key[i] = 0u;
        }
        if (lane == j) my_w = s_win;
        if (lane == 0) ids[(int64_t)t * k + j] = e;
    }
    const float sum = wave_sum(lane < k ? my_w : 0.f);
    const float w = norm ? my_w / sum : my_w;
    if (lane < k) wout[(int64_t)t * k + lane] = w * scale;
    if (s_out && lane < k) s_out[(int64_t)t * k + lane] = my_w;
}

// Routing replay (miles page "Step-5-Preview", section 5.2 Algorithm: the
// trainer reruns the rollout's expert choices).  The k ids of each token
// come from the caller, clamped to [0, E-1] as the selection's own guard
// does; only the weights are computed, from the current raw scores, with the
// same arithmetic as topk_kernel (partial logits added in split order,
// s = 1/(1+exp(-a)), a wave sum over the k slots), so replaying the router's
// own choice gives back its weights bit for bit.  One wavefront per token;
// lane j < k owns slot j.
__global__ __launch_bounds__(256) void replay_kernel(const float* __restrict__ logits, int nsplit,
                                                     const int32_t* __restrict__ ids_in, int T, int E, int k,
                                                     float scale, int norm, float* __restrict__ wout,
                                                     int32_t* __restrict__ ids_out, float* __restrict__ s_out) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    float s = 0.f;
    if (lane < k) {
        const int e = min(max(ids_in[(int64_t)t * k + lane], 0), E - 1);
        if (ids_out) ids_out[(int64_t)t * k + lane] = e;
        const float* lg = logits + (int64_t)t * E + e;
        float part[8];
        float a = 0.f;
        for (int z0 = 0; z0 < nsplit; z0 += 8) {
#pragma unroll
            for (int z = 0; z < 8; ++z) part[z] = z0 + z < nsplit ? lg[(int64_t)(z0 + z) * T * E] : 0.f;
#pragma unroll
            for (int z = 0; z < 8; ++z)
                if (z0 + z < nsplit) a += part[z];
        }
        s = 1.0f / (1.0f + expf(-a));
    }
    const float sum = wave_sum(lane < k ? s : 0.f);
    const float w = norm ? s / sum : s;
    if (lane < k) wout[(int64_t)t * k + lane] = w * scale;
    if (s_out && lane < k) s_out[(int64_t)t * k + lane] = s;
}

// Static balanced routing (AutoModel page, benchmark table): pair
// p = t*k + j goes to expert p mod E, so every expert gets floor(T*k/E) or
// one more pair and a token's k experts are distinct (k <= E).
__global__ __launch_bounds__(256) void balanced_ids_kernel(int32_t* __restrict__ ids, int64_t P, int E) {
    for (int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x; p < P; p += (int64_t)gridDim.x * 256)
        ids[p] = (int32_t)(p % E);
}

hipError_t launch_replay_weights(const float* logits, int nsplit, const int32_t* ids, int T, int E, int k,
                                 float scale, int norm, float* w, hipStream_t s, int32_t* ids_out, float* s_out) {
    if (T <= 0) return hipSuccess;
    replay_kernel<<<(T + 3) / 4, 256, 0, s>>>(logits, nsplit, ids, T, E, k, scale, norm, w, ids_out, s_out);
    return hipGetLastError();
}

hipError_t launch_balanced_ids(int32_t* ids, int64_t P, int E, hipStream_t s) {
    if (P <= 0) return hipSuccess;
    const int64_t need = (P + 255) / 256;
    const int64_t blocks = need < 2048 ? need : 2048;
    balanced_ids_kernel<<<(unsigned)blocks, 256, 0, s>>>(ids, P, E);
    return hipGetLastError();
}

template <int BATCH, int NPL>
static void launch_topk_n(const float* logits, int nsplit, const float* bias, int T, int E, int k, float scale,
                          int norm, int32_t* ids, float* w, hipStream_t s, float* s_out) {
    topk_kernel<BATCH, NPL><<<(T + 3) / 4, 256, 0, s>>>(logits, nsplit, bias, T, E, k, scale, norm, ids, w, s_out);
}

template <int BATCH>
static void launch_topk_b(const float* logits, int nsplit, const float* bias, int T, int E, int k, float scale,
                          int norm, int32_t* ids, float* w, hipStream_t s, float* s_out) {
    if (E <= 128) launch_topk_n<BATCH, 2>(logits, nsplit, bias, T, E, k, scale, norm, ids, w, s, s_out);
    else if (E <= 256) launch_topk_n<BATCH, 4>(logits, nsplit, bias, T, E, k, scale, norm, ids, w, s, s_out);
    else if (E <= 384) launch_topk_n<BATCH, 6>(logits, nsplit, bias, T, E, k, scale, norm, ids, w, s, s_out);
    else if (E <= 512) launch_topk_n<BATCH, 8>(logits, nsplit, bias, T, E, k, scale, norm, ids, w, s, s_out);
    else launch_topk_n<BATCH, TOPK_MAX_PER_LANE>(logits, nsplit, bias, T, E, k, scale, norm, ids, w, s, s_out);
}

hipError_t launch_topk(const float* logits, int nsplit, const float* bias, int T, int E, int k, float scale,
                       int norm, int32_t* ids, float* w, hipStream_t s, float* s_out) {
    if (T <= 0) return hipSuccess;
    if (nsplit > 1)
        launch_topk_b<8>(logits, nsplit, bias, T, E, k, scale, norm, ids, w, s, s_out);
    else
        launch_topk_b<1>(logits, nsplit, bias, T, E, k, scale, norm, ids, w, s, s_out);
    return hipGetLastError();
}

}  // namespace moe
