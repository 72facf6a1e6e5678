// router.hip -- router logits on gfx950:  logits[T, E] = x[T, H] . W_g[E, H]^T
// in fp32 from bf16 operands (the gate is computed in FP32: page "MAX 中
// Step-3.5-Flash 架构解析…", section "MoE：共享专家、sigmoid 路由与激活裁剪").
//
// A small GEMM (2*T*E*H flops, about 1% of the layer), so it uses no LDS: each
// wave owns a (16*TM tokens) x (16*TN experts) tile and feeds
// v_mfma_f32_16x16x32_bf16 straight from global memory (x rows and router
// rows stay in L2), with the next K slice's loads issued before the current
// slice's MFMAs.  Few registers per wave, so many waves per SIMD hide the
// load latency.  K order inside a 32-wide slice: lane group g = lane >> 4
// takes 8-element chunk g, for both operands.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

template <int TM, int TN>
__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ wg,
                                                            float* __restrict__ logits, int T, int E, int H) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t0 = blockIdx.x * 16 * TM;
    const int e0 = (blockIdx.y * 4 + wave) * 16 * TN;
    if (e0 >= E) return;                          // no barriers: a wave may leave alone
    const int r = lane & 15, kc = (lane >> 4) * 8;
    const uint16_t* ap[TM];
    const uint16_t* bp[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) ap[i] = x + (int64_t)min(t0 + 16 * i + r, T - 1) * H + kc;
#pragma unroll
    for (int j = 0; j < TN; ++j) bp[j] = wg + (int64_t)min(e0 + 16 * j + r, E - 1) * H + kc;

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    bf16x8 a[TM], b[TN], an[TM], bn[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) a[i] = *(const bf16x8*)(ap[i]);
#pragma unroll
    for (int j = 0; j < TN; ++j) b[j] = *(const bf16x8*)(bp[j]);
    for (int k0 = 32; k0 <= H; k0 += 32) {
        const int kn = min(k0, H - 32);           // the last step re-reads its own slice
#pragma unroll
        for (int i = 0; i < TM; ++i) an[i] = *(const bf16x8*)(ap[i] + kn);
#pragma unroll
        for (int j = 0; j < TN; ++j) bn[j] = *(const bf16x8*)(bp[j] + kn);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < TM; ++i) a[i] = an[i];
#pragma unroll
        for (int j = 0; j < TN; ++j) b[j] = bn[j];
    }
    // lane holds expert column (lane & 15), token rows 4*(lane >> 4) + v
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int e = e0 + 16 * j + (lane & 15);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int t = t0 + 16 * i + 4 * (lane >> 4) + v;
                if (t < T && e < E) logits[(int64_t)t * E + e] = acc[i][j][v];
            }
        }
}

hipError_t launch_router_logits(const void* x, const void* w_router, float* logits, int T, int E, int H,
                                hipStream_t s) {
    if (T <= 0) return hipSuccess;
    const uint16_t* xp = (const uint16_t*)x;
    const uint16_t* wp = (const uint16_t*)w_router;
    if (T >= 1024) {
        dim3 grid((T + 31) / 32, (E + 255) / 256);        // wave: 32 tokens x 64 experts
        router_logits_kernel<2, 4><<<grid, 256, 0, s>>>(xp, wp, logits, T, E, H);
    } else {
        dim3 grid((T + 15) / 16, (E + 63) / 64);          // wave: 16 tokens x 16 experts
        router_logits_kernel<1, 1><<<grid, 256, 0, s>>>(xp, wp, logits, T, E, H);
    }
    return hipGetLastError();
}

}  // namespace moe
