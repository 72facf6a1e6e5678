// router.hip -- router logits on gfx950:  logits[T, E] = x[T, H] . W_g[E, H]^T
// in fp32 from bf16 operands (the gate is computed in FP32: page "MAX 中
// Step-3.5-Flash 架构解析…", section "MoE：共享专家、sigmoid 路由与激活裁剪").
//
// A small GEMM (2*T*E*H flops, about 1% of the layer).  From 512 tokens it
// runs on the dense instance of the grouped expert GEMM (64-token tiles,
// direct-to-LDS DMA, fp32 out).  Below that, few tokens leave too little
// work per wave for that kernel, and router_logits_kernel below is used: no
// LDS, each wave owns a 16-token x 16-expert tile and feeds
// v_mfma_f32_16x16x32_bf16 straight from global memory (x rows and router
// rows stay in L2), with the loads of up to 16 K slices issued before their
// MFMAs; K is split over `nsplit` blocks (blockIdx.z) that write
// partial logits [nsplit][T][E], summed in split order by the top-k kernel,
// so the dependent chain per wave is short.  K order inside a 32-wide slice:
// lane group g = lane >> 4 takes 8-element chunk g, for both operands.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

template <int TM, int TN>
__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ wg,
                                                            float* __restrict__ logits, int T, int E, int H) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // this block's K range: [kz * H/nsplit, (kz + 1) * H/nsplit)
    const int hk = H / gridDim.z, kz = blockIdx.z;
    x += (int64_t)kz * hk;
    wg += (int64_t)kz * hk;
    logits += (int64_t)kz * T * E;
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

    // all loads of up to CH slices are issued before their MFMAs, so a wave
    // waits for memory once per CH slices (once in all when H/nsplit <= 512)
    constexpr int CH = 16;
    for (int k0 = 0; k0 < hk; k0 += 32 * CH) {
        bf16x8 a[CH][TM], b[CH][TN];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int kk = min(k0 + 32 * c, hk - 32);   // past the end: a re-read, not multiplied
#pragma unroll
            for (int i = 0; i < TM; ++i) a[c][i] = *(const bf16x8*)(ap[i] + kk);
#pragma unroll
            for (int j = 0; j < TN; ++j) b[c][j] = *(const bf16x8*)(bp[j] + kk);
        }
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            if (k0 + 32 * c < hk) {
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[c][i], b[c][j], acc[i][j], 0, 0, 0);
            }
        }
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

int router_splits(int64_t T, int H) {
    if (T >= 512) return 1;
    int n = 8;
    while (n > 1 && H % (32 * n)) n >>= 1;
    return n;
}

hipError_t launch_router_logits(const void* x, const void* w_router, float* logits, int T, int E, int H,
                                hipStream_t s) {
    if (T <= 0) return hipSuccess;
    const int nsplit = router_splits(T, H);
    if (nsplit == 1 && T >= 512) {
        GroupedArgs a;
        a.A = x;
        a.a_nrows = T;
        a.W = w_router;
        a.C = logits;
        a.M = T;
        a.N = E;
        a.K = H;
        a.bm = 64;
        a.rot_group = -2;           // the K order the fused RMSNorm + router pass repeats
        return launch_grouped_down(a, true, s);
    }
    dim3 grid((T + 15) / 16, (E + 63) / 64, nsplit);   // wave: 16 tokens x 16 experts x H/nsplit
    router_logits_kernel<1, 1><<<grid, 256, 0, s>>>((const uint16_t*)x, (const uint16_t*)w_router, logits, T, E,
                                                    H);
    return hipGetLastError();
}

}  // namespace moe
