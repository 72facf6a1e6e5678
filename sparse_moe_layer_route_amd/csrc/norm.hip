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

// ---- the RMSNorm fused with the router logits ------------------------------
// One block of 8 waves per 32 tokens.  First each wave takes the mean square
// of four rows exactly as rmsnorm_regs_kernel<16> does (the same loads and
// sums: the same scale bits).  Then, 256 columns at a time, the block
// normalises the 32 rows' chunk (the same fp32 products and rounding as the
// separate pass, so x gets the same bf16 bits), writes it to x and to LDS,
// and multiplies it into the logits of all experts with
// v_mfma_f32_16x16x32_bf16: wave w owns the 16-expert tiles w, w + 8, ...
// for both 16-token tiles.  Router rows come straight from global memory
// (L2), loaded at the start of each chunk so they land while the chunk is
// normalised.  The MFMA operands, their lanes' K chunks and the order of the
// K slices (chunks from router_chunk_rot(64-token tile), slices in order
// inside) are those of the dense 64 x 128 GEMM instance the router uses from
// 512 tokens, so the logits are the same fp32 bits too.  The residual rows
// are read twice (once for the scale, once per chunk); x is written once and
// never read back.  H <= 4096, H % 256 == 0, E <= 384.
constexpr int RN_TOK = 32;
constexpr int RN_CHUNK = 256;
constexpr int RN_PITCH = RN_CHUNK + 8;      // bf16 per LDS row: 16 bytes of padding spread the fragment reads
constexpr int RN_MAX_TILES = 3;             // expert tiles per wave: E <= 384

__global__ __launch_bounds__(512) void rmsnorm_router_kernel(const float* __restrict__ r, const float* __restrict__ g,
                                                             float eps, const uint16_t* __restrict__ wr,
                                                             uint16_t* __restrict__ x, float* __restrict__ logits,
                                                             int T, int E, int H) {
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][RN_TOK * RN_PITCH];
    __shared__ float inv_s[RN_TOK];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t0 = blockIdx.x * RN_TOK;
    const int n4 = H / 4;
    // ---- the rows' scales: wave w takes rows 4 w .. 4 w + 3
    for (int rr = 0; rr < 4; ++rr) {
        const int lr = 4 * wave + rr, t = t0 + lr;
        float inv = 0.f;
        if (t < T) {
            const float4* row = (const float4*)(r + (int64_t)t * H);
            float4 v[16];
#pragma unroll
            for (int j = 0; j < 16; ++j)
                if (lane + 64 * j < n4) v[j] = row[lane + 64 * j];
            float ss = 0.f;
#pragma unroll
            for (int j = 0; j < 16; ++j)
                if (lane + 64 * j < n4) ss += v[j].x * v[j].x + v[j].y * v[j].y + v[j].z * v[j].z + v[j].w * v[j].w;
            ss = wave_sum(ss);
            inv = 1.0f / sqrtf(ss / (float)H + eps);
        }
        if (lane == 0) inv_s[lr] = inv;
    }
    // ---- chunks: normalise, then multiply
    const int nc = H / RN_CHUNK;
    const int rc = router_chunk_rot(t0 / 64, nc);
    const int fr = lane & 15, fc = 8 * (lane >> 4);
    const int ntw = (E / 16 + (E % 16 ? 1 : 0) - wave + 7) / 8;   // expert tiles of this wave
    f32x4 acc[RN_MAX_TILES][2];
#pragma unroll
    for (int j = 0; j < RN_MAX_TILES; ++j) acc[j][0] = acc[j][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    // normalisation work of a thread: row nr, float4 columns i4 + 16 q of the chunk (q < 4)
    const int nr = threadIdx.x >> 4, i4 = threadIdx.x & 15;
    const float4* g4 = (const float4*)g;
    __syncthreads();                                                 // inv_s
    const float inv_row = inv_s[nr];
    const bool row_ok = t0 + nr < T;
    const float* rrow = r + (int64_t)min(t0 + nr, T - 1) * H;
    auto chunk_of = [&](int c) { return (rc + c < nc ? rc + c : rc + c - nc) * RN_CHUNK; };
    // residual values of the next chunk in registers, router fragments half a
    // chunk (4 slices) ahead: loads are in flight while the current ones are used
    float4 rv[RN_CHUNK / 64];
    auto load_r = [&](int k0) {
#pragma unroll
        for (int q = 0; q < RN_CHUNK / 64; ++q) rv[q] = ((const float4*)(rrow + k0))[i4 + 16 * q];
    };
    bf16x8 bA[RN_MAX_TILES][4], bB[RN_MAX_TILES][4];
    auto load_w = [&](int k0, bf16x8 (*bb)[4]) {
#pragma unroll
        for (int j = 0; j < RN_MAX_TILES; ++j) {
            if (j < ntw) {
                const int e = min(16 * (wave + 8 * j) + fr, E - 1);
                const uint16_t* wrow = wr + (int64_t)e * H + k0 + fc;
#pragma unroll
                for (int q = 0; q < 4; ++q) bb[j][q] = *(const bf16x8*)(wrow + 32 * q);
            }
        }
    };
    auto mul = [&](const uint16_t* xa, const bf16x8 (*bb)[4]) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const bf16x8 a0 = *(const bf16x8*)(xa + 32 * q);
            const bf16x8 a1 = *(const bf16x8*)(xa + 16 * RN_PITCH + 32 * q);
#pragma unroll
            for (int j = 0; j < RN_MAX_TILES; ++j) {
                if (j < ntw) {
                    acc[j][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bb[j][q], acc[j][0], 0, 0, 0);
                    acc[j][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bb[j][q], acc[j][1], 0, 0, 0);
                }
            }
        }
    };
    load_r(chunk_of(0));
    load_w(chunk_of(0), bA);
    for (int c = 0; c < nc; ++c) {
        const int k0 = chunk_of(c);
        // normalise the chunk into LDS buffer c & 1 (and x)
        uint2* xl = (uint2*)(xs[c & 1] + nr * RN_PITCH);
        uint2* out = (uint2*)(x + (int64_t)(t0 + nr) * H + k0);
        const float4* gc = g4 + (k0 >> 2);
#pragma unroll
        for (int q = 0; q < RN_CHUNK / 64; ++q) {
            const int f = i4 + 16 * q;
            uint2 o = make_uint2(0u, 0u);
            if (row_ok) {
                const float4 v = rv[q];
                const float4 w = gc[f];
                o.x = pack_bf16x2(v.x * inv_row * (1.0f + w.x), v.y * inv_row * (1.0f + w.y));
                o.y = pack_bf16x2(v.z * inv_row * (1.0f + w.z), v.w * inv_row * (1.0f + w.w));
                out[f] = o;
            }
            xl[f] = o;
        }
        if (c + 1 < nc) load_r(chunk_of(c + 1));
        __syncthreads();            // the chunk is in LDS (the other buffer was last read a chunk ago)
        const uint16_t* xa = xs[c & 1] + fr * RN_PITCH + fc;
        load_w(k0 + 128, bB);
        mul(xa, bA);
        if (c + 1 < nc) load_w(chunk_of(c + 1), bA);
        mul(xa + 128, bB);
    }
    // lane holds tokens 16 i + 4 (lane >> 4) + v of expert 16 (wave + 8 j) + (lane & 15)
#pragma unroll
    for (int j = 0; j < RN_MAX_TILES; ++j) {
        if (j >= ntw) continue;
        const int e = 16 * (wave + 8 * j) + fr;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int t = t0 + 16 * i + 4 * (lane >> 4) + v;
                if (t < T && e < E) logits[(int64_t)t * E + e] = acc[j][i][v];
            }
    }
}

bool rmsnorm_router_fusable(int64_t T, int H, int E) {
    return T >= 512 && H <= 4096 && H % RN_CHUNK == 0 && E <= 16 * 8 * RN_MAX_TILES;
}

hipError_t launch_rmsnorm_router(const float* resid, const float* norm_weight, float eps, const void* w_router,
                                 void* x, float* logits, int T, int E, int H, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    if (!rmsnorm_router_fusable(T, H, E)) return hipErrorInvalidValue;
    rmsnorm_router_kernel<<<(unsigned)((T + RN_TOK - 1) / RN_TOK), 512, 0, s>>>(
        resid, norm_weight, eps, (const uint16_t*)w_router, (uint16_t*)x, logits, T, E, H);
    return hipGetLastError();
}

}  // namespace moe
