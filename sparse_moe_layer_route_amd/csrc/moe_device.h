// moe_device.h -- device-side helpers shared by the gfx950 kernels of the
// MoE-layer forward (bf16 packing, MFMA fragment types, wave reductions).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t v) {
    return __uint_as_float(((uint32_t)v) << 16);
}

// round-to-nearest-even fp32 -> bf16 (NaN stays NaN)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// fp32 -> fp16, round to nearest even, finite values beyond the fp16 range
// saturate to +-65504 (NaN stays NaN)
__device__ __forceinline__ _Float16 f32_to_f16_sat(float f) {
    const float m = 65504.0f;
    float c = f > m ? m : (f < -m ? -m : f);
    return (_Float16)c;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

// Clipped SwiGLU: silu(g) * u without a limit; with limit L > 0 both factors
// are clipped, silu(g) from above at L and u to [-L, L].
__device__ __forceinline__ float swiglu_clip(float g, float u, float L) {
    float sg = silu(g);
    if (L > 0.0f) {
        sg = fminf(sg, L);
        u = fminf(fmaxf(u, -L), L);
    }
    return sg * u;
}

// Derivatives of swiglu_clip with respect to g and u.  Each clamp passes the
// gradient where its input lies in its range, ends included, else none.
__device__ __forceinline__ void swiglu_clip_grad(float g, float u, float L, float& dg, float& du) {
    const float sg = 1.0f / (1.0f + __expf(-g));
    const float sl = g * sg;
    const float dsl = sg * (1.0f + g * (1.0f - sg));
    if (L > 0.0f) {
        const float uc = fminf(fmaxf(u, -L), L);
        dg = sl <= L ? uc * dsl : 0.0f;
        du = (u >= -L && u <= L) ? fminf(sl, L) : 0.0f;
    } else {
        dg = u * dsl;
        du = sl;
    }
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// Wave-wide max / min of a 32-bit unsigned value through DPP lane moves
// (VALU only): quad permutes, row rotates, then row broadcasts 15 and 31
// carry the result into lane 63, which is read back to every lane.
__device__ __forceinline__ uint32_t dpp_max(uint32_t v, uint32_t d) { return v > d ? v : d; }
__device__ __forceinline__ uint32_t dpp_min(uint32_t v, uint32_t d) { return v < d ? v : d; }

#define MOE_DPP_REDUCE(OP, ID)                                                                        \
    v = OP(v, (uint32_t)__builtin_amdgcn_update_dpp((int)(ID), (int)v, 0xB1, 0xF, 0xF, false));     \
    v = OP(v, (uint32_t)__builtin_amdgcn_update_dpp((int)(ID), (int)v, 0x4E, 0xF, 0xF, false));     \
    v = OP(v, (uint32_t)__builtin_amdgcn_update_dpp((int)(ID), (int)v, 0x124, 0xF, 0xF, false));    \
    v = OP(v, (uint32_t)__builtin_amdgcn_update_dpp((int)(ID), (int)v, 0x128, 0xF, 0xF, false));    \
    v = OP(v, (uint32_t)__builtin_amdgcn_update_dpp((int)(ID), (int)v, 0x142, 0xA, 0xF, false));    \
    v = OP(v, (uint32_t)__builtin_amdgcn_update_dpp((int)(ID), (int)v, 0x143, 0xC, 0xF, false));    \
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) { MOE_DPP_REDUCE(dpp_max, 0u) }
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) { MOE_DPP_REDUCE(dpp_min, 0xFFFFFFFFu) }
#undef MOE_DPP_REDUCE

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        uint64_t w = __shfl_xor(v, o, kWave);
        v = w > v ? w : v;
    }
    return v;
}

}  // namespace moe
