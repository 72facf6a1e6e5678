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

// ---- expert output rows: fp16 values with a power-of-two scale per 128 columns ----
// A row of H values is H fp16 numbers, then one int8 exponent e per 128
// columns (then zeros to a multiple of 16 bytes); value = fp16 * 2^e.  e
// scales the group's largest magnitude into [2^14, 2^15) (rounding to fp16
// may carry it to 2^15), so no finite value overflows and every
// value keeps fp16's 11 significant bits relative to its group's largest
// (scaling by a power of two commutes with the rounding, so where plain
// fp16 neither overflows nor underflows the stored value is the same).
__host__ __device__ __forceinline__ int64_t yrow_bytes(int H) { return 2 * (int64_t)H + ((H + 127) / 128 + 15) / 16 * 16; }
// exponent for a group whose largest magnitude is amax (>= 0, NaN-free)
__device__ __forceinline__ int yrow_exp(float amax) {
    const int ex = (int)((__float_as_uint(amax) >> 23) & 0xffu) - 127;   // floor(log2 amax); -127 for 0 and subnormals
    return min(max(ex - 14, -126), 113);
}
// zero the padding after a row's exponents (called by the thread that writes
// the row's first exponent), so rows are fully defined bytes
__device__ __forceinline__ void yrow_zero_pad(char* row, int H) {
    for (int64_t b = 2 * (int64_t)H + (H + 127) / 128; b < yrow_bytes(H); ++b) row[b] = 0;
}
// 2^e for e in [-126, 127]
__device__ __forceinline__ float exp2_int(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

// 16-byte chunk swizzle of row r (r & 15) of a tile held as 128-byte LDS
// rows (one K slice per row, a DMA of whole lines): LDS chunk p holds global
// chunk p ^ line_swz(r).  Chosen by search so that the fragment reads (lane
// l: row l & 15, chunk (l >> 4) or 4 + (l >> 4)) hit distinct 16-byte bank
// groups under every LDS service order that fits the bank-conflict
// counter's readings on both this and the 64-row layout of the bf16 tiles
// (8 lanes per cycle over 256 bytes; lanes l, l+16, l+32, l+48 together over
// 128 or 256 bytes; 32 lanes over 512 bytes).  The simpler 2 ((r & 15) >> 2)
// is conflict-free only under the last and measured 2-way.
__device__ __forceinline__ int line_swz(int r) {
    return ((((r ^ (r >> 1) ^ (r >> 3)) & 1) << 2) | (((r >> 2) & 1) << 1));
}

// The router's K order from 512 tokens: the 64-token tile m adds its K
// chunks of 256 (8 slices of 32) starting at chunk router_chunk_rot(m, nc)
// of nc, wrapping around, slices in order inside a chunk.  Tiles start at
// different chunks (their rows' reads spread over the HBM channels); every
// expert column of a tile uses the same order, which the fused RMSNorm +
// router pass repeats chunk by chunk.
__host__ __device__ __forceinline__ int router_chunk_rot(int m, int nc) { return (m * 5 + 3) % nc; }

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

// max over lanes l, l ^ 16, l ^ 32, l ^ 48 (two lane-swap moves, VALU only)
__device__ __forceinline__ float max_lanes_xor16_32(float m) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
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
