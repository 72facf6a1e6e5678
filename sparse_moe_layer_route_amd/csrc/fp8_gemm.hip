// fp8_gemm.hip -- routed experts with FP8 E4M3 weights on gfx950.
//
// The routed expert weights are OCP E4M3FN codes with one fp32 scale per
// 128 x 128 block (miles page "Step-5-Preview", section 1 Model
// Introduction); a weight is code * scale.  The inputs of both projections
// (x, and h) are quantised per (row, 128 columns) to E4M3FN with scale
// amax / 448 (1 when amax is 0), so both projections run on FP8 MFMA:
//
//   out[r, n] = sum over 128-wide K blocks kb of
//               s_a[r, kb] * s_w[n / 128, kb] * sum_{k in kb} qa[r, k] * qw[n, k]
//
// One v_mfma_f32_16x16x128_f8f6f4 covers exactly one K block of a 16 x 16
// output tile, so each MFMA result is scaled and added to the fp32
// accumulator straight away.
//
// Layout and staging (the bf16 kernel's choices, with bytes for elements):
//   * x is quantised once per token (quant_rows_kernel); the first projection
//     gathers the code rows of its permuted rows (token = pair / k) as the
//     bf16 kernel gathers x; activation scales are stored K-block-major,
//     s_a[kb][row], and gathered per row into LDS by 4-byte DMA;
//   * block tile 128 rows x 256 weight rows, K slices of 128 bytes (one
//     scale block), 3-stage LDS ring filled by direct global->LDS DMA from
//     inline asm with explicit vmcnt waits (see grouped_gemm.hip);
//   * each DMA instruction moves 16 rows x 64 B with every 4 lanes reading
//     64 contiguous bytes of one row, and LDS blocks sit at offsets that keep
//     the MFMA fragment reads free of bank conflicts (as in grouped_gemm.hip);
//   * 8 waves as 2 along M x 4 along N, each 64 rows (16-row tiles wm + 2i)
//     x 64 columns; weight-block scales are wave-uniform scalar loads.
// The first projection's epilogue applies the clipped SwiGLU, takes each
// row's amax over the block's 128 h columns (one K block of the second
// projection) across the 4 N waves through LDS, and writes the E4M3 codes of
// h and their scales s_h[kb][row].
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace f8 {

constexpr int BM = 128, BN = 256, BKB = 128;      // K slice = 128 bytes = one scale block
constexpr int NW = 8, NT = NW * 64;
constexpr int TM = 4, TN = 4;
constexpr int STAGES = 3;
// A DMA block is 16 rows x 64 B (half of a 128-byte K slice).  The 4 blocks
// of one (64-row group, half) start at these byte offsets: 16-byte bank
// groups 0, 1, 16, 17 (mod 32), which keeps both 16-byte reads of every
// 32-lane fragment pass free of bank conflicts.
__device__ constexpr int BOFF[4] = {0, 1024 + 16, 2048 + 256, 3072 + 272};
constexpr int GROUP = 3072 + 272 + 1024;
constexpr int A_BYTES = 4 * GROUP;                 // 128 rows: 2 row groups x 2 halves
constexpr int B_BYTES = 8 * GROUP;                 // 256 weight rows
constexpr int SA_OFF = A_BYTES + B_BYTES;          // 128 row scales (two 256-byte DMAs)
constexpr int STAGE_BYTES = SA_OFF + 512;
constexpr int NXCD = 8;

enum { SWIGLU = 0, OUT_F16 = 1 };

struct Params {
    const uint8_t* A;           // activation codes [a_nrows][K]
    const int32_t* a_rows;      // row r reads A row a_rows[r] / a_div (nullptr: row r)
    int a_div, a_nrows;
    const float* As;            // activation scales [K/128][a_ld], indexed like A's rows
    int a_ld;
    const uint8_t* W;           // weight codes [groups][Nw][K]
    const float* Ws;            // weight scales [groups][Nw/128][K/128]
    int64_t w_group_stride;     // bytes between groups' weights
    int64_t ws_group_stride;    // floats between groups' scales
    void* C;                    // SWIGLU: h codes [rows][N]; OUT_F16: fp16 [rows][N]
    float* Cs;                  // SWIGLU: h scales [N/128][c_ld]
    int c_ld;
    int N, K;
    float limit;
    const int32_t* offsets;
    const int32_t* tile_start;
    int groups;
    int n_tiles;
};

typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ void dma16(const void* g, unsigned lds_off) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_off), "v"(g) : "memory");
}
__device__ __forceinline__ void dma4(const void* g, unsigned lds_off) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(lds_off), "v"(g) : "memory");
}

template <int n>
__device__ __forceinline__ void wait_vm() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

// fp32 -> E4M3FN byte, round to nearest even (|v| <= 448 by construction)
__device__ __forceinline__ uint32_t to_e4m3(float v) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.0f, 0, false) & 0xffu;
}

template <int MODE>
__global__ __launch_bounds__(NT, 1) void kernel(Params p) {
    __shared__ __attribute__((aligned(1024))) unsigned char smem[STAGES * STAGE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;

    // ---- work item: (expert, n-tile, m-tile), m fastest, per-XCD ranges
    int g, n_tile, row0, row_end;
    {
        const int b = blockIdx.x;
        const int xcd = b % NXCD, slot = b / NXCD;
        const int ntiles = p.tile_start[p.groups];
        const int total = ntiles * p.n_tiles;
        const int per = (total + NXCD - 1) / NXCD;
        if (slot >= per) return;
        const int w = xcd * per + slot;
        if (w >= total) return;
        int lo = 0, hi = p.groups - 1;
        while (lo < hi) {
            int mid = (lo + hi + 1) >> 1;
            if (p.tile_start[mid] * p.n_tiles <= w) lo = mid; else hi = mid - 1;
        }
        g = lo;
        const int mt = p.tile_start[g + 1] - p.tile_start[g];
        const int local = w - p.tile_start[g] * p.n_tiles;
        n_tile = local / mt;
        // rows split evenly over the group's mt tiles (each <= BM rows): the
        // m-tiles of one weight panel stay in step and share it in L2
        const int m_tile = local % mt;
        const int cnt = p.offsets[g + 1] - p.offsets[g];
        row0 = p.offsets[g] + (int)(((int64_t)m_tile * cnt) / mt);
        row_end = p.offsets[g] + (int)(((int64_t)(m_tile + 1) * cnt) / mt);
    }
    const int valid = min(row_end - row0, BM);
    const int K = p.K, KB = K / BKB;
    const uint8_t* Wg = p.W + (int64_t)g * p.w_group_stride;
    const float* Wsg = p.Ws + (int64_t)g * p.ws_group_stride;

    // source row of tile row r (rows past the group's end repeat its last row)
    auto src_row = [&](int r) {
        const int pr = row0 + min(r, valid - 1);
        const int sr = p.a_rows ? p.a_rows[pr] / p.a_div : pr;
        return min(max(sr, 0), p.a_nrows - 1);
    };

    // ---- DMA sources (at k = 0).  Every 4 lanes read 64 contiguous bytes
    // of one row (lane l: row quad l >> 2, 16 bytes at (l & 3) * 16 of the
    // block's half); block b of row group g holds rows 64g + 16t + 4b + i
    // for quad 4t + i.  Wave w moves A blocks 2w, 2w+1 and B blocks
    // 4w .. 4w+3 of every slice; waves 0 and 1 also move the scales of tile
    // rows 64w + lane.
    const int quad = lane >> 2, chunk = lane & 3;
    auto block_row = [&](int blk) { return 64 * (blk >> 3) + 16 * (quad >> 2) + 4 * (blk & 3) + (quad & 3); };
    auto block_lds = [&](int blk) { return (blk >> 2) * GROUP + BOFF[blk & 3]; };
    const uint8_t* a_src[2];
    unsigned a_lds[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int blk = 2 * wave + q;                           // 0..15: (row group, half, block)
        a_src[q] = p.A + (int64_t)src_row(block_row(blk)) * K + 64 * ((blk >> 2) & 1) + 16 * chunk;
        a_lds[q] = block_lds(blk);
    }
    const uint8_t* b_src[4];
    unsigned b_lds[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int blk = 4 * wave + q;                           // 0..31
        const int r = block_row(blk);                           // tile column 0..255
        int wrow;
        if (MODE == SWIGLU) {
            // 64-column wave groups: 32 gate columns, then the matching 32 up columns
            const int wg = r >> 6, u = r & 63;
            const int hcol = min(n_tile * (BN / 2) + 32 * wg + (u & 31), p.N - 1);
            wrow = (u < 32) ? hcol : p.N + hcol;
        } else {
            wrow = min(n_tile * BN + r, p.N - 1);
        }
        b_src[q] = Wg + (int64_t)wrow * K + 64 * ((blk >> 2) & 1) + 16 * chunk;
        b_lds[q] = A_BYTES + block_lds(blk);
    }
    const float* sa_src = p.As + src_row(64 * (wave & 1) + lane);

    const unsigned lds_base = (unsigned)(size_t)(lds_u8*)smem;
    // this wave's DMA q of slice kt into `stage`: q 0, 1 A blocks, 2 .. 5 W
    // blocks, 6 the row scales (waves 0 and 1 only)
    auto issue_q = [&](int kt, int stage, int q) {
        const int k0 = kt * BKB;
        const unsigned sb = lds_base + stage * STAGE_BYTES;
        if (q < 2) dma16(a_src[q] + k0, __builtin_amdgcn_readfirstlane(sb + a_lds[q]));
        else if (q < 6) dma16(b_src[q - 2] + k0, __builtin_amdgcn_readfirstlane(sb + b_lds[q - 2]));
        else if (wave < 2) dma4(sa_src + (int64_t)kt * p.a_ld, __builtin_amdgcn_readfirstlane(sb + SA_OFF + 256 * wave));
    };
    // LDS offset of this lane's 32 bytes (two 16-byte reads, +0 and +16) in
    // 16-row tile tau = 4g + t: row r = lane & 15 from block r >> 2 of
    // half (lane >> 5), bytes 32 * ((lane >> 4) & 1) of that half
    const int fr = lane & 15;
    const unsigned lane_off = (lane >> 5) * GROUP + BOFF[fr >> 2] + 64 * (fr & 3) + 32 * ((lane >> 4) & 1);
    auto tile_off = [&](int tau) { return (unsigned)((tau >> 2) * 2 * GROUP + 256 * (tau & 3)) + lane_off; };

    const int ntile_valid = (valid + 15) >> 4;
    int n_i = 0;
#pragma unroll
    for (int i = 0; i < TM; ++i) n_i += (wm + 2 * i < ntile_valid) ? 1 : 0;
    n_i = __builtin_amdgcn_readfirstlane(n_i);

    // weight-scale block rows of this wave's columns (wave-uniform); all 64
    // columns of a wave (32 + 32 for the gate/up pairs) sit in one 128-row block
    int sw_row[2];
    if (MODE == SWIGLU) {
        const int hbase = min(n_tile * (BN / 2) + 32 * wn, p.N - 1);
        sw_row[0] = hbase / 128;
        sw_row[1] = (p.N + hbase) / 128;
    } else {
        sw_row[0] = sw_row[1] = min(n_tile * BN + 64 * wn, p.N - 1) / 128;
    }
    sw_row[0] = __builtin_amdgcn_readfirstlane(sw_row[0]);
    sw_row[1] = __builtin_amdgcn_readfirstlane(sw_row[1]);
    const float* swa_p = Wsg + (int64_t)sw_row[0] * KB;
    const float* swb_p = Wsg + (int64_t)sw_row[1] * KB;
    // lane c holds the scales of K blocks 64 m + c for the current chunk m;
    // loaded before any DMA is in flight (and every 64 slices after), so the
    // compiler's wait for them never drains the ring
    float swa_v = lane < KB ? swa_p[lane] : 0.f;
    float swb_v = lane < KB ? swb_p[lane] : 0.f;
    asm volatile("" ::"v"(swa_v), "v"(swb_v));

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // fragments and row scales of one slice
    i32x8 bfr[TN], afr[TM];
    f32x4 sa[TM];
    const int crow = (lane >> 4) * 4;
    auto read_frags = [&](int stage) {
        const unsigned char* st = smem + stage * STAGE_BYTES;
        const float* sa_l = (const float*)(st + SA_OFF);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const unsigned char* f = st + A_BYTES + tile_off(4 * wn + j);
            const u32x4 lo = *(const u32x4*)f, hi = *(const u32x4*)(f + 16);
            bfr[j] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            if (i < n_i) {
                const int tile = wm + 2 * i;
                const unsigned char* f = st + tile_off(tile);
                const u32x4 lo = *(const u32x4*)f, hi = *(const u32x4*)(f + 16);
                afr[i] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                sa[i] = *(const f32x4*)(sa_l + 16 * tile + crow);
            }
        }
    };

    // Slice s sits in stage s % STAGES.  Step kt multiplies slice kt from
    // registers; its stage then takes slice kt + STAGES (its fragments were
    // read during step kt-1), and the fragments of slice kt+1 are read into
    // the same registers once this step's MFMAs have been issued, so the LDS
    // latency overlaps the MFMAs.  The DMAs sit between the MFMA groups:
    // issued in one burst after the barrier they queue at the wave's issue
    // and hold back its MFMAs.  Clamped re-reads past the end keep the DMA
    // count per step fixed, which the waits rely on.
#pragma unroll
    for (int s = 0; s < STAGES; ++s)
#pragma unroll
        for (int q = 0; q < 7; ++q) issue_q(min(s, KB - 1), s, q);
    if (wave < 2) wait_vm<7 * (STAGES - 1)>(); else wait_vm<6 * (STAGES - 1)>();
    __builtin_amdgcn_s_barrier();
    read_frags(0);

    for (int kt = 0; kt < KB; ++kt) {
        // slice kt+1 has landed (at most slice kt+2's DMAs outstanding), and
        // this wave's reads of slice kt are done
        if (wave < 2) wait_vm<7>(); else wait_vm<6>();
        __builtin_amdgcn_s_waitcnt(0xc07f);       // lgkmcnt(0), vmcnt/expcnt untouched
        __builtin_amdgcn_s_barrier();
        const int kn = min(kt + STAGES, KB - 1), sn = kt % STAGES;

        if ((kt & 63) == 0 && kt > 0) {
            swa_v = kt + lane < KB ? swa_p[kt + lane] : 0.f;
            swb_v = kt + lane < KB ? swb_p[kt + lane] : 0.f;
            asm volatile("" ::"v"(swa_v), "v"(swb_v));
        }
        const float swa = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(swa_v), kt & 63));
        const float swb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(swb_v), kt & 63));
        // The MFMAs of 16-row tile i go to temporaries; tile i-1's results
        // are scaled and added while they run (so no MFMA result is consumed
        // right after issue), and the DMAs sit between the groups.  The next
        // slice's fragments are read after the last group is issued; the last
        // tile's results are scaled after that, with its row scales kept.
        f32x4 r[2][TN];
        f32x4 sa_last = sa[TM - 1];
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        auto scale_add = [&](int i, const f32x4* ri, f32x4 sai) {
            const f32x4 sga = sai * swa, sgb = sai * swb;
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] += ri[j] * ((MODE == SWIGLU && j >= TN / 2) ? sgb : sga);
        };
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            issue_q(kn, sn, 2 * i);
            if (2 * i + 1 < 7) issue_q(kn, sn, 2 * i + 1);
            if (i < n_i) {
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    // E8M0 scale 127 = 1.0 on both operands; the fp32 block scales follow
                    r[i & 1][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(afr[i], bfr[j], z, 0, 0, 0, 127, 0, 127);
            }
            if (i > 0 && i - 1 < n_i) scale_add(i - 1, r[(i - 1) & 1], sa[i - 1]);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (kt + 1 < KB) read_frags((kt + 1) % STAGES);
        if (TM - 1 < n_i) scale_add(TM - 1, r[(TM - 1) & 1], sa_last);
    }
    wait_vm<0>();

    const int ccol = lane & 15;
    if (MODE == SWIGLU) {
        // this wave's h: rows of tiles wm + 2i, h columns 32 wn + 16 j + ccol (j < 2)
        float hv[TM][2][4];
        float* amax_l = (float*)smem;                          // [128 rows][4 waves along N]
        __syncthreads();                                       // every wave is done with the ring
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                float m = 0.f;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    hv[i][j][v] = swiglu_clip(acc[i][j][v], acc[i][j + 2][v], p.limit);
                    m = fmaxf(m, fabsf(hv[i][j][v]));
                }
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));   // the row's 16 lanes
                if (ccol == 0) amax_l[(16 * (wm + 2 * i) + crow + v) * 4 + wn] = m;
            }
        __syncthreads();
        uint8_t* Hq = (uint8_t*)p.C;
        const int kb = n_tile;                                  // K block of the second projection
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            if (i >= n_i) continue;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int lr = 16 * (wm + 2 * i) + crow + v;
                const f32x4 m4 = *(const f32x4*)(amax_l + lr * 4);
                const float amax = fmaxf(fmaxf(m4.x, m4.y), fmaxf(m4.z, m4.w));
                const float s = amax > 0.f ? amax / 448.0f : 1.0f;
                if (lr < valid) {
                    if (wn == 0 && ccol == 0) p.Cs[(int64_t)kb * p.c_ld + row0 + lr] = s;
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int hcol = n_tile * (BN / 2) + 32 * wn + 16 * j + ccol;
                        if (hcol < p.N) Hq[(int64_t)(row0 + lr) * p.N + hcol] = (uint8_t)to_e4m3(hv[i][j][v] / s);
                    }
                }
            }
        }
    } else {
        _Float16* Y = (_Float16*)p.C;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            if (i >= n_i) continue;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int col = n_tile * BN + 64 * wn + 16 * j + ccol;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int lr = 16 * (wm + 2 * i) + crow + v;
                    if (lr < valid && col < p.N) Y[(int64_t)(row0 + lr) * p.N + col] = f32_to_f16_sat(acc[i][j][v]);
                }
            }
        }
    }
}

// Quantise each row of x per 128 columns: one block per row, 16 elements per
// thread, so a 128-wide group is 8 consecutive threads.  xs is
// K-block-major: xs[kb * ld + row].
__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t* __restrict__ x, int H,
                                                         uint8_t* __restrict__ xq, float* __restrict__ xs, int ld) {
    const int r = blockIdx.x;
    const uint16_t* xr = x + (int64_t)r * H;
    for (int c0 = threadIdx.x * 16; c0 < H; c0 += 256 * 16) {
        float v[16];
        const u32x4 a = *(const u32x4*)(xr + c0), b = *(const u32x4*)(xr + c0 + 8);
        const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        float m = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
            m = fmaxf(m, fmaxf(fabsf(v[2 * i]), fabsf(v[2 * i + 1])));
        }
#pragma unroll
        for (int o = 1; o < 8; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
        const float s = m > 0.f ? m / 448.0f : 1.0f;
        uint32_t q[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            q[i] = to_e4m3(v[4 * i] / s) | (to_e4m3(v[4 * i + 1] / s) << 8) | (to_e4m3(v[4 * i + 2] / s) << 16) |
                   (to_e4m3(v[4 * i + 3] / s) << 24);
        *(u32x4*)(xq + (int64_t)r * H + c0) = u32x4{q[0], q[1], q[2], q[3]};
        if ((threadIdx.x & 7) == 0) xs[(int64_t)(c0 / 128) * ld + r] = s;
    }
}

}  // namespace f8

hipError_t launch_quant_rows(const void* x, int rows, int H, void* xq, float* xs, int ld, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    f8::quant_rows_kernel<<<rows, 256, 0, s>>>((const uint16_t*)x, H, (uint8_t*)xq, xs, ld);
    return hipGetLastError();
}

int fp8_tile_m() { return f8::BM; }

static int f8_grid(int64_t work) { return (int)((work + f8::NXCD - 1) / f8::NXCD * f8::NXCD); }

hipError_t launch_fp8_up(const void* xq, const float* xs, int xs_ld, const int32_t* a_rows, int a_div,
                         int a_nrows, const void* w13, const float* w13s, void* hq, float* hs, int hs_ld, int N,
                         int K, float limit, const int32_t* offsets, const int32_t* tile_start, int groups,
                         int max_tiles, hipStream_t s) {
    f8::Params p{};
    p.A = (const uint8_t*)xq;
    p.a_rows = a_rows;
    p.a_div = a_div > 0 ? a_div : 1;
    p.a_nrows = a_nrows;
    p.As = xs;
    p.a_ld = xs_ld;
    p.W = (const uint8_t*)w13;
    p.Ws = w13s;
    p.w_group_stride = (int64_t)2 * N * K;
    p.ws_group_stride = (int64_t)(2 * N / 128) * (K / 128);
    p.C = hq;
    p.Cs = hs;
    p.c_ld = hs_ld;
    p.N = N;
    p.K = K;
    p.limit = limit;
    p.offsets = offsets;
    p.tile_start = tile_start;
    p.groups = groups;
    p.n_tiles = (2 * N) / f8::BN;
    if (max_tiles <= 0) return hipSuccess;
    f8::kernel<f8::SWIGLU><<<f8_grid((int64_t)max_tiles * p.n_tiles), f8::NT, 0, s>>>(p);
    return hipGetLastError();
}

hipError_t launch_fp8_down(const void* hq, const float* hs, int hs_ld, int rows, const void* w2, const float* w2s,
                           void* y, int N, int K, const int32_t* offsets, const int32_t* tile_start, int groups,
                           int max_tiles, hipStream_t s) {
    f8::Params p{};
    p.A = (const uint8_t*)hq;
    p.a_rows = nullptr;
    p.a_div = 1;
    p.a_nrows = rows;
    p.As = hs;
    p.a_ld = hs_ld;
    p.W = (const uint8_t*)w2;
    p.Ws = w2s;
    p.w_group_stride = (int64_t)N * K;
    p.ws_group_stride = (int64_t)(N / 128) * (K / 128);
    p.C = y;
    p.N = N;
    p.K = K;
    p.offsets = offsets;
    p.tile_start = tile_start;
    p.groups = groups;
    p.n_tiles = (N + f8::BN - 1) / f8::BN;
    if (max_tiles <= 0) return hipSuccess;
    f8::kernel<f8::OUT_F16><<<f8_grid((int64_t)max_tiles * p.n_tiles), f8::NT, 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace moe
