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
// Layout and staging (the bf16 256-row tiles' choices, with bytes for elements):
//   * x is quantised once per token (quant_rows_kernel); the first projection
//     gathers the code rows of its permuted rows (token = pair / k) as the
//     bf16 kernel gathers x; activation scales are stored K-block-major,
//     s_a[kb][row], and gathered per row into LDS by 4-byte DMA;
//   * block tile 128 rows x 256 weight rows, K slices of 128 bytes (one
//     scale block, one whole line of every row), 3-stage LDS ring filled by
//     direct global->LDS DMA from inline asm with explicit vmcnt waits;
//   * each DMA instruction moves 8 rows x 128 B, the 16-byte chunks of a
//     row swizzled by line_swz so that the fragment reads are free of bank
//     conflicts (the layout of grouped_gemm.hip's 256-row tiles);
//   * 8 waves as 2 along M x 4 along N, each 64 rows (16-row tiles wm + 2i)
//     x 64 columns; weight-block scales are wave-uniform scalar loads;
//   * the fragments of the next slice are read while this slice's MFMAs
//     run, each into its register as soon as the register is free.
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
constexpr int A_BYTES = BM * BKB;                  // 128 rows of 128 B
constexpr int B_BYTES = BN * BKB;                  // 256 weight rows of 128 B
constexpr int SA_OFF = A_BYTES + B_BYTES;          // 128 row scales (two 256-byte DMAs)
constexpr int STAGE_BYTES = SA_OFF + 1024;         // (1 KiB aligned)
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
    void* C;                    // SWIGLU: h codes [rows][N]; OUT_F16: scaled fp16 rows of c_row_bytes
    float* Cs;                  // SWIGLU: h scales [N/128][c_ld]
    int c_ld;
    int N, K;
    int64_t c_row_bytes;
    float limit;
    const int32_t* offsets;
    const int32_t* tile_start;
    int groups;
    int n_tiles;
    const int4* items;          // optional: per work item {group, first row, rows, n-tile}
    const int* xcd_start;       // with items: XCD x runs items xcd_start[x] .. xcd_start[x + 1] - 1
};

typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// one 1 KiB block: lane l's 16 bytes from base + off land at LDS byte
// lds_off + 16 l (base wave-uniform, off this lane's 32-bit byte offset)
__device__ __forceinline__ void dma16s(const void* base, unsigned off, unsigned lds_off) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_off), "v"(off), "s"(base) : "memory");
}
__device__ __forceinline__ void dma4(const void* g, unsigned lds_off) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(lds_off), "v"(g) : "memory");
}

template <int n>
__device__ __forceinline__ void wait_vm() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

// clipped SwiGLU with silu(g) = g * rcp(1 + exp(-g)), the hardware
// reciprocal (1 ulp) in place of a division: the epilogue's VALU work is
// most of its time
__device__ __forceinline__ float swiglu_clip_fast(float g, float u, float L) {
    float sg = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
    if (L > 0.0f) {
        sg = fminf(sg, L);
        u = fminf(fmaxf(u, -L), L);
    }
    return sg * u;
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
    if (p.items) {
        // one load from the item table (written by a one-block launch first)
        const int b = blockIdx.x;
        const int xcd = b % NXCD, slot = b / NXCD;
        const int r0 = __builtin_amdgcn_readfirstlane(p.xcd_start[xcd]);
        if (slot >= __builtin_amdgcn_readfirstlane(p.xcd_start[xcd + 1]) - r0) return;
        const int4 d = p.items[r0 + slot];
        g = __builtin_amdgcn_readfirstlane(d.x);
        row0 = __builtin_amdgcn_readfirstlane(d.y);
        row_end = row0 + __builtin_amdgcn_readfirstlane(d.z);
        n_tile = __builtin_amdgcn_readfirstlane(d.w);
    } else {
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

    // ---- DMA sources.  One DMA instruction moves 8 rows x 128 B: lanes
    // 8q .. 8q+7 read the whole 128-byte line of row q; lane l reads chunk
    // (l & 7) ^ line_swz(row) and lands at LDS byte 16 l, so LDS chunk c of
    // a row holds global chunk c ^ line_swz(row).  Wave w moves A rows
    // 16w .. 16w+15 and W rows 32w .. 32w+31 of every slice.  Offsets are
    // 32-bit from wave-uniform bases (the launch checks the ranges).
    const int dq = lane >> 3;
    unsigned a_off[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int r = 16 * wave + 8 * q + dq;
        a_off[q] = (unsigned)src_row(r) * (unsigned)K + 16u * ((lane & 7) ^ line_swz(r & 15));
    }
    unsigned b_off[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int r = 32 * wave + 8 * q + dq;                   // tile column 0..255
        int wrow;
        if (MODE == SWIGLU) {
            // 64-column wave groups: 32 gate columns, then the matching 32 up columns
            const int wg = r >> 6, u = r & 63;
            const int hcol = min(n_tile * (BN / 2) + 32 * wg + (u & 31), p.N - 1);
            wrow = (u < 32) ? hcol : p.N + hcol;
        } else {
            wrow = min(n_tile * BN + r, p.N - 1);
        }
        b_off[q] = (unsigned)wrow * (unsigned)K + 16u * ((lane & 7) ^ line_swz(r & 15));
    }
    const float* sa_src = p.As + src_row(64 * (wave & 1) + lane);

    const unsigned lds_base = (unsigned)(size_t)(lds_u8*)smem;
    // this wave's DMA q of slice kt into `stage`: q 0, 1 A blocks, 2 .. 5 W
    // blocks, 6 the row scales (waves 0 and 1 only)
    auto issue_q = [&](int kt, int stage, int q) {
        const int k0 = kt * BKB;
        const unsigned sb = lds_base + stage * STAGE_BYTES;
        if (q < 2) dma16s(p.A + k0, a_off[q], __builtin_amdgcn_readfirstlane(sb + 1024 * (2 * wave + q)));
        else if (q < 6) dma16s(Wg + k0, b_off[q - 2], __builtin_amdgcn_readfirstlane(sb + A_BYTES + 1024 * (4 * wave + q - 2)));
        else if (wave < 2) dma4(sa_src + (int64_t)kt * p.a_ld, __builtin_amdgcn_readfirstlane(sb + SA_OFF + 256 * wave));
    };
    // A lane's 32 bytes of a fragment (row lane & 15 of a 16-row tile) are
    // global chunks (lane >> 4) and 4 + (lane >> 4) of the row: the same K
    // order in both operands, so the MFMA still sums the slice's 128 products
    // of every (row, column); the two reads hit distinct bank groups
    // (line_swz).  off0 is opaque so that no part of it is kept apart.
    const int fr = lane & 15;
    unsigned off0 = 128 * fr + 16 * ((lane >> 4) ^ line_swz(fr));
    asm volatile("" : "+v"(off0));

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

    // Fragments and row scales of one slice.  The MFMAs take the W fragment
    // as their first operand, so the tile comes out transposed: lane l holds
    // row l & 15 of its 16-row tile and 4 consecutive columns 4 (l >> 4) + v,
    // and one activation scale per tile covers all four.
    i32x8 bfr[TN], afr[TM];
    float sa[TM];
    const int quad4 = 4 * (lane >> 4);
    auto read_frag = [&](const unsigned char* f) {
        const u32x4 lo = *(const u32x4*)(f + off0), hi = *(const u32x4*)(f + (off0 ^ 64u));
        return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    };
    auto stage_ptr = [&](int kt) { return smem + (kt % STAGES) * STAGE_BYTES; };
    auto read_a = [&](int kt, int i) { afr[i] = read_frag(stage_ptr(kt) + 2048 * (wm + 2 * i)); };
    auto read_sa = [&](int kt, int i) {
        sa[i] = ((const float*)(stage_ptr(kt) + SA_OFF))[16 * (wm + 2 * i) + fr];
    };
    auto read_b = [&](int kt, int j) { bfr[j] = read_frag(stage_ptr(kt) + A_BYTES + 2048 * (4 * wn + j)); };

    // Slice s sits in stage s % STAGES.  Step kt multiplies slice kt from
    // registers; its stage then takes slice kt + STAGES (its fragments were
    // read during step kt-1).  Slice kt+1 has landed when step kt starts, so
    // its fragments are read during step kt, each as soon as its register
    // is free: a tile's A fragment right after the tile's MFMAs are issued,
    // its row scale after its products are scaled, and the W fragments after
    // the last tile's MFMAs (reading them all after the MFMAs, as a block,
    // serialised the LDS reads with the MFMAs: 1.72 against 1.38 ms for the
    // first projection at the Step-5 prefill).
    // The DMAs sit between the MFMA groups: issued in one burst after the
    // barrier they queue at the wave's issue and hold back its MFMAs.
    // Clamped re-reads past the end keep the DMA count per step fixed, which
    // the waits rely on.
#pragma unroll
    for (int s = 0; s < STAGES; ++s)
#pragma unroll
        for (int q = 0; q < 7; ++q) issue_q(min(s, KB - 1), s, q);
    if (wave < 2) wait_vm<7 * (STAGES - 1)>(); else wait_vm<6 * (STAGES - 1)>();
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int j = 0; j < TN; ++j) read_b(0, j);
#pragma unroll
    for (int i = 0; i < TM; ++i) { read_a(0, i); read_sa(0, i); }

    for (int kt = 0; kt < KB; ++kt) {
        // slice kt+1 has landed (at most slice kt+2's DMAs outstanding), and
        // this wave's reads of slice kt are done
        if (wave < 2) wait_vm<7>(); else wait_vm<6>();
        __builtin_amdgcn_s_waitcnt(0xc07f);       // lgkmcnt(0), vmcnt/expcnt untouched
        __builtin_amdgcn_s_barrier();
        const int kn = min(kt + STAGES, KB - 1), sn = kt % STAGES;
        const int kt1 = min(kt + 1, KB - 1);      // (the last step re-reads its own slice; unused)

        if ((kt & 63) == 0 && kt > 0) {
            swa_v = kt + lane < KB ? swa_p[kt + lane] : 0.f;
            swb_v = kt + lane < KB ? swb_p[kt + lane] : 0.f;
            asm volatile("" ::"v"(swa_v), "v"(swb_v));
        }
        const float swa = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(swa_v), kt & 63));
        const float swb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(swb_v), kt & 63));
        // The MFMAs of 16-row tile i go to temporaries; tile i-1's results
        // are scaled and added while they run (so no MFMA result is consumed
        // right after issue).  The reads are unconditional (a branch around
        // them costs more than the LDS bytes of tiles past the valid rows).
        f32x4 r[2][TN];
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        auto scale_add = [&](int i) {
            const float sga = sa[i] * swa, sgb = sa[i] * swb;
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] += r[i & 1][j] * ((MODE == SWIGLU && j >= TN / 2) ? sgb : sga);
        };
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            issue_q(kn, sn, 2 * i);
            if (2 * i + 1 < 7) issue_q(kn, sn, 2 * i + 1);
            if (i < n_i) {
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    // E8M0 scale 127 = 1.0 on both operands; the fp32 block scales follow
                    r[i & 1][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bfr[j], afr[i], z, 0, 0, 0, 127, 0, 127);
            }
            read_a(kt1, i);
            if (i == TM - 1) {
#pragma unroll
                for (int j = 0; j < TN; ++j) read_b(kt1, j);
            }
            if (i > 0 && i - 1 < n_i) scale_add(i - 1);
            if (i > 0) read_sa(kt1, i - 1);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (TM - 1 < n_i) scale_add(TM - 1);
        read_sa(kt1, TM - 1);
    }
    wait_vm<0>();

    if (MODE == SWIGLU) {
        // this wave's h: rows 16 (wm + 2i) + fr, h columns 32 wn + 16 j + quad4 + v (j < 2)
        float hv[TM][2][4];
        float* amax_l = (float*)smem;                          // [128 rows][4 waves along N]
        __syncthreads();                                       // every wave is done with the ring
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            float m = 0.f;
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    hv[i][j][v] = swiglu_clip_fast(acc[i][j][v], acc[i][j + 2][v], p.limit);
                    m = fmaxf(m, fabsf(hv[i][j][v]));
                }
            m = max_lanes_xor16_32(m);                          // the row's 4 lanes
            if (quad4 == 0) amax_l[(16 * (wm + 2 * i) + fr) * 4 + wn] = m;
        }
        __syncthreads();
        uint8_t* Hq = (uint8_t*)p.C;
        const int kb = n_tile;                                  // K block of the second projection
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            if (i >= n_i) continue;
            const int lr = 16 * (wm + 2 * i) + fr;
            const f32x4 m4 = *(const f32x4*)(amax_l + lr * 4);
            const float amax = fmaxf(fmaxf(m4.x, m4.y), fmaxf(m4.z, m4.w));
            const float s = amax > 0.f ? amax / 448.0f : 1.0f;
            const float rs = 1.0f / s;
            if (lr < valid) {
                if (wn == 0 && quad4 == 0) p.Cs[(int64_t)kb * p.c_ld + row0 + lr] = s;
                uint32_t code[2];
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    code[j] = to_e4m3(hv[i][j][0] * rs) | (to_e4m3(hv[i][j][1] * rs) << 8) |
                              (to_e4m3(hv[i][j][2] * rs) << 16) | (to_e4m3(hv[i][j][3] * rs) << 24);
                const int hc0 = n_tile * (BN / 2) + 32 * wn;
                if (hc0 + 32 <= p.N) {
                    // both h tiles through one lane swap: lanes with (lane >> 4)
                    // even take 8 codes of tile 0, the odd ones 8 of tile 1
                    const auto sw = __builtin_amdgcn_permlane16_swap(code[0], code[1], false, false);
                    const int hcol = hc0 + 16 * ((lane >> 4) & 1) + 4 * ((lane >> 4) & ~1);
                    *(uint2*)(Hq + (int64_t)(row0 + lr) * p.N + hcol) = make_uint2(sw[0], sw[1]);
                } else {
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int hcol = hc0 + 16 * j + quad4;
                        if (hcol < p.N) *(uint32_t*)(Hq + (int64_t)(row0 + lr) * p.N + hcol) = code[j];
                    }
                }
            }
        }
    } else {
        // scaled fp16 rows: a 128-column exponent group is two waves along N;
        // each row's largest magnitude over the wave's 64 columns goes
        // through LDS to its partner wave
        float* red = (float*)smem;                              // [128 rows][4 waves along N]
        __syncthreads();                                       // every wave is done with the ring
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int lr = 16 * (wm + 2 * i) + fr;
            float m = 0.f;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int col = n_tile * BN + 64 * wn + 16 * j + quad4;
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (i < n_i && lr < valid && col < p.N) m = fmaxf(m, fabsf(acc[i][j][v]));
            }
            m = max_lanes_xor16_32(m);                          // the row's 4 lanes
            if (quad4 == 0) red[lr * 4 + wn] = m;
        }
        __syncthreads();
        const int gw = wn & ~1;                                 // first wave of this wave's group
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            if (i >= n_i) continue;
            const int lr = 16 * (wm + 2 * i) + fr;
            if (lr >= valid) continue;
            const int ex = yrow_exp(fmaxf(red[lr * 4 + gw], red[lr * 4 + gw + 1]));
            const float sc = exp2_int(-ex);
            char* row = (char*)p.C + (int64_t)(row0 + lr) * p.c_row_bytes;
            const int wc0 = n_tile * BN + 64 * wn;
            if (wc0 + 64 <= p.N) {
                // tiles j and j+1 through one lane swap, 16 bytes per lane
                // (the grouped bf16 kernel's second projection does the same)
#pragma unroll
                for (int j = 0; j < TN; j += 2) {
                    const f16x4 a4 = {(_Float16)(acc[i][j][0] * sc), (_Float16)(acc[i][j][1] * sc),
                                      (_Float16)(acc[i][j][2] * sc), (_Float16)(acc[i][j][3] * sc)};
                    const f16x4 b4 = {(_Float16)(acc[i][j + 1][0] * sc), (_Float16)(acc[i][j + 1][1] * sc),
                                      (_Float16)(acc[i][j + 1][2] * sc), (_Float16)(acc[i][j + 1][3] * sc)};
                    const uint2 a = __builtin_bit_cast(uint2, a4), b = __builtin_bit_cast(uint2, b4);
                    const auto s0 = __builtin_amdgcn_permlane16_swap(a.x, b.x, false, false);
                    const auto s1 = __builtin_amdgcn_permlane16_swap(a.y, b.y, false, false);
                    const int col = wc0 + 16 * (j + ((lane >> 4) & 1)) + 4 * ((lane >> 4) & ~1);
                    *(uint4*)(row + 2 * col) = make_uint4(s0[0], s1[0], s0[1], s1[1]);
                }
            } else {
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int col = wc0 + 16 * j + quad4;
                    if (col < p.N) {
                        const f16x4 o = {(_Float16)(acc[i][j][0] * sc), (_Float16)(acc[i][j][1] * sc),
                                         (_Float16)(acc[i][j][2] * sc), (_Float16)(acc[i][j][3] * sc)};
                        *(f16x4*)(row + 2 * col) = o;
                    }
                }
            }
            const int gcol = n_tile * BN + 64 * gw;
            if (wn == gw && quad4 == 0 && gcol < p.N) {
                row[2 * p.N + (gcol >> 7)] = (char)ex;
                if (gcol == 0) yrow_zero_pad(row, p.N);
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
                         int max_tiles, void* items, hipStream_t s) {
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
    if ((int64_t)a_nrows * K > UINT32_MAX || (int64_t)2 * N * K > UINT32_MAX) return hipErrorInvalidValue;
    if (items) {
        const hipError_t e = launch_item_table(offsets, tile_start, groups, 0, p.n_tiles, false, items, s);
        if (e != hipSuccess) return e;
        p.xcd_start = (const int*)items;
        p.items = (const int4*)((const char*)items + 64);
    }
    f8::kernel<f8::SWIGLU><<<f8_grid((int64_t)max_tiles * p.n_tiles), f8::NT, 0, s>>>(p);
    return hipGetLastError();
}

hipError_t launch_fp8_down(const void* hq, const float* hs, int hs_ld, int rows, const void* w2, const float* w2s,
                           void* y, int N, int K, const int32_t* offsets, const int32_t* tile_start, int groups,
                           int max_tiles, void* items, hipStream_t s) {
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
    p.c_row_bytes = yrow_bytes(N);
    p.offsets = offsets;
    p.tile_start = tile_start;
    p.groups = groups;
    p.n_tiles = (N + f8::BN - 1) / f8::BN;
    if (max_tiles <= 0) return hipSuccess;
    if ((int64_t)rows * K > UINT32_MAX || (int64_t)N * K > UINT32_MAX) return hipErrorInvalidValue;
    if (items) {
        const hipError_t e = launch_item_table(offsets, tile_start, groups, 0, p.n_tiles, false, items, s);
        if (e != hipSuccess) return e;
        p.xcd_start = (const int*)items;
        p.items = (const int4*)((const char*)items + 64);
    }
    f8::kernel<f8::OUT_F16><<<f8_grid((int64_t)max_tiles * p.n_tiles), f8::NT, 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace moe
