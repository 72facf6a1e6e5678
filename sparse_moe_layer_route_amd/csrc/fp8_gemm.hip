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
//
// The grid is persistent: at most one block per CU, each walking a stride of
// its XCD's range of the work-item table.  While an item runs its last three
// K steps, their ring stages take the next item's first three slices (its
// descriptor read by scalar loads in step 0, its gathered row indices and
// weight-block scales brought into LDS by DMA in step 1), so the next item
// starts with its operands landed and its prologue's DMA latency hides behind
// this item's epilogue.  Second projection at the Step-5 prefill: 0.80 ->
// 0.69 ms; the first projection, whose item loop is three times longer, is
// unchanged by it (and slower without it inside the same persistent walk).
#include <type_traits>
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
    const int4* items;          // per work item {group, first row, rows, n-tile}
    const int* xcd_start;       // XCD x runs items xcd_start[x] .. xcd_start[x + 1] - 1
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

// LDS after the operand ring: the epilogue's row maxima, and the next work
// item's gathered row indices and weight-block scales (brought in by DMA
// while the current item runs)
constexpr int RING_BYTES = STAGES * STAGE_BYTES;
constexpr int AUX_RED = RING_BYTES;                 // [128 rows][4 waves along N] floats
constexpr int AUX_ROWS = AUX_RED + 2048;            // 128 source-row entries
constexpr int AUX_SW = AUX_ROWS + 512;              // per wave: 2 rows of 64 weight-block scales
constexpr int SMEM_BYTES = AUX_SW + NW * 512;
// Items of at least this many K slices take the next item's first slices
// into the ring during their own last steps (the descriptor, row indices and
// scales are fetched in steps 0 and 1, the addresses made before step KB - 3).
constexpr int PIPE_MIN_KB = 8;

typedef const __attribute__((address_space(4))) int cint;

struct Item {
    int g, n_tile, row0, valid;
};

template <int MODE>
__global__ __launch_bounds__(NT, 1) void kernel(Params p) {
    __shared__ __attribute__((aligned(1024))) unsigned char smem[SMEM_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;

    // ---- this block's work items: slot, slot + slots, ... of its XCD's
    // range of the item table (written by a one-block launch first)
    const int xcd = blockIdx.x % NXCD, slot = blockIdx.x / NXCD, slots = gridDim.x / NXCD;
    const int r0 = __builtin_amdgcn_readfirstlane(p.xcd_start[xcd]);
    const int nit = __builtin_amdgcn_readfirstlane(p.xcd_start[xcd + 1]) - r0;
    if (slot >= nit) return;
    // the table is not written while this kernel runs: read it through the
    // scalar path, which the vector-memory counters the K loop's waits rely
    // on do not see
    cint* items = (cint*)(p.items + r0);          // 4 ints per item
    auto load_item = [&](int s) {
        Item it;
        it.g = __builtin_amdgcn_readfirstlane(items[4 * s]);
        it.row0 = __builtin_amdgcn_readfirstlane(items[4 * s + 1]);
        it.valid = __builtin_amdgcn_readfirstlane(min(items[4 * s + 2], BM));
        it.n_tile = __builtin_amdgcn_readfirstlane(items[4 * s + 3]);
        return it;
    };
    const int K = p.K, KB = K / BKB;
    // the second projection reads h rows in place (no gather)
    const bool gathered = MODE == SWIGLU && p.a_rows != nullptr;
    const unsigned lds_base = (unsigned)(size_t)(lds_u8*)smem;
    const int dq = lane >> 3;

    // weight-scale block rows of this wave's columns (wave-uniform); all 64
    // columns of a wave (32 + 32 for the gate/up pairs) sit in one 128-row block
    auto sw_rows = [&](const Item& it, int& ra, int& rb) {
        if (MODE == SWIGLU) {
            const int hbase = min(it.n_tile * (BN / 2) + 32 * wn, p.N - 1);
            ra = hbase / 128;
            rb = (p.N + hbase) / 128;
        } else {
            ra = rb = min(it.n_tile * BN + 64 * wn, p.N - 1) / 128;
        }
    };
    // DMAs of an item's row indices (waves 0 and 1: entry e = tile row e,
    // clamped to the item's rows) and of this wave's two weight-scale rows
    // (K blocks 0 .. 63, lane c block c), into the aux LDS
    auto aux_dmas = [&](const Item& it) {
        if (gathered && wave < 2)
            dma4(p.a_rows + it.row0 + min(64 * wave + lane, it.valid - 1),
                 __builtin_amdgcn_readfirstlane(lds_base + AUX_ROWS + 256 * wave));
        int ra, rb;
        sw_rows(it, ra, rb);
        const float* wsg = p.Ws + (int64_t)it.g * p.ws_group_stride;
        const int c = min(lane, KB - 1);
        dma4(wsg + (int64_t)ra * KB + c, __builtin_amdgcn_readfirstlane(lds_base + AUX_SW + 512 * wave));
        dma4(wsg + (int64_t)rb * KB + c, __builtin_amdgcn_readfirstlane(lds_base + AUX_SW + 512 * wave + 256));
    };
    const int n_aux = (gathered && wave < 2) ? 3 : 2;   // aux DMAs of this wave per item

    // ---- DMA sources of the item whose slices are being issued.  One DMA
    // instruction moves 8 rows x 128 B: lanes 8q .. 8q+7 read the whole
    // 128-byte line of row q; lane l reads chunk (l & 7) ^ line_swz(row) and
    // lands at LDS byte 16 l, so LDS chunk c of a row holds global chunk
    // c ^ line_swz(row).  Wave w moves A rows 16w .. 16w+15 and W rows
    // 32w .. 32w+31 of every slice.  Offsets are 32-bit from wave-uniform
    // bases (the launch checks the ranges).
    unsigned a_off[2], b_off[4];
    const float* sa_src;
    const uint8_t* Wg;
    auto src_row = [&](const Item& it, int r) {          // from the aux row entries
        int sr;
        if (gathered) sr = ((const int*)(smem + AUX_ROWS))[r] / p.a_div;
        else sr = it.row0 + min(r, it.valid - 1);
        return min(max(sr, 0), p.a_nrows - 1);
    };
    auto make_addrs = [&](const Item& it) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int r = 16 * wave + 8 * q + dq;
            a_off[q] = (unsigned)src_row(it, r) * (unsigned)K + 16u * ((lane & 7) ^ line_swz(r & 15));
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = 32 * wave + 8 * q + dq;               // tile column 0..255
            int wrow;
            if (MODE == SWIGLU) {
                // 64-column wave groups: 32 gate columns, then the matching 32 up columns
                const int wg = r >> 6, u = r & 63;
                const int hcol = min(it.n_tile * (BN / 2) + 32 * wg + (u & 31), p.N - 1);
                wrow = (u < 32) ? hcol : p.N + hcol;
            } else {
                wrow = min(it.n_tile * BN + r, p.N - 1);
            }
            b_off[q] = (unsigned)wrow * (unsigned)K + 16u * ((lane & 7) ^ line_swz(r & 15));
        }
        sa_src = p.As + src_row(it, 64 * (wave & 1) + lane);
        Wg = p.W + (int64_t)it.g * p.w_group_stride;
    };
    // this wave's DMA q of slice ks into `stage`: q 0, 1 A blocks, 2 .. 5 W
    // blocks, 6 the row scales (waves 0 and 1 only)
    auto issue_q = [&](int ks, int stage, int q) {
        const int k0 = ks * BKB;
        const unsigned sb = lds_base + stage * STAGE_BYTES;
        if (q < 2) dma16s(p.A + k0, a_off[q], __builtin_amdgcn_readfirstlane(sb + 1024 * (2 * wave + q)));
        else if (q < 6) dma16s(Wg + k0, b_off[q - 2], __builtin_amdgcn_readfirstlane(sb + A_BYTES + 1024 * (4 * wave + q - 2)));
        else if (wave < 2) dma4(sa_src + (int64_t)ks * p.a_ld, __builtin_amdgcn_readfirstlane(sb + SA_OFF + 256 * wave));
    };

    // A lane's 32 bytes of a fragment (row lane & 15 of a 16-row tile) are
    // global chunks (lane >> 4) and 4 + (lane >> 4) of the row: the same K
    // order in both operands, so the MFMA still sums the slice's 128 products
    // of every (row, column); the two reads hit distinct bank groups
    // (line_swz).  off0 is opaque so that no part of it is kept apart.
    const int fr = lane & 15;
    unsigned off0 = 128 * fr + 16 * ((lane >> 4) ^ line_swz(fr));
    asm volatile("" : "+v"(off0));
    const int quad4 = 4 * (lane >> 4);

    // ---- the first item: its aux data, addresses and first slices
    Item cur = load_item(slot);
    aux_dmas(cur);
    wait_vm<0>();
    __syncthreads();
    make_addrs(cur);
    int sbase = 0;                                    // stage of the item's slice 0
#pragma unroll
    for (int s = 0; s < STAGES; ++s)
#pragma unroll
        for (int q = 0; q < 7; ++q) issue_q(min(s, KB - 1), s, q);
    if (wave < 2) wait_vm<7 * (STAGES - 1)>(); else wait_vm<6 * (STAGES - 1)>();
    __builtin_amdgcn_s_barrier();

    for (int s = slot; s < nit; s += slots) {
        const bool has_next = s + slots < nit;
        const bool pipe = has_next && KB >= PIPE_MIN_KB;
        const int row0 = cur.row0, valid = cur.valid, n_tile = cur.n_tile;
        const int ntile_valid = (valid + 15) >> 4;
        int n_i = 0;
#pragma unroll
        for (int i = 0; i < TM; ++i) n_i += (wm + 2 * i < ntile_valid) ? 1 : 0;
        n_i = __builtin_amdgcn_readfirstlane(n_i);
        // lane c holds the scales of K blocks 64 m + c for the current chunk m
        // (the first chunk from the aux LDS; later ones loaded every 64 slices)
        int swr_a, swr_b;
        sw_rows(cur, swr_a, swr_b);
        const float* Wsg = p.Ws + (int64_t)cur.g * p.ws_group_stride;
        const float* swa_p = Wsg + (int64_t)swr_a * KB;
        const float* swb_p = Wsg + (int64_t)swr_b * KB;
        float swa_v = ((const float*)(smem + AUX_SW + 512 * wave))[lane];
        float swb_v = ((const float*)(smem + AUX_SW + 512 * wave + 256))[lane];

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
        auto read_frag = [&](const unsigned char* f) {
            const u32x4 lo = *(const u32x4*)(f + off0), hi = *(const u32x4*)(f + (off0 ^ 64u));
            return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        };
        auto stage_ptr = [&](int kt) { return smem + ((sbase + kt) % STAGES) * STAGE_BYTES; };
        auto read_a = [&](int kt, int i) { afr[i] = read_frag(stage_ptr(kt) + 2048 * (wm + 2 * i)); };
        auto read_sa = [&](int kt, int i) {
            sa[i] = ((const float*)(stage_ptr(kt) + SA_OFF))[16 * (wm + 2 * i) + fr];
        };
        auto read_b = [&](int kt, int j) { bfr[j] = read_frag(stage_ptr(kt) + A_BYTES + 2048 * (4 * wn + j)); };

        // slice 0 has landed (the previous item's last wait and barrier, or the
        // first item's prologue)
#pragma unroll
        for (int j = 0; j < TN; ++j) read_b(0, j);
#pragma unroll
        for (int i = 0; i < TM; ++i) { read_a(0, i); read_sa(0, i); }

        Item nxt = cur;
        // Slice kt sits in stage (sbase + kt) % STAGES.  Step kt multiplies
        // slice kt from registers; its stage then takes slice kt + STAGES --
        // of this item, or past its end the next item's first slices (pipe),
        // or clamped re-reads of the last slice (which keep the DMA count per
        // step fixed, as the waits rely on).  Slice kt+1 has landed when step
        // kt starts, so its fragments are read during step kt, each as soon
        // as its register is free: a tile's A fragment right after the tile's
        // MFMAs are issued, its row scale after its products are scaled, and
        // the W fragments after the last tile's MFMAs.  The DMAs sit between
        // the MFMA groups: issued in one burst after the barrier they queue at
        // the wave's issue and hold back its MFMAs.
        // PH 0: steps 0 .. 2 (the next item's descriptor and aux DMAs; in the
        // second projection also the steady steps), PH 1: the steady steps
        // (this item's slices only), PH 2: the last three steps (the next
        // item's first slices, or clamped re-reads); each phase is compiled on
        // its own, so the first projection's steady loop carries no step tests
        auto step = [&](auto ph_tag, int kt) {
            constexpr int PH = decltype(ph_tag)::value;
            // slice kt+1 has landed (at most the DMAs issued in step kt-1 are
            // outstanding: the slice's own and, in step 1 of a pipelined item,
            // the next item's aux DMAs, issued before them), and this wave's
            // reads of slice kt are done.  Stores of the previous item's
            // epilogue are not counted: they only make a wait longer.
            if (PH == 0 && pipe && kt == 2) {
                if (wave < 2) {
                    if (n_aux == 3) wait_vm<10>(); else wait_vm<9>();
                } else {
                    wait_vm<8>();
                }
            } else {
                if (wave < 2) wait_vm<7>(); else wait_vm<6>();
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);       // lgkmcnt(0), vmcnt/expcnt untouched
            __builtin_amdgcn_s_barrier();
            if (PH == 0 && pipe) {
                if (kt == 0) nxt = load_item(s + slots);
                if (kt == 1) aux_dmas(nxt);           // before this step's slice DMAs
            }
            const int sn = (sbase + kt) % STAGES;
            const int kn = PH == 1 ? kt + STAGES : kt + STAGES < KB ? kt + STAGES : (pipe ? kt + STAGES - KB : KB - 1);
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
                };
        using P0 = std::integral_constant<int, 0>;
        using P1 = std::integral_constant<int, 1>;
        using P2 = std::integral_constant<int, 2>;
        const int t_begin = max(0, KB - STAGES);
        if constexpr (MODE == SWIGLU) {
            // the head steps on their own (in the second projection's shorter
            // loop a third copy costs more registers than it saves)
            const int h_end = min(STAGES, t_begin);
            for (int kt = 0; kt < h_end; ++kt) step(P0{}, kt);
            for (int kt = h_end; kt < t_begin; ++kt) step(P1{}, kt);
        } else {
            for (int kt = 0; kt < t_begin; ++kt) step(P0{}, kt);
        }
        // the next item's addresses replace this item's once its last slice
        // is issued (step KB - STAGES - 1)
        if (pipe) make_addrs(nxt);
        for (int kt = t_begin; kt < KB; ++kt) step(P2{}, kt);
        // the last step waited for slice KB: with pipe the next item's slice 0
        if (!pipe) wait_vm<0>();

        if (MODE == SWIGLU) {
            // this wave's h: rows 16 (wm + 2i) + fr, h columns 32 wn + 16 j + quad4 + v (j < 2)
            float hv[TM][2][4];
            float* amax_l = (float*)(smem + AUX_RED);          // [128 rows][4 waves along N]
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
                m = max_lanes_xor16_32(m);                      // the row's 4 lanes
                if (quad4 == 0) amax_l[(16 * (wm + 2 * i) + fr) * 4 + wn] = m;
            }
            __syncthreads();
            uint8_t* Hq = (uint8_t*)p.C;
            const int kb = n_tile;                              // K block of the second projection
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                if (i >= n_i) continue;
                const int lr = 16 * (wm + 2 * i) + fr;
                const f32x4 m4 = *(const f32x4*)(amax_l + lr * 4);
                const float amax = fmaxf(fmaxf(m4.x, m4.y), fmaxf(m4.z, m4.w));
                const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
                const float rs = 1.0f / sc;
                if (lr < valid) {
                    if (wn == 0 && quad4 == 0) p.Cs[(int64_t)kb * p.c_ld + row0 + lr] = sc;
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
            float* red = (float*)(smem + AUX_RED);             // [128 rows][4 waves along N]
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
                m = max_lanes_xor16_32(m);                      // the row's 4 lanes
                if (quad4 == 0) red[lr * 4 + wn] = m;
            }
            __syncthreads();
            const int gw = wn & ~1;                             // first wave of this wave's group
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

        // ---- on to the next item
        if (pipe) {
            // its addresses are made and its first slices in the ring
            cur = nxt;
            sbase = (sbase + KB) % STAGES;
        } else if (has_next) {
            cur = load_item(s + slots);
            __syncthreads();                              // every wave is done with the ring and aux rows
            aux_dmas(cur);
            wait_vm<0>();
            __syncthreads();
            make_addrs(cur);
            sbase = 0;
#pragma unroll
            for (int st = 0; st < STAGES; ++st)
#pragma unroll
                for (int q = 0; q < 7; ++q) issue_q(min(st, KB - 1), st, q);
            if (wave < 2) wait_vm<7 * (STAGES - 1)>(); else wait_vm<6 * (STAGES - 1)>();
            __builtin_amdgcn_s_barrier();
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

static int f8_grid(int64_t work) { const int64_t g = (work + f8::NXCD - 1) / f8::NXCD * f8::NXCD; return (int)(g < 256 ? g : 256); }

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
    if (!items) return hipErrorInvalidValue;           // the kernel walks the item table
    {
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
    if (!items) return hipErrorInvalidValue;           // the kernel walks the item table
    {
        const hipError_t e = launch_item_table(offsets, tile_start, groups, 0, p.n_tiles, false, items, s);
        if (e != hipSuccess) return e;
        p.xcd_start = (const int*)items;
        p.items = (const int4*)((const char*)items + 64);
    }
    f8::kernel<f8::OUT_F16><<<f8_grid((int64_t)max_tiles * p.n_tiles), f8::NT, 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace moe
