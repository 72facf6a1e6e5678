// grouped_gemm.hip -- the routed experts' weight-streaming GEMMs on gfx950.
//
//   C[r, n] = sum_k A[src(r), k] * W_e[n, k]      for every row r of expert e
//
// Mode SWIGLU (first projection): the block's 256 weight rows are 128 gate
// rows and the matching 128 up rows, and the epilogue writes
// h = act(gate, up, L) in bf16 (clipped SwiGLU).  Mode F16 / F32 (second
// projection, shared expert): plain output.
//
// Block tile (rows x weight rows): 256 x 256 for batches with many rows per
// expert, 64 x 256 / 64 x 128 for few.  8 waves (two per SIMD); 256-row
// tiles as 4 along M x 2 along N, each wave 64 rows x 128 columns of
// 16x16x32 bf16 MFMA tiles.  Choices, each measured on MI355X:
//   * Operands go global -> LDS by direct DMA (global_load_lds_dwordx4), so
//     no registers stage them.  The DMA is issued from inline asm and its
//     completion is waited for explicitly (s_waitcnt vmcnt before the
//     barrier of the step that reads it): the compiler cannot tell which LDS
//     reads depend on which DMA and would otherwise wait for all of them at
//     every step.  The instruction has no destination register.
//   * 256-row tiles: K slices of 64, each DMA instruction 8 rows x 128 B
//     (whole lines), A in 2 LDS stages and W in 3 (160 KiB, no padding: an
//     XOR swizzle of the 16-byte chunks keeps the fragment reads free of
//     bank conflicts).  Each half slice's MFMAs run in four groups with this
//     wave's DMAs and next fragment reads between them; issued as one burst
//     after the barrier they held back the MFMAs (2.58 -> 2.43 ms for the
//     Step-5 prefill's first projection).
//   * 64-row tiles: K slices of 32, each DMA instruction 16 rows x 64 B
//     (4 lanes per row: spreading 16 lanes over 16 rows ran the address unit
//     at a quarter of the rate), 6 padded stages whose block offsets keep the
//     fragment reads (lane l: row l & 15, 16 bytes of chunk l >> 4) free of
//     bank conflicts.
//   * The fragments of the next (half) slice are read into registers while
//     the MFMAs of the current one run.
//   * 16-row tiles are dealt to the waves along M round-robin (tile t to
//     wave t % WM), so an expert's valid rows spread evenly over the SIMDs;
//     tiles past the expert's last row skip their MFMAs.
//   * A rows are gathered straight from x by the DMA (row_to_pair / k); no
//     permuted copy of x is written.
//   * Work order: (expert, n-tile, m-tile) with m fastest, so the m-tiles
//     that stream one weight panel are dispatched together and share it in
//     L2 (against n fastest: 2.34 -> 2.10 ms for the Step-5 prefill's first
//     projection, whose experts of up to 705 rows take up to 3 m-tiles);
//     each XCD (blocks b with b % 8 == x) takes a contiguous range of that
//     list.  256-row launches read each item's (expert, first row, rows,
//     n-tile) from a table a one-block launch writes first (one load instead
//     of a binary search over the tile plan: 2.10 -> 2.02 ms).
#include <type_traits>
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace gg {

constexpr int BK = 32;    // K slice of the 64-row tiles
constexpr int BK2 = 64;   // K slice of the 256-row tiles
// One DMA block is 16 rows x 64 B.  The 4 blocks of a 64-row group start at
// these byte offsets: 16-byte bank groups 0, 2, 16, 18 (mod 32), which makes
// every 32-lane pass of a fragment read touch 32 distinct bank groups.
__device__ constexpr int BLK_OFF[4] = {0, 1024 + 32, 2048 + 256, 3072 + 288};
constexpr int GROUP = 3072 + 288 + 1024;   // 4 blocks = 64 rows of one K slice
constexpr int NXCD = 8;

// Tile shapes (rows BM x weight rows BN):
//   256 x 256 (prefill): 8 waves as 4 along M x 2 along N, each 64 x 128;
//   64 x 256 (few rows per expert): 8 waves along N, each 64 x 32, so no
//     DMA and no LDS go to rows that are not there;
//   64 x 128 (few rows, plain output): 8 waves along N, each 64 x 16 -- twice
//     the work items, for launches whose item count would leave a ragged
//     last round on 256 CUs.
template <int BM, int BN>
struct Shape {
    static constexpr int NW = 8;                       // waves per block
    static constexpr int NT = NW * 64;                 // threads per block
    static constexpr int WM = BM / 64;                 // waves along M
    static constexpr int WN = NW / WM;                 // waves along N
    static constexpr int TM = BM / 16 / WM;            // 16-row tiles per wave
    static constexpr int TN = BN / 16 / WN;            // 16-col tiles per wave
    static constexpr int GW = BN / WN;                 // columns per wave
    static constexpr int NA = BM / 16;                 // A DMA blocks per slice
    static constexpr int NB = BN / 16;                 // B DMA blocks per slice
    static constexpr int A_OPERAND = (BM / 64) * GROUP;
    static constexpr int STAGE_BYTES = A_OPERAND + (BN / 64) * GROUP;
    static constexpr int STAGES = BM == 256 ? 4 : 6;
    // epilogue staging through LDS (BM 256): rows per pass
    static constexpr int EPI_ROWS = 128;
    // operand LDS: 256-row tiles hold A in 2 and W in 3 stages of K 64
    // (128 B per row); 64-row tiles STAGES stages of K 32
    static constexpr int OPER = BM == 256 ? 2 * BM * 128 + 3 * BN * 128 : STAGES * STAGE_BYTES;
    static constexpr int SMEM = OPER > EPI_ROWS * (BN + 4) * 4 ? OPER : EPI_ROWS * (BN + 4) * 4;
};

// SWIGLU_SAVE: SWIGLU that also writes the pre-activations (gu_out)
enum { SWIGLU = 0, OUT_F16 = 1, OUT_F32 = 2, SWIGLU_SAVE = 3 };
constexpr bool is_swiglu(int mode) { return mode == SWIGLU || mode == SWIGLU_SAVE; }

struct Params {
    const uint16_t* A;          // bf16 activations
    const int32_t* a_rows;      // gather: A row = a_rows[r] / a_div; nullptr: row r
    int a_div;
    int a_nrows;                // rows of A (gather clamp)
    const uint16_t* W;          // bf16 weights [groups][Nw][K]
    int64_t w_group_stride;
    void* C;
    int N;                      // output columns (SWIGLU: h width, W has 2N rows)
    int K;
    float limit;
    const int32_t* offsets;     // [groups+1] row offsets; nullptr: dense with M rows
    const int32_t* tile_start;  // [groups+2] BM-tile plan (grouped)
    int groups;
    int M;                      // dense rows
    int n_tiles;                // BN tiles along N (SWIGLU: of 2N weight rows)
    // optional extra group (index `groups`): extra_rows rows after
    // offsets[groups], its own weights and clip limit -- the shared expert
    // run in the same launch; when A is gathered (a_rows), the extra group's
    // A row is row - offsets[groups] (the token) instead
    int extra_rows;
    const uint16_t* W_extra;
    float limit_extra;
    uint16_t* gu_out;           // SWIGLU (optional): the pre-activations [rows][2N] bf16, gate then up
    const int4* items;          // grouped (optional): per work item {group, first row, rows, n-tile}
    const int* xcd_start;       // with items: XCD x runs routed items xcd_start[x] .. xcd_start[x + 1] - 1
    int64_t c_row_bytes;        // OUT_F16: bytes per output row (scaled fp16 rows)
    int rot_group;              // dense (>= 0): take the K rotation of group rot_group, so a dense
                                // launch adds in the order of that group's grouped launch;
                                // -2: the router's order (router_chunk_rot by 64-row tile)
};

typedef __attribute__((address_space(3))) unsigned char lds_u8;

// one 1 KiB block: lane l's 16 bytes from g land at LDS byte lds_off + 16*l
__device__ __forceinline__ void dma_frag(const void* g, unsigned lds_off) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_off), "v"(g) : "memory");
}

// the same from a wave-uniform 64-bit base plus this lane's 32-bit byte offset
__device__ __forceinline__ void dma_frag_s(const void* base, unsigned off, unsigned lds_off) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_off), "v"(off), "s"(base) : "memory");
}

// two fp32 -> packed bf16 by the gfx950 conversion instruction (one
// v_cvt_pk_bf16_f32, round to nearest even like f32_to_bf16; NaN stays NaN)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2_hw(float lo, float hi) {
    const bf16x2_t b = __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t);
    return __builtin_bit_cast(uint32_t, b);
}

// wait until at most n vector-memory operations of this wave are outstanding
template <int n>
__device__ __forceinline__ void wait_vm() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

// Work items: grouped, (group, n-tile, m-tile) with m fastest, from the tile
// plan; dense, (n-tile, m-tile).  The routed items and the extra group's are
// two segments, each cut into 8 contiguous ranges, one per XCD (block b runs
// on XCD b % 8), so the blocks that share a weight panel run on one L2: the
// extra group's in equal shares, the routed ones by the item table's
// cost-balanced ranges (equal shares of the count without a table).  An XCD
// runs its extra-group items (full tiles) first, then its routed ones.
struct Segments {
    int total1, per1, total2, per2;           // routed / extra items, per-XCD range lengths
};
template <bool GROUPED, int BM>
__device__ __forceinline__ Segments segments(const Params& p) {
    Segments g;
    if (GROUPED) {
        g.total1 = p.tile_start[p.groups] * p.n_tiles;
        g.total2 = p.extra_rows > 0 ? (p.tile_start[p.groups + 1] - p.tile_start[p.groups]) * p.n_tiles : 0;
    } else {
        g.total1 = ((p.M + BM - 1) / BM) * p.n_tiles;
        g.total2 = 0;
    }
    g.per1 = (g.total1 + NXCD - 1) / NXCD;
    g.per2 = (g.total2 + NXCD - 1) / NXCD;
    return g;
}

// one work item w of the list
template <int MODE, bool GROUPED, int BM, int BN>
__device__ __forceinline__ void run_item(const Params& p, int w, unsigned char* smem) {
    using S = Shape<BM, BN>;
    constexpr int STAGES = S::STAGES, STAGE_BYTES = S::STAGE_BYTES, TN = S::TN, TM = S::TM, NW = S::NW,
                  NT = S::NT;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / S::WN, wn = wave % S::WN;

    // ---- decode the work item ------------------------------------------
    int g = 0, m_tile = 0, n_tile, row0, row_end;
    if (GROUPED) {
        if (p.items) {
            const int4 d = p.items[w];
            g = __builtin_amdgcn_readfirstlane(d.x);
            row0 = __builtin_amdgcn_readfirstlane(d.y);
            row_end = row0 + __builtin_amdgcn_readfirstlane(d.z);
            n_tile = __builtin_amdgcn_readfirstlane(d.w);
        } else {
            // group owning work item w: largest g with tile_start[g]*n_tiles <= w
            int lo = 0, hi = p.groups + (p.extra_rows > 0 ? 1 : 0) - 1;
            while (lo < hi) {
                int mid = (lo + hi + 1) >> 1;
                if (p.tile_start[mid] * p.n_tiles <= w) lo = mid; else hi = mid - 1;
            }
            g = lo;
            const int mt = p.tile_start[g + 1] - p.tile_start[g];
            const int local = w - p.tile_start[g] * p.n_tiles;
            n_tile = local / mt;
            m_tile = local % mt;
            // the group's rows are split evenly over its mt tiles (each at most
            // BM rows, as mt = ceil(rows / BM)): the m-tiles of one weight panel
            // then do the same work at the same pace
            const int base = p.offsets[g];
            const int cnt = (g < p.groups ? p.offsets[g + 1] : base + p.extra_rows) - base;
            row0 = base + (int)(((int64_t)m_tile * cnt) / mt);
            row_end = base + (int)(((int64_t)(m_tile + 1) * cnt) / mt);
        }
    } else {
        const int mt = (p.M + BM - 1) / BM;
        n_tile = w / mt;
        m_tile = w % mt;
        row0 = m_tile * BM;
        row_end = p.M;
    }
    const bool extra = GROUPED && g == p.groups;
    const int valid = min(row_end - row0, BM);
    const int K = p.K;
    const uint16_t* Wg = extra ? p.W_extra : p.W + (int64_t)g * p.w_group_stride;
    const float limit = extra ? p.limit_extra : p.limit;
    // K-slice rotation: the K loop starts at slice `rot`.  Weight and x rows
    // are 8 KiB apart in the Step-5 shapes, so one K slice of all rows of a
    // tile sits on few HBM channels; blocks that start at different slices
    // spread over the channels (measured: 5.0 -> 6.4 TB/s for this DMA
    // pattern).  One rotation per expert (per n-tile when dense) keeps the
    // blocks that share an A tile (grouped) or a weight panel (dense) in step.
    // K slices: 64 (128 B of a row) for 256-row tiles, 32 for 64-row tiles
    const int nk = K / (BM == 256 ? BK2 : BK);   // K % 64 == 0
    // (the router's dense launch, rot_group -2, takes the chunk order of
    // router_chunk_rot by 64-row tile: 8 slices of 32 per chunk)
    const int rot = GROUPED ? (g + 1) * 37 % nk
                    : (p.rot_group == -2 && nk % 8 == 0) ? 8 * router_chunk_rot(m_tile, nk / 8)
                    : ((p.rot_group >= 0 ? p.rot_group : n_tile) + 1) * 37 % nk;

    // valid 16-row tiles of this wave: tiles wm + WM i with 16 (wm + WM i) < valid
    const int ntile_valid = (valid + 15) >> 4;
    int n_i = 0;
#pragma unroll
    for (int i = 0; i < TM; ++i) n_i += (wm + S::WM * i < ntile_valid) ? 1 : 0;
    n_i = __builtin_amdgcn_readfirstlane(n_i);

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    if constexpr (BM == 256) {
        // ---- 256-row tiles: K slices of 64, whole 128-byte lines per DMA ----
        // One DMA instruction moves 8 rows x 128 B: lanes 8q .. 8q+7 read the
        // 128-byte line of row q, so every request is a whole line (half the
        // L2 requests of 64-byte pieces for the same bytes).  A block lands at
        // LDS byte 16 l per lane l, i.e. rows of 128 B back to back; lane l
        // reads the line's 16-byte chunk (l & 7) ^ line_swz(row), so LDS
        // chunk p of a row holds global chunk p ^ line_swz(row).  A fragment
        // read (lane l: row l & 15 of a 16-row tile, K chunk 4 sub + (l >> 4))
        // is then free of bank conflicts (see line_swz).  LDS: A in 2 stages,
        // W in 3 (W is the operand that streams from HBM, so it gets the
        // longer lead), 160 KiB.
        // Wave w moves A blocks 4w .. 4w+3 (rows 32w .. 32w+31) and W blocks
        // 4w .. 4w+3 of every slice.
        constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;
        constexpr int NQA = BM / 8 / NW, NQB = BN / 8 / NW;      // DMA blocks per wave
        const int dq = lane >> 3;                                 // row within the DMA block
        // A blocks of a wave whose rows all lie past the valid ones are not
        // moved (their tiles are not multiplied; a 16-row tile that is only
        // partly valid reads clamped copies, or stale LDS for rows of a block
        // not moved, which only reach output rows that are not written)
        const bool a_mine = 32 * wave < valid;
        // sources as 32-bit byte offsets from a wave-uniform base (gathered
        // rows: all of A, which the launch checks is under 4 GiB; otherwise
        // the tile's first row)
        const bool gather = GROUPED && p.a_rows;
        const uint16_t* a_base = gather ? p.A : p.A + (int64_t)row0 * K;
        unsigned a_off[NQA];
#pragma unroll
        for (int q = 0; q < NQA; ++q) {
            const int r = 8 * (NQA * wave + q) + dq;              // tile row 0..255
            const int c = (lane & 7) ^ line_swz(r & 15);
            int ar = min(r, valid - 1);
            if (gather) {
                ar += row0;
                ar = extra ? ar - p.offsets[p.groups] : p.a_rows[ar] / p.a_div;
                ar = min(max(ar, 0), p.a_nrows - 1);
            }
            a_off[q] = (unsigned)ar * (unsigned)(2 * K) + 16u * c;
        }
        // W rows of this wave's DMA q: wave-uniform w_add + min(w_base + 8 q +
        // dq, w_last), computed at each DMA from two lane values (the four
        // offsets would hold registers through the loop).  SwiGLU: the wave's
        // 32 columns of a slice are gate rows (waves 4g, 4g+1 of column group
        // g) or the matching up rows (4g+2, 4g+3).
        int w_add, w_base, w_last;
        if (is_swiglu(MODE)) {
            w_add = (wave & 3) < 2 ? 0 : p.N;
            w_base = n_tile * (BN / 2) + (S::GW / 2) * (8 * NQB * wave / S::GW) + 32 * (wave & 1);
            w_last = p.N - 1;
        } else {
            w_add = 0;
            w_base = n_tile * BN + 32 * wave;
            w_last = p.N - 1;
        }
        static_assert(NQB == 4 && S::GW == 128, "the W row formula assumes 32 columns per wave and slice");
        // chunk of even / odd q (tile column 8 (4 wave + q) + dq: row 8 (q & 1) + dq of its 16)
        const unsigned b_chunk0 = 16u * ((lane & 7) ^ line_swz(dq));
        const unsigned b_chunk1 = 16u * ((lane & 7) ^ line_swz(8 + dq));
        auto b_off = [&](int q) {
            const int wrow = w_add + min(w_base + 8 * q + dq, w_last);
            return (unsigned)wrow * (unsigned)(2 * K) + ((q & 1) ? b_chunk1 : b_chunk0);
        };
        const unsigned lds_base = (unsigned)(size_t)(lds_u8*)smem;
        auto issue_a = [&](int kt, int stage) {
            const int ks = kt + rot < nk ? kt + rot : kt + rot - nk;
            const unsigned sb = lds_base + stage * A_BYTES + NQA * wave * 1024;
            if (a_mine) {
#pragma unroll
                for (int q = 0; q < NQA; ++q)
                    dma_frag_s(a_base + ks * BK2, a_off[q], __builtin_amdgcn_readfirstlane(sb + 1024 * q));
            }
        };
        auto issue_b = [&](int kt, int stage) {
            const int ks = kt + rot < nk ? kt + rot : kt + rot - nk;
            const unsigned sb = lds_base + 2 * A_BYTES + stage * B_BYTES + NQB * wave * 1024;
#pragma unroll
            for (int q = 0; q < NQB; ++q)
                dma_frag_s(Wg + ks * BK2, b_off(q), __builtin_amdgcn_readfirstlane(sb + 1024 * q));
        };
        // lane's byte offset in a 16-row tile for K chunk 4 sub + (lane >> 4)
        const int fr = lane & 15, sw = line_swz(fr);
        unsigned off0 = 128 * fr + 16 * ((lane >> 4) ^ sw);
        // opaque to the compiler: otherwise it keeps 128 fr apart through the
        // item loop, spills it, and its reload after the prologue barrier
        // waits for every DMA in flight (vmcnt 0)
        asm volatile("" : "+v"(off0));
        const unsigned off1 = off0 ^ 64u;         // chunk 4 + c: (c ^ sw) ^ 4
        // The loop is compiled once per count of this wave's valid 16-row
        // tiles (0..TM): a wave reads only the fragments its MFMAs use,
        // with no branch inside the loop (a branch around the reads breaks
        // the interleaved schedule).
        auto kloop = [&](auto ni_tag) {
            constexpr int NI = decltype(ni_tag)::value;
            bf16x8 xa[TM], xb[TN], ya[TM], yb[TN];
            auto read_frags = [&](int kt, unsigned off, bf16x8* a, bf16x8* b) {
                const unsigned char* sa = smem + (kt & 1) * A_BYTES;
                const unsigned char* sb = smem + 2 * A_BYTES + (kt % 3) * B_BYTES;
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    if (NI > 0) b[j] = *(const bf16x8*)(sb + 2048 * (wn * TN + j) + off);
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    if (i < NI) a[i] = *(const bf16x8*)(sa + 2048 * (wm + S::WM * i) + off);
            };
            // Slice kt's A sits in stage kt % 2, its W in stage kt % 3.  Step kt
            // multiplies the slice's two K halves; between them (its reads done,
            // slice kt+1 landed) the barrier frees its stages, which take A of
            // kt+2 and W of kt+3 (clamped re-reads past the end keep the DMA count
            // per step fixed, which the waits rely on).  DMAs complete in order and
            // the last ones issued before step kt's wait are the previous step's
            // A of kt+1, then W of kt+2: at most NQB outstanding means A and W of
            // slice kt+1 have landed.
            issue_a(0, 0);
            issue_b(0, 0);
            issue_a(min(1, nk - 1), 1);
            issue_b(min(1, nk - 1), 1);
            issue_b(min(2, nk - 1), 2);
            if (a_mine) wait_vm<2 * NQB + NQA>(); else wait_vm<2 * NQB>();
            __builtin_amdgcn_s_barrier();
            read_frags(0, off0, xa, xb);
            // The MFMAs take the W fragment as their first operand, so the tile
            // comes out transposed: lane l holds row l & 15 and 4 consecutive
            // columns, which the epilogue stores as whole 8- or 16-byte pieces.
            // Each half step runs its MFMAs in TM groups (one 16-row tile each)
            // and puts this wave's memory instructions between the groups: the
            // LDS reads of the other half's fragments, and after the barrier two
            // DMAs per group (A in the first half of the groups, W in the
            // second).  Issued in one burst they queue at the wave's issue (the
            // address and LDS units take one instruction at a time from all
            // waves) and hold back its MFMAs.
            static_assert(TM == NQA && TM == NQB && TM % 2 == 0 && TN % TM == 0, "two DMAs per 16-row tile group");
            constexpr int JG = TN / TM;               // W fragments read per group
            for (int kt = 0; kt < nk; ++kt) {
                {
                    const unsigned char* sa = smem + (kt & 1) * A_BYTES;
                    const unsigned char* sb = smem + 2 * A_BYTES + (kt % 3) * B_BYTES;
#pragma unroll
                    for (int i = 0; i < TM; ++i) {
                        if (i < NI) ya[i] = *(const bf16x8*)(sa + 2048 * (wm + S::WM * i) + off1);
#pragma unroll
                        for (int jj = 0; jj < JG; ++jj)
                            if (NI > 0) yb[JG * i + jj] = *(const bf16x8*)(sb + 2048 * (wn * TN + JG * i + jj) + off1);
                        if (i < NI) {
#pragma unroll
                            for (int j = 0; j < TN; ++j)
                                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb[j], xa[i], acc[i][j], 0, 0, 0);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
                wait_vm<NQB>();                       // slice kt+1 has landed
                __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's reads of slice kt are done
                __builtin_amdgcn_s_barrier();
                {
                    const int ka = min(kt + 2, nk - 1), kb = min(kt + 3, nk - 1);
                    const int ksa = ka + rot < nk ? ka + rot : ka + rot - nk;
                    const int ksb = kb + rot < nk ? kb + rot : kb + rot - nk;
                    const unsigned da = lds_base + (kt & 1) * A_BYTES + NQA * wave * 1024;
                    const unsigned db = lds_base + 2 * A_BYTES + (kt % 3) * B_BYTES + NQB * wave * 1024;
                    const unsigned char* sa = smem + ((kt + 1) & 1) * A_BYTES;
                    const unsigned char* sb = smem + 2 * A_BYTES + ((kt + 1) % 3) * B_BYTES;
                    const bool more = kt + 1 < nk;
#pragma unroll
                    for (int i = 0; i < TM; ++i) {
                        // all A DMAs of the step before all W DMAs: the wait
                        // above relies on W being the last NQB issued
                        if (i < TM / 2) {
                            if (a_mine) {
                                dma_frag_s(a_base + ksa * BK2, a_off[2 * i],
                                           __builtin_amdgcn_readfirstlane(da + 2048 * i));
                                dma_frag_s(a_base + ksa * BK2, a_off[2 * i + 1],
                                           __builtin_amdgcn_readfirstlane(da + 2048 * i + 1024));
                            }
                        } else {
                            const int q = 2 * (i - TM / 2);
                            dma_frag_s(Wg + ksb * BK2, b_off(q), __builtin_amdgcn_readfirstlane(db + 1024 * q));
                            dma_frag_s(Wg + ksb * BK2, b_off(q + 1),
                                       __builtin_amdgcn_readfirstlane(db + 1024 * (q + 1)));
                        }
                        if (more) {
                            if (i < NI) xa[i] = *(const bf16x8*)(sa + 2048 * (wm + S::WM * i) + off0);
#pragma unroll
                            for (int jj = 0; jj < JG; ++jj)
                                if (NI > 0)
                                    xb[JG * i + jj] = *(const bf16x8*)(sb + 2048 * (wn * TN + JG * i + jj) + off0);
                        }
                        if (i < NI) {
#pragma unroll
                            for (int j = 0; j < TN; ++j)
                                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(yb[j], ya[i], acc[i][j], 0, 0, 0);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
        };
        switch (n_i) {
            case 0: kloop(std::integral_constant<int, 0>{}); break;
            case 1: kloop(std::integral_constant<int, 1>{}); break;
            case 2: kloop(std::integral_constant<int, 2>{}); break;
            case 3: kloop(std::integral_constant<int, 3>{}); break;
            default: kloop(std::integral_constant<int, TM>{}); break;
        }
        wait_vm<0>();
    } else {
    // ---- DMA sources.  One DMA instruction moves a block of 16 rows x 64 B
    // (one K slice of 32): lane l reads 16 B of row quad l >> 2 at chunk
    // l & 3, so every 4 lanes read 64 contiguous bytes (the address unit
    // then runs at ~4x the rate of 16 distinct rows per 16 lanes), and lands
    // at LDS byte 16*l of the block.  Block b (0..3) of row group g (64 rows)
    // holds tile rows 64g + 16t + 4b + i for quad 4t + i, so the 16 rows of
    // a 16-row MFMA tile come 4 apiece from the 4 blocks; with the block
    // offsets of BLK_OFF, each 32-lane pass of a ds_read_b128 hits 32
    // distinct bank groups.  Wave w moves B blocks (BN/128) w + q and A blocks
    // 2w, 2w+1 (BM 256) or A block w for w < 4 (BM 64) of every slice.
    // Grouped 64-row tiles hold A differently: block b is the 16-row MFMA
    // tile b (quad q = its row q, chunks XOR-swizzled by (q >> 2) & 3), so a
    // tile of few rows (decode: ~15 per expert) moves one A block per slice
    // instead of four.  (The counter reads some bank conflicts for it; dense
    // 64-row launches, whose tiles are full, keep the layout above.)
    constexpr int A_PER_WAVE = S::NA >= NW ? S::NA / NW : 1;
    // A blocks hold only valid rows of their group (BM 256) or tile (BM 64):
    // a wave whose rows all lie past the valid ones moves none (those rows
    // are never multiplied)
    constexpr bool A_TILED = BM == 64 && GROUPED;
    const bool a_mine = S::NA >= NW ? 64 * ((A_PER_WAVE * wave) >> 2) < valid
                                    : (wave < S::NA && (!A_TILED || 16 * wave < valid));
    const int quad = lane >> 2, chunk = lane & 3;
    auto block_row = [&](int blk) { return 64 * (blk >> 2) + 16 * (quad >> 2) + 4 * (blk & 3) + (quad & 3); };
    const uint16_t* a_src[A_PER_WAVE];
    unsigned a_lds[A_PER_WAVE];
#pragma unroll
    for (int q = 0; q < A_PER_WAVE; ++q) {
        const int blk = S::NA >= NW ? A_PER_WAVE * wave + q : min(wave, S::NA - 1);
        // the gathered activation row (clamped inside the group, and to A)
        int ar = row0 + min(A_TILED ? 16 * blk + quad : block_row(blk), valid - 1);
        if (GROUPED && p.a_rows) {
            // gathered rows (first projection): pair / k, or the token itself
            // for the extra group; otherwise A rows are the output rows
            ar = extra ? ar - p.offsets[p.groups] : p.a_rows[ar] / p.a_div;
            ar = min(max(ar, 0), p.a_nrows - 1);
        }
        a_src[q] = p.A + (int64_t)ar * K + (A_TILED ? chunk ^ ((quad >> 2) & 3) : chunk) * 8;
        a_lds[q] = (blk >> 2) * GROUP + BLK_OFF[blk & 3];
    }
    constexpr int B_PER_WAVE = S::NB / NW;
    const uint16_t* b_src[B_PER_WAVE];
    unsigned b_lds[B_PER_WAVE];
#pragma unroll
    for (int q = 0; q < B_PER_WAVE; ++q) {
        const int blk = B_PER_WAVE * wave + q;            // 0 .. NB-1
        const int r = block_row(blk);                     // tile column 0..255
        int wrow;
        if (is_swiglu(MODE)) {
            // each wave's GW columns: GW/2 gate columns, then the matching GW/2 up columns
            const int grp = r / S::GW, u = r % S::GW;
            const int hcol = min(n_tile * (BN / 2) + (S::GW / 2) * grp + u % (S::GW / 2), p.N - 1);
            wrow = (u < S::GW / 2) ? hcol : p.N + hcol;
        } else {
            wrow = min(n_tile * BN + r, p.N - 1);
        }
        b_src[q] = Wg + (int64_t)wrow * K + chunk * 8;
        b_lds[q] = S::A_OPERAND + (blk >> 2) * GROUP + BLK_OFF[blk & 3];
    }
    const unsigned lds_base = (unsigned)(size_t)(lds_u8*)smem;
    auto issue = [&](int kt, int stage) {
        const int ks = kt + rot < nk ? kt + rot : kt + rot - nk;
        const int k0 = ks * BK;
        const unsigned sb = lds_base + stage * STAGE_BYTES;
        if (a_mine) {
#pragma unroll
            for (int q = 0; q < A_PER_WAVE; ++q) dma_frag(a_src[q] + k0, __builtin_amdgcn_readfirstlane(sb + a_lds[q]));
        }
#pragma unroll
        for (int q = 0; q < B_PER_WAVE; ++q) dma_frag(b_src[q] + k0, __builtin_amdgcn_readfirstlane(sb + b_lds[q]));
    };
    // LDS byte offset of this lane's 16 B in 16-row tile tau = 4g + t:
    // g * GROUP + 256 t + lane_off (row r = lane & 15 from block r >> 2,
    // quad 4t + (r & 3); chunk lane >> 4)
    const int fr = lane & 15;
    const unsigned lane_off = BLK_OFF[fr >> 2] + 64 * (fr & 3) + 16 * (lane >> 4);
    auto tile_off = [&](int tau) { return (unsigned)((tau >> 2) * GROUP + 256 * (tau & 3)) + lane_off; };
    // grouped 64-row tiles' A: tile tau is block tau, row fr at 64 fr, chunk swizzled
    const unsigned a64_off = 64 * fr + 16 * ((lane >> 4) ^ ((fr >> 2) & 3));
    auto a_tile_off = [&](int tau) { return A_TILED ? (unsigned)BLK_OFF[tau & 3] + a64_off : tile_off(tau); };


    // prologue: slices 0 .. STAGES-1 in flight, one per stage (clamped re-reads
    // past the end keep the per-step DMA count fixed, which the waits below
    // rely on)
#pragma unroll
    for (int s = 0; s < STAGES; ++s) issue(min(s, nk - 1), s);

    // fragments of one slice, double-buffered in registers: the LDS reads of
    // slice kt+1 are issued before the MFMAs of slice kt, so they overlap
    bf16x8 fa[2][TM], fb[2][TN];
    auto read_frags = [&](int stage, bf16x8* a, bf16x8* b) {
        const unsigned char* st = smem + stage * STAGE_BYTES;
#pragma unroll
        for (int j = 0; j < TN; ++j) b[j] = *(const bf16x8*)(st + S::A_OPERAND + tile_off(wn * TN + j));
#pragma unroll
        for (int i = 0; i < TM; ++i)   // rows past the end hold clamped copies: reading them is safe
            a[i] = *(const bf16x8*)(st + a_tile_off(wm + S::WM * i));
    };
    auto mfmas = [&](const bf16x8* a, const bf16x8* b) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            if (i < n_i) {
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
            }
        }
    };
    // DMAs per slice of this wave: B_PER_WAVE + A_PER_WAVE if it moves A blocks
    constexpr int D_HI = B_PER_WAVE + A_PER_WAVE, D_LO = B_PER_WAVE;
    // one step: slice kt's fragments are in registers (cur), so its stage is
    // free: refill it with slice kt+STAGES, make slice kt+1 visible, read it
    // (nxt), multiply slice kt.  Slices kt+1 .. kt+STAGES occupy the stages,
    // so each DMA has STAGES-1 steps to land.
    auto step = [&](int kt, const bf16x8* ca, const bf16x8* cb, bf16x8* na, bf16x8* nb) {
        // slices kt+2 .. kt+STAGES-1 may stay in flight; this wave's reads of
        // slice kt have completed (its stage is refilled after the barrier)
        if (a_mine) wait_vm<D_HI * (STAGES - 2)>(); else wait_vm<D_LO * (STAGES - 2)>();
        __builtin_amdgcn_s_waitcnt(0xc07f);       // lgkmcnt(0), vmcnt/expcnt untouched
        __builtin_amdgcn_s_barrier();
        issue(min(kt + STAGES, nk - 1), kt % STAGES);
        read_frags((kt + 1 < nk ? kt + 1 : kt) % STAGES, na, nb);
        mfmas(ca, cb);
    };

    if (a_mine) wait_vm<D_HI * (STAGES - 1)>(); else wait_vm<D_LO * (STAGES - 1)>();
    __builtin_amdgcn_s_barrier();
    read_frags(0, fa[0], fb[0]);
    for (int kt = 0; kt < nk; kt += 2) {
        step(kt, fa[0], fb[0], fa[1], fb[1]);
        step(kt + 1, fa[1], fb[1], fa[0], fb[0]);
    }
    wait_vm<0>();
    }

    // ---- epilogue ----------------------------------------------------------
    // 64-row tiles: lane holds column (lane & 15), rows 4 (lane >> 4) + v.
    // 256-row tiles (weights as the MFMAs' first operand): lane holds row
    // lane & 15 and the 4 consecutive columns 4 (lane >> 4) + v.
    const int ccol = lane & 15, crow = (lane >> 4) * 4;
    if (BM == 256) {
        // SwiGLU: each lane stores its 4 h values (and, when kept, the 4
        // gate and 4 up values) as 8 contiguous bytes straight from
        // registers (2.36 against 2.42 ms staged, Step-5 first projection);
        // so do the scaled fp16 rows (below).  The fp32 output goes through
        // LDS and is written as whole rows of 256 columns, which measured
        // faster for it (105 against 108 us for the dense 8192-row second
        // projection).
        const int lrow = lane & 15, lcol = 4 * (lane >> 4);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            if (i >= n_i) continue;
            const int lr = 16 * (wm + S::WM * i) + lrow;
            if (lr >= valid) continue;
            const int64_t r = row0 + lr;
            const int hc0 = n_tile * (BN / 2) + (S::GW / 2) * wn;
            if (MODE == SWIGLU && hc0 + S::GW / 2 <= p.N) {
                // the wave's h columns all inside N: h tiles j and j+1 through
                // one lane swap (as the second projection's rows below), 16
                // bytes per lane
#pragma unroll
                for (int j = 0; j < TN / 2; j += 2) {
                    float ha[4], hb[4];
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        ha[v] = swiglu_clip(acc[i][j][v], acc[i][j + TN / 2][v], limit);
                        hb[v] = swiglu_clip(acc[i][j + 1][v], acc[i][j + 1 + TN / 2][v], limit);
                    }
                    const auto s0 = __builtin_amdgcn_permlane16_swap(pack_bf16x2_hw(ha[0], ha[1]),
                                                                     pack_bf16x2_hw(hb[0], hb[1]), false, false);
                    const auto s1 = __builtin_amdgcn_permlane16_swap(pack_bf16x2_hw(ha[2], ha[3]),
                                                                     pack_bf16x2_hw(hb[2], hb[3]), false, false);
                    const int hcol = hc0 + 16 * (j + ((lane >> 4) & 1)) + 4 * ((lane >> 4) & ~1);
                    *(uint4*)((uint16_t*)p.C + r * p.N + hcol) = make_uint4(s0[0], s1[0], s0[1], s1[1]);
                }
            } else if (is_swiglu(MODE)) {
#pragma unroll
                for (int j = 0; j < TN / 2; ++j) {
                    const int hcol = n_tile * (BN / 2) + (S::GW / 2) * wn + 16 * j + lcol;
                    if (hcol >= p.N) continue;
                    uint2 hv;
                    if (MODE == SWIGLU_SAVE) {
                        uint16_t gq[4], uq[4];
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            gq[v] = f32_to_bf16(acc[i][j][v]);
                            uq[v] = f32_to_bf16(acc[i][j + TN / 2][v]);
                        }
                        *(uint2*)(p.gu_out + r * 2 * p.N + hcol) =
                            make_uint2(gq[0] | ((uint32_t)gq[1] << 16), gq[2] | ((uint32_t)gq[3] << 16));
                        *(uint2*)(p.gu_out + r * 2 * p.N + p.N + hcol) =
                            make_uint2(uq[0] | ((uint32_t)uq[1] << 16), uq[2] | ((uint32_t)uq[3] << 16));
                        float hh[4];
#pragma unroll
                        for (int v = 0; v < 4; ++v) hh[v] = swiglu_clip(bf16_to_f32(gq[v]), bf16_to_f32(uq[v]), limit);
                        hv = make_uint2(pack_bf16x2(hh[0], hh[1]), pack_bf16x2(hh[2], hh[3]));
                    } else {
                        float hh[4];
#pragma unroll
                        for (int v = 0; v < 4; ++v) hh[v] = swiglu_clip(acc[i][j][v], acc[i][j + TN / 2][v], limit);
                        hv = make_uint2(pack_bf16x2_hw(hh[0], hh[1]), pack_bf16x2_hw(hh[2], hh[3]));
                    }
                    *(uint2*)((uint16_t*)p.C + r * p.N + hcol) = hv;
                }
            }
        }
        if constexpr (MODE == OUT_F16) {
            // scaled fp16 rows straight from the registers: a wave's 128
            // columns are one exponent group, so a row's largest magnitude
            // is the max over the lane's 32 values and its 3 sibling lanes
            // (lane swaps, no LDS).  Staged through LDS as the fp32 output
            // is, with its bank conflicts, the second projection took
            // 1.33 ms against 1.21 ms at the Step-5 prefill.  A wave whose
            // columns all lie inside N stores without per-column checks.
            const int c0 = n_tile * BN + S::GW * wn;
            auto epi = [&](auto full_tag) {
                constexpr bool full = decltype(full_tag)::value;
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    if (i >= n_i) continue;
                    const int lr = 16 * (wm + S::WM * i) + lrow;
                    float m = 0.f;
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        const int col = c0 + 16 * j + lcol;
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            if (full || col + v < p.N) m = fmaxf(m, fabsf(acc[i][j][v]));
                    }
                    m = max_lanes_xor16_32(m);
                    if (lr >= valid) continue;
                    const int ex = yrow_exp(m);
                    const float sc = exp2_int(-ex);
                    char* row = (char*)p.C + (int64_t)(row0 + lr) * p.c_row_bytes;
                    typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
                    if constexpr (full) {
                        // tiles j and j+1 through one lane swap: lanes with
                        // (lane >> 4) even take columns 4 (lane >> 4) .. +7 of
                        // tile j, the odd ones the same 8 columns of tile
                        // j+1, so each lane stores 16 bytes
                        const bool odd = (lane >> 4) & 1;
#pragma unroll
                        for (int j = 0; j < TN; j += 2) {
                            f16x4 a4, b4;
#pragma unroll
                            for (int v = 0; v < 4; ++v) {
                                a4[v] = (_Float16)(acc[i][j][v] * sc);
                                b4[v] = (_Float16)(acc[i][j + 1][v] * sc);
                            }
                            const uint2 a = __builtin_bit_cast(uint2, a4), b = __builtin_bit_cast(uint2, b4);
                            const auto s0 = __builtin_amdgcn_permlane16_swap(a.x, b.x, false, false);
                            const auto s1 = __builtin_amdgcn_permlane16_swap(a.y, b.y, false, false);
                            // even rows of lanes keep their tile-j columns and take the
                            // partner's next 4; odd rows take the partner's tile-(j+1)
                            // columns before their own
                            const uint4 q = make_uint4(s0[0], s1[0], s0[1], s1[1]);
                            const int col = c0 + 16 * (j + (odd ? 1 : 0)) + 4 * ((lane >> 4) & ~1);
                            *(uint4*)(row + 2 * col) = q;
                        }
                    } else {
#pragma unroll
                        for (int j = 0; j < TN; ++j) {
                            const int col = c0 + 16 * j + lcol;
                            if (col < p.N) {
                                f16x4 h4;
#pragma unroll
                                for (int v = 0; v < 4; ++v) h4[v] = (_Float16)(acc[i][j][v] * sc);
                                *(f16x4*)(row + 2 * col) = h4;
                            }
                        }
                    }
                    if (lcol == 0 && c0 < p.N) {
                        row[2 * p.N + (c0 >> 7)] = (char)ex;
                        if (c0 == 0) yrow_zero_pad(row, p.N);
                    }
                }
            };
            if (c0 + S::GW <= p.N) epi(std::true_type{}); else epi(std::false_type{});
        } else if (!is_swiglu(MODE)) {
            // plain fp32 output: through LDS, EPI_ROWS rows at a time (16-byte
            // writes of each lane's 4 columns), then whole rows, 16 bytes per
            // lane
            constexpr int PITCH = BN + 4;
            constexpr int EPI_ROWS = S::EPI_ROWS;
            constexpr int IPP = EPI_ROWS / 16 / S::WM;
            float* stage = (float*)smem;
            __syncthreads();
#pragma unroll
            for (int pass = 0; pass < BM / EPI_ROWS; ++pass) {
#pragma unroll
                for (int ii = 0; ii < IPP; ++ii) {
                    const int i = IPP * pass + ii;
                    const int pr = 16 * (wm + S::WM * ii) + lrow;
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        *(f32x4*)&stage[pr * PITCH + S::GW * wn + 16 * j + lcol] = acc[i][j];
                }
                __syncthreads();
                constexpr int PER_ROW = BN / 4;
                const int c = (tid % PER_ROW) * 4;
                const int col = n_tile * BN + c;
#pragma unroll 4
                for (int q = 0; q < EPI_ROWS * PER_ROW / NT; ++q) {
                    const int pr = tid / PER_ROW + (NT / PER_ROW) * q;
                    const int lr = EPI_ROWS * pass + pr;
                    if (lr < valid && col < p.N)
                        *(float4*)((float*)p.C + (int64_t)(row0 + lr) * p.N + col) = *(const float4*)&stage[pr * PITCH + c];
                }
                __syncthreads();
            }
        }
        return;
    }
    if (is_swiglu(MODE)) {
        uint16_t* H = (uint16_t*)p.C;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            if (i >= n_i) continue;
#pragma unroll
            for (int j = 0; j < TN / 2; ++j) {
                const int hcol = n_tile * (BN / 2) + (S::GW / 2) * wn + 16 * j + ccol;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int lr = 16 * (wm + S::WM * i) + crow + v;
                    if (lr < valid && hcol < p.N) {
                        const int64_t r = row0 + lr;
                        if (MODE == SWIGLU_SAVE) {
                            // kept for the backward; the activation uses the same rounded values
                            const uint16_t gq = f32_to_bf16(acc[i][j][v]);
                            const uint16_t uq = f32_to_bf16(acc[i][j + TN / 2][v]);
                            p.gu_out[r * 2 * p.N + hcol] = gq;
                            p.gu_out[r * 2 * p.N + p.N + hcol] = uq;
                            H[r * p.N + hcol] = f32_to_bf16(swiglu_clip(bf16_to_f32(gq), bf16_to_f32(uq), limit));
                        } else {
                            H[r * p.N + hcol] = f32_to_bf16(swiglu_clip(acc[i][j][v], acc[i][j + TN / 2][v], limit));
                        }
                    }
                }
            }
        }
    } else if (MODE == OUT_F32) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            if (i >= n_i) continue;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int col = n_tile * BN + S::GW * wn + 16 * j + ccol;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int lr = 16 * (wm + S::WM * i) + crow + v;
                    if (lr < valid && col < p.N) ((float*)p.C)[(int64_t)(row0 + lr) * p.N + col] = acc[i][j][v];
                }
            }
        }
    } else if constexpr (BM == 64 && BN == 128 && S::WM == 1) {
        // scaled fp16 rows (64-row tiles, 128 columns = one exponent group
        // per tile): each row's largest magnitude over the wave's columns,
        // then over the waves through LDS, sets the group's exponent
        float* red = (float*)smem;                 // [NW waves][64 rows]
        __syncthreads();                           // every wave is done with the operand ring
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                float m = 0.f;
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int col = n_tile * BN + S::GW * wn + 16 * j + ccol;
                    const int lr = 16 * i + crow + v;
                    if (i < n_i && lr < valid && col < p.N) m = fmaxf(m, fabsf(acc[i][j][v]));
                }
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
                if (ccol == 0) red[wave * 64 + 16 * i + crow + v] = m;
            }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            if (i >= n_i) continue;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int lr = 16 * i + crow + v;
                if (lr >= valid) continue;
                float m = 0.f;
#pragma unroll
                for (int w8 = 0; w8 < NW; ++w8) m = fmaxf(m, red[w8 * 64 + lr]);
                const int ex = yrow_exp(m);
                const float sc = exp2_int(-ex);
                char* row = (char*)p.C + (int64_t)(row0 + lr) * p.c_row_bytes;
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int col = n_tile * BN + S::GW * wn + 16 * j + ccol;
                    if (col < p.N) *(_Float16*)(row + 2 * col) = (_Float16)(acc[i][j][v] * sc);
                }
                if (wave == 0 && ccol == 0) {
                    row[2 * p.N + n_tile] = (char)ex;
                    if (n_tile == 0) yrow_zero_pad(row, p.N);
                }
            }
        }
    }
}

// GROUPED: rows come in expert groups (offsets + tile plan); otherwise one
// dense group of M rows.  Separate instances also keep the uses apart in
// kernel traces.  Block (xcd, slot) runs the items at slots slot, slot +
// slots, ... of its XCD's ranges (one item when the grid covers them).
template <int MODE, bool GROUPED, int BM, int BN>
__global__ __launch_bounds__((Shape<BM, BN>::NT), 1) void kernel(Params p) {
    using S = Shape<BM, BN>;
    static_assert(!is_swiglu(MODE) || S::TN % 2 == 0, "SwiGLU pairs gate and up tiles inside a wave");
    static_assert(MODE != OUT_F16 || BM == 256 || (BM == 64 && BN == 128), "scaled fp16 rows: 256-row or 64 x 128 tiles");
    __shared__ __attribute__((aligned(1024))) unsigned char smem[S::SMEM];
    const Segments sg = segments<GROUPED, BM>(p);
    const int xcd = blockIdx.x % NXCD, slots = gridDim.x / NXCD;
    // routed items of this XCD: a contiguous range of the list, from the
    // item table's cost-balanced split or an equal split of the count
    int r0 = xcd * sg.per1, rn = sg.per1;
    if (GROUPED && p.xcd_start) {
        r0 = __builtin_amdgcn_readfirstlane(p.xcd_start[xcd]);
        rn = __builtin_amdgcn_readfirstlane(p.xcd_start[xcd + 1]) - r0;
    }
    for (int s = blockIdx.x / NXCD; s < sg.per2 + rn; s += slots) {
        int w;
        if (s < sg.per2) {
            w = xcd * sg.per2 + s;
            if (w >= sg.total2) continue;
            w += sg.total1;
        } else {
            w = r0 + (s - sg.per2);
            if (w >= sg.total1) continue;
        }
        run_item<MODE, GROUPED, BM, BN>(p, w, smem);
        __syncthreads();                          // LDS is reused by the next item
    }
}

// blocks for `work` items in two segments: one more slot per XCD than the
// items need, since each segment rounds its per-XCD range up
static int grid_blocks(int64_t work) {
    const int64_t per = (work + NXCD - 1) / NXCD + 1;
    return (int)(per * NXCD);
}

// The work items of a grouped launch, {group, first row, rows, n-tile}.  A
// group's rows are split evenly over its m-tiles (each at most bm rows, as
// the tile plan counts ceil(rows / bm) of them), so the m-tiles that share a
// weight panel do the same work at the same pace; a group's items are
// n-tile-major, m-tile fastest.  The routed groups are dealt to the 8 XCDs
// by cost, so that every XCD gets about the same work: ranked by cost (an
// item costs ITEM_COST0 + its rows, the weight panel's stream counted in
// rows' worth of time), they go to XCDs 0..7, 7..0, 0..7, ... in rank order,
// and each XCD's groups lie contiguous in the list (xcd_start gives the
// ranges), heavy and light alternating.  Without `balance` the items stay
// in group order and the ranges are equal shares of their count.  The extra group's items follow the routed ones; the
// kernel splits them evenly over the XCDs.  One block of 1024 threads.
constexpr int ITEM_COST0 = 224;

__global__ __launch_bounds__(1024) void item_table_kernel(const int32_t* __restrict__ offsets,
                                                         const int32_t* __restrict__ tile_start, int groups,
                                                         int extra_rows, int n_tiles, int balance,
                                                         int* __restrict__ xcd_start, int4* __restrict__ items) {
    __shared__ int32_t ts[1026];
    __shared__ int32_t cost[1024], rank_of[1024], by_rank[1024];
    __shared__ int32_t cnt_at[NXCD][128], off_at[NXCD][128];
    __shared__ int32_t xs[NXCD + 1];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ng = groups + (extra_rows > 0 ? 1 : 0);
    for (int g = tid; g <= ng; g += blockDim.x) ts[g] = tile_start[g];
    for (int i = tid; i < NXCD * 128; i += blockDim.x) cnt_at[i / 128][i % 128] = 0;
    // rank i goes to XCD x(i) as its (i / 8)-th heaviest group; an XCD's k
    // groups run heaviest, lightest, second heaviest, second lightest, ...,
    // so that items bound by the MFMAs and items bound by the weight stream
    // overlap in time on every XCD
    auto xcd_of = [](int i) { const int pos = i % NXCD; return ((i / NXCD) & 1) ? NXCD - 1 - pos : pos; };
    const int last = groups > 0 ? (groups - 1) / NXCD : 0;         // the last round
    auto groups_of = [&](int x) {
        const int pos = (last & 1) ? NXCD - 1 - x : x;
        return groups > 0 ? last + (pos <= (groups - 1) % NXCD ? 1 : 0) : 0;
    };
    auto slot_of = [&](int i) {
        const int j = i / NXCD, k = groups_of(xcd_of(i));
        return j < (k + 1) / 2 ? 2 * j : 2 * (k - 1 - j) + 1;
    };
    __syncthreads();
    if (balance) {                              // (uniform over the block)
    for (int g = tid; g < groups; g += blockDim.x)
        cost[g] = n_tiles * ((ts[g + 1] - ts[g]) * ITEM_COST0 + (offsets[g + 1] - offsets[g]));
    __syncthreads();
    // rank: descending cost, ties to the lower group
    for (int g = tid; g < groups; g += blockDim.x) {
        const int c = cost[g];
        int r = 0;
        for (int h = 0; h < groups; ++h) {
            const int ch = cost[h];
            r += (ch > c || (ch == c && h < g)) ? 1 : 0;
        }
        rank_of[g] = r;
        by_rank[r] = g;
    }
    __syncthreads();
    for (int i = tid; i < groups; i += blockDim.x) {
        const int g = by_rank[i];
        cnt_at[xcd_of(i)][slot_of(i)] = (ts[g + 1] - ts[g]) * n_tiles;
    }
    __syncthreads();
    // exclusive scan of each XCD's item counts over its groups (wave x, two per lane)
    if (wave < NXCD) {
        const int a = cnt_at[wave][2 * lane], b = cnt_at[wave][2 * lane + 1];
        int incl = a + b;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int v = __shfl_up(incl, o, 64);
            if (lane >= o) incl += v;
        }
        const int excl = incl - a - b;
        off_at[wave][2 * lane] = excl;
        off_at[wave][2 * lane + 1] = excl + a;
        if (lane == 63) xs[wave + 1] = incl;
    }
    __syncthreads();
    if (tid == 0) {
        xs[0] = 0;
        for (int x = 0; x < NXCD; ++x) xs[x + 1] += xs[x];
    }
    __syncthreads();
    if (tid <= NXCD) xcd_start[tid] = xs[tid];
    } else if (tid <= NXCD) {
        // group order: equal shares of the routed items' count
        const int total1 = ts[groups] * n_tiles, per = (total1 + NXCD - 1) / NXCD;
        xcd_start[tid] = min(tid * per, total1);
    }
    const int total = ts[ng];
    for (int i = tid; i < total; i += blockDim.x) {
        int lo = 0, hi = ng - 1;                // the group g with ts[g] <= i < ts[g + 1]
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (ts[mid] <= i) lo = mid; else hi = mid - 1;
        }
        const int g = lo, t0 = ts[g], mt = ts[g + 1] - t0, m = i - t0;
        const int base = offsets[min(g, groups)];
        const int cnt = (g < groups ? offsets[g + 1] : base + extra_rows) - base;
        const int a = (int)(((int64_t)m * cnt) / mt), b = (int)(((int64_t)(m + 1) * cnt) / mt);
        int64_t first;
        if (g < groups && balance) {
            const int r = rank_of[g], x = xcd_of(r);
            first = (int64_t)xs[x] + off_at[x][slot_of(r)];
        } else {
            first = (int64_t)t0 * n_tiles;      // in group order (the extra group after all routed items)
        }
        int4* out = items + first + m;
        for (int n = 0; n < n_tiles; ++n) out[n * mt] = make_int4(g, base + a, b - a, n);
    }
}

template <int MODE, int BM, int BN>
void launch(Params p, int64_t tiles, hipStream_t s) {
    p.n_tiles = is_swiglu(MODE) ? (2 * p.N + BN - 1) / BN : (p.N + BN - 1) / BN;
    if (p.items) {
        // the first projection's routed groups are dealt to the XCDs by cost
        // (measured: 2.18 -> 2.16 ms at the Step-5 prefill); the second
        // projection keeps them in group order, equal shares of the count
        // (dealt by cost it ran slower)
        const int balance = is_swiglu(MODE) ? 1 : 0;
        item_table_kernel<<<1, 1024, 0, s>>>(p.offsets, p.tile_start, p.groups, p.extra_rows, p.n_tiles, balance,
                                             (int*)p.xcd_start, (int4*)p.items);
        if (!balance) p.xcd_start = nullptr;
    }
    // the second projection's 256-row items run on a persistent grid, one
    // block per CU walking a stride of its XCD's items (1,150 -> 1,133 us at
    // the Step-5 prefill: no block launch per item); the first projection's
    // items differ too much in cost for a fixed stride and keep one block each
    int nb = grid_blocks(tiles * p.n_tiles);
    if (MODE == OUT_F16 && BM == 256 && p.offsets && nb > 256) nb = 256;
    if (p.offsets) kernel<MODE, true, BM, BN><<<nb, Shape<BM, BN>::NT, 0, s>>>(p);
    else kernel<MODE, false, BM, BN><<<nb, Shape<BM, BN>::NT, 0, s>>>(p);
}

}  // namespace gg

// the XCD ranges (16 ints), then the items
size_t grouped_item_bytes(int64_t max_tiles, int n_tiles) { return 64 + (size_t)max_tiles * n_tiles * 16; }

hipError_t launch_item_table(const int32_t* offsets, const int32_t* tile_start, int groups, int extra_rows,
                             int n_tiles, bool balance, void* buf, hipStream_t s) {
    gg::item_table_kernel<<<1, 1024, 0, s>>>(offsets, tile_start, groups, extra_rows, n_tiles, balance ? 1 : 0,
                                             (int*)buf, (int4*)((char*)buf + 64));
    return hipGetLastError();
}
int64_t expert_row_bytes(int H) { return yrow_bytes(H); }

int grouped_tile_m(int64_t rows, int groups) {
    // 64-row tiles when the groups average under 48 rows (decode-like
    // batches), else 256-row tiles
    return rows < (int64_t)48 * groups ? 64 : 256;
}

hipError_t launch_grouped_up(const GroupedArgs& a, hipStream_t s) {
    gg::Params p{};
    p.A = (const uint16_t*)a.A;
    p.a_rows = a.a_rows;
    p.a_div = a.a_div > 0 ? a.a_div : 1;
    p.a_nrows = a.a_nrows;
    p.W = (const uint16_t*)a.W;
    p.w_group_stride = a.w_group_stride;
    p.C = a.C;
    p.N = a.N;
    p.K = a.K;
    p.limit = a.limit;
    p.offsets = a.offsets;
    p.tile_start = a.tile_start;
    p.groups = a.groups;
    p.M = a.M;
    p.extra_rows = a.extra_rows;
    p.W_extra = (const uint16_t*)a.W_extra;
    p.limit_extra = a.limit_extra;
    p.gu_out = (uint16_t*)a.gu_out;
    p.rot_group = a.rot_group;
    p.items = (a.bm == 256 && a.offsets && a.items) ? (const int4*)((const char*)a.items + 64) : nullptr;
    p.xcd_start = p.items ? (const int*)a.items : nullptr;
    const int64_t tiles = a.offsets ? a.max_tiles : (a.M + a.bm - 1) / a.bm;
    if (tiles <= 0) return hipSuccess;
    // 256-row tiles address gathered A rows and one group's weights by 32-bit
    // byte offsets
    if (a.bm == 256 && ((a.a_rows && (int64_t)a.a_nrows * a.K * 2 >= (int64_t(1) << 32)) ||
                        (int64_t)2 * a.N * a.K * 2 >= (int64_t(1) << 32)))
        return hipErrorInvalidValue;
    if (a.gu_out) {
        if (a.bm == 64) gg::launch<gg::SWIGLU_SAVE, 64, 256>(p, tiles, s);
        else gg::launch<gg::SWIGLU_SAVE, 256, 256>(p, tiles, s);
    } else {
        if (a.bm == 64) gg::launch<gg::SWIGLU, 64, 256>(p, tiles, s);
        else gg::launch<gg::SWIGLU, 256, 256>(p, tiles, s);
    }
    return hipGetLastError();
}

hipError_t launch_grouped_down(const GroupedArgs& a, bool c_fp32, hipStream_t s) {
    gg::Params p{};
    p.A = (const uint16_t*)a.A;
    p.a_rows = nullptr;
    p.a_div = 1;
    p.a_nrows = a.a_nrows;
    p.W = (const uint16_t*)a.W;
    p.w_group_stride = a.w_group_stride;
    p.C = a.C;
    p.N = a.N;
    p.K = a.K;
    p.offsets = a.offsets;
    p.tile_start = a.tile_start;
    p.groups = a.groups;
    p.M = a.M;
    p.extra_rows = a.extra_rows;
    p.W_extra = (const uint16_t*)a.W_extra;
    p.rot_group = a.rot_group;
    p.items = (a.bm == 256 && a.offsets && a.items) ? (const int4*)((const char*)a.items + 64) : nullptr;
    p.xcd_start = p.items ? (const int*)a.items : nullptr;
    p.c_row_bytes = yrow_bytes(a.N);
    const int64_t tiles = a.offsets ? a.max_tiles : (a.M + a.bm - 1) / a.bm;
    if (tiles <= 0) return hipSuccess;
    if (a.bm == 256 && (int64_t)a.N * a.K * 2 >= (int64_t(1) << 32)) return hipErrorInvalidValue;
    // 64-row tiles: 128-column tiles double the work items of these
    // (HBM-bound) launches, which evens out the last round on 256 CUs
    if (c_fp32) {
        if (a.bm == 64) gg::launch<gg::OUT_F32, 64, 128>(p, tiles, s);
        else gg::launch<gg::OUT_F32, 256, 256>(p, tiles, s);
    } else {
        if (a.bm == 64) gg::launch<gg::OUT_F16, 64, 128>(p, tiles, s);
        else gg::launch<gg::OUT_F16, 256, 256>(p, tiles, s);
    }
    return hipGetLastError();
}

}  // namespace moe
