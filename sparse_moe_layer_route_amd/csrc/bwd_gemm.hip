// bwd_gemm.hip -- the grouped GEMMs of the layer's backward on gfx950.
//
//   C[m, n] = sum_k A(m, k) * B(k, n)
//
// The backward's products read operands that the forward reads the other way
// round: the expert weights W2 [H][I] and W13 [2I][H] are contracted over
// their row index (data gradients), and the saved activations are
// contracted over the token rows (weight gradients).  Both land in LDS
// K-major -- rows of k, the m or n index contiguous -- and reach the MFMA
// through ds_read_b64_tr_b16, gfx950's transposing LDS read: in each group of
// 16 lanes, lane i receives element i & 3 of the 8 bytes that lane
// 4j + (i >> 2) addressed, for j = 0..3.  Lane s reading row k0 + (s >> 2),
// columns c0 + 4 (s & 3) .. +3 therefore hands lane i the 4 values
// B[k0 .. k0+3][c0 + i], half of a 16x16x32 MFMA fragment.
//
// Instances:
//   * DGRAD (groups partition the rows M, like the forward): A is K-
//     contiguous rows (the output gradient rows dy, or dgu), B is the group's
//     weight [K][N].  Epilogues: ACT -- the clipped SwiGLU's backward with
//     the saved pre-activations gu, giving dgu (bf16 [rows][2N]); F32 --
//     plain fp32 rows.
//   * WGRAD (groups partition the contraction K = the group's rows): A and
//     B are K-major row sets (dy or dgu, and h or the x rows in row order);
//     every group, empty ones included, writes its full fp32 [M][N] gradient.
//
// Each wave computes 64 x 128 of the output with 16x16x32 bf16 MFMA; operands
// go global -> LDS by direct DMA (inline asm, explicit vmcnt waits) and the
// fragments of slice k+1 are read while slice k multiplies -- the forward
// kernel's scheme.  Block tile 256 x 256, 8 waves (4 along M x 2 along N),
// 4 LDS stages, one block per CU.  (A 128 x 256 weight-gradient tile with 4
// waves, two blocks per CU, measured slower: 21.9 against 18.0 ms for the
// Step-5 prefill backward.)
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

namespace bg {

constexpr int BK = 32;
constexpr int BN = 256;
constexpr int TM = 4, TN = 8;           // 16-row / 16-col tiles per wave (64 x 128)
constexpr int NXCD = 8;
// K-contiguous operand (16 rows x 64 B per DMA block), as in the forward
// kernel: the 4 blocks of a 64-row group at bank groups 0, 2, 16, 18
__device__ constexpr int BLK_OFF[4] = {0, 1024 + 32, 2048 + 256, 3072 + 288};
constexpr int GROUP = 3072 + 288 + 1024;
constexpr int KC_BYTES = 4 * GROUP;     // 256 rows x one K slice
// K-major operand: 4 slabs of 64 columns x 4 blocks of 8 k-rows (one DMA
// block each: 128 B per row, lane-consecutive), k-row r of a slice holding
// the row's 16-byte chunk c at position c ^ km_swz(r).  The swizzle was
// found by search: the transposing reads are free of bank conflicts under
// every LDS service order that fits the conflict counter's readings (16 or
// 32 consecutive lanes, or lanes l and l + 32, over 128 to 512 bytes).  The
// earlier 32-byte skew between blocks fitted only a 32-lane, 512-byte order
// and measured 1.2-1.6 conflict cycles per LDS instruction.
constexpr int KB_PITCH = 1024;
constexpr int SLAB = 4 * KB_PITCH;
constexpr int KM_BYTES = 4 * SLAB;
// epilogue staging: rows of 256 fp32 with a 16-byte skew per row, so the 4
// row groups of an MFMA store land on distinct banks
constexpr int EPI_PITCH = 256 + 4;

template <bool WGRAD>
struct Tile {
    static constexpr int NW = 8;                        // waves per block
    static constexpr int BM = 256;
    static constexpr int WM = BM / 64;                  // waves along M
    static constexpr int WN = NW / WM;                  // waves along N (2)
    static constexpr int NA = BM / 16;                  // A DMA blocks per slice
    static constexpr int NB = BN / 16;                  // B DMA blocks per slice
    static constexpr int A_PER_WAVE = NA / NW;
    static constexpr int B_PER_WAVE = NB / NW;
    static constexpr int A_BYTES = WGRAD ? (BM / 64) * SLAB : KC_BYTES;
    static constexpr int STAGE_BYTES = A_BYTES + KM_BYTES;
    static constexpr int STAGES = 4;
    static constexpr int EPI_ROWS = 128;                // rows per staging pass
    static constexpr int SMEM = STAGES * STAGE_BYTES > EPI_ROWS * EPI_PITCH * 4 ? STAGES * STAGE_BYTES
                                                                                 : EPI_ROWS * EPI_PITCH * 4;
    static_assert(WN == 2 && NA % NW == 0 && NB % NW == 0, "tile shape");
};

enum { ACT = 0, F32 = 1 };

struct Params {
    const uint16_t* A;          // DGRAD: [rows][K] K-contiguous; WGRAD: [rows][M] K-major
    int64_t lda;
    const uint16_t* B;          // DGRAD: weights [groups][K][N]; WGRAD: [rows][N] K-major
    int64_t ldb;
    int64_t b_group_stride;
    const uint16_t* B_extra;    // DGRAD: the extra group's weight [K][N]
    const uint16_t* zero_row;   // WGRAD: >= max(M, N) zero values, read for k rows past a group's end
    void* C;
    int64_t ldc;
    int64_t c_group_stride;     // WGRAD: per-group output stride
    void* C_extra;              // WGRAD: the extra group's output
    const uint16_t* gu;         // ACT: saved pre-activations [rows][2N], gate then up
    float limit, limit_extra;
    int M, N, K;                // DGRAD: N, K (M from the groups); WGRAD: M, N (K from the groups)
    const int32_t* offsets;     // [groups+1]
    const int32_t* tile_start;  // DGRAD: 256-row tile plan [groups+2]
    int groups;
    int extra_rows;             // rows of the extra group after offsets[groups] (0: none)
    int m_tiles, n_tiles;
};

typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef short v4s __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void dma_frag(const void* g, unsigned lds_off) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_off), "v"(g) : "memory");
}

template <int n>
__device__ __forceinline__ void wait_vm() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

// chunk swizzle of k-row r (0..31) of a K-major slice
__device__ __forceinline__ int km_swz(int r) {
    return (2 * ((r ^ (r >> 3) ^ (r >> 4)) & 1)) | (4 * (((r >> 1) ^ (r >> 4)) & 1));
}

// The 8 bytes that lane s (of its 16-lane group g) reads for the 16-column
// tile at column c0 are in k-row r = 8g + 4 half + (s >> 2), chunk
// (c0 & 63) / 8 + ((s & 3) >> 1), bytes 8 (s & 1) of it.  The chunk's high
// bits come from c0 alone, so the offset is this lane's base for the half
// XOR 16 (c0 & 63) / 8, plus the slab.
struct KmLane {
    unsigned half0, half1;
};
__device__ __forceinline__ KmLane km_lane(int lane) {
    const int g = lane >> 4, s = lane & 15;
    KmLane kl;
    const int r0 = 8 * g + (s >> 2), r1 = r0 + 4;
    kl.half0 = (unsigned)(g * KB_PITCH + (r0 & 7) * 128 + 16 * (((s & 3) >> 1) ^ km_swz(r0)) + 8 * (s & 1));
    kl.half1 = (unsigned)(g * KB_PITCH + (r1 & 7) * 128 + 16 * (((s & 3) >> 1) ^ km_swz(r1)) + 8 * (s & 1));
    return kl;
}

// a 16x16x32 fragment from a K-major operand: two transposing reads
__device__ __forceinline__ bf16x8 km_frag(const unsigned char* base, int c0, const KmLane& kl) {
    const unsigned x = 16u * ((c0 & 63) >> 3);
    const unsigned char* slab = base + (c0 >> 6) * SLAB;
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(
        (lds_u8*)(slab + (kl.half0 ^ x))));
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(
        (lds_u8*)(slab + (kl.half1 ^ x))));
    typedef short v8s __attribute__((ext_vector_type(8)));
    const v8s v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

template <bool WGRAD, int EPI>
__device__ __forceinline__ void run_item(const Params& p, int w, unsigned char* smem) {
    using S = Tile<WGRAD>;
    constexpr int NW = S::NW, BM = S::BM, WM = S::WM, WN = S::WN, STAGES = S::STAGES;
    constexpr int A_PER_WAVE = S::A_PER_WAVE, B_PER_WAVE = S::B_PER_WAVE, D = A_PER_WAVE + B_PER_WAVE;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;

    // ---- the work item -------------------------------------------------
    int g, m_tile, n_tile;
    int row0 = 0, valid = BM;        // DGRAD: the tile's rows
    int k_begin = 0, k_end = p.K;    // WGRAD: the group's rows
    {
        if (WGRAD) {
            const int per_g = p.m_tiles * p.n_tiles;
            g = w / per_g;
            const int local = w - g * per_g;
            n_tile = local / p.m_tiles;
            m_tile = local % p.m_tiles;
            k_begin = p.offsets[g];
            k_end = g < p.groups ? p.offsets[g + 1] : k_begin + p.extra_rows;
        } else {
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
            const int base = p.offsets[g];
            const int cnt = (g < p.groups ? p.offsets[g + 1] : base + p.extra_rows) - base;
            row0 = base + (int)(((int64_t)m_tile * cnt) / mt);
            valid = base + (int)(((int64_t)(m_tile + 1) * cnt) / mt) - row0;
        }
    }
    const bool extra = g == p.groups;
    const int nk = WGRAD ? (k_end - k_begin + BK - 1) / BK : p.K / BK;

    // ---- DMA sources ----------------------------------------------------
    const uint16_t* Bg = WGRAD ? p.B : (extra ? p.B_extra : p.B + (int64_t)g * p.b_group_stride);
    // K-contiguous A (DGRAD): block b of the 16 (16 rows x 64 B), rows as in
    // the forward kernel
    const int quad = lane >> 2, chunk = lane & 3;
    auto block_row = [&](int blk) { return 64 * (blk >> 2) + 16 * (quad >> 2) + 4 * (blk & 3) + (quad & 3); };
    // K-major blocks b: slab b >> 2, k block b & 3; lane l: k row
    // 8 (b & 3) + (l >> 3), 16-byte chunk l & 7 of the slab's row
    const uint16_t* a_src[A_PER_WAVE];   // DGRAD: A row source (the slice offset is added per slice)
    int a_col[A_PER_WAVE], a_row[A_PER_WAVE];
    unsigned a_lds[A_PER_WAVE];
#pragma unroll
    for (int q = 0; q < A_PER_WAVE; ++q) {
        const int blk = A_PER_WAVE * wave + q;
        const int kb = blk & 3, slab = blk >> 2;
        a_row[q] = 8 * kb + (lane >> 3);
        a_col[q] = 0;
        a_src[q] = p.A;
        if (WGRAD) {
            a_col[q] = min(m_tile * BM + slab * 64, p.M - 64) + ((lane & 7) ^ km_swz(a_row[q])) * 8;
            a_lds[q] = slab * SLAB + kb * KB_PITCH + 16 * lane;
        } else {
            const int ar = row0 + min(block_row(blk), valid - 1);
            a_src[q] = p.A + (int64_t)ar * p.lda + chunk * 8;
            a_lds[q] = (blk >> 2) * GROUP + BLK_OFF[blk & 3];
        }
    }
    int b_col[B_PER_WAVE], b_row_k[B_PER_WAVE];
    unsigned b_lds[B_PER_WAVE];
#pragma unroll
    for (int q = 0; q < B_PER_WAVE; ++q) {
        const int blk = B_PER_WAVE * wave + q;
        const int kb = blk & 3, slab = blk >> 2;
        b_row_k[q] = 8 * kb + (lane >> 3);
        b_col[q] = min(n_tile * BN + slab * 64, p.N - 64) + ((lane & 7) ^ km_swz(b_row_k[q])) * 8;
        b_lds[q] = S::A_BYTES + slab * SLAB + kb * KB_PITCH + 16 * lane;
    }
    const unsigned lds_base = (unsigned)(size_t)(lds_u8*)smem;
    // row r of the K-major sources (WGRAD: the group's rows, zeros past the end)
    auto b_row = [&](int r) -> const uint16_t* {
        if (!WGRAD) return Bg + (int64_t)r * p.ldb;
        if (r >= k_end) return p.zero_row;
        return p.B + (int64_t)r * p.ldb;
    };
    // this wave's DMA q of slice kt (A blocks first, then B) into `stage`
    auto issue_q = [&](int kt, int stage, int q) {
        const unsigned sb = lds_base + stage * S::STAGE_BYTES;
        const int k0 = k_begin + kt * BK;
        if (q < A_PER_WAVE) {
            if (WGRAD) {
                const int r = k0 + a_row[q];
                const uint16_t* as = (r < k_end ? p.A + (int64_t)r * p.lda : p.zero_row) + a_col[q];
                dma_frag(as, __builtin_amdgcn_readfirstlane(sb + a_lds[q]));
            } else {
                dma_frag(a_src[q] + k0, __builtin_amdgcn_readfirstlane(sb + a_lds[q]));
            }
        } else {
            const int qb = q - A_PER_WAVE;
            dma_frag(b_row(k0 + b_row_k[qb]) + b_col[qb], __builtin_amdgcn_readfirstlane(sb + b_lds[qb]));
        }
    };
    auto issue = [&](int kt, int stage) {
#pragma unroll
        for (int q = 0; q < D; ++q) issue_q(kt, stage, q);
    };

    // fragment offsets of the K-contiguous A (DGRAD)
    const int fr = lane & 15;
    const unsigned lane_off = BLK_OFF[fr >> 2] + 64 * (fr & 3) + 16 * (lane >> 4);
    auto tile_off = [&](int tau) { return (unsigned)((tau >> 2) * GROUP + 256 * (tau & 3)) + lane_off; };

    // DGRAD: 16-row tiles past the tile's valid rows skip their MFMAs
    int n_i = TM;
    if (!WGRAD) {
        const int ntile_valid = (valid + 15) >> 4;
        n_i = 0;
#pragma unroll
        for (int i = 0; i < TM; ++i) n_i += (wm + WM * i < ntile_valid) ? 1 : 0;
        n_i = __builtin_amdgcn_readfirstlane(n_i);
    }

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (nk > 0) {
#pragma unroll
        for (int s = 0; s < STAGES - 1; ++s) issue(min(s, nk - 1), s);

        bf16x8 fa[2][TM], fb[2][TN];
        const KmLane kml = km_lane(lane);
        // group i of a slice's fragments: A tile wm + WM i and B tiles JG i ..
        static_assert(D == TM && TN % TM == 0, "one DMA per 16-row tile group");
        constexpr int JG = TN / TM;
        auto read_group = [&](const unsigned char* st, int i, bf16x8* a, bf16x8* b) {
            const int tau = wm + WM * i;          // 16-row tile of the block
            if (WGRAD) a[i] = km_frag(st, 16 * tau, kml);
            else a[i] = *(const bf16x8*)(st + tile_off(tau));
#pragma unroll
            for (int jj = 0; jj < JG; ++jj)
                b[JG * i + jj] = km_frag(st + S::A_BYTES, 128 * wn + 16 * (JG * i + jj), kml);
        };
        // The MFMAs run in TM groups (one 16-row tile each) with this wave's
        // DMA and next fragment reads between them: issued in one burst after
        // the barrier they queue at the wave's issue and hold back its MFMAs.
        auto step = [&](int kt, const bf16x8* ca, const bf16x8* cb, bf16x8* na, bf16x8* nb) {
            wait_vm<D * (STAGES - 3)>();
            __builtin_amdgcn_s_barrier();
            const int kn = min(kt + STAGES - 1, nk - 1), sn = (kt + STAGES - 1) % STAGES;
            const unsigned char* st = smem + ((kt + 1 < nk ? kt + 1 : kt) % STAGES) * S::STAGE_BYTES;
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                issue_q(kn, sn, i);
                read_group(st, i, na, nb);
                if (i < n_i) {
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ca[i], cb[j], acc[i][j], 0, 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        wait_vm<D * (STAGES - 2)>();
        __builtin_amdgcn_s_barrier();
#pragma unroll
        for (int i = 0; i < TM; ++i) read_group(smem, i, fa[0], fb[0]);
        int kt = 0;
        for (; kt + 1 < nk; kt += 2) {
            step(kt, fa[0], fb[0], fa[1], fb[1]);
            step(kt + 1, fa[1], fb[1], fa[0], fb[0]);
        }
        if (kt < nk) step(kt, fa[0], fb[0], fa[1], fb[1]);
        wait_vm<0>();
    }

    // ---- epilogue through LDS ---------------------------------------------
    // An MFMA lane holds column lane & 15 of rows 4 (lane >> 4) + v: stored
    // straight from registers, each instruction would write 64-byte pieces of
    // 4 rows.  Instead the tile goes to LDS EPI_ROWS rows at a time (the
    // operand stages are free by now), and each wave then writes whole rows
    // with 16 bytes per lane.  (The weight gradients written straight from a
    // transposed tile, 16 bytes per lane in 64-byte row pieces, took the
    // Step-5 prefill backward from 14.0 to 16.8 ms.)
    constexpr int EPI_ROWS = S::EPI_ROWS;
    constexpr int IPP = EPI_ROWS / 16 / WM;        // 16-row tiles of a wave per pass
    const int ccol = lane & 15, crow = (lane >> 4) * 4;
    float* stage = (float*)smem;
    __syncthreads();                              // every wave is done with the operand stages
    const float L = extra ? p.limit_extra : p.limit;
#pragma unroll
    for (int pass = 0; pass < BM / EPI_ROWS; ++pass) {
#pragma unroll
        for (int ii = 0; ii < IPP; ++ii) {
            const int i = pass * IPP + ii;
            const int lr0 = 16 * (wm + WM * ii) + crow;   // row within the pass
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    stage[(lr0 + v) * EPI_PITCH + 128 * wn + 16 * j + ccol] = acc[i][j][v];
        }
        __syncthreads();
        if (WGRAD || EPI == F32) {
            // EPI_ROWS rows x 64 float4; thread t: float4 t % 64 of rows t / 64 + NW q
            float* C = WGRAD ? (float*)(extra ? p.C_extra : (float*)p.C + (int64_t)g * p.c_group_stride)
                             : (float*)p.C;
            const int c4 = (tid & 63) * 4;
            const int col = n_tile * BN + c4;
#pragma unroll 4
            for (int q = 0; q < EPI_ROWS / NW; ++q) {
                const int pr = (tid >> 6) + NW * q;
                const int lr = EPI_ROWS * pass + pr;
                const float4 v = *(const float4*)&stage[pr * EPI_PITCH + c4];
                if (col < p.N) {
                    if (WGRAD) {
                        const int m = m_tile * BM + lr;
                        // written once and not read here: non-temporal stores
                        const f32x4 vv = {v.x, v.y, v.z, v.w};
                        if (m < p.M) __builtin_nontemporal_store(vv, (f32x4*)&C[(int64_t)m * p.ldc + col]);
                    } else if (lr < valid) {
                        *(float4*)&C[(int64_t)(row0 + lr) * p.ldc + col] = v;
                    }
                }
            }
        } else {
            // dh -> dgu: 8 columns per thread (16-byte loads of gu, stores of dgu)
            uint16_t* Dg = (uint16_t*)p.C;
            const int c8 = (tid & 31) * 8;
            const int col = n_tile * BN + c8;
#pragma unroll 2
            for (int q = 0; q < EPI_ROWS * 32 / (NW * 64); ++q) {
                const int pr = (tid >> 5) + (NW * 2) * q;
                const int lr = EPI_ROWS * pass + pr;
                if (lr < valid && col < p.N) {
                    const int64_t r = row0 + lr;
                    const float* sv = &stage[pr * EPI_PITCH + c8];
                    const uint4 gq = *(const uint4*)(p.gu + r * 2 * p.N + col);
                    const uint4 uq = *(const uint4*)(p.gu + r * 2 * p.N + p.N + col);
                    const uint32_t gw[4] = {gq.x, gq.y, gq.z, gq.w}, uw[4] = {uq.x, uq.y, uq.z, uq.w};
                    uint32_t dg_out[4], du_out[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float dg0, du0, dg1, du1;
                        swiglu_clip_grad(bf16_to_f32((uint16_t)(gw[e] & 0xffff)),
                                         bf16_to_f32((uint16_t)(uw[e] & 0xffff)), L, dg0, du0);
                        swiglu_clip_grad(bf16_to_f32((uint16_t)(gw[e] >> 16)), bf16_to_f32((uint16_t)(uw[e] >> 16)),
                                         L, dg1, du1);
                        const float dh0 = sv[2 * e], dh1 = sv[2 * e + 1];
                        dg_out[e] = pack_bf16x2(dh0 * dg0, dh1 * dg1);
                        du_out[e] = pack_bf16x2(dh0 * du0, dh1 * du1);
                    }
                    *(uint4*)(Dg + r * 2 * p.N + col) = make_uint4(dg_out[0], dg_out[1], dg_out[2], dg_out[3]);
                    *(uint4*)(Dg + r * 2 * p.N + p.N + col) = make_uint4(du_out[0], du_out[1], du_out[2], du_out[3]);
                }
            }
        }
        __syncthreads();                          // the next pass reuses the staging area
    }
}

// Work items: WGRAD (group, n-tile, m-tile); DGRAD (group, n-tile, m-tile)
// from the tile plan.  Each XCD (blocks b with b % 8 == x) takes a
// contiguous range, so the blocks that share an operand share an L2.
template <bool WGRAD, int EPI>
__global__ __launch_bounds__(Tile<WGRAD>::NW * 64, 1) void kernel(Params p) {
    __shared__ __attribute__((aligned(1024))) unsigned char smem[Tile<WGRAD>::SMEM];
    int total;
    if (WGRAD) total = (p.groups + (p.extra_rows > 0 ? 1 : 0)) * p.m_tiles * p.n_tiles;
    else total = p.tile_start[p.groups + (p.extra_rows > 0 ? 1 : 0)] * p.n_tiles;
    const int per = (total + NXCD - 1) / NXCD;
    const int xcd = blockIdx.x % NXCD, slots = gridDim.x / NXCD;
    for (int s = blockIdx.x / NXCD; s < per; s += slots) {
        const int w = xcd * per + s;
        if (w >= total) break;
        run_item<WGRAD, EPI>(p, w, smem);
        __syncthreads();
    }
}

template <bool WGRAD, int EPI>
static hipError_t launch(const BwdArgs& a, hipStream_t s) {
    Params p{};
    p.A = (const uint16_t*)a.A;
    p.lda = a.lda;
    p.B = (const uint16_t*)a.B;
    p.ldb = a.ldb;
    p.b_group_stride = a.b_group_stride;
    p.B_extra = (const uint16_t*)a.B_extra;
    p.zero_row = (const uint16_t*)a.zero_row;
    p.C = a.C;
    p.ldc = a.ldc;
    p.c_group_stride = a.c_group_stride;
    p.C_extra = a.C_extra;
    p.gu = (const uint16_t*)a.gu;
    p.limit = a.limit;
    p.limit_extra = a.limit_extra;
    p.M = a.M;
    p.N = a.N;
    p.K = a.K;
    p.offsets = a.offsets;
    p.tile_start = a.tile_start;
    p.groups = a.groups;
    p.extra_rows = a.extra_rows;
    p.n_tiles = (a.N + BN - 1) / BN;
    p.m_tiles = (a.M + Tile<WGRAD>::BM - 1) / Tile<WGRAD>::BM;
    int64_t items = WGRAD ? (int64_t)(a.groups + (a.extra_rows > 0 ? 1 : 0)) * p.m_tiles * p.n_tiles
                          : (int64_t)a.max_tiles * p.n_tiles;
    if (items <= 0) return hipSuccess;
    const int64_t blocks = (items + NXCD - 1) / NXCD * NXCD;
    kernel<WGRAD, EPI><<<(unsigned)blocks, Tile<WGRAD>::NW * 64, 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace bg

hipError_t launch_bwd_dgrad(const BwdArgs& a, bool act, hipStream_t s) {
    return act ? bg::launch<false, bg::ACT>(a, s) : bg::launch<false, bg::F32>(a, s);
}

hipError_t launch_bwd_wgrad(const BwdArgs& a, hipStream_t s) { return bg::launch<true, bg::F32>(a, s); }

}  // namespace moe
