// gemm.hip -- block-scaled FP8 GEMM for gfx950 (Fprop, Dgrad, Wgrad, grouped).
//
// C[m][n] = sum_j sA[j][m] * sB(n, j) * P_j[m][n], where P_j is the FP32 sum
// of the FP8 products of 128-element K slab j. This is the pages' promotion
// scheme: partial products of one 128-element interval (page inprokorea.com
// free board, passage on the four-WGMMA accumulation interval) are moved into
// full-precision FP32 accumulators, where the per-group scales are applied
// (page "Deepseek Ai News Expert Interview", passage on copying partial
// results to FP32 registers; page "Is aI Hitting a Wall?", passage on the
// dequantization overhead).
//
// gfx950 mapping: one v_mfma_f32_16x16x128_f8f6f4 consumes exactly one slab
// for a 16x16 subtile and returns P_j in fresh registers (C operand 0); the
// promotion is one v_fma_f32 per output element per slab on the vector ALU,
// overlapped with the next subtile's MFMA. The interval is set by the
// scales: measured on gfx950, chaining the MFMA accumulator across slabs
// gives the same error as promoting each slab, and what precision is lost
// is lost inside the instruction's own 128-product sum.
//
// Tiling: 256 (m) x BN (n) block tiles, BN = 256 or 224, 8 waves (4 along
// m x 2 along n), 64 x BN/2 per wave. BN = 224 makes N = 7168 (Dgrad, Wgrad)
// an exact multiple, so those grids are whole waves of the 256 CUs. Each
// 128-byte K slab of the A and B tiles is copied global -> LDS by the direct
// LDS-DMA load (global_load_lds_dwordx4) -- two stages, or for grouped-over-M
// tiles two A and three B stages -- with 16-byte chunks XOR-swizzled by row.
//
// Modes: one GEMM; grouped over M (MoE Fprop/Dgrad); grouped over K (MoE
// Wgrad); one GEMM of several rounds of whole tiles, run by one looping block
// per CU that copies each next tile's first slab during the last slab of the
// tile before (Dgrad-like shapes: short K, several rounds).
// Two more dense variants accumulate in place across slabs instead
// of promoting: microscaling operands (E8M0 block scales applied by the
// scaled MFMA) and one scale per tensor (applied in the epilogue).
// The MFMA computes the transposed tile: its row operand is B (n), its column
// operand is A (m), so every lane holds four consecutive n of one m -- one A
// scale per lane per m-subtile, and the B block scale is wave-uniform per
// 16-column subtile. Waves whose rows are all past the real rows (grouped
// padding, ragged M) skip their MFMAs.
#include "fp8q.h"
#include "gemm_common.h"

#include <algorithm>
#include <mutex>

// Cache policy of the LDS-DMA copies: the expert weights of a grouped-over-M
// GEMM are streamed from HBM once per m-tile, so they are loaded
// non-temporal (NT, bit 1 of the cache-policy operand on gfx950); everything
// else keeps the default policy. Paired on one MI355X, NT weights took the
// MoE grouped GEMM from 372 to 359 us; NT on the B operand of dense GEMMs,
// which is re-read from L2 by the tiles of a band, made Dgrad 14% slower.
constexpr int kPolicyDefault = 0;
constexpr int kPolicyNonTemporal = 2;

namespace fp8q {
namespace {

// ---------------------------------------------------------------- LDS
// Every stage of every operand is its own __shared__ array. The copy of slab
// j+1 into one stage and the fragment reads of slab j from the other then
// touch provably distinct objects, so the compiler's wait insertion lets the
// reads proceed while the copy is in flight; a stage is fenced explicitly
// (vmcnt(0) + barrier) before it is read.

// The arrays live at namespace scope; a kernel's LDS holds only the ones
// it uses. Two-stage kernels (dense): A, B, A scales and B scales in stages
// 0 and 1 (135168 bytes). Three-stage kernels (grouped): A in stages 0 and
// 1, B in stages 0, 1 and 2, scales in registers (163840 bytes).
__shared__ __attribute__((aligned(1024))) uint8_t lds_a0[kTileBytes];
__shared__ __attribute__((aligned(1024))) uint8_t lds_a1[kTileBytes];
__shared__ __attribute__((aligned(1024))) uint8_t lds_b0[kTileBytes];
__shared__ __attribute__((aligned(1024))) uint8_t lds_b1[kTileBytes];
__shared__ __attribute__((aligned(1024))) uint8_t lds_b2[kTileBytes];
__shared__ __attribute__((aligned(16))) float lds_sa0[kBM];
__shared__ __attribute__((aligned(16))) float lds_sa1[kBM];
__shared__ __attribute__((aligned(16))) float lds_sb0[kBNMax];
__shared__ __attribute__((aligned(16))) float lds_sb1[kBNMax];

template <int S>
__device__ __forceinline__ uint8_t* stage_a() {
    if constexpr (S == 0) return lds_a0; else return lds_a1;
}
template <int S>
__device__ __forceinline__ uint8_t* stage_b() {
    if constexpr (S == 0) return lds_b0;
    else if constexpr (S == 1) return lds_b1;
    else return lds_b2;
}
template <int S>
__device__ __forceinline__ float* stage_sa() {
    if constexpr (S == 0) return lds_sa0; else return lds_sa1;
}
template <int S>
__device__ __forceinline__ float* stage_sb() {
    if constexpr (S == 0) return lds_sb0; else return lds_sb1;
}

// ---------------------------------------------------------------- the kernel

// MX: microscaling operands (OCP MX, E4M3 elements): each row's 32-element
// K blocks carry E8M0 scales, one uint32 per row and slab (byte b = block
// 4j + b); the scaled MFMA applies them and accumulates in place, with no
// promotion step. Copies and scale staging are those of per-row scales.
// TENSOR: one scale per operand (a_scale[0], b_scale[0]); the whole K sum is
// accumulated inside the MFMA accumulators and scaled once in the epilogue.
template <int BN, bool ROWSCALE, bool OUT_F32, int MODE, bool MX = false, bool TENSOR = false>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(Params p) {
    constexpr bool GROUPED = MODE == kGroupedM;
    constexpr bool ROUNDS = MODE == kDenseRounds;
    static_assert(!MX || (ROWSCALE && MODE == kDense), "microscaling: dense, per-row staging");
    static_assert(!TENSOR || (ROWSCALE && MODE == kDense && !MX), "per-tensor: dense, no staged scales");
    constexpr bool INPLACE = MX || TENSOR;  // MFMA accumulates across slabs
    static_assert(BN == 256 || BN == 224, "n tile");
    constexpr int WN = BN / 2;        // n extent of one wave
    constexpr int NSUB = WN / 16;     // n-subtiles per wave
    // With 224-wide tiles a wave's 112 columns can straddle two 128-wide
    // weight blocks; each 16-column subtile still lies inside one block.
    constexpr bool STRADDLE = !ROWSCALE && (WN % 128 != 0);
    static_assert(!ROUNDS || (!MX && !TENSOR), "rounds: promoted block or row scales");

    // Grouped tiles stream each expert's weights from HBM once: they keep two
    // B slabs in flight (three B stages) and take their scales through
    // registers; dense tiles, whose operands mostly hit L2, use two stages.
    constexpr bool DEEP = GROUPED;
    static_assert(!DEEP || (!ROWSCALE && BN == 256), "three-stage tiles: block scales, 256 wide");

    TileRows tr;
    if constexpr (MODE == kGroupedM) {
        if (!grouped_tile<BN>(p, tr)) return;
    } else if constexpr (MODE == kGroupedK) {
        if (!grouped_k_tile<BN>(p, tr)) return;
    } else {
        if (!dense_tile<BN>(p, 0, tr)) return;
    }

    // Several rounds: this block's tiles one after another. The last step of
    // a tile copies the next tile's first slab (and its scales) instead of a
    // slab of its own, so the next tile starts computing at once while the
    // stores of the tile before are still in flight.
    bool prefetched = false;
    for (int it = 0;; ++it) {
        TileRows nx;
        bool has_next = false;
        if constexpr (ROUNDS) has_next = dense_tile<BN>(p, it + 1, nx);

        const int tid = threadIdx.x;
        const int lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int wm = wave >> 1, wn = wave & 1;
        const int slabs = tr.slabs;
        const int64_t m_last = p.m - 1;
        const int64_t n_last = p.n - 1;

        // ---- LDS-DMA sources: wave w copies rows [32w, 32w+32) of both tiles,
        // 8 rows (1 KB) per instruction; lane l -> row 8i + l/8, chunk l%8.
        // Rows past the tile or the matrix are clamped to valid rows (loaded,
        // never used). Addresses are a wave-uniform base (tile origin + slab) plus
        // a 32-bit per-lane offset, which maps onto the saddr + voffset form.
        const uint8_t* const tileA = p.a + tr.m0 * p.lda + (int64_t)tr.slab0 * kSlab;
        const uint8_t* const tileB = tr.b + tr.n0 * p.ldb + (int64_t)tr.slab0 * kSlab;
        // In a grouped tile, A rows past the tile's real rows only feed outputs
        // that are written as zeros or not at all (an output row depends on its
        // own A row only): every lane of such an 8-row chunk reads the same
        // 128-byte line, so the copy costs one L2 line instead of 1 KB.
        const int a_rows = (int)min((int64_t)kBM, min(tr.real_end, tr.row_hi) - tr.m0);
        uint32_t offA[4], offB[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 32 * wave + 8 * i + (lane >> 3);
            const int chunk = swz_chunk(lane & 7, row);
            const int src = (GROUPED && 32 * wave + 8 * i >= a_rows) ? max(a_rows - 1, 0) : row;
            offA[i] = (uint32_t)((min(tr.m0 + src, m_last) - tr.m0) * p.lda) + chunk * 16;
            offB[i] = (uint32_t)((min(tr.n0 + min(row, BN - 1), n_last) - tr.n0) * p.ldb) + chunk * 16;
        }
        // Scales: waves 0-3 copy the slab's 256 A scales (64 each) into the sA
        // area. Waves 4-7 copy B scales into the sB area: with per-row scaling the
        // slab's B scales (64 each); with 128x128 blocks, lane l copies the scale
        // of n-block (n0/128 + l%4), the at most three blocks a tile touches.
        const int64_t ld_s = wave < 4 ? p.ld_as : (ROWSCALE ? p.ld_bs : 1);
        // the wave's scale source of tile t's first slab: a base and a lane offset
        auto scale_src = [&](const TileRows& t, const float*& base, uint32_t& off) {
            if (wave < 4) {
                base = p.a_scale + t.m0;
                off = (uint32_t)(min(t.m0 + 64 * wave + lane, m_last) - t.m0) * 4u;
            } else if (ROWSCALE) {
                base = t.b_scale + t.n0;
                off = (uint32_t)(min(t.n0 + min(64 * (wave - 4) + lane, BN - 1), n_last) - t.n0) * 4u;
            } else {
                base = t.b_scale;
                off = (uint32_t)(min(t.n0 / 128 + (lane & 3), n_last / 128) * p.ld_bs) * 4u;
            }
            base += (int64_t)t.slab0 * ld_s;
        };
        const float* scale_base;
        uint32_t offS;
        scale_src(tr, scale_base, offS);

        // What one step copies: A and B slab bases and the wave's scale source.
        struct CopySrc {
            const uint8_t* a;
            const uint8_t* b;
            const uint8_t* s;
            uint32_t offs;
        };
        auto src_of = [&](int j) {
            return CopySrc{tileA + (int64_t)j * kSlab, tileB + (int64_t)j * kSlab,
                           reinterpret_cast<const uint8_t*>(scale_base + (int64_t)j * ld_s), offS};
        };
        // the next tile's first slab (rounds; every tile whole, so the lane
        // offsets of the A and B copies are those of this tile)
        CopySrc next0 = src_of(0);
        if constexpr (ROUNDS) {
            if (has_next) {
                const float* nb;
                uint32_t no;
                scale_src(nx, nb, no);
                next0 = CopySrc{p.a + nx.m0 * p.lda, nx.b + nx.n0 * p.ldb, reinterpret_cast<const uint8_t*>(nb), no};
            }
        }

        // Part i (0..3) of this wave's copy of slab j into stage st: 8 rows of
        // A and 8 rows of B; part 3 also carries the scales. Computing waves
        // spread the parts over their first n-subtiles, which keeps the LDS-DMA
        // writes from bunching up behind the barrier.
        // Three-stage kernels recompute the offsets of each copy (a few VALU
        // operations at the step boundary) instead of holding eight registers
        // through the MFMA loop.
        auto a_off = [&](int i) -> uint32_t {
            if constexpr (!DEEP) return offA[i];
            const int row = 32 * wave + 8 * i + (lane >> 3);
            const int src = 32 * wave + 8 * i >= a_rows ? max(a_rows - 1, 0) : row;
            return (uint32_t)((min(tr.m0 + src, m_last) - tr.m0) * p.lda) + swz_chunk(lane & 7, row) * 16;
        };
        auto b_off = [&](int i) -> uint32_t {
            if constexpr (!DEEP) return offB[i];
            const int row = 32 * wave + 8 * i + (lane >> 3);
            return (uint32_t)((min(tr.n0 + min(row, BN - 1), n_last) - tr.n0) * p.ldb) + swz_chunk(lane & 7, row) * 16;
        };
        auto copy_a_from = [&](const uint8_t* ga, auto st, int i) {
            uint8_t* base = stage_a<decltype(st)::value>() + 32 * wave * kSlab;
            // (offset computed outside the builtin's argument list: a lambda
            // call there keeps the host pass from emitting the kernel's stub)
            const uint32_t off = a_off(i);
            __builtin_amdgcn_global_load_lds(ga + off, (lds_void*)(base + i * 8 * kSlab), 16, 0, kPolicyDefault);
        };
        auto copy_b_from = [&](const uint8_t* gb, auto st, int i) {
            uint8_t* base = stage_b<decltype(st)::value>() + 32 * wave * kSlab;
            const uint32_t off = b_off(i);
            __builtin_amdgcn_global_load_lds(gb + off, (lds_void*)(base + i * 8 * kSlab), 16, 0,
                                             GROUPED ? kPolicyNonTemporal : kPolicyDefault);
        };
        auto copy_a = [&](int j, auto st, int i) { copy_a_from(tileA + (int64_t)j * kSlab, st, i); };
        auto copy_b = [&](int j, auto st, int i) { copy_b_from(tileB + (int64_t)j * kSlab, st, i); };
        auto issue_part = [&](const CopySrc& src, auto st, int i) {
            copy_a_from(src.a, st, i);
            copy_b_from(src.b, st, i);
            if constexpr (!DEEP && !TENSOR) {
                if (i == 3) {
                    constexpr int S = decltype(st)::value;
                    float* dst = wave < 4 ? stage_sa<S>() + 64 * wave : stage_sb<S>() + 64 * (wave - 4);
                    __builtin_amdgcn_global_load_lds(src.s + src.offs, (lds_void*)dst, 4, 0, 0);
                }
            }
        };
        auto issue = [&](const CopySrc& src, auto st) {
#pragma unroll
            for (int i = 0; i < 4; ++i) issue_part(src, st, i);
        };
        CopySrc nsrc = src_of(0);  // what the current step prefetches

        // ---- fragment addresses: lane (i = l%16, g = l/16) reads 32 bytes of
        // row i, the 16-byte chunks g and g + 4 of every 16-row subtile. In the
        // 16x16x128 FP8 MFMA the 32 bytes of lane group g are K[16g, 16g+16) and
        // K[64+16g, 64+16g+16) of the slab, and the scale of K block b (32
        // elements) comes from lane group b (measured on gfx950); with chunks g
        // and g + 4, block b is chunks 2b and 2b+1 -- the microscaling
        // quantizer's block b. The unscaled MFMA is blind to the order (A and B
        // share it), and this order reads LDS without bank conflicts (counted:
        // chunks 2g and 2g+1 cost ~11M conflict cycles per Dense Fprop GEMM).
        const int fi = lane & 15, fg = lane >> 4;
        const uint32_t off0 = fi * kSlab + swz_chunk(fg, fi) * 16;
        const uint32_t off1 = fi * kSlab + swz_chunk(fg + 4, fi) * 16;
        const uint32_t fragA = wm * kWaveM * kSlab;
        const uint32_t fragB = wn * WN * kSlab;
        // Block scales: the wave's first column lies in n-block nb0; sB holds the
        // tile's blocks from n0/128 on. Subtiles T < split are in nb0, the rest in
        // nb0 + 1 (only possible when STRADDLE).
        const int64_t wcol = tr.n0 + wn * WN;
        const int nb_rel = (int)(wcol / 128 - tr.n0 / 128);
        const int split = (int)((128 - (wcol & 127)) / 16);

        // Real rows of the wave (grouped padding, ragged M): m-subtiles past them
        // skip their MFMAs. act is wave-uniform.
        const int64_t wrow = tr.m0 + wm * kWaveM;
        const int64_t live = min(tr.real_end, tr.row_hi) - wrow;
        const int act = (int)max((int64_t)0, min((int64_t)kMSub, (live + 15) / 16));

        v4f acc[NSUB][kMSub];
#pragma unroll
        for (int t = 0; t < NSUB; ++t)
#pragma unroll
            for (int s = 0; s < kMSub; ++s) acc[t][s] = v4f{0.f, 0.f, 0.f, 0.f};

        const v4f zero = {0.f, 0.f, 0.f, 0.f};

        // Three-stage kernel: the lane's four A scales and the wave's B block
        // scale of slab j, loaded into registers one step ahead.
        const int row_a0 = (int)(wrow - tr.m0) + fi;       // the lane's row in m-subtile 0
        const int row_a_last = (int)(m_last - tr.m0);
        const float* const bscale_row = tr.b_scale + min(wcol, n_last) / 128 * p.ld_bs + tr.slab0;
        auto load_scales = [&](int j, float (&sa)[kMSub], float& sb) {
            const float* as = p.a_scale + tr.m0 + (int64_t)(tr.slab0 + j) * p.ld_as;
#pragma unroll
            for (int s = 0; s < kMSub; ++s) sa[s] = as[min(row_a0 + 16 * s, row_a_last)];
            sb = bscale_row[j];
        };

        // Block-scale dense kernels defer the promotion of each slab's last
        // subtile into the next slab (carry_p * carry_f; zero before the first).
        constexpr bool DEFER = !ROWSCALE && !DEEP;
        v4f carry_p[kMSub];
        float carry_f[kMSub];
#pragma unroll
        for (int s = 0; s < kMSub; ++s) {
            carry_p[s] = zero;
            carry_f[s] = 0.f;
        }

        // One slab of MFMAs + promotion for the first ACT m-subtiles of the wave,
        // on A stage AS and B stage BS (two-stage kernels: AS = BS, scales from
        // LDS; three-stage kernels: the products sA * sB come in sab_in).
        auto compute = [&](auto a_tag, auto b_tag, auto act_tag, const float (&sab_in)[kMSub]) {
            constexpr int ST = decltype(a_tag)::value;
            constexpr int BS = decltype(b_tag)::value;
            constexpr int ACT = decltype(act_tag)::value;
            const uint8_t* const la = stage_a<ST>() + fragA;
            const uint8_t* const lb = stage_b<BS>() + fragB;
            const float* const lsa = stage_sa<ST % 2>() + wm * kWaveM + fi;
            const float* const lsb = stage_sb<ST % 2>();
            // B fragment of n-subtile T (and, with per-row B scales, the lane's
            // four scales)
            auto read_b = [&](auto t_tag, v8i& bf, v4f& sbv) {
                constexpr int T = decltype(t_tag)::value;
                bf = ld_frag(lb + T * 2048 + off0, lb + T * 2048 + off1);
                if constexpr (ROWSCALE)
                    sbv = *reinterpret_cast<const v4f*>(lsb + wn * WN + 4 * fg + 16 * T);
            };
            v8i fr[2];
            v4f fsb[2];
            v4f pc[kMSub], pp[kMSub];
            v4f sbp;
            // Reads in the order the first MFMAs use them -- B fragment 0, A
            // fragments 0..3, then the scales (first needed by the promotion in
            // subtile 1) -- so the first MFMA waits for four reads, not all.
            read_b(std::integral_constant<int, 0>{}, fr[0], fsb[0]);
            v8i am[kMSub];
            float sa[kMSub];
#pragma unroll
            for (int s = 0; s < kMSub; ++s) am[s] = ld_frag(la + s * 2048 + off0, la + s * 2048 + off1);
#pragma unroll
            for (int s = 0; s < kMSub; ++s) sa[s] = DEEP ? 0.f : lsa[16 * s];
            const float sb0 = (ROWSCALE || DEEP) ? 0.f : lsb[nb_rel];
            const float sb1 = (ROWSCALE || !STRADDLE) ? 0.f : lsb[nb_rel + 1];
            float sab0[kMSub], sab1[kMSub];
            // Software pipeline over the n-subtiles: while the MFMAs of subtile T
            // run, the fragment of T+1 is in flight and the partials of T-1 are
            // promoted (acc += P * sA * sB), one FMA group after each MFMA.
            auto promote = [&](auto t_tag, const v4f& sbn) {
                constexpr int T = decltype(t_tag)::value;
#pragma unroll
                for (int s = 0; s < ACT; ++s) {
                    if constexpr (ROWSCALE) {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            acc[T][s][r] = __builtin_fmaf(pp[s][r], sa[s] * sbn[r], acc[T][s][r]);
                    } else {
                        float f = sab0[s];
                        if constexpr (STRADDLE) f = T < split ? sab0[s] : sab1[s];
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[T][s][r] = __builtin_fmaf(pp[s][r], f, acc[T][s][r]);
                    }
                }
            };
            __builtin_amdgcn_sched_barrier(0);
            unroll(std::make_integer_sequence<int, NSUB>{}, [&](auto t_tag) {
                constexpr int T = decltype(t_tag)::value;
                constexpr int NEXT_READS = ROWSCALE ? 3 : 2;
                const v8i bf = fr[T & 1];
                if constexpr (T + 1 < NSUB)
                    read_b(std::integral_constant<int, T + 1>{}, fr[(T + 1) & 1], fsb[(T + 1) & 1]);
                if constexpr (!GROUPED && T < 4)
                    issue_part(nsrc, std::integral_constant<int, ST ^ 1>{}, T);
#pragma unroll
                for (int s = 0; s < ACT; ++s)
                    pc[s] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, am[s], zero, 0, 0, 0, 0, 0, 0);
                if constexpr (T == 0) {
                    // the previous slab's last subtile (deferred), then this
                    // slab's scale products
                    if constexpr (DEFER) {
#pragma unroll
                        for (int s = 0; s < ACT; ++s)
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                acc[NSUB - 1][s][r] = __builtin_fmaf(carry_p[s][r], carry_f[s], acc[NSUB - 1][s][r]);
                    }
#pragma unroll
                    for (int s = 0; s < kMSub; ++s) {
                        sab0[s] = DEEP ? sab_in[s] : sa[s] * sb0;
                        if constexpr (STRADDLE) sab1[s] = sa[s] * sb1;
                    }
                } else {
                    promote(std::integral_constant<int, T - 1>{}, sbp);
                }
                // Order: the first MFMA (its wait covers only the fragment read
                // one subtile earlier), the next fragment's reads, this subtile's
                // copy part, then the FMA group of one m-subtile after each MFMA.
                constexpr int FMAS = ROWSCALE ? 8 : (STRADDLE ? 5 : 4);
                constexpr bool HAS_FMAS = T > 0 || DEFER;
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if constexpr (T + 1 < NSUB) __builtin_amdgcn_sched_group_barrier(0x100, NEXT_READS, 0);
                if constexpr (!GROUPED && T < 4) __builtin_amdgcn_sched_group_barrier(0x020, T == 3 ? 3 : 2, 0);
                if constexpr (HAS_FMAS) __builtin_amdgcn_sched_group_barrier(0x002, T > 0 ? FMAS : 4, 0);
#pragma unroll
                for (int s = 1; s < ACT; ++s) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if constexpr (HAS_FMAS) __builtin_amdgcn_sched_group_barrier(0x002, T > 0 ? FMAS : 4, 0);
                }
#pragma unroll
                for (int s = 0; s < ACT; ++s) pp[s] = pc[s];
                sbp = fsb[T & 1];
                __builtin_amdgcn_sched_barrier(0);
            });
            if constexpr (DEFER) {
                // the last subtile is promoted at the start of the next slab,
                // where the VALU otherwise waits for the fragment reads
#pragma unroll
                for (int s = 0; s < kMSub; ++s) {
                    carry_p[s] = pp[s];
                    carry_f[s] = (!STRADDLE || NSUB - 1 < split) ? sab0[s] : sab1[s];
                }
            } else {
                promote(std::integral_constant<int, NSUB - 1>{}, sbp);
            }
            __builtin_amdgcn_sched_barrier(0);
        };

        // One slab of the in-place GEMMs. Microscaling: the scaled MFMA takes
        // each lane's E8M0 byte (lane group g supplies block g's byte, see the
        // fragment addresses) and accumulates into acc directly. Per-tensor: the
        // plain MFMA accumulates into acc directly.
        auto compute_inplace = [&](auto a_tag, auto act_tag) {
            constexpr int ST = decltype(a_tag)::value;
            constexpr int ACT = decltype(act_tag)::value;
            const uint8_t* const la = stage_a<ST>() + fragA;
            const uint8_t* const lb = stage_b<ST>() + fragB;
            const uint32_t* const lsa = reinterpret_cast<const uint32_t*>(stage_sa<ST>()) + wm * kWaveM + fi;
            const uint32_t* const lsb = reinterpret_cast<const uint32_t*>(stage_sb<ST>()) + wn * WN + fi;
            const int shift = 8 * fg;
            v8i fr[2];
            uint32_t sbw[2];
            fr[0] = ld_frag(lb + off0, lb + off1);
            sbw[0] = MX ? lsb[0] : 0u;
            v8i am[kMSub];
            int sae[kMSub];
#pragma unroll
            for (int s = 0; s < kMSub; ++s) am[s] = ld_frag(la + s * 2048 + off0, la + s * 2048 + off1);
#pragma unroll
            for (int s = 0; s < kMSub; ++s) sae[s] = MX ? (int)((lsa[16 * s] >> shift) & 0xFFu) : 0;
            __builtin_amdgcn_sched_barrier(0);
            unroll(std::make_integer_sequence<int, NSUB>{}, [&](auto t_tag) {
                constexpr int T = decltype(t_tag)::value;
                const v8i bf = fr[T & 1];
                const int sbe = MX ? (int)((sbw[T & 1] >> shift) & 0xFFu) : 0;
                if constexpr (T + 1 < NSUB) {
                    fr[(T + 1) & 1] = ld_frag(lb + (T + 1) * 2048 + off0, lb + (T + 1) * 2048 + off1);
                    if constexpr (MX) sbw[(T + 1) & 1] = lsb[16 * (T + 1)];
                }
                if constexpr (T < 4) issue_part(nsrc, std::integral_constant<int, ST ^ 1>{}, T);
#pragma unroll
                for (int s = 0; s < ACT; ++s) {
                    // (zero scale operands select the unscaled instruction)
                    if constexpr (MX)
                        acc[T][s] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, am[s], acc[T][s], 0, 0,
                                                                                    0, sbe, 0, sae[s]);
                    else
                        acc[T][s] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, am[s], acc[T][s], 0, 0,
                                                                                    0, 0, 0, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if constexpr (T + 1 < NSUB) __builtin_amdgcn_sched_group_barrier(0x100, MX ? 3 : 2, 0);
                if constexpr (T < 4) __builtin_amdgcn_sched_group_barrier(0x020, T == 3 ? 3 : 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, ACT - 1, 0);
                __builtin_amdgcn_sched_barrier(0);
            });
        };

        // The K loop for a wave with ACT live m-subtiles (ACT = 0: the wave only
        // does its share of the copies and the barriers).
        auto mainloop = [&](auto act_tag) {
            constexpr int ACT = decltype(act_tag)::value;
            const float no_sab[kMSub] = {0.f, 0.f, 0.f, 0.f};
            // A step waits for its slab at its start; with several rounds at its
            // end instead (the same wait, for the copy it issued), so that the
            // last step of a tile leaves the next tile's first slab ready and the
            // tile's stores are never waited for.
            auto step = [&](auto stage_tag, int j) {
                constexpr int ST = decltype(stage_tag)::value;
                if constexpr (!ROUNDS) wait_dma_and_barrier<0>();
                // Prefetch the next slab into the other stage: spread over the
                // first n-subtiles, or all at once for a wave without MFMA work.
                // The last step copies the next tile's first slab there (rounds)
                // or re-loads its own slab (never read), keeping the body
                // branch-free.
                nsrc = src_of(min(j + 1, slabs - 1));
                if constexpr (ROUNDS) {
                    // (values, not lvalues: a select between two objects' fields
                    // would keep every local of the kernel in scratch memory)
                    const bool cross = j + 1 >= slabs && has_next;
                    nsrc = CopySrc{pick(cross, next0.a, nsrc.a), pick(cross, next0.b, nsrc.b),
                                   pick(cross, next0.s, nsrc.s), pick(cross, next0.offs, nsrc.offs)};
                }
                if constexpr (ACT == 0) issue(nsrc, std::integral_constant<int, ST ^ 1>{});
                if constexpr (ACT > 0) {
                    if constexpr (INPLACE)
                        compute_inplace(stage_tag, act_tag);
                    else
                        compute(stage_tag, stage_tag, act_tag, no_sab);
                }
                if constexpr (ROUNDS) wait_dma_and_barrier<0>();
            };
            if (slabs > 0 && !prefetched) {
                issue(src_of(0), std::integral_constant<int, 0>{});
                if constexpr (ROUNDS) wait_dma_and_barrier<0>();
            }
            int j = 0;
            for (; j + 2 <= slabs; j += 2) {
                step(std::integral_constant<int, 0>{}, j);
                step(std::integral_constant<int, 1>{}, j + 1);
            }
            if (j < slabs) step(std::integral_constant<int, 0>{}, j);
            if constexpr (DEFER && ACT > 0) {
#pragma unroll
                for (int s = 0; s < ACT; ++s)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        acc[NSUB - 1][s][r] = __builtin_fmaf(carry_p[s][r], carry_f[s], acc[NSUB - 1][s][r]);
            }
        };

        // Three-stage K loop: slab j lives in A stage j % 2 and B stage j % 3.
        // Step j waits until only this wave's youngest copy (the 4 B parts of
        // slab j + 1) may still be in flight, then prefetches the scales and A of
        // slab j + 1 and the B of slab j + 2, in that order (the wait count
        // relies on it). Clamped slab indices keep the tail branch-free.
        auto mainloop_deep = [&](auto act_tag) {
            constexpr int ACT = decltype(act_tag)::value;
            float sa_nx[kMSub], sb_nx;
            auto copy_all_a = [&](int jj, auto st) {
#pragma unroll
                for (int i = 0; i < 4; ++i) copy_a(jj, st, i);
            };
            auto copy_all_b = [&](int jj, auto st) {
#pragma unroll
                for (int i = 0; i < 4; ++i) copy_b(jj, st, i);
            };
            auto step = [&](auto a_tag, auto b_tag, int j) {
                constexpr int AS = decltype(a_tag)::value;
                constexpr int BS = decltype(b_tag)::value;
                wait_dma_and_barrier<4>();
                float sab[kMSub];
#pragma unroll
                for (int s = 0; s < kMSub; ++s) sab[s] = sa_nx[s] * sb_nx;
                load_scales(min(j + 1, slabs - 1), sa_nx, sb_nx);
                copy_all_a(min(j + 1, slabs - 1), std::integral_constant<int, AS ^ 1>{});
                __builtin_amdgcn_sched_barrier(0);
                copy_all_b(min(j + 2, slabs - 1), std::integral_constant<int, (BS + 2) % 3>{});
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (ACT > 0) compute(a_tag, b_tag, act_tag, sab);
            };
            using I0 = std::integral_constant<int, 0>;
            using I1 = std::integral_constant<int, 1>;
            using I2 = std::integral_constant<int, 2>;
            if (slabs == 0) return;
            load_scales(0, sa_nx, sb_nx);
            copy_all_a(0, I0{});
            __builtin_amdgcn_sched_barrier(0);
            copy_all_b(0, I0{});
            __builtin_amdgcn_sched_barrier(0);
            copy_all_b(min(1, slabs - 1), I1{});
            __builtin_amdgcn_sched_barrier(0);
            int j = 0;
            for (; j + 6 <= slabs; j += 6) {
                step(I0{}, I0{}, j);
                step(I1{}, I1{}, j + 1);
                step(I0{}, I2{}, j + 2);
                step(I1{}, I0{}, j + 3);
                step(I0{}, I1{}, j + 4);
                step(I1{}, I2{}, j + 5);
            }
            const int rem = slabs - j;
            if (rem > 0) step(I0{}, I0{}, j);
            if (rem > 1) step(I1{}, I1{}, j + 1);
            if (rem > 2) step(I0{}, I2{}, j + 2);
            if (rem > 3) step(I1{}, I0{}, j + 3);
            if (rem > 4) step(I0{}, I1{}, j + 4);
        };
        if constexpr (GROUPED) {
            // expert tails: only the live m-subtiles do MFMA work
            switch (act) {
                case 4: mainloop_deep(std::integral_constant<int, 4>{}); break;
                case 3: mainloop_deep(std::integral_constant<int, 3>{}); break;
                case 2: mainloop_deep(std::integral_constant<int, 2>{}); break;
                case 1: mainloop_deep(std::integral_constant<int, 1>{}); break;
                default: mainloop_deep(std::integral_constant<int, 0>{}); break;
            }
        } else if (ROUNDS || act > 0) {
            mainloop(std::integral_constant<int, 4>{});  // ragged-M rows are computed and dropped
        } else {
            mainloop(std::integral_constant<int, 0>{});
        }
        // Drain the last (unused) prefetches before the block's LDS can be reused
        // (with several rounds every step has waited for its copy already).
        if constexpr (!ROUNDS) __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));

        // ---- epilogue: lane holds C[m][n..n+3] for each (n-subtile, m-subtile).
        // (k == 0: the scales may be NULL and are not read; C is zero)
        const float alpha = (TENSOR && p.k > 0) ? p.a_scale[0] * p.b_scale[0] : 1.0f;
        if constexpr (GROUPED) {
            if (tr.piece >= 0) {
                // a K piece of a split tile: the FP32 partial in fragment order
                // (one store instruction writes 1 KB), for the fix-up kernel
                v4f* const dst = reinterpret_cast<v4f*>(p.split_ws) +
                                 ((int64_t)tr.piece * 8 + wave) * (NSUB * kMSub * 64) + lane;
#pragma unroll
                for (int t = 0; t < NSUB; ++t)
#pragma unroll
                    for (int s = 0; s < kMSub; ++s) dst[(t * kMSub + s) * 64] = acc[t][s];
                return;
            }
        }
        if constexpr (ROUNDS) {
            // whole tiles: no edge guards (their branches would keep these loops
            // rolled inside the tile loop)
#pragma unroll
            for (int s = 0; s < kMSub; ++s) {
                const int64_t m = wrow + s * 16 + fi;
#pragma unroll
                for (int t = 0; t < NSUB; ++t) {
                    const int64_t n = wcol + t * 16 + 4 * fg;
                    const v4f v = acc[t][s];
                    if constexpr (OUT_F32) {
                        *reinterpret_cast<v4f*>(reinterpret_cast<float*>(tr.c) + m * p.ldc + n) = v;
                    } else {
                        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(tr.c) + m * p.ldc + n) =
                            make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                    }
                }
            }
        } else {
#pragma unroll
            for (int s = 0; s < kMSub; ++s) {
                const int64_t m = wrow + s * 16 + fi;
                if (m >= tr.row_hi) continue;
                const bool pad = m >= tr.real_end;
#pragma unroll
                for (int t = 0; t < NSUB; ++t) {
                    const int64_t n = wcol + t * 16 + 4 * fg;
                    if (n >= tr.n0 + BN) continue;
                    v4f v = pad ? zero : acc[t][s];
                    if constexpr (TENSOR) v = v * alpha;
                    if constexpr (OUT_F32) {
                        float* dst = reinterpret_cast<float*>(tr.c) + m * p.ldc + n;
                        if (n + 3 < p.n) {
                            *reinterpret_cast<v4f*>(dst) = v;
                        } else {
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                if (n + r < p.n) dst[r] = v[r];
                        }
                    } else {
                        uint16_t* dst = reinterpret_cast<uint16_t*>(tr.c) + m * p.ldc + n;
                        const uint32_t lo = pack_bf16x2(v[0], v[1]), hi = pack_bf16x2(v[2], v[3]);
                        if (n + 3 < p.n) {
                            *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
                        } else {
                            const uint16_t h[4] = {(uint16_t)lo, (uint16_t)(lo >> 16), (uint16_t)hi,
                                                   (uint16_t)(hi >> 16)};
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                if (n + r < p.n) dst[r] = h[r];
                        }
                    }
                }
            }
        }
        if (!has_next) break;
        tr = nx;
        prefetched = true;
    }
}

// Sum of the K pieces of each split tile of a grouped GEMM's last round
// (see tail_split), in piece order, stored to C as the GEMM stores a whole
// tile: rows past row_hi untouched, padding rows zero. The work is cut into
// units of 256 output vectors (an eighth of one GEMM wave's 64 x 128 outputs,
// in its fragment order), 64 per tail tile; block b takes units b, b + grid,
// ..., one vector per thread: the blocks get equal shares, every load
// instruction reads 1 KB contiguous per wave, and a unit's partial loads and
// its tile record (written by the tile's first piece) are in flight together.
// When nothing was split the blocks return after the scan.
constexpr int kFixupThreads = 256;
constexpr int kFixupBlocks = 1024;

template <bool OUT_F32>
__global__ __launch_bounds__(kFixupThreads) void grouped_fixup_kernel(Params p) {
    constexpr int BN = 256, WN = BN / 2, NSUB = WN / 16;
    constexpr int kItems = NSUB * kMSub * 64;           // one GEMM wave's partial, in v4f
    constexpr int kUnits = 8 * kItems / kFixupThreads;  // units per tile
    const TailSplit ts = tail_split<BN>(p);
    if (ts.split < 2) return;
    const v4f* const part = reinterpret_cast<const v4f*>(p.split_ws);
    for (int unit = (int)blockIdx.x; unit < ts.tiles * kUnits; unit += (int)gridDim.x) {
        const int r = unit / kUnits;
        const int flat = (unit % kUnits) * kFixupThreads + (int)threadIdx.x;  // in [0, 8 kItems)
        const int w = flat / kItems, item = flat % kItems;
        v4f pv[kMaxSplit];
#pragma unroll
        for (int i = 0; i < kMaxSplit; ++i)
            if (i < ts.split) pv[i] = part[((int64_t)(i * ts.tiles + r) * 8 + w) * kItems + item];
        const TailRecord tr = p.split_records[r];
        const int lane = item & 63, s = (item >> 6) % kMSub, t = (item >> 6) / kMSub;
        const int64_t m = tr.m0 + (w >> 1) * kWaveM + s * 16 + (lane & 15);
        const int64_t n = tr.n0 + (w & 1) * WN + t * 16 + 4 * (lane >> 4);
        // (offsets that break the contract can leave a piece unrun and its
        // record from an earlier call: the stores still stay inside C)
        if (m >= tr.row_hi || m >= p.m || tr.m0 < 0 || tr.n0 < 0) continue;
        v4f v = {0.f, 0.f, 0.f, 0.f};
        if (m < tr.real_end) {
#pragma unroll
            for (int i = 0; i < kMaxSplit; ++i)
                if (i < ts.split) v += pv[i];
        }
        if constexpr (OUT_F32) {
            float* dst = reinterpret_cast<float*>(p.c) + m * p.ldc + n;
            if (n + 3 < p.n) {
                *reinterpret_cast<v4f*>(dst) = v;
            } else {
                for (int q = 0; q < 4; ++q)
                    if (n + q < p.n) dst[q] = v[q];
            }
        } else {
            uint16_t* dst = reinterpret_cast<uint16_t*>(p.c) + m * p.ldc + n;
            const uint32_t lo = pack_bf16x2(v[0], v[1]), hi = pack_bf16x2(v[2], v[3]);
            if (n + 3 < p.n) {
                *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
            } else {
                const uint16_t h[4] = {(uint16_t)lo, (uint16_t)(lo >> 16), (uint16_t)hi, (uint16_t)(hi >> 16)};
                for (int q = 0; q < 4; ++q)
                    if (n + q < p.n) dst[q] = h[q];
            }
        }
    }
}

// blocks: the dense slots rounded up to a multiple of 8.
template <int BN>
hipError_t dispatch_dense(const GemmProblem& g, int64_t blocks, hipStream_t stream) {
    const Params p = to_params(g);
    const dim3 grid((unsigned)blocks), block(kThreads);
    if (g.b_rowscale) {
        if (g.out_f32)
            hipLaunchKernelGGL((gemm_kernel<BN, true, true, kDense>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((gemm_kernel<BN, true, false, kDense>), grid, block, 0, stream, p);
    } else {
        if (g.out_f32)
            hipLaunchKernelGGL((gemm_kernel<BN, false, true, kDense>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((gemm_kernel<BN, false, false, kDense>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

// A dense GEMM of several rounds of whole tiles: 256 blocks, one per CU,
// each looping over its tiles (see dense_tile).
template <int BN>
hipError_t dispatch_rounds(const GemmProblem& g, hipStream_t stream) {
    const Params p = to_params(g);
    const dim3 grid(256), block(kThreads);
    if (g.b_rowscale) {
        if (g.out_f32)
            hipLaunchKernelGGL((gemm_kernel<BN, true, true, kDenseRounds>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((gemm_kernel<BN, true, false, kDenseRounds>), grid, block, 0, stream, p);
    } else {
        if (g.out_f32)
            hipLaunchKernelGGL((gemm_kernel<BN, false, true, kDenseRounds>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((gemm_kernel<BN, false, false, kDenseRounds>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

// Microscaling dense GEMM (per-row E8M0 scale words on both operands).
template <int BN>
hipError_t dispatch_mx(const GemmProblem& g, int64_t blocks, hipStream_t stream) {
    const Params p = to_params(g);
    const dim3 grid((unsigned)blocks), block(kThreads);
    if (g.out_f32)
        hipLaunchKernelGGL((gemm_kernel<BN, true, true, kDense, true>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((gemm_kernel<BN, true, false, kDense, true>), grid, block, 0, stream, p);
    return hipGetLastError();
}

// Per-tensor scaled dense GEMM (whole-K accumulation in the MFMA).
template <int BN>
hipError_t dispatch_tensor(const GemmProblem& g, int64_t blocks, hipStream_t stream) {
    const Params p = to_params(g);
    const dim3 grid((unsigned)blocks), block(kThreads);
    if (g.out_f32)
        hipLaunchKernelGGL((gemm_kernel<BN, true, true, kDense, false, true>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((gemm_kernel<BN, true, false, kDense, false, true>), grid, block, 0, stream, p);
    return hipGetLastError();
}

// blocks: a multiple of 256 (see grouped_tile). Grouped GEMMs take 128x128
// block scales only.
constexpr int64_t kRecordBytes = kTailRecords * (int64_t)sizeof(TailRecord);
constexpr int64_t kPartBytes = kSplitFloats * (int64_t)sizeof(float);
static_assert(FP8Q_GROUPED_WORKSPACE_BYTES == kRecordBytes + kMaxPieces * kPartBytes,
              "the workspace size in fp8q.h holds every record and partial a call can use");

hipError_t dispatch_grouped(const GemmProblem& g, int64_t blocks, hipStream_t stream) {
    Params p = to_params(g);
    // workspace: the tile records, then as many partial tiles as fit (two at
    // least, or no split)
    const int64_t pieces = g.workspace ? std::min<int64_t>((g.workspace_bytes - kRecordBytes) / kPartBytes, kMaxPieces) : 0;
    if (pieces >= 2) {
        p.split_records = static_cast<TailRecord*>(g.workspace);
        p.split_ws = reinterpret_cast<float*>(static_cast<char*>(g.workspace) + kRecordBytes);
        p.split_pieces = (int32_t)pieces;
    }
    const dim3 grid((unsigned)blocks), block(kThreads);
    if (g.out_f32)
        hipLaunchKernelGGL((gemm_kernel<256, false, true, kGroupedM>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((gemm_kernel<256, false, false, kGroupedM>), grid, block, 0, stream, p);
    if (p.split_ws == nullptr) return hipGetLastError();
    const dim3 fgrid(kFixupBlocks), fblock(kFixupThreads);
    if (g.out_f32)
        hipLaunchKernelGGL((grouped_fixup_kernel<true>), fgrid, fblock, 0, stream, p);
    else
        hipLaunchKernelGGL((grouped_fixup_kernel<false>), fgrid, fblock, 0, stream, p);
    return hipGetLastError();
}

// blocks: a multiple of 256 (see grouped_k_tile). Grouped-over-K GEMMs take
// per-row (128x1) scales on both operands, as Wgrad does.
template <int BN>
hipError_t dispatch_grouped_k(const GemmProblem& g, int64_t blocks, hipStream_t stream) {
    const Params p = to_params(g);
    const dim3 grid((unsigned)blocks), block(kThreads);
    if (g.out_f32)
        hipLaunchKernelGGL((gemm_kernel<BN, true, true, kGroupedK>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((gemm_kernel<BN, true, false, kGroupedK>), grid, block, 0, stream, p);
    return hipGetLastError();
}

// Time of a dense grid in units of one 256-wide tile's work: the number of
// rounds of the 256 CUs times the tile width (all tiles share K and BM).
int64_t grid_cost(int64_t m, int64_t n, int64_t bn) {
    const int64_t tiles = ((m + kBM - 1) / kBM) * ((n + bn - 1) / bn);
    return (tiles + 255) / 256 * bn;
}

}  // namespace

// Several rounds of whole 224-wide tiles, with an even number of slabs: one
// looping block per CU. (Paired on one MI355X, bit-identical output: Dgrad
// 4096 x 7168 x 2048 took 64.2 against 65.4 us, and 8192 x 7168 x 2048 118.9
// against 123.7 us; a 256-wide looping tile, which needs a few more registers
// than the kernel has, gained nothing on 8192 x 4096 x 7168.)
bool use_rounds(const GemmProblem& g) {
    const int64_t tiles = ((g.m + kBM - 1) / kBM) * ((g.n + 223) / 224);
    const int64_t slabs = g.k / kSlab;
    return tiles > 256 && g.m % kBM == 0 && g.n % 224 == 0 && slabs >= 2 && slabs % 2 == 0;
}

hipError_t launch_gemm(const GemmProblem& g, hipStream_t stream) {
    // 224-wide n tiles when the grid then takes less time on the 256 CUs,
    // e.g. N = 7168 = 32 x 224 (Dgrad, Wgrad); otherwise 256-wide.
    if (grid_cost(g.m, g.n, 224) < grid_cost(g.m, g.n, 256)) {
        if (use_rounds(g)) return dispatch_rounds<224>(g, stream);
        const int64_t tiles = ((g.m + kBM - 1) / kBM) * ((g.n + 223) / 224);
        return dispatch_dense<224>(g, (tiles + 7) / 8 * 8, stream);
    }
    const int64_t tiles = ((g.m + kBM - 1) / kBM) * ((g.n + 255) / 256);
    return dispatch_dense<256>(g, (tiles + 7) / 8 * 8, stream);
}

hipError_t launch_grouped_gemm(const GemmProblem& g, hipStream_t stream) {
    // Upper bound on the tile count: every 256-row m-tile of an expert holds at
    // least 128 of its rows, so there are at most m_total / 128 of them.
    const int64_t tiles = (g.m / 128) * ((g.n + 255) / 256);
    return dispatch_grouped(g, (tiles + 255) / 256 * 256, stream);
}

hipError_t launch_grouped_k_gemm(const GemmProblem& g, hipStream_t stream) {
    // Every expert has the same output tiles; 224-wide when that tiles N
    // better (N = 7168), as for a dense GEMM.
    const int bn = grid_cost(g.m, g.n, 224) < grid_cost(g.m, g.n, 256) ? 224 : 256;
    const int64_t per = ((g.m + kBM - 1) / kBM) * ((g.n + bn - 1) / bn);
    const int64_t blocks = (per * g.groups + 255) / 256 * 256;
    return bn == 224 ? dispatch_grouped_k<224>(g, blocks, stream)
                     : dispatch_grouped_k<256>(g, blocks, stream);
}

hipError_t launch_gemm_mx(const GemmProblem& g, hipStream_t stream) {
    if (grid_cost(g.m, g.n, 224) < grid_cost(g.m, g.n, 256)) {
        const int64_t tiles = ((g.m + kBM - 1) / kBM) * ((g.n + 223) / 224);
        return dispatch_mx<224>(g, (tiles + 7) / 8 * 8, stream);
    }
    const int64_t tiles = ((g.m + kBM - 1) / kBM) * ((g.n + 255) / 256);
    return dispatch_mx<256>(g, (tiles + 7) / 8 * 8, stream);
}

hipError_t launch_gemm_tensor(const GemmProblem& g, hipStream_t stream) {
    if (grid_cost(g.m, g.n, 224) < grid_cost(g.m, g.n, 256)) {
        const int64_t tiles = ((g.m + kBM - 1) / kBM) * ((g.n + 223) / 224);
        return dispatch_tensor<224>(g, (tiles + 7) / 8 * 8, stream);
    }
    const int64_t tiles = ((g.m + kBM - 1) / kBM) * ((g.n + 255) / 256);
    return dispatch_tensor<256>(g, (tiles + 7) / 8 * 8, stream);
}

// Scratch of the allocation-free grouped GEMM (fp8_grouped_gemm_noalloc): the
// largest workspace a call uses, one copy on every GPU the library runs on,
// held until the process ends. In host code the array's name is a host-side
// stand-in, not a device address: host code uses only the address that
// hipGetSymbolAddress gives with the device current, kept per device.
__device__ __align__(256) uint8_t scratch[FP8Q_GROUPED_WORKSPACE_BYTES];

constexpr int kMaxScratchDevices = 64;

hipError_t grouped_scratch(void** ptr) {
    static std::mutex mu;
    static void* per_device[kMaxScratchDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (per_device[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        per_device[dev] = p;
    }
    *ptr = per_device[dev];
    return hipSuccess;
}

}  // namespace fp8q
