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
// overlapped with the next subtile's MFMA. There is no limited-precision
// accumulator to protect: the FP32 MFMA sum of a slab is already exact-ish,
// and the interval is set by the scales, not by the hardware.
//
// Tiling: 256 (m) x 256 (n) block tile, 8 waves (4 along m x 2 along n),
// 64 x 128 per wave. Each 128-byte K slab of the A and B tiles is copied
// global -> LDS by the direct LDS-DMA load (global_load_lds_dwordx4), double
// buffered, with 16-byte chunks XOR-swizzled by row so that fragment reads
// are bank-conflict free. The MFMA computes the transposed tile: its row
// operand is B (n), its column operand is A (m), so every lane holds four
// consecutive n of one m -- one A scale per lane per m-subtile, and the B
// block scale is wave-uniform.
#include "fp8q_device.h"
#include "launch.h"

#include <type_traits>

namespace fp8q {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kSlab = 128;  // K elements per promotion interval
constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kThreads = 512;
constexpr int kWaveM = 64;
constexpr int kWaveN = 128;
constexpr int kMSub = kWaveM / 16;
constexpr int kNSub = kWaveN / 16;

// LDS map (bytes): A stage 0 | A stage 1 | B stage 0 | B stage 1 |
//                  sA stage 0 | sA stage 1 | sB stage 0 | sB stage 1.
constexpr int kTileBytes = kBM * kSlab;
constexpr int kOffA = 0;
constexpr int kOffB = 2 * kTileBytes;
constexpr int kOffSA = 4 * kTileBytes;
constexpr int kOffSB = kOffSA + 2 * kBM * 4;
constexpr int kLdsBytes = kOffSB + 2 * kBN * 4;

// Physical 16-byte chunk of logical chunk c in LDS row `row`.
__device__ __forceinline__ int swz_chunk(int c, int row) { return c ^ (row & 7); }

struct Params {
    int64_t m, n, k;
    const uint8_t* a;
    int64_t lda;
    const float* a_scale;
    int64_t ld_as;
    const uint8_t* b;
    int64_t ldb;
    const float* b_scale;
    int64_t ld_bs;
    void* c;
    int64_t ldc;
    int32_t groups;
    const int32_t* group_offsets;
    const int32_t* group_rows;
    int64_t stride_b;
    int64_t stride_bs;
};

// Which rows of the output a block tile owns.
struct TileRows {
    int64_t m0;        // first row of the tile
    int64_t row_hi;    // rows >= row_hi belong to someone else: not stored
    int64_t real_end;  // rows in [real_end, row_hi) are padding: stored as 0
    int64_t n0;
    const uint8_t* b;
    const float* b_scale;
};

// Dense tile order: block -> XCD x = block % 8 gets the contiguous slot
// range [x*per, (x+1)*per); slots walk 4-row bands of tiles so the blocks
// resident on one XCD share A and B panels in its L2.
__device__ __forceinline__ bool dense_tile(const Params& p, TileRows& t) {
    const int tiles_m = (int)((p.m + kBM - 1) / kBM);
    const int tiles_n = (int)((p.n + kBN - 1) / kBN);
    const int total = tiles_m * tiles_n;
    const int per = (total + 7) / 8;
    const int slot = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
    if (slot >= total) return false;
    constexpr int G = 4;
    const int group = slot / (G * tiles_n);
    const int first_m = group * G;
    const int gm = min(tiles_m - first_m, G);
    const int within = slot - group * G * tiles_n;
    const int tm = first_m + within % gm;
    const int tn = within / gm;
    t.m0 = (int64_t)tm * kBM;
    t.row_hi = p.m;
    t.real_end = p.m;
    t.n0 = (int64_t)tn * kBN;
    t.b = p.b;
    t.b_scale = p.b_scale;
    return true;
}

// Grouped tile order: expert e's segment [off[e], off[e+1]) is cut into
// 256-row m-tiles (the last may hold only 128 rows); slots run expert-major,
// then n-tile, then m-tile, so consecutive slots on one XCD reuse the same
// 256 x K panel of W_e.
__device__ __forceinline__ bool grouped_tile(const Params& p, TileRows& t) {
    const int tiles_n = (int)(p.n / kBN + (p.n % kBN != 0));
    int total = 0;
    for (int e = 0; e < p.groups; ++e) {
        const int seg = p.group_offsets[e + 1] - p.group_offsets[e];
        total += (seg + kBM - 1) / kBM * tiles_n;
    }
    const int per = (total + 7) / 8;
    int slot = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
    if (slot >= total) return false;
    for (int e = 0; e < p.groups; ++e) {
        const int beg = p.group_offsets[e], end = p.group_offsets[e + 1];
        const int cnt = (end - beg + kBM - 1) / kBM;
        if (slot < cnt * tiles_n) {
            const int tn = slot / cnt, mt = slot - tn * cnt;
            t.m0 = beg + (int64_t)mt * kBM;
            // offsets that break the contract must not move stores outside C
            if (t.m0 < 0 || t.m0 >= p.m) return false;
            t.row_hi = min(min((int64_t)end, t.m0 + kBM), p.m);
            const int real = p.group_rows ? p.group_rows[e] : end - beg;
            t.real_end = beg + (int64_t)real;
            t.n0 = (int64_t)tn * kBN;
            t.b = p.b + e * p.stride_b;
            t.b_scale = p.b_scale + e * p.stride_bs;
            return true;
        }
        slot -= cnt * tiles_n;
    }
    return false;
}

// ---------------------------------------------------------------- LDS reads
// Fragment reads are inline asm with their own s_waitcnt: the compiler would
// otherwise wait for every outstanding LDS-DMA load (including the prefetch
// of the next slab) before any LDS read, serialising load and compute. The
// DMA of a stage is fenced explicitly (vmcnt(0) + barrier) before it is read.

// A fragments of the four m-subtiles plus the lane's four A scales and the
// wave's B block scale (or, with per-row B scales, an unused value).
template <int ST>
__device__ __forceinline__ void read_a_frags(uint32_t v0, uint32_t v1, uint32_t vs, uint32_t vsb,
                                             v8i (&am)[kMSub], float (&sa)[kMSub], float& sb) {
    v4i l0, h0, l1, h1, l2, h2, l3, h3;
    float f0, f1, f2, f3, fb;
    asm volatile(
        "ds_read_b128 %0, %13 offset:%15\n\t"
        "ds_read_b128 %1, %14 offset:%15\n\t"
        "ds_read_b128 %2, %13 offset:%16\n\t"
        "ds_read_b128 %3, %14 offset:%16\n\t"
        "ds_read_b128 %4, %13 offset:%17\n\t"
        "ds_read_b128 %5, %14 offset:%17\n\t"
        "ds_read_b128 %6, %13 offset:%18\n\t"
        "ds_read_b128 %7, %14 offset:%18\n\t"
        "ds_read_b32 %8, %19 offset:%20\n\t"
        "ds_read_b32 %9, %19 offset:%21\n\t"
        "ds_read_b32 %10, %19 offset:%22\n\t"
        "ds_read_b32 %11, %19 offset:%23\n\t"
        "ds_read_b32 %12, %24 offset:%25\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(l0), "=&v"(h0), "=&v"(l1), "=&v"(h1), "=&v"(l2), "=&v"(h2), "=&v"(l3), "=&v"(h3),
          "=&v"(f0), "=&v"(f1), "=&v"(f2), "=&v"(f3), "=&v"(fb)
        : "v"(v0), "v"(v1), "n"(ST * kTileBytes + 0 * 2048), "n"(ST * kTileBytes + 1 * 2048),
          "n"(ST * kTileBytes + 2 * 2048), "n"(ST * kTileBytes + 3 * 2048), "v"(vs),
          "n"(ST * kBM * 4 + 0), "n"(ST * kBM * 4 + 64), "n"(ST * kBM * 4 + 128),
          "n"(ST * kBM * 4 + 192), "v"(vsb), "n"(ST * kBN * 4)
        : "memory");
    am[0] = __builtin_shufflevector(l0, h0, 0, 1, 2, 3, 4, 5, 6, 7);
    am[1] = __builtin_shufflevector(l1, h1, 0, 1, 2, 3, 4, 5, 6, 7);
    am[2] = __builtin_shufflevector(l2, h2, 0, 1, 2, 3, 4, 5, 6, 7);
    am[3] = __builtin_shufflevector(l3, h3, 0, 1, 2, 3, 4, 5, 6, 7);
    sa[0] = f0;
    sa[1] = f1;
    sa[2] = f2;
    sa[3] = f3;
    sb = fb;
}

// A B fragment in flight: issued by issue_b_frag, completed by wait_b_frag.
// The wait takes the destination registers as in/out operands, so nothing
// can read them (and the compiler cannot reuse them) before the data landed.
struct BFrag {
    v4i lo, hi;
    v4f sb;  // per-row B scales of the lane's four n (per-row scaling only)
};

template <bool ROWSCALE, int ST, int T>
__device__ __forceinline__ void issue_b_frag(uint32_t v0, uint32_t v1, uint32_t vs, BFrag& f) {
    if (ROWSCALE) {
        asm volatile(
            "ds_read_b128 %0, %3 offset:%5\n\t"
            "ds_read_b128 %1, %4 offset:%5\n\t"
            "ds_read_b128 %2, %6 offset:%7"
            : "=&v"(f.lo), "=&v"(f.hi), "=&v"(f.sb)
            : "v"(v0), "v"(v1), "n"(ST * kTileBytes + T * 2048), "v"(vs), "n"(ST * kBN * 4 + T * 64)
            : "memory");
    } else {
        asm volatile(
            "ds_read_b128 %0, %2 offset:%4\n\t"
            "ds_read_b128 %1, %3 offset:%4"
            : "=&v"(f.lo), "=&v"(f.hi)
            : "v"(v0), "v"(v1), "n"(ST * kTileBytes + T * 2048)
            : "memory");
    }
}

template <bool ROWSCALE>
__device__ __forceinline__ void wait_b_frag(BFrag& f) {
    if (ROWSCALE)
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(f.lo), "+v"(f.hi), "+v"(f.sb) : : "memory");
    else
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(f.lo), "+v"(f.hi) : : "memory");
}

__device__ __forceinline__ void wait_dma_and_barrier() {
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---------------------------------------------------------------- the kernel

template <bool ROWSCALE, bool OUT_F32, bool GROUPED>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(Params p) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kLdsBytes];

    TileRows tr;
    if (GROUPED ? !grouped_tile(p, tr) : !dense_tile(p, tr)) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int slabs = (int)(p.k / kSlab);
    const int64_t m_last = (GROUPED ? p.m : p.m) - 1;
    const int64_t n_last = p.n - 1;

    // ---- LDS-DMA sources: wave w copies rows [32w, 32w+32) of both tiles,
    // 8 rows (1 KB) per instruction; lane l -> row 8i + l/8, chunk l%8.
    // Addresses are a wave-uniform base (tile origin + slab) plus a 32-bit
    // per-lane offset, which maps onto the saddr + voffset load form.
    const uint8_t* const tileA = p.a + tr.m0 * p.lda;
    const uint8_t* const tileB = tr.b + tr.n0 * p.ldb;
    uint32_t offA[4], offB[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 32 * wave + 8 * i + (lane >> 3);
        const int chunk = swz_chunk(lane & 7, row);
        offA[i] = (uint32_t)((min(tr.m0 + row, m_last) - tr.m0) * p.lda) + chunk * 16;
        offB[i] = (uint32_t)((min(tr.n0 + row, n_last) - tr.n0) * p.ldb) + chunk * 16;
    }
    // Scales: waves 0-3 copy the slab's 256 A scales (64 each) into the sA
    // area. Waves 4-7 copy B scales into the sB area: with per-row scaling the
    // slab's 256 B scales (64 each); with 128x128 blocks, lane l copies the
    // scale of n-block (n0/128 + l%2) (only wave 4's first two are read).
    const float* scale_base;
    int64_t ld_s;
    uint32_t offS;
    if (wave < 4) {
        scale_base = p.a_scale + tr.m0;
        ld_s = p.ld_as;
        offS = (uint32_t)(min(tr.m0 + 64 * wave + lane, m_last) - tr.m0) * 4u;
    } else if (ROWSCALE) {
        scale_base = tr.b_scale + tr.n0;
        ld_s = p.ld_bs;
        offS = (uint32_t)(min(tr.n0 + 64 * (wave - 4) + lane, n_last) - tr.n0) * 4u;
    } else {
        scale_base = tr.b_scale;
        ld_s = 1;
        offS = (uint32_t)(min(tr.n0 / 128 + (lane & 1), n_last / 128) * p.ld_bs) * 4u;
    }
    const int lds_s = wave < 4 ? kOffSA + 64 * 4 * wave : kOffSB + 64 * 4 * (wave - 4);

    auto issue = [&](int j, int st) {
        uint8_t* base_a = smem + kOffA + st * kTileBytes + 32 * wave * kSlab;
        uint8_t* base_b = smem + kOffB + st * kTileBytes + 32 * wave * kSlab;
        const uint8_t* ga = tileA + (int64_t)j * kSlab;
        const uint8_t* gb = tileB + (int64_t)j * kSlab;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            __builtin_amdgcn_global_load_lds(ga + offA[i], (lds_void*)(base_a + i * 8 * kSlab), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(gb + offB[i], (lds_void*)(base_b + i * 8 * kSlab), 16, 0, 0);
        }
        const uint8_t* gs = reinterpret_cast<const uint8_t*>(scale_base + (int64_t)j * ld_s);
        __builtin_amdgcn_global_load_lds(gs + offS, (lds_void*)(smem + lds_s + st * kBM * 4), 4, 0, 0);
    };

    // ---- fragment addresses: lane (i = l%16, g = l/16) reads 32 bytes of
    // row i at logical chunks 2g and 2g+1 of every 16-row subtile.
    const int fi = lane & 15, fg = lane >> 4;
    const uint32_t lds0 = lds_addr(smem);
    const uint32_t off0 = fi * kSlab + swz_chunk(2 * fg, fi) * 16;
    const uint32_t off1 = fi * kSlab + swz_chunk(2 * fg + 1, fi) * 16;
    const uint32_t vA0 = lds0 + kOffA + wm * kWaveM * kSlab + off0;
    const uint32_t vA1 = lds0 + kOffA + wm * kWaveM * kSlab + off1;
    const uint32_t vB0 = lds0 + kOffB + wn * kWaveN * kSlab + off0;
    const uint32_t vB1 = lds0 + kOffB + wn * kWaveN * kSlab + off1;
    const uint32_t vSA = lds0 + kOffSA + (wm * kWaveM + fi) * 4;
    const uint32_t vSB = lds0 + kOffSB + (wn * kWaveN + 4 * fg) * 4;
    // The wave's 128 n rows are exactly one 128x128 weight block (n-block wn
    // of the tile), whose scale wave 4 copied to sB[wn].
    const uint32_t vSBblk = lds0 + kOffSB + wn * 4;

    v4f acc[kNSub][kMSub];
#pragma unroll
    for (int t = 0; t < kNSub; ++t)
#pragma unroll
        for (int s = 0; s < kMSub; ++s) acc[t][s] = v4f{0.f, 0.f, 0.f, 0.f};

    const v4f zero = {0.f, 0.f, 0.f, 0.f};

    auto step = [&](auto stage_tag, int j) {
        constexpr int ST = decltype(stage_tag)::value;
        wait_dma_and_barrier();
        // Prefetch the next slab into the other stage. The last step re-loads
        // its own slab there instead (never read), keeping the body branch-free.
        issue(min(j + 1, slabs - 1), ST ^ 1);
        v8i am[kMSub];
        float sa[kMSub], sb;
        read_a_frags<ST>(vA0, vA1, vSA, vSBblk, am, sa, sb);
        float sab[kMSub];
#pragma unroll
        for (int s = 0; s < kMSub; ++s) sab[s] = sa[s] * sb;

        // Software pipeline over the 8 n-subtiles: while the MFMAs of subtile
        // T run, the fragment of T+1 is in flight and the partials of T-1 are
        // promoted (acc += P * sA * sB), one FMA group after each MFMA.
        BFrag fr[2];
        v4f pc[kMSub], pp[kMSub];
        v4f sbp;
        issue_b_frag<ROWSCALE, ST, 0>(vB0, vB1, vSB, fr[0]);
        auto tile = [&](auto t_tag) {
            constexpr int T = decltype(t_tag)::value;
            BFrag& cur = fr[T & 1];
            wait_b_frag<ROWSCALE>(cur);
            if (T + 1 < kNSub) issue_b_frag<ROWSCALE, ST, (T + 1) % kNSub>(vB0, vB1, vSB, fr[(T + 1) & 1]);
            const v8i bf = __builtin_shufflevector(cur.lo, cur.hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
            for (int s = 0; s < kMSub; ++s) {
                pc[s] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, am[s], zero, 0, 0, 0, 0, 0, 0);
                if constexpr (T > 0) {
                    if (ROWSCALE) {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            acc[T - 1][s][r] = __builtin_fmaf(pp[s][r], sa[s] * sbp[r], acc[T - 1][s][r]);
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            acc[T - 1][s][r] = __builtin_fmaf(pp[s][r], sab[s], acc[T - 1][s][r]);
                    }
                }
            }
            if constexpr (T > 0) {
                // one MFMA, then the FMA group of one m-subtile, four times
#pragma unroll
                for (int s = 0; s < kMSub; ++s) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, ROWSCALE ? 8 : 4, 0);
                }
            }
#pragma unroll
            for (int s = 0; s < kMSub; ++s) pp[s] = pc[s];
            sbp = cur.sb;
            __builtin_amdgcn_sched_barrier(0);
        };
        tile(std::integral_constant<int, 0>{});
        tile(std::integral_constant<int, 1>{});
        tile(std::integral_constant<int, 2>{});
        tile(std::integral_constant<int, 3>{});
        tile(std::integral_constant<int, 4>{});
        tile(std::integral_constant<int, 5>{});
        tile(std::integral_constant<int, 6>{});
        tile(std::integral_constant<int, 7>{});
#pragma unroll
        for (int s = 0; s < kMSub; ++s) {
            if (ROWSCALE) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[kNSub - 1][s][r] = __builtin_fmaf(pp[s][r], sa[s] * sbp[r], acc[kNSub - 1][s][r]);
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[kNSub - 1][s][r] = __builtin_fmaf(pp[s][r], sab[s], acc[kNSub - 1][s][r]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    if (slabs > 0) issue(0, 0);
    int j = 0;
    for (; j + 2 <= slabs; j += 2) {
        step(std::integral_constant<int, 0>{}, j);
        step(std::integral_constant<int, 1>{}, j + 1);
    }
    if (j < slabs) step(std::integral_constant<int, 0>{}, j);
    // Drain the last (unused) prefetch before the block's LDS can be reused.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // ---- epilogue: lane holds C[m][n..n+3] for each (n-subtile, m-subtile).
#pragma unroll
    for (int s = 0; s < kMSub; ++s) {
        const int64_t m = tr.m0 + wm * kWaveM + s * 16 + fi;
        if (m >= tr.row_hi) continue;
        const bool pad = m >= tr.real_end;
#pragma unroll
        for (int t = 0; t < kNSub; ++t) {
            const int64_t n = tr.n0 + wn * kWaveN + t * 16 + 4 * fg;
            v4f v = pad ? zero : acc[t][s];
            if (OUT_F32) {
                float* dst = reinterpret_cast<float*>(p.c) + m * p.ldc + n;
                if (n + 3 < p.n) {
                    *reinterpret_cast<v4f*>(dst) = v;
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < p.n) dst[r] = v[r];
                }
            } else {
                uint16_t* dst = reinterpret_cast<uint16_t*>(p.c) + m * p.ldc + n;
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

Params to_params(const GemmProblem& g) {
    Params p;
    p.m = g.m;
    p.n = g.n;
    p.k = g.k;
    p.a = g.a;
    p.lda = g.lda;
    p.a_scale = g.a_scale;
    p.ld_as = g.ld_as;
    p.b = g.b;
    p.ldb = g.ldb;
    p.b_scale = g.b_scale;
    p.ld_bs = g.ld_bs;
    p.c = g.c;
    p.ldc = g.ldc;
    p.groups = g.groups;
    p.group_offsets = g.group_offsets;
    p.group_rows = g.group_rows;
    p.stride_b = g.stride_b;
    p.stride_bs = g.stride_bs;
    return p;
}

template <bool GROUPED>
hipError_t dispatch(const GemmProblem& g, int64_t slots, hipStream_t stream) {
    const Params p = to_params(g);
    const int64_t blocks = (slots + 7) / 8 * 8;
    const dim3 grid((unsigned)blocks), block(kThreads);
    if (g.b_rowscale) {
        if (g.out_f32)
            hipLaunchKernelGGL((gemm_kernel<true, true, GROUPED>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((gemm_kernel<true, false, GROUPED>), grid, block, 0, stream, p);
    } else {
        if (g.out_f32)
            hipLaunchKernelGGL((gemm_kernel<false, true, GROUPED>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((gemm_kernel<false, false, GROUPED>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmProblem& g, hipStream_t stream) {
    const int64_t tiles = ((g.m + kBM - 1) / kBM) * ((g.n + kBN - 1) / kBN);
    return dispatch<false>(g, tiles, stream);
}

hipError_t launch_grouped_gemm(const GemmProblem& g, hipStream_t stream) {
    // Upper bound on the tile count: every 256-row m-tile of an expert holds at
    // least 128 of its rows, so there are at most m_total / 128 of them.
    const int64_t tiles = (g.m / 128) * ((g.n + kBN - 1) / kBN);
    return dispatch<true>(g, tiles, stream);
}

}  // namespace fp8q
