// gemm_common.h -- pieces shared by the block-scaled FP8 GEMM kernels of
// libfp8q (internal): kernel parameters, the output-tile schedulers (dense,
// grouped over M for MoE Fprop/Dgrad, grouped over K for MoE Wgrad), the
// LDS swizzle and small device helpers.
#pragma once

#include "fp8q_device.h"
#include "launch.h"

#include <type_traits>
#include <utility>

namespace fp8q {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kSlab = 128;  // K elements per promotion interval
constexpr int kBM = 256;
constexpr int kBNMax = 256;  // LDS is laid out for the widest n tile
constexpr int kThreads = 512;
constexpr int kWaveM = 64;
constexpr int kMSub = kWaveM / 16;

// LDS per stage: one 256x128-byte tile of A, one of B, 256 A scales and up
// to 256 B scales (two stages: 135168 bytes).
constexpr int kTileBytes = kBM * kSlab;

// Physical 16-byte chunk of logical chunk c in LDS row `row` (rows are 128
// bytes). A fragment read has each 16-lane quarter of the wave fetch one
// chunk from 16 consecutive rows; XOR with (row >> 1) & 7 sends those 16
// reads to 16 different 16-byte bank groups (rows 2r and 2r+1 already sit
// in opposite halves of the 64 banks). With the fragment order below
// (chunks g and g + 4) the counters show no bank conflicts at all. Tiles
// and subtiles start at multiples of 16 rows, so tile-relative and
// subtile-relative rows give the same chunk.
__device__ __forceinline__ int swz_chunk(int c, int row) { return c ^ ((row >> 1) & 7); }

// Where the K pieces of a split tile (see tail_split) write: a record of the
// tile's rows, from its first piece, and one FP32 partial tile per piece.
struct TailRecord {
    int64_t m0, row_hi, real_end, n0;
};
constexpr int kMaxPieces = 256;    // the pieces fill at most one round of slots
constexpr int kTailRecords = 256;  // one per tile of that round
constexpr int kSplitFloats = kBM * kBNMax;  // one partial tile

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
    int64_t stride_c_bytes;  // grouped over K: distance between expert outputs
    // grouped over M, K-split last round: the tiles' records, the FP32 partial
    // tiles (NULL: no split) and how many of them fit
    TailRecord* split_records;
    float* split_ws;
    int32_t split_pieces;
};

// Which rows of the output a block tile owns.
struct TileRows {
    int64_t m0;        // first row of the tile
    int64_t row_hi;    // rows >= row_hi belong to someone else: not stored
    int64_t real_end;  // rows in [real_end, row_hi) are padding: stored as 0
    int64_t n0;
    const uint8_t* b;
    const float* b_scale;
    int slab0;         // first K slab of the tile's contraction
    int slabs;         // number of K slabs
    void* c;           // output matrix the tile belongs to
    int piece;         // >= 0: a K piece of a split tile, stored as FP32 partial `piece`
};

// Kernel modes: one GEMM; grouped over M (MoE Fprop/Dgrad: experts own row
// segments, one weight each); grouped over K (MoE Wgrad: experts own token
// segments of the contraction, one output each); one GEMM whose tiles take
// several rounds of the CUs, run by one block per CU that loops over its
// tiles (every tile whole: M and N multiples of the tile, an even number of
// slabs) and fetches each next tile's first slab under the stores of the
// tile before.
constexpr int kDense = 0;
constexpr int kGroupedM = 1;
constexpr int kGroupedK = 2;
constexpr int kDenseRounds = 3;

// Dense tile order: slot s belongs to XCD s / per, where per = ceil(tiles/8);
// block b runs on XCD b % 8, and its i-th tile (one-tile-per-block launches:
// its only tile, i = 0) is slot (b % 8) * per + b / 8 + 32 i. Within an XCD,
// slots walk 4-row bands of tiles, so the blocks resident on one XCD share A
// and B panels in its L2. Rounds of a looping grid of 256 blocks take the
// same slots at the same time as a grid of one block per tile would.
template <int BN>
__device__ __forceinline__ bool dense_tile(const Params& p, int i, TileRows& t) {
    const int tiles_m = (int)((p.m + kBM - 1) / kBM);
    const int tiles_n = (int)((p.n + BN - 1) / BN);
    const int total = tiles_m * tiles_n;
    const int per = (total + 7) / 8;
    const int q = (int)(blockIdx.x / 8) + 32 * i;
    const int slot = (int)(blockIdx.x % 8) * per + q;
    if (q >= per || slot >= total) return false;
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
    t.n0 = (int64_t)tn * BN;
    t.b = p.b;
    t.b_scale = p.b_scale;
    t.slab0 = 0;
    t.slabs = (int)(p.k / kSlab);
    t.c = p.c;
    t.piece = -1;
    return true;
}

// Grouped tiles. Expert e's segment [off[e], off[e+1]) is cut into 256-row
// m-tiles: whole tiles of real rows, then a tail tile whose first 1-4 64-row
// quarters hold real rows, then tiles of padding only (written as zeros).
// Slots run expert by expert, inside an expert by n-tile and then m-tile, so
// the m-tiles that share a 256 x K panel of W_e -- the tail included -- are
// consecutive and run together on one XCD, where the panel is fetched into
// L2 once. (Every tile streams the same K x 256 weight panel, and its padding
// rows cost one repeated line, so a tile with 128 real rows still takes about
// 3/4 of a full tile's time: ordering by tile size buys no balance, and
// measured ~5% slower than this order.)
// Experts run last to first: the grouped weight quantizer writes them first
// to last, so right after it the last experts' codes are the ones still held
// by the memory-side cache. Measured on one MI355X in the quantize-then-GEMM
// step: 388.6 against 400.0 us for the MoE Fprop GEMM (bit-identical output),
// and no difference when GEMMs run back to back.
struct ExpertSplit {
    int beg;    // first row of the segment
    int tiles;  // m-tiles of the segment
};

__device__ __forceinline__ ExpertSplit expert_split(const Params& p, int e) {
    ExpertSplit x;
    x.beg = p.group_offsets[e];
    const int seg = max(p.group_offsets[e + 1] - x.beg, 0);
    x.tiles = (seg + kBM - 1) / kBM;
    return x;
}

// The experts are found by a scan over the wave rather than a walk over the
// offsets (a chain of dependent scalar loads, one round trip per expert, at
// the start of every block): lane l takes the expert at position base + l of
// the order, one load each.
// Tiles of that expert (zero past the last one):
__device__ __forceinline__ int lane_expert_tiles(const Params& p, int base, int tiles_n) {
    const int pos = base + (int)(threadIdx.x & 63);
    if (pos >= p.groups) return 0;
    return expert_split(p, p.groups - 1 - pos).tiles * tiles_n;
}

__device__ __forceinline__ int wave_inclusive_sum(int v) {
    const int lane = (int)(threadIdx.x & 63);
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int u = __shfl_up(v, d);
        if (lane >= d) v += u;
    }
    return v;
}

// Tile `slot` of the grouped order (see above), or false past the last tile.
// Every lane of the wave must take part.
template <int BN>
__device__ __forceinline__ bool grouped_slot(const Params& p, int slot, TileRows& t) {
    const int tiles_n = (int)((p.n + BN - 1) / BN);
    for (int base = 0; base < p.groups; base += 64) {
        const int cnt = lane_expert_tiles(p, base, tiles_n);
        const int incl = wave_inclusive_sum(cnt);
        const int chunk = __builtin_amdgcn_readfirstlane(__shfl(incl, 63));
        if (slot < chunk) {
            // the first lane whose running total passes the slot holds its expert
            const unsigned long long hit = __ballot(incl > slot);
            const int l = __builtin_amdgcn_readfirstlane(__ffsll(hit) - 1);
            slot -= __builtin_amdgcn_readfirstlane(__shfl(incl - cnt, l));
            const int e = p.groups - 1 - (base + l);
            const ExpertSplit x = expert_split(p, e);
            const int k = x.tiles;
            const int tn = slot / k, mt = slot % k;
            const int end = x.beg + max(p.group_offsets[e + 1] - x.beg, 0);
            t.m0 = x.beg + (int64_t)mt * kBM;
            // offsets that break the contract must not move stores outside C
            if (t.m0 < 0 || t.m0 >= p.m) return false;
            t.row_hi = min(min((int64_t)end, t.m0 + kBM), p.m);
            const int seg = end - x.beg;
            const int real = p.group_rows ? min(max(p.group_rows[e], 0), seg) : seg;
            t.real_end = x.beg + (int64_t)real;
            t.n0 = (int64_t)tn * BN;
            t.b = p.b + e * p.stride_b;
            t.b_scale = p.b_scale + e * p.stride_bs;
            t.slab0 = 0;
            t.slabs = (int)(p.k / kSlab);
            t.c = p.c;
            t.piece = -1;
            return true;
        }
        slot -= chunk;
    }
    return false;
}

// The last, partial round of a grouped GEMM: its `tiles` tiles (slots from
// `first` on) leave most CUs idle for a whole tile time, so each is cut into
// `split` pieces of about K / split. Piece i of tail tile r takes slot
// first + i * tiles + r (the same piece of neighbouring tiles -- which share
// weight or activation panels -- run side by side on one XCD) and stores its
// FP32 partial as partial i * tiles + r; a second kernel adds a tile's
// partials in piece order. split = 1: no split (no workspace, a last round
// more than half full, or too few slabs).
constexpr int kMaxSplit = 8;
constexpr int kMinSplitSlabs = 4;

struct TailSplit {
    int first;
    int tiles;
    int split;
};

template <int BN>
__device__ __forceinline__ TailSplit tail_split(const Params& p) {
    const int tiles_n = (int)((p.n + BN - 1) / BN);
    int total = 0;
    for (int base = 0; base < p.groups; base += 64)
        total += __builtin_amdgcn_readfirstlane(__shfl(wave_inclusive_sum(lane_expert_tiles(p, base, tiles_n)), 63));
    TailSplit ts;
    ts.first = total / 256 * 256;
    ts.tiles = total - ts.first;
    ts.split = 1;
    if (p.split_ws != nullptr && ts.tiles > 0) {
        const int s = min(min(256 / ts.tiles, kMaxSplit),
                          min(p.split_pieces / ts.tiles, (int)(p.k / kSlab) / kMinSplitSlabs));
        ts.split = max(s, 1);
    }
    return ts;
}

// Block b runs on XCD b % 8; round r of that XCD's 32 CUs takes the 32
// consecutive slots 256 r + 32 (b % 8) + [0, 32). Every round is then spread
// evenly over the XCDs and panel reuse stays inside one L2. The grid is a
// multiple of 256 blocks, so this is a bijection onto its slots (the pieces
// of a split last round fill at most the 256 slots of that round).
template <int BN>
__device__ __forceinline__ bool grouped_tile(const Params& p, TileRows& t) {
    const int q = (int)(blockIdx.x >> 3);
    const int slot = ((q >> 5) << 8) + ((int)(blockIdx.x & 7) << 5) + (q & 31);
    if (p.split_ws != nullptr) {
        const TailSplit ts = tail_split<BN>(p);
        if (ts.split > 1 && slot >= ts.first) {
            const int u = slot - ts.first;
            if (u >= ts.tiles * ts.split) return false;
            const int r = u % ts.tiles, i = u / ts.tiles;
            if (!grouped_slot<BN>(p, ts.first + r, t)) return false;
            const int slabs = t.slabs;
            t.slab0 = i * slabs / ts.split;
            t.slabs = (i + 1) * slabs / ts.split - t.slab0;
            t.piece = u;
            if (i == 0 && threadIdx.x == 0) p.split_records[r] = TailRecord{t.m0, t.row_hi, t.real_end, t.n0};
            return true;
        }
    }
    return grouped_slot<BN>(p, slot, t);
}

// Grouped-over-K tiles (MoE Wgrad): expert e contracts over its token segment
// [off[e], off[e+1]) (a multiple of 128: whole slabs) and owns the output
// matrix c + e * stride_c. Every expert has the same tiles_m x tiles_n tiles;
// slots run expert by expert, inside an expert in the dense order (bands of
// 4 m-tiles). Blocks take slots in XCD rounds as grouped_tile does, so the
// 32 tiles an XCD runs together share the expert's A and B panels in L2.
// An expert without rows still writes its (zero) output.
template <int BN>
__device__ __forceinline__ bool grouped_k_tile(const Params& p, TileRows& t) {
    const int tiles_m = (int)((p.m + kBM - 1) / kBM);
    const int tiles_n = (int)((p.n + BN - 1) / BN);
    const int per = tiles_m * tiles_n;
    const int q = (int)(blockIdx.x >> 3);
    const int slot = ((q >> 5) << 8) + ((int)(blockIdx.x & 7) << 5) + (q & 31);
    if (slot >= per * p.groups) return false;
    const int e = slot / per;
    const int within_e = slot - e * per;
    constexpr int G = 4;
    const int group = within_e / (G * tiles_n);
    const int first_m = group * G;
    const int gm = min(tiles_m - first_m, G);
    const int within = within_e - group * G * tiles_n;
    const int beg = p.group_offsets[e];
    const int seg = max(p.group_offsets[e + 1] - beg, 0);
    // offsets that break the contract must not move reads outside A and B
    if (beg < 0 || (int64_t)beg + seg > p.k) return false;
    t.m0 = (int64_t)(first_m + within % gm) * kBM;
    t.row_hi = p.m;
    t.real_end = p.m;
    t.n0 = (int64_t)(within / gm) * BN;
    t.b = p.b;
    t.b_scale = p.b_scale;
    t.slab0 = beg / kSlab;
    t.slabs = seg / kSlab;
    t.c = static_cast<char*>(p.c) + (int64_t)e * p.stride_c_bytes;
    t.piece = -1;
    return true;
}

// s_waitcnt with vmcnt = N (0..63: low four bits in [3:0], high two in
// [15:14]) and the other counters left at their maxima.
constexpr int waitcnt_vm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

template <int N>
__device__ __forceinline__ void wait_dma_and_barrier() {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(N));
    __builtin_amdgcn_s_barrier();
}

__device__ __forceinline__ v8i ld_frag(const uint8_t* p0, const uint8_t* p1) {
    const v4i lo = *reinterpret_cast<const v4i*>(p0);
    const v4i hi = *reinterpret_cast<const v4i*>(p1);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// c ? a : b on values
template <class T>
__device__ __forceinline__ T pick(bool c, T a, T b) {
    return c ? a : b;
}

template <int... Is, class F>
__device__ __forceinline__ void unroll(std::integer_sequence<int, Is...>, F&& f) {
    (f(std::integral_constant<int, Is>{}), ...);
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
    p.stride_c_bytes = g.stride_c * (g.out_f32 ? 4 : 2);
    p.split_records = nullptr;
    p.split_ws = nullptr;
    p.split_pieces = 0;
    return p;
}

}  // namespace
}  // namespace fp8q
