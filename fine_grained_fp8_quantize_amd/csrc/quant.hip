// quant.hip -- fine-grained FP8 (E4M3) quantization kernels for gfx950.
//
// Groups (page dssusan.co.kr Q&A board, passage on Figure 7(a)): 1x128 tiles
// for activations (per token per 128 channels), 128x128 blocks for weights;
// 128x1 token tiles for the Wgrad operands. Every group gets one FP32 scale
// s = amax / 448 and its elements become E4M3 codes of x / s (page "Deepseek
// Ai News Expert Interview", passages on E4M3 for all tensors and on sharing
// exponent bits within small groups). The kernels are HBM-bound: 2 bytes
// read, 1 byte written and 4/128 (or 4/16384) bytes of scale per element
// (the re-tile of a cached FP8 activation reads 1 byte instead of 2). Also
// here: the scatter form of the 1x128 kernel (quantize before dispatch), the
// microscaling quantizer, the weight quantizer over several experts in one
// launch, one launch that quantizes a layer's activation and weight, and
// launches that make both Wgrad operands in 128x1 tiles (from bf16, or dY
// from bf16 and X from the FP8 cache).
#include "fp8q_device.h"
#include "launch.h"

namespace fp8q {
namespace {

// ------------------------------------------------------------------ 1x128

// One wave quantizes 8 rows of two adjacent 128-column slabs (16 tiles).
// Lane 32*rr + 16*sj + c holds the 16-byte chunk c (8 bf16) of slab sj of
// rows 2u + rr, u = 0..3, so each 1x128 tile is one DPP row of 16 lanes and
// its amax reduces in-row. Codes are stored non-temporal (16 lanes write one
// whole 128-byte line). Paired on one MI355X against 16 rows of one slab
// per wave and plain stores, bit-identical output: dY [10112][4096] 25.3 ->
// 23.0 us, the MoE dispatch scatter (8192 x 7168, top-8) 41.4 -> 39.3 us,
// Dense Fprop X + W in one launch 31.4 -> 29.4 us.
//
// SCATTER (quantize before dispatch): source row t is quantized once and
// its codes and scale are stored to every destination row dst[t][k] >= 0,
// k < topk, of the expert-sorted layout (page "Eliminate Deepseek Ai News For
// Good", passage on quantizing activations before the MoE dispatch).
constexpr int kActWavesPerBlock = 4;
constexpr int kMaxTopk = 8;  // destinations per source row (scatter)

// Work units of the 1x128 and microscaling quantizers: one wave takes 8
// rows x 2 slabs (16 tiles), so that every load instruction reads 512
// contiguous bytes of each of two rows.
__host__ __device__ constexpr int64_t act_units(int64_t rows, int64_t slabs) {
    return (rows + 7) / 8 * ((slabs + 1) / 2);
}

// 8-byte non-temporal store (whole 128-byte lines per 16 lanes at the call
// sites)
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store_nt8(uint8_t* p, uint32_t lo, uint32_t hi) {
    __builtin_nontemporal_store(u32x2_t{lo, hi}, reinterpret_cast<u32x2_t*>(p));
}

// The body of one 256-thread block (block index `block`); kernels below
// call it, alone or next to the weight body.
template <bool SCATTER>
__device__ __forceinline__ void act_1x128_body(
    const uint16_t* __restrict__ x, int64_t rows, int64_t slabs, int64_t ld_x,
    uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ scale, int64_t ld_s,
    int64_t units, const int32_t* __restrict__ dst, int topk, int64_t m_total, int64_t block) {
    const int lane = threadIdx.x & 63;
    const int64_t unit = block * kActWavesPerBlock + (threadIdx.x >> 6);
    if (unit >= units) return;  // whole wave
    // lane l: slab 2 p + (l / 16) % 2, rows 8 rg + 2 u + l / 32 (u = 0..3),
    // columns 8 (l % 16) .. +7 of the slab; a DPP row of 16 lanes is one tile
    const int64_t pairs = (slabs + 1) / 2;
    const int64_t rg = unit / pairs;
    const int64_t j = 2 * (unit - rg * pairs) + ((lane >> 4) & 1);
    const bool jvalid = j < slabs;  // the last pair of an odd slab count has one slab
    const int rr = lane >> 5, c = lane & 15;

    uint4 v[4];
    int64_t row[4];
    bool live[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        row[u] = rg * 8 + u * 2 + rr;
        live[u] = row[u] < rows && jvalid;
        v[u] = make_uint4(0, 0, 0, 0);
        if (live[u])
            v[u] = load_nt16(x + row[u] * ld_x + j * 128 + c * 8);
    }
    // destinations of the lane's four rows, loaded alongside the data
    int32_t d[SCATTER ? 4 : 1][SCATTER ? kMaxTopk : 1];
    if constexpr (SCATTER) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int k = 0; k < kMaxTopk; ++k)
                d[u][k] = (row[u] < rows && k < topk) ? dst[row[u] * topk + k] : -1;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const uint32_t mask = 0x7FFF7FFFu;
        uint32_t m = pk_max_u16(pk_max_u16(v[u].x & mask, v[u].y & mask),
                                pk_max_u16(v[u].z & mask, v[u].w & mask));
        m = row16_max(umax32(m & 0xFFFFu, m >> 16));
        const GroupScale g = group_scale(m);

        float a[8] = {bf16_lo(v[u].x), bf16_hi(v[u].x), bf16_lo(v[u].y), bf16_hi(v[u].y),
                      bf16_lo(v[u].z), bf16_hi(v[u].z), bf16_lo(v[u].w), bf16_hi(v[u].w)};
        float qv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) qv[i] = quot_fast(__builtin_fabsf(a[i]), g);
        if (g.slow) {
#pragma unroll
            for (int i = 0; i < 8; ++i) qv[i] = quot_slow(__builtin_fabsf(a[i]), g);
        }
        const uint32_t w0 = pack_e4m3x4(qv[0], qv[1], qv[2], qv[3], bf16x4_sign_bytes(v[u].x, v[u].y));
        const uint32_t w1 = pack_e4m3x4(qv[4], qv[5], qv[6], qv[7], bf16x4_sign_bytes(v[u].z, v[u].w));
        if (live[u]) {
            if constexpr (SCATTER) {
#pragma unroll
                for (int k = 0; k < kMaxTopk; ++k) {
                    const int64_t dk = d[u][k];
                    if (dk < 0 || dk >= m_total) continue;  // not routed here (or out of contract)
                    store_nt8(q + dk * ld_q + j * 128 + c * 8, w0, w1);
                    if (c == 0) scale[j * ld_s + dk] = g.s;
                }
            } else {
                store_nt8(q + row[u] * ld_q + j * 128 + c * 8, w0, w1);
                if (c == 0) scale[j * ld_s + row[u]] = g.s;
            }
        }
    }
}

template <bool SCATTER>
__global__ __launch_bounds__(256) void quant_act_1x128_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t slabs, int64_t ld_x,
    uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ scale, int64_t ld_s,
    int64_t units, const int32_t* __restrict__ dst, int topk, int64_t m_total) {
    act_1x128_body<SCATTER>(x, rows, slabs, ld_x, q, ld_q, scale, ld_s, units, dst, topk, m_total,
                            (int64_t)blockIdx.x);
}

// ------------------------------------------------------------ MX (1x32)

// Microscaling variant (page "Deepseek Ai News Expert Interview", passage
// likening the fine-grained groups to microscaling formats): 32 consecutive
// elements of a row share an E8M0 power-of-two scale 2^e with
// e = floor(log2(amax)) - 8 (8: exponent of E4M3's largest normal), clamped
// to [-127, 127], -127 for an all-zero block; codes are E4M3_RNE_sat(x / 2^e).
// Same wave layout as the 1x128 kernel (8 rows x 2 slabs per wave, one slab
// of one row per 16 lanes); a 32-element block is one quad of lanes. The
// scale of row r, slab j is one uint32: byte b = block 4j + b.
// The body of one 256-thread block (block index `block`); the kernels below
// call it for one matrix, or for both GEMM operands in one grid.
__device__ __forceinline__ void mx_1x32_body(
    const uint16_t* __restrict__ x, int64_t rows, int64_t slabs, int64_t ld_x,
    uint8_t* __restrict__ q, int64_t ld_q, uint32_t* __restrict__ scale, int64_t ld_s,
    int64_t units, int64_t block) {
    const int lane = threadIdx.x & 63;
    const int64_t unit = block * kActWavesPerBlock + (threadIdx.x >> 6);
    if (unit >= units) return;  // whole wave
    const int64_t pairs = (slabs + 1) / 2;
    const int64_t rg = unit / pairs;
    const int64_t j = 2 * (unit - rg * pairs) + ((lane >> 4) & 1);
    const bool jvalid = j < slabs;
    const int rr = lane >> 5, c = lane & 15;

    uint4 v[4];
    int64_t row[4];
    bool live[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        row[u] = rg * 8 + u * 2 + rr;
        live[u] = row[u] < rows && jvalid;
        v[u] = make_uint4(0, 0, 0, 0);
        if (live[u])
            v[u] = load_nt16(x + row[u] * ld_x + j * 128 + c * 8);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const uint32_t mask = 0x7FFF7FFFu;
        uint32_t m = pk_max_u16(pk_max_u16(v[u].x & mask, v[u].y & mask),
                                pk_max_u16(v[u].z & mask, v[u].w & mask));
        m = quad_max(umax32(m & 0xFFFFu, m >> 16));  // amax bits of the lane's block
        // floor(log2(amax)) from the bf16 bits: the unbiased exponent of a
        // normal, or the top mantissa bit of a subnormal (value mant * 2^-133)
        const int ebits = (int)(m >> 7);
        const int fl2 = ebits != 0 ? ebits - 127 : (31 - __builtin_clz(m | 1u)) - 133;
        int e = m == 0 ? -127 : fl2 - 8;
        e = e < -127 ? -127 : (e > 127 ? 127 : e);
        // 2^-e as a float: normal for -e >= -126, else the subnormal 2^-127
        const float factor = __builtin_bit_cast(float, -e >= -126 ? (uint32_t)(127 - e) << 23 : 0x00400000u);
        float a[8] = {bf16_lo(v[u].x), bf16_hi(v[u].x), bf16_lo(v[u].y), bf16_hi(v[u].y),
                      bf16_lo(v[u].z), bf16_hi(v[u].z), bf16_lo(v[u].w), bf16_hi(v[u].w)};
        float qv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) qv[i] = __builtin_fabsf(a[i]) * factor;  // exact
        const uint32_t w0 = pack_e4m3x4(qv[0], qv[1], qv[2], qv[3], bf16x4_sign_bytes(v[u].x, v[u].y));
        const uint32_t w1 = pack_e4m3x4(qv[4], qv[5], qv[6], qv[7], bf16x4_sign_bytes(v[u].z, v[u].w));
        if (live[u]) {
            store_nt8(q + row[u] * ld_q + j * 128 + c * 8, w0, w1);
            if ((c & 3) == 0)
                reinterpret_cast<uint8_t*>(scale + j * ld_s + row[u])[c >> 2] = (uint8_t)(e + 127);
        }
    }
}

__global__ __launch_bounds__(256) void quant_mx_1x32_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t slabs, int64_t ld_x,
    uint8_t* __restrict__ q, int64_t ld_q, uint32_t* __restrict__ scale, int64_t ld_s,
    int64_t units) {
    mx_1x32_body(x, rows, slabs, ld_x, q, ld_q, scale, ld_s, units, (int64_t)blockIdx.x);
}

// Both operands of the microscaling GEMM in one grid: blocks below a_blocks
// take units of the first matrix, the rest units of the second.
struct MxArgs {
    const uint16_t* x;
    int64_t rows, slabs, ld_x;
    uint8_t* q;
    int64_t ld_q;
    uint32_t* scale;
    int64_t ld_s, units;
};

__global__ __launch_bounds__(256) void quant_mx_1x32_pair_kernel(MxArgs a, int64_t a_blocks, MxArgs b) {
    const int64_t blk = (int64_t)blockIdx.x;
    const bool first = blk < a_blocks;
    const MxArgs& o = first ? a : b;
    mx_1x32_body(o.x, o.rows, o.slabs, o.ld_x, o.q, o.ld_q, o.scale, o.ld_s, o.units, first ? blk : blk - a_blocks);
}

// ------------------------------------------------------------------ 128x1

// One 256-thread block quantizes a 128-token x 128-channel panel: thread
// (token group r = t/16, channel chunk g = t%16) loads 8 tokens x 8 channels.
// Column amax: per-thread max over its 8 tokens, cross-lane max inside the
// wave, then across the 4 waves through LDS. Codes are transposed through LDS
// so that each output row (one channel, 128 consecutive tokens) is written
// with full 16-byte stores.
constexpr int kTrStride = 144;  // bytes per transposed row (128 + 16 pad)

// LDS of one 128x128 panel block: the amax partials of the 4 waves, the
// 128 scales and their reciprocals, and the transposed codes.
template <int R>
struct PanelLds {
    uint32_t (*red)[16][R];
    float* s_sh;
    float* y_sh;
    uint8_t* tr;
};

// The body of one 256-thread block (panel index `block`); the kernels below
// call it, alone or beside another operand in one grid.
__device__ __forceinline__ void act_128x1_body(
    const uint16_t* __restrict__ x, int64_t tokens, int64_t cols, int64_t ld_x,
    uint8_t* __restrict__ qt, int64_t ld_q, float* __restrict__ scale, int64_t ld_s,
    int64_t cblocks, int64_t block, PanelLds<4> lds) {
    uint32_t (*const red)[16][4] = lds.red;
    float* const s_sh = lds.s_sh;
    float* const y_sh = lds.y_sh;
    uint8_t* const tr = lds.tr;

    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int g = t & 15, r = t >> 4;
    const int64_t tb = block / cblocks, cb = block - tb * cblocks;
    const int64_t t0 = tb * 128, c0 = cb * 128;
    const int64_t ch = c0 + 8 * g;
    const bool valid = ch < cols;  // cols % 8 == 0: a chunk is all in or all out

    uint4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        v[i] = make_uint4(0, 0, 0, 0);
        if (valid)
            v[i] = load_nt16(x + (t0 + 8 * r + i) * ld_x + ch);
    }
    const uint32_t mask = 0x7FFF7FFFu;
    uint32_t m[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        m[0] = pk_max_u16(m[0], v[i].x & mask);
        m[1] = pk_max_u16(m[1], v[i].y & mask);
        m[2] = pk_max_u16(m[2], v[i].z & mask);
        m[3] = pk_max_u16(m[3], v[i].w & mask);
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        m[d] = pk_max_u16(m[d], (uint32_t)__shfl_xor((int)m[d], 16));
        m[d] = pk_max_u16(m[d], (uint32_t)__shfl_xor((int)m[d], 32));
    }
    if ((lane >> 4) == 0) {
#pragma unroll
        for (int d = 0; d < 4; ++d) red[w][g][d] = m[d];
    }
    __syncthreads();
    if (t < 128) {
        const int chunk = t >> 3, pair = (t & 7) >> 1;
        uint32_t mm = 0;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) mm = pk_max_u16(mm, red[ww][chunk][pair]);
        const uint32_t bits = (t & 1) ? (mm >> 16) : (mm & 0xFFFFu);
        const GroupScale gs = group_scale(bits);
        s_sh[t] = gs.s;
        y_sh[t] = gs.y;
        if (c0 + t < cols) scale[tb * ld_s + c0 + t] = gs.s;
    }
    __syncthreads();

    if (valid) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            GroupScale gs;
            gs.s = s_sh[8 * g + k];
            gs.y = y_sh[8 * g + k];
            gs.slow = !(gs.s >= kSmallScale);
            const int d = k >> 1;
            float a[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t word = d == 0 ? v[i].x : d == 1 ? v[i].y : d == 2 ? v[i].z : v[i].w;
                a[i] = (k & 1) ? bf16_hi(word) : bf16_lo(word);
            }
            float qv[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) qv[i] = quot_fast(__builtin_fabsf(a[i]), gs);
            if (gs.slow) {
#pragma unroll
                for (int i = 0; i < 8; ++i) qv[i] = quot_slow(__builtin_fabsf(a[i]), gs);
            }
            uint32_t wd[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                wd[i] = d == 0 ? v[i].x : d == 1 ? v[i].y : d == 2 ? v[i].z : v[i].w;
            const uint32_t byte = (k & 1) ? 3u : 1u;
            const uint32_t s0 = gather_byte4(wd[0], wd[1], wd[2], wd[3], byte);
            const uint32_t s1 = gather_byte4(wd[4], wd[5], wd[6], wd[7], byte);
            const uint32_t w0 = pack_e4m3x4(qv[0], qv[1], qv[2], qv[3], s0);
            const uint32_t w1 = pack_e4m3x4(qv[4], qv[5], qv[6], qv[7], s1);
            *reinterpret_cast<uint2*>(&tr[(8 * g + k) * kTrStride + 8 * r]) = make_uint2(w0, w1);
        }
    }
    __syncthreads();
    const int cc = t >> 1, h = t & 1;
    if (c0 + cc < cols) {
        uint8_t* dst = qt + (c0 + cc) * ld_q + t0 + 64 * h;
        const uint8_t* src = &tr[cc * kTrStride + 64 * h];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<uint4*>(dst + 16 * i) = *reinterpret_cast<const uint4*>(src + 16 * i);
    }
}

__global__ __launch_bounds__(256) void quant_act_128x1_kernel(
    const uint16_t* __restrict__ x, int64_t tokens, int64_t cols, int64_t ld_x,
    uint8_t* __restrict__ qt, int64_t ld_q, float* __restrict__ scale, int64_t ld_s,
    int64_t cblocks) {
    __shared__ uint32_t red[4][16][4];
    __shared__ float s_sh[128];
    __shared__ float y_sh[128];
    __shared__ __attribute__((aligned(16))) uint8_t tr[128 * kTrStride];
    act_128x1_body(x, tokens, cols, ld_x, qt, ld_q, scale, ld_s, cblocks, (int64_t)blockIdx.x,
                   PanelLds<4>{red, s_sh, y_sh, tr});
}

// Both Wgrad operands (dY and X, one token count) in one grid: blocks below
// a_blocks take panels of the first, the rest panels of the second.
struct Act128Args {
    const uint16_t* x;
    int64_t cols, ld_x;
    uint8_t* qt;
    int64_t ld_q;
    float* scale;
    int64_t ld_s, cblocks;
};

__global__ __launch_bounds__(256) void quant_act_128x1_pair_kernel(int64_t tokens, Act128Args a,
                                                                   int64_t a_blocks, Act128Args b) {
    __shared__ uint32_t red[4][16][4];
    __shared__ float s_sh[128];
    __shared__ float y_sh[128];
    __shared__ __attribute__((aligned(16))) uint8_t tr[128 * kTrStride];
    const int64_t blk = (int64_t)blockIdx.x;
    const bool first = blk < a_blocks;  // block-uniform: the barriers inside stay whole
    const Act128Args& o = first ? a : b;
    act_128x1_body(o.x, tokens, o.cols, o.ld_x, o.qt, o.ld_q, o.scale, o.ld_s, o.cblocks,
                   first ? blk : blk - a_blocks, PanelLds<4>{red, s_sh, y_sh, tr});
}

// ------------------------------------------------- cached activation re-tile

// A cached FP8 activation (1x128 codes and scales from the forward pass)
// re-tiled into the 128x1 token tiles Wgrad takes (page "Is aI Hitting a
// Wall?", passage on keeping activations in FP8 for the backward pass): each
// value is dequantized to binary32, v = fl32(dec(q) * s_token), and the v are
// quantized in 128x1 tiles exactly as quant_act_128x1_kernel quantizes bf16.
// One 256-thread block takes a 128-token x 128-channel panel; thread (token
// group r = t/16, channel chunk g = t%16) loads 8 tokens x 8 channels of
// codes (one 8-byte load per token) and the 8 tokens' scales. The code of an
// output element keeps the sign bit of the input code (s_token >= 0).
__device__ __forceinline__ void retile_128x1_body(
    const uint8_t* __restrict__ q, int64_t ld_q, const float* __restrict__ scale, int64_t ld_s,
    uint8_t* __restrict__ qt, int64_t ld_qt, float* __restrict__ scale_t, int64_t ld_st,
    int64_t cblocks, int64_t block, PanelLds<8> lds) {
    uint32_t (*const red)[16][8] = lds.red;
    float* const s_sh = lds.s_sh;
    float* const y_sh = lds.y_sh;
    uint8_t* const tr = lds.tr;

    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int g = t & 15, r = t >> 4;
    const int64_t tb = block / cblocks, cb = block - tb * cblocks;
    const int64_t t0 = tb * 128, c0 = cb * 128;

    uint2 code[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 c = __builtin_nontemporal_load(
            reinterpret_cast<const u32x2*>(q + (t0 + 8 * r + i) * ld_q + c0 + 8 * g));
        code[i] = make_uint2(c.x, c.y);
    }
    // scale[slab cb][token]: the thread's 8 tokens are 32 contiguous bytes
    const float4* sp = reinterpret_cast<const float4*>(scale + cb * ld_s + t0 + 8 * r);
    const float4 s_lo = sp[0], s_hi = sp[1];
    const float st[8] = {s_lo.x, s_lo.y, s_lo.z, s_lo.w, s_hi.x, s_hi.y, s_hi.z, s_hi.w};

    // v = fl32(dec(q) * s_token) for token i, channels 4h..4h+3 (h = 0, 1).
    // The values are made twice (amax pass, quotient pass) rather than held
    // across the barrier: fewer registers, more blocks and loads in flight.
    typedef float f4 __attribute__((ext_vector_type(4)));
    auto dequant4 = [&](int i, int h) -> f4 {
        typedef float f2 __attribute__((ext_vector_type(2)));
        const uint32_t word = h ? code[i].y : code[i].x;
        const f2 d0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, false);
        const f2 d1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, true);
        return f4{d0.x * st[i], d0.y * st[i], d1.x * st[i], d1.y * st[i]};
    };
    // Column amax: over the thread's 8 tokens, the wave's 4 token groups
    // (lanes 16 and 32 apart), then the 4 waves through LDS. Magnitudes of
    // finite non-negative floats order as their bit patterns.
    float mf[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const f4 v = dequant4(i, h);
#pragma unroll
            for (int c = 0; c < 4; ++c) mf[4 * h + c] = __builtin_fmaxf(mf[4 * h + c], __builtin_fabsf(v[c]));
        }
    }
    uint32_t m[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        uint32_t mm = __float_as_uint(mf[k]);
        mm = umax32(mm, (uint32_t)__shfl_xor((int)mm, 16));
        mm = umax32(mm, (uint32_t)__shfl_xor((int)mm, 32));
        m[k] = mm;
    }
    if ((lane >> 4) == 0) {
#pragma unroll
        for (int k = 0; k < 8; ++k) red[w][g][k] = m[k];
    }
    __syncthreads();
    if (t < 128) {
        const int chunk = t >> 3, kk = t & 7;
        uint32_t mm = 0;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) mm = umax32(mm, red[ww][chunk][kk]);
        const GroupScale gs = group_scale_f32(__uint_as_float(mm));
        s_sh[t] = gs.s;
        y_sh[t] = gs.y;
        scale_t[tb * ld_st + c0 + t] = gs.s;
    }
    __syncthreads();
    // (an empty asm marks the code words as changed, so the compiler makes
    // the values again here instead of keeping 64 of them live)
#pragma unroll
    for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(code[i].x), "+v"(code[i].y));

#pragma unroll
    for (int k = 0; k < 8; ++k) {
        GroupScale gs;
        gs.s = s_sh[8 * g + k];
        gs.y = y_sh[8 * g + k];
        gs.slow = !(gs.s >= kSmallScale);
        float av[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) av[i] = __builtin_fabsf(dequant4(i, k >> 2)[k & 3]);
        float qv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) qv[i] = quot_fast(av[i], gs);
        if (gs.slow) {
#pragma unroll
            for (int i = 0; i < 8; ++i) qv[i] = quot_slow(av[i], gs);
        }
        uint32_t wd[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) wd[i] = k < 4 ? code[i].x : code[i].y;
        const uint32_t byte = (uint32_t)(k & 3);
        const uint32_t s0 = gather_byte4(wd[0], wd[1], wd[2], wd[3], byte);
        const uint32_t s1 = gather_byte4(wd[4], wd[5], wd[6], wd[7], byte);
        const uint32_t w0 = pack_e4m3x4(qv[0], qv[1], qv[2], qv[3], s0);
        const uint32_t w1 = pack_e4m3x4(qv[4], qv[5], qv[6], qv[7], s1);
        *reinterpret_cast<uint2*>(&tr[(8 * g + k) * kTrStride + 8 * r]) = make_uint2(w0, w1);
    }
    __syncthreads();
    const int cc = t >> 1, h = t & 1;
    uint8_t* dst = qt + (c0 + cc) * ld_qt + t0 + 64 * h;
    const uint8_t* src = &tr[cc * kTrStride + 64 * h];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        *reinterpret_cast<uint4*>(dst + 16 * i) = *reinterpret_cast<const uint4*>(src + 16 * i);
}

__global__ __launch_bounds__(256) void retile_128x1_kernel(
    const uint8_t* __restrict__ q, int64_t ld_q, const float* __restrict__ scale, int64_t ld_s,
    uint8_t* __restrict__ qt, int64_t ld_qt, float* __restrict__ scale_t, int64_t ld_st,
    int64_t cblocks) {
    __shared__ uint32_t red[4][16][8];
    __shared__ float s_sh[128];
    __shared__ float y_sh[128];
    __shared__ __attribute__((aligned(16))) uint8_t tr[128 * kTrStride];
    retile_128x1_body(q, ld_q, scale, ld_s, qt, ld_qt, scale_t, ld_st, cblocks, (int64_t)blockIdx.x,
                      PanelLds<8>{red, s_sh, y_sh, tr});
}

// The Wgrad operands when X comes from the FP8 activation cache, in one
// grid: blocks below a_blocks quantize panels of dY in 128x1 tiles, the rest
// re-tile panels of the cached X. Both bodies share one set of LDS arrays,
// sized for the larger.
struct RetileArgs {
    const uint8_t* q;
    int64_t ld_q;
    const float* scale;
    int64_t ld_s;
    uint8_t* qt;
    int64_t ld_qt;
    float* scale_t;
    int64_t ld_st, cblocks;
};

__global__ __launch_bounds__(256) void quant_retile_128x1_kernel(int64_t tokens, Act128Args a, int64_t a_blocks,
                                                                 RetileArgs b) {
    __shared__ uint32_t red[4][16][8];
    __shared__ float s_sh[128];
    __shared__ float y_sh[128];
    __shared__ __attribute__((aligned(16))) uint8_t tr[128 * kTrStride];
    const int64_t blk = (int64_t)blockIdx.x;
    if (blk < a_blocks)  // block-uniform: the barriers inside stay whole
        act_128x1_body(a.x, tokens, a.cols, a.ld_x, a.qt, a.ld_q, a.scale, a.ld_s, a.cblocks, blk,
                       PanelLds<4>{reinterpret_cast<uint32_t(*)[16][4]>(red), s_sh, y_sh, tr});
    else
        retile_128x1_body(b.q, b.ld_q, b.scale, b.ld_s, b.qt, b.ld_qt, b.scale_t, b.ld_st, b.cblocks,
                          blk - a_blocks, PanelLds<8>{red, s_sh, y_sh, tr});
}

// ---------------------------------------------------------------- 128x128

// Several weight matrices (experts) in one launch: group e starts at the
// base pointers plus e times these strides (elements); work units (single
// 128x128 blocks or pairs of them) per group.
struct WeightGroups {
    int64_t units;
    int64_t w, q, s, qt, st;
};

// Grids of at least kStageTBlocks weight blocks (8 per CU) write the
// transposed copy through LDS (STAGE_T kernels): measured, 32 MoE experts quantize in
// 724 instead of 754 us that way, while a single 2048x7168 weight (896
// blocks, too few to hide the extra barrier) takes 15.0 instead of 14.0 us.
// Kernels without the staging hold no LDS for it. Grids of at least
// kPairBlocks weight blocks (16 per CU) take pairs of blocks per workgroup;
// smaller grids keep single-block units, which end the grid more evenly.
constexpr int64_t kPairBlocks = 4096;
constexpr int64_t kStageTBlocks = 2048;

// One 256-thread block quantizes one 128x128 weight block: thread (row group
// rg = t/16, chunk g = t%16) holds rows 8rg..8rg+7 x columns 8g..8g+7. The
// optional transposed copy is produced from the thread's 8x8 byte tile with
// byte permutes, so block (bn, bk) of W^T gets exactly the same codes. (The
// unit of grids too small for pairs of blocks to balance over the CUs.)
template <bool STAGE_T>
__device__ __forceinline__ void weight_block_body(
    const uint16_t* __restrict__ w, int64_t kblocks, int64_t ld_w,
    uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ scale, int64_t ld_s,
    uint8_t* __restrict__ q_t, int64_t ld_qt, float* __restrict__ scale_t, int64_t ld_st,
    WeightGroups grp, int64_t block) {
    __shared__ uint32_t red[4];
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int g = t & 15, rg = t >> 4;
    // group (expert) of this block, then its block (bn, bk)
    const int64_t e = block / grp.units, local = block - e * grp.units;
    w += e * grp.w;
    q += e * grp.q;
    scale += e * grp.s;
    if (q_t != nullptr) {
        q_t += e * grp.qt;
        scale_t += e * grp.st;
    }
    const int64_t bn = local / kblocks, bk = local - bn * kblocks;
    const int64_t n0 = bn * 128 + 8 * rg, k0 = bk * 128 + 8 * g;

    uint4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        v[i] = load_nt16(w + (n0 + i) * ld_w + k0);
    const uint32_t mask = 0x7FFF7FFFu;
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        m = pk_max_u16(m, pk_max_u16(pk_max_u16(v[i].x & mask, v[i].y & mask),
                                     pk_max_u16(v[i].z & mask, v[i].w & mask)));
    m = wave_max(umax32(m & 0xFFFFu, m >> 16));
    if (lane == 0) red[wv] = m;
    __syncthreads();
    m = umax32(umax32(red[0], red[1]), umax32(red[2], red[3]));
    const GroupScale gs = group_scale(m);

    uint32_t code[8][2];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float a[8] = {bf16_lo(v[i].x), bf16_hi(v[i].x), bf16_lo(v[i].y), bf16_hi(v[i].y),
                      bf16_lo(v[i].z), bf16_hi(v[i].z), bf16_lo(v[i].w), bf16_hi(v[i].w)};
        float qv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[e] = quot_fast(__builtin_fabsf(a[e]), gs);
        if (gs.slow) {
#pragma unroll
            for (int e = 0; e < 8; ++e) qv[e] = quot_slow(__builtin_fabsf(a[e]), gs);
        }
        code[i][0] = pack_e4m3x4(qv[0], qv[1], qv[2], qv[3], bf16x4_sign_bytes(v[i].x, v[i].y));
        code[i][1] = pack_e4m3x4(qv[4], qv[5], qv[6], qv[7], bf16x4_sign_bytes(v[i].z, v[i].w));
        store_nt8(q + (n0 + i) * ld_q + k0, code[i][0], code[i][1]);
    }
    if (t == 0) scale[bn * ld_s + bk] = gs.s;
    if (q_t != nullptr && !STAGE_T) {
        if (t == 0) scale_t[bk * ld_st + bn] = gs.s;
        // Column kk of the 8x8 tile = byte (kk % 4) of word (kk / 4) of rows 0..7.
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const int d = kk >> 2;
            const uint32_t byte = (uint32_t)(kk & 3);
            const uint32_t lo = gather_byte4(code[0][d], code[1][d], code[2][d], code[3][d], byte);
            const uint32_t hi = gather_byte4(code[4][d], code[5][d], code[6][d], code[7][d], byte);
            *reinterpret_cast<uint2*>(q_t + (k0 + kk) * ld_qt + bn * 128 + 8 * rg) = make_uint2(lo, hi);
        }
    }
    if constexpr (STAGE_T) {
        if (q_t != nullptr) {  // block-uniform: the barrier below is reached by all or none
            // The transposed block goes through LDS so that every store writes
            // whole 128-byte rows of q_t. Column kk of the thread's 8x8 tile =
            // byte (kk % 4) of word (kk / 4) of rows 0..7.
            __shared__ __attribute__((aligned(16))) uint8_t trw[128 * kTrStride];
            if (t == 0) scale_t[bk * ld_st + bn] = gs.s;
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const int d = kk >> 2;
                const uint32_t byte = (uint32_t)(kk & 3);
                const uint32_t lo = gather_byte4(code[0][d], code[1][d], code[2][d], code[3][d], byte);
                const uint32_t hi = gather_byte4(code[4][d], code[5][d], code[6][d], code[7][d], byte);
                *reinterpret_cast<uint2*>(&trw[(8 * g + kk) * kTrStride + 8 * rg]) = make_uint2(lo, hi);
            }
            __syncthreads();
            // thread t writes half h of transposed row kr (64 bytes)
            const int kr = t >> 1, h = t & 1;
            uint8_t* dst = q_t + (bk * 128 + kr) * ld_qt + bn * 128 + 64 * h;
            const uint8_t* src = &trw[kr * kTrStride + 64 * h];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<uint4*>(dst + 16 * i) = *reinterpret_cast<const uint4*>(src + 16 * i);
        }
    }
}

// One 256-thread block quantizes two horizontally adjacent 128x128 weight
// blocks, (bn, 2p) and (bn, 2p + 1); the second exists only when the number
// of K blocks is even or p is not the last pair. Lane l of wave wv works on
// block sel = (l / 16) % 2, rows 16 rb .. 16 rb + 15 with rb = 2 wv + l / 32,
// columns 8 g .. 8 g + 7 with g = l % 16. Every load instruction then reads
// 512 contiguous bytes of each of two rows, and codes are stored
// non-temporal. (A streaming probe of this traffic, 2 B read and 1 B written
// per element over the 32 MoE experts, measured 457 us this way against
// 512 us with one block per workgroup -- 4 rows x 256 bytes per load -- and
// plain stores; each code store instruction covers whole 128-byte lines.)
// The optional transposed copy is produced from the thread's
// 16x8 byte tile with byte permutes, so block (bk, bn) of W^T gets exactly
// the same codes.
template <bool STAGE_T>
__device__ __forceinline__ void weight_pair_body(
    const uint16_t* __restrict__ w, int64_t kblocks, int64_t ld_w,
    uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ scale, int64_t ld_s,
    uint8_t* __restrict__ q_t, int64_t ld_qt, float* __restrict__ scale_t, int64_t ld_st,
    WeightGroups grp, int64_t unit) {
    __shared__ uint32_t red[4][2];
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int sel = (lane >> 4) & 1, g = lane & 15, rb = 2 * wv + (lane >> 5);
    // group (expert) of this unit, then its pair of blocks
    const int64_t e = unit / grp.units, local = unit - e * grp.units;
    w += e * grp.w;
    q += e * grp.q;
    scale += e * grp.s;
    if (q_t != nullptr) {
        q_t += e * grp.qt;
        scale_t += e * grp.st;
    }
    const int64_t pairs = (kblocks + 1) / 2;
    const int64_t bn = local / pairs, bk0 = 2 * (local - bn * pairs);
    const int64_t bk = bk0 + sel;
    const bool valid = bk < kblocks;  // lane-divergent only in the last pair of an odd row
    const int64_t n0 = bn * 128 + 16 * rb, k0 = bk * 128 + 8 * g;

    uint4 v[16];
    if (valid) {
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = load_nt16(w + (n0 + i) * ld_w + k0);
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = make_uint4(0u, 0u, 0u, 0u);
    }
    const uint32_t mask = 0x7FFF7FFFu;
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        m = pk_max_u16(m, pk_max_u16(pk_max_u16(v[i].x & mask, v[i].y & mask),
                                     pk_max_u16(v[i].z & mask, v[i].w & mask)));
    // a DPP row of 16 lanes is one (row band, block); lanes l and l ^ 32 hold
    // the wave's two row bands of the same block
    m = row16_max(umax32(m & 0xFFFFu, m >> 16));
    m = umax32(m, (uint32_t)__shfl_xor((int)m, 32));
    if ((lane & 47) == 0) red[wv][sel] = m;  // lanes 0 (block 0) and 16 (block 1)
    __syncthreads();
    m = umax32(umax32(red[0][sel], red[1][sel]), umax32(red[2][sel], red[3][sel]));
    const GroupScale gs = group_scale(m);
    const bool writes_scale = valid && wv == 0 && (lane & 47) == 0;

    uint32_t code[16][2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        float a[8] = {bf16_lo(v[i].x), bf16_hi(v[i].x), bf16_lo(v[i].y), bf16_hi(v[i].y),
                      bf16_lo(v[i].z), bf16_hi(v[i].z), bf16_lo(v[i].w), bf16_hi(v[i].w)};
        float qv[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) qv[c] = quot_fast(__builtin_fabsf(a[c]), gs);
        if (gs.slow) {
#pragma unroll
            for (int c = 0; c < 8; ++c) qv[c] = quot_slow(__builtin_fabsf(a[c]), gs);
        }
        code[i][0] = pack_e4m3x4(qv[0], qv[1], qv[2], qv[3], bf16x4_sign_bytes(v[i].x, v[i].y));
        code[i][1] = pack_e4m3x4(qv[4], qv[5], qv[6], qv[7], bf16x4_sign_bytes(v[i].z, v[i].w));
        if (valid) store_nt8(q + (n0 + i) * ld_q + k0, code[i][0], code[i][1]);
    }
    if (writes_scale) scale[bn * ld_s + bk] = gs.s;
    if (q_t == nullptr) return;

    // Column kk of the thread's tile, rows 0..15: byte kk % 4 of word kk / 4
    // of each row, four rows per word.
    auto column = [&](int kk, uint32_t (&c4)[4]) {
        const int d = kk >> 2;
        const uint32_t byte = (uint32_t)(kk & 3);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            c4[j] = gather_byte4(code[4 * j][d], code[4 * j + 1][d], code[4 * j + 2][d], code[4 * j + 3][d], byte);
    };
    if (writes_scale) scale_t[bk * ld_st + bn] = gs.s;
    // (The transposed copy keeps plain stores: a store instruction here
    // covers parts of many 128-byte lines, and non-temporal partial-line
    // stores measured 4x slower.)
    if constexpr (!STAGE_T) {
        if (valid) {
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                uint32_t c4[4];
                column(kk, c4);
                *reinterpret_cast<uint4*>(q_t + (k0 + kk) * ld_qt + n0) = make_uint4(c4[0], c4[1], c4[2], c4[3]);
            }
        }
    } else {
        // Staged: both transposed blocks go through LDS; then each store
        // instruction of the block writes 32 whole 128-byte rows (8 lanes per
        // row). (q_t and the kernel variant are block-uniform, so the barrier
        // is reached by all threads.)
        __shared__ __attribute__((aligned(16))) uint8_t trw[2][128 * kTrStride];
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            uint32_t c4[4];
            column(kk, c4);
            *reinterpret_cast<uint4*>(&trw[sel][(8 * g + kk) * kTrStride + 16 * rb]) =
                make_uint4(c4[0], c4[1], c4[2], c4[3]);
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int idx = 256 * i + t;  // (transposed block, row, 16-byte chunk)
            const int ws = idx >> 10, kr = (idx >> 3) & 127, c = idx & 7;
            if (bk0 + ws < kblocks)
                *reinterpret_cast<uint4*>(q_t + ((bk0 + ws) * 128 + kr) * ld_qt + bn * 128 + 16 * c) =
                    *reinterpret_cast<const uint4*>(&trw[ws][kr * kTrStride + 16 * c]);
        }
    }
}

// Work unit `unit` of a weight grid: a pair of blocks (PAIR) or one block.
template <bool STAGE_T, bool PAIR>
__device__ __forceinline__ void weight_unit(
    const uint16_t* __restrict__ w, int64_t kblocks, int64_t ld_w,
    uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ scale, int64_t ld_s,
    uint8_t* __restrict__ q_t, int64_t ld_qt, float* __restrict__ scale_t, int64_t ld_st,
    WeightGroups grp, int64_t unit) {
    if constexpr (PAIR)
        weight_pair_body<STAGE_T>(w, kblocks, ld_w, q, ld_q, scale, ld_s, q_t, ld_qt, scale_t, ld_st, grp, unit);
    else
        weight_block_body<STAGE_T>(w, kblocks, ld_w, q, ld_q, scale, ld_s, q_t, ld_qt, scale_t, ld_st, grp, unit);
}

template <bool STAGE_T, bool PAIR>
__global__ __launch_bounds__(256) void quant_weight_kernel(
    const uint16_t* __restrict__ w, int64_t kblocks, int64_t ld_w,
    uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ scale, int64_t ld_s,
    uint8_t* __restrict__ q_t, int64_t ld_qt, float* __restrict__ scale_t, int64_t ld_st,
    WeightGroups grp) {
    weight_unit<STAGE_T, PAIR>(w, kblocks, ld_w, q, ld_q, scale, ld_s, q_t, ld_qt, scale_t, ld_st, grp,
                               (int64_t)blockIdx.x);
}

// ----------------------------------------------- activation + weight, one launch

// A Linear layer's two operands in one launch: blocks [0, act_blocks) run
// the 1x128 activation body, the rest the 128x128 weight body (block-uniform
// branch). The arithmetic is that of the two kernels above, bit for bit; one
// launch saves a launch gap and overlaps the two ramps and tails.
struct ActArgs {
    const uint16_t* x;
    int64_t rows, slabs, ld_x;
    uint8_t* q;
    int64_t ld_q;
    float* scale;
    int64_t ld_s, units;
};

struct WeightArgs {
    const uint16_t* w;
    int64_t kblocks, ld_w;
    uint8_t* q;
    int64_t ld_q;
    float* scale;
    int64_t ld_s;
    uint8_t* q_t;
    int64_t ld_qt;
    float* scale_t;
    int64_t ld_st;
};

template <bool STAGE_T, bool PAIR>
__global__ __launch_bounds__(256) void quant_act_weight_kernel(ActArgs a, int64_t act_blocks, WeightArgs wa,
                                                               WeightGroups grp) {
    const int64_t b = (int64_t)blockIdx.x;
    // weight blocks first (they are the larger work items) unless they also
    // write the transposed copy: measured, that case finishes sooner with the
    // activation tiles first
    const bool weight_first = wa.q_t == nullptr;
    const bool is_weight = weight_first ? b < grp.units : b >= act_blocks;
    const int64_t i = b - (is_weight ? (weight_first ? 0 : act_blocks) : (weight_first ? grp.units : 0));
    if (is_weight)
        weight_unit<STAGE_T, PAIR>(wa.w, wa.kblocks, wa.ld_w, wa.q, wa.ld_q, wa.scale, wa.ld_s, wa.q_t, wa.ld_qt,
                                   wa.scale_t, wa.ld_st, grp, i);
    else
        act_1x128_body<false>(a.x, a.rows, a.slabs, a.ld_x, a.q, a.ld_q, a.scale, a.ld_s, a.units, nullptr, 0,
                              (int64_t)0, i);
}

}  // namespace

// ------------------------------------------------------------------ launch

hipError_t launch_quant_act_1x128(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                                  uint8_t* q, int64_t ld_q, float* scale, int64_t ld_s,
                                  hipStream_t stream) {
    const int64_t slabs = cols / 128;
    const int64_t units = act_units(rows, slabs);
    const int64_t blocks = (units + kActWavesPerBlock - 1) / kActWavesPerBlock;
    hipLaunchKernelGGL(quant_act_1x128_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       x, rows, slabs, ld_x, q, ld_q, scale, ld_s, units, nullptr, 0, (int64_t)0);
    return hipGetLastError();
}

hipError_t launch_quant_act_scatter(const uint16_t* x, int64_t tokens, int64_t cols, int64_t ld_x,
                                    int topk, const int32_t* dst_rows, int64_t m_total, uint8_t* q,
                                    int64_t ld_q, float* scale, int64_t ld_s, hipStream_t stream) {
    const int64_t slabs = cols / 128;
    const int64_t units = act_units(tokens, slabs);
    const int64_t blocks = (units + kActWavesPerBlock - 1) / kActWavesPerBlock;
    hipLaunchKernelGGL(quant_act_1x128_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       x, tokens, slabs, ld_x, q, ld_q, scale, ld_s, units, dst_rows, topk, m_total);
    return hipGetLastError();
}

hipError_t launch_quant_mx(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q,
                           int64_t ld_q, uint32_t* scale, int64_t ld_s, hipStream_t stream) {
    const int64_t slabs = cols / 128;
    const int64_t units = act_units(rows, slabs);
    const int64_t blocks = (units + kActWavesPerBlock - 1) / kActWavesPerBlock;
    hipLaunchKernelGGL(quant_mx_1x32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       x, rows, slabs, ld_x, q, ld_q, scale, ld_s, units);
    return hipGetLastError();
}

hipError_t launch_quant_mx_pair(const uint16_t* x0, int64_t rows0, int64_t cols0, int64_t ld_x0, uint8_t* q0,
                                int64_t ld_q0, uint32_t* s0, int64_t ld_s0, const uint16_t* x1, int64_t rows1,
                                int64_t cols1, int64_t ld_x1, uint8_t* q1, int64_t ld_q1, uint32_t* s1,
                                int64_t ld_s1, hipStream_t stream) {
    MxArgs a{x0, rows0, cols0 / 128, ld_x0, q0, ld_q0, s0, ld_s0, 0};
    MxArgs b{x1, rows1, cols1 / 128, ld_x1, q1, ld_q1, s1, ld_s1, 0};
    a.units = act_units(rows0, a.slabs);
    b.units = act_units(rows1, b.slabs);
    const int64_t a_blocks = (a.units + kActWavesPerBlock - 1) / kActWavesPerBlock;
    const int64_t blocks = a_blocks + (b.units + kActWavesPerBlock - 1) / kActWavesPerBlock;
    hipLaunchKernelGGL(quant_mx_1x32_pair_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a, a_blocks, b);
    return hipGetLastError();
}

hipError_t launch_quant_act_128x1(const uint16_t* x, int64_t tokens, int64_t cols, int64_t ld_x,
                                  uint8_t* qt, int64_t ld_q, float* scale, int64_t ld_s,
                                  hipStream_t stream) {
    const int64_t cblocks = (cols + 127) / 128;
    const int64_t blocks = tokens / 128 * cblocks;
    hipLaunchKernelGGL(quant_act_128x1_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       x, tokens, cols, ld_x, qt, ld_q, scale, ld_s, cblocks);
    return hipGetLastError();
}

hipError_t launch_quant_act_128x1_pair(int64_t tokens, const uint16_t* x0, int64_t cols0, int64_t ld_x0,
                                       uint8_t* q0, int64_t ld_q0, float* s0, int64_t ld_s0,
                                       const uint16_t* x1, int64_t cols1, int64_t ld_x1, uint8_t* q1,
                                       int64_t ld_q1, float* s1, int64_t ld_s1, hipStream_t stream) {
    Act128Args a{x0, cols0, ld_x0, q0, ld_q0, s0, ld_s0, (cols0 + 127) / 128};
    Act128Args b{x1, cols1, ld_x1, q1, ld_q1, s1, ld_s1, (cols1 + 127) / 128};
    const int64_t a_blocks = tokens / 128 * a.cblocks;
    const int64_t blocks = a_blocks + tokens / 128 * b.cblocks;
    hipLaunchKernelGGL(quant_act_128x1_pair_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, tokens, a,
                       a_blocks, b);
    return hipGetLastError();
}

hipError_t launch_quant_retile_128x1(int64_t tokens, const uint16_t* x0, int64_t cols0, int64_t ld_x0,
                                     uint8_t* q0, int64_t ld_q0, float* s0, int64_t ld_s0, const uint8_t* xq,
                                     int64_t cols1, int64_t ld_xq, const float* xs, int64_t ld_xs, uint8_t* q1,
                                     int64_t ld_q1, float* s1, int64_t ld_s1, hipStream_t stream) {
    Act128Args a{x0, cols0, ld_x0, q0, ld_q0, s0, ld_s0, (cols0 + 127) / 128};
    RetileArgs b{xq, ld_xq, xs, ld_xs, q1, ld_q1, s1, ld_s1, cols1 / 128};
    const int64_t a_blocks = tokens / 128 * a.cblocks;
    const int64_t blocks = a_blocks + tokens / 128 * b.cblocks;
    hipLaunchKernelGGL(quant_retile_128x1_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, tokens, a,
                       a_blocks, b);
    return hipGetLastError();
}

hipError_t launch_retile_128x1(const uint8_t* q, int64_t tokens, int64_t cols, int64_t ld_q,
                               const float* scale, int64_t ld_s, uint8_t* qt, int64_t ld_qt,
                               float* scale_t, int64_t ld_st, hipStream_t stream) {
    const int64_t cblocks = cols / 128;
    const int64_t blocks = tokens / 128 * cblocks;
    hipLaunchKernelGGL(retile_128x1_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       q, ld_q, scale, ld_s, qt, ld_qt, scale_t, ld_st, cblocks);
    return hipGetLastError();
}

hipError_t launch_quant_act_weight(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q,
                                   int64_t ld_q, float* scale, int64_t ld_s, const uint16_t* w, int64_t n,
                                   int64_t k, int64_t ld_w, uint8_t* wq, int64_t ld_wq, float* ws, int64_t ld_ws,
                                   uint8_t* wq_t, int64_t ld_wqt, float* ws_t, int64_t ld_wst,
                                   hipStream_t stream) {
    ActArgs a;
    a.x = x;
    a.rows = rows;
    a.slabs = cols / 128;
    a.ld_x = ld_x;
    a.q = q;
    a.ld_q = ld_q;
    a.scale = scale;
    a.ld_s = ld_s;
    a.units = act_units(rows, a.slabs);
    const int64_t act_blocks = (a.units + kActWavesPerBlock - 1) / kActWavesPerBlock;
    WeightArgs wa;
    wa.w = w;
    wa.kblocks = k / 128;
    wa.ld_w = ld_w;
    wa.q = wq;
    wa.ld_q = ld_wq;
    wa.scale = ws;
    wa.ld_s = ld_ws;
    wa.q_t = wq_t;
    wa.ld_qt = ld_wqt;
    wa.scale_t = ws_t;
    wa.ld_st = ld_wst;
    // Pairs of blocks when the weight blocks run first (no transposed copy):
    // the activation tiles then fill the tail. With the transposed copy the
    // activation tiles go first, and the weights keep the finer single-block
    // units for the tail.
    const bool pair = wq_t == nullptr;
    const bool stage = wq_t != nullptr && n / 128 * wa.kblocks >= kStageTBlocks;
    WeightGroups grp;
    grp.units = n / 128 * (pair ? (wa.kblocks + 1) / 2 : wa.kblocks);
    grp.w = grp.q = grp.s = grp.qt = grp.st = 0;
    const dim3 grid((unsigned)(act_blocks + grp.units)), block(256);
    if (pair)
        hipLaunchKernelGGL((quant_act_weight_kernel<false, true>), grid, block, 0, stream, a, act_blocks, wa, grp);
    else if (stage)
        hipLaunchKernelGGL((quant_act_weight_kernel<true, false>), grid, block, 0, stream, a, act_blocks, wa, grp);
    else
        hipLaunchKernelGGL((quant_act_weight_kernel<false, false>), grid, block, 0, stream, a, act_blocks, wa, grp);
    return hipGetLastError();
}

hipError_t launch_quant_weight(int64_t groups, const uint16_t* w, int64_t n, int64_t k, int64_t ld_w,
                               int64_t stride_w, uint8_t* q, int64_t ld_q, int64_t stride_q, float* scale,
                               int64_t ld_s, int64_t stride_s, uint8_t* q_t, int64_t ld_qt, int64_t stride_qt,
                               float* scale_t, int64_t ld_st, int64_t stride_st, hipStream_t stream) {
    const int64_t kblocks = k / 128;
    const int64_t blocks = groups * (n / 128) * kblocks;
    // Pairs of blocks for grids of at least 16 blocks per CU; smaller grids
    // keep single-block units, which balance better over the CUs.
    const bool pair = blocks >= kPairBlocks;
    const bool stage = q_t != nullptr && blocks >= kStageTBlocks;
    WeightGroups grp;
    grp.units = n / 128 * (pair ? (kblocks + 1) / 2 : kblocks);
    grp.w = stride_w;
    grp.q = stride_q;
    grp.s = stride_s;
    grp.qt = stride_qt;
    grp.st = stride_st;
    const dim3 grid((unsigned)(groups * grp.units)), block(256);
    if (pair && stage)
        hipLaunchKernelGGL((quant_weight_kernel<true, true>), grid, block, 0, stream, w, kblocks, ld_w, q, ld_q,
                           scale, ld_s, q_t, ld_qt, scale_t, ld_st, grp);
    else if (pair)
        hipLaunchKernelGGL((quant_weight_kernel<false, true>), grid, block, 0, stream, w, kblocks, ld_w, q, ld_q,
                           scale, ld_s, q_t, ld_qt, scale_t, ld_st, grp);
    else if (stage)
        hipLaunchKernelGGL((quant_weight_kernel<true, false>), grid, block, 0, stream, w, kblocks, ld_w, q, ld_q,
                           scale, ld_s, q_t, ld_qt, scale_t, ld_st, grp);
    else
        hipLaunchKernelGGL((quant_weight_kernel<false, false>), grid, block, 0, stream, w, kblocks, ld_w, q, ld_q,
                           scale, ld_s, q_t, ld_qt, scale_t, ld_st, grp);
    return hipGetLastError();
}

}  // namespace fp8q
