// api.cpp -- the C ABI of libfp8q (declared in include/fp8q.h).
//
// Every entry point validates its arguments on the host, returns a status
// code without launching anything on error, and otherwise enqueues the
// kernels on the caller's stream. Nothing here allocates, frees or
// synchronizes.
#include "fp8q.h"

#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdlib.h>

#include <vector>

#include "launch.h"

namespace {

thread_local int g_last_hip_error = 0;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int hip_status(hipError_t e) {
    if (e == hipSuccess) return FP8Q_OK;
    g_last_hip_error = (int)e;
    return FP8Q_ERR_HIP;
}

// A grid of more than 2^31 - 1 blocks is not launchable.
bool grid_ok(int64_t blocks) { return blocks >= 0 && blocks <= 0x7FFFFFFFLL; }

// Bytes [lo, hi) a row-major rows x cols matrix of elem-byte elements with
// leading dimension ld occupies (rows, cols > 0).
struct Span {
    uintptr_t lo, hi;
};
Span span(const void* p, int64_t rows, int64_t cols, int64_t ld, int64_t elem) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return {lo, lo + (uintptr_t)(((rows - 1) * ld + cols) * elem)};
}
bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

// FP8Q_DEBUG=1 in the environment (read on every grouped call): the grouped
// entry points copy the device arrays that describe the expert segments to
// the host and check the contract their kernels trust. This synchronizes
// the caller's stream, so it is off by default.
bool debug_checks() {
    const char* v = getenv("FP8Q_DEBUG");
    return v && v[0] == '1' && v[1] == '\0';
}

// group_offsets[0] == 0, non-decreasing multiples of 128 ending at total;
// 0 <= group_rows[e] <= segment e (when given).
int check_segments_on_host(int32_t groups, const int32_t* group_offsets, const int32_t* group_rows, int64_t total,
                           hipStream_t stream) {
    std::vector<int32_t> off(groups + 1), rows(group_rows ? groups : 0);
    hipError_t e = hipMemcpyAsync(off.data(), group_offsets, off.size() * sizeof(int32_t), hipMemcpyDeviceToHost,
                                  stream);
    if (e == hipSuccess && group_rows)
        e = hipMemcpyAsync(rows.data(), group_rows, rows.size() * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_status(e);
    if (off[0] != 0 || off[groups] != total) return FP8Q_ERR_SHAPE;
    for (int32_t g = 0; g < groups; ++g) {
        if (off[g + 1] < off[g] || off[g + 1] % 128 != 0) return FP8Q_ERR_SHAPE;
        if (group_rows && (rows[g] < 0 || rows[g] > off[g + 1] - off[g])) return FP8Q_ERR_SHAPE;
    }
    return FP8Q_OK;
}

// rows * ld < FP8Q_MAX_SCALE_SPAN without overflowing int64 (a scale array of
// `rows` rows with leading dimension ld, in floats)
bool scale_span_ok(int64_t rows, int64_t ld) { return rows <= 0 || ld < FP8Q_MAX_SCALE_SPAN / rows; }

}  // namespace

extern "C" {

const char* fp8q_status_string(int status) {
    switch (status) {
        case FP8Q_OK: return "ok";
        case FP8Q_ERR_NULL: return "a required pointer is NULL";
        case FP8Q_ERR_SHAPE: return "bad shape (negative size, divisibility or leading dimension)";
        case FP8Q_ERR_ALIGN: return "pointer or leading dimension breaks the required alignment";
        case FP8Q_ERR_ENUM: return "enum argument out of range";
        case FP8Q_ERR_HIP: return "HIP launch failed (see fp8q_last_hip_error)";
        default: return "unknown status";
    }
}

int fp8q_last_hip_error(void) { return g_last_hip_error; }

int fp8_quantize_act(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, int tiling,
                     uint8_t* q, int64_t ld_q, float* scale, int64_t ld_s, hipStream_t stream) {
    if (tiling != FP8Q_TILE_1x128 && tiling != FP8Q_TILE_128x1) return FP8Q_ERR_ENUM;
    if (rows < 0 || cols < 0) return FP8Q_ERR_SHAPE;
    if (rows == 0 || cols == 0) return FP8Q_OK;
    if (!x || !q || !scale) return FP8Q_ERR_NULL;
    if (ld_x < cols) return FP8Q_ERR_SHAPE;
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(scale, 4) || ld_x % 8 != 0 || ld_q % 16 != 0)
        return FP8Q_ERR_ALIGN;
    if (tiling == FP8Q_TILE_1x128) {
        if (cols % 128 != 0 || ld_q < cols || ld_s < rows) return FP8Q_ERR_SHAPE;
        if (!grid_ok((rows + 15) / 16 * (cols / 128) / 4 + 1)) return FP8Q_ERR_SHAPE;
        return hip_status(fp8q::launch_quant_act_1x128(x, rows, cols, ld_x, q, ld_q, scale, ld_s, stream));
    }
    if (rows % 128 != 0 || cols % 8 != 0 || ld_q < rows || ld_s < cols) return FP8Q_ERR_SHAPE;
    if (!grid_ok(rows / 128 * ((cols + 127) / 128))) return FP8Q_ERR_SHAPE;
    return hip_status(fp8q::launch_quant_act_128x1(x, rows, cols, ld_x, q, ld_q, scale, ld_s, stream));
}

int fp8_quantize_act_scatter(const uint16_t* x, int64_t tokens, int64_t cols, int64_t ld_x,
                             int32_t topk, const int32_t* dst_rows, int64_t m_total, uint8_t* q,
                             int64_t ld_q, float* scale, int64_t ld_s, hipStream_t stream) {
    if (tokens < 0 || cols < 0 || m_total < 0 || topk < 1 || topk > 8) return FP8Q_ERR_SHAPE;
    if (tokens == 0 || cols == 0 || m_total == 0) return FP8Q_OK;
    if (!x || !dst_rows || !q || !scale) return FP8Q_ERR_NULL;
    if (cols % 128 != 0 || ld_x < cols || ld_q < cols || ld_s < m_total) return FP8Q_ERR_SHAPE;
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(scale, 4) || !aligned(dst_rows, 4) ||
        ld_x % 8 != 0 || ld_q % 16 != 0)
        return FP8Q_ERR_ALIGN;
    if (!grid_ok((tokens + 15) / 16 * (cols / 128) / 4 + 1)) return FP8Q_ERR_SHAPE;
    return hip_status(fp8q::launch_quant_act_scatter(x, tokens, cols, ld_x, topk, dst_rows, m_total, q,
                                                     ld_q, scale, ld_s, stream));
}

int fp8_quantize_weight_grouped(int32_t groups, const uint16_t* w, int64_t n, int64_t k, int64_t ld_w,
                                int64_t stride_w, uint8_t* q, int64_t ld_q, int64_t stride_q, float* scale,
                                int64_t ld_s, int64_t stride_s, uint8_t* q_t, int64_t ld_qt,
                                int64_t stride_qt, float* scale_t, int64_t ld_st, int64_t stride_st,
                                hipStream_t stream) {
    if (groups < 0 || n < 0 || k < 0) return FP8Q_ERR_SHAPE;
    if (groups == 0 || n == 0 || k == 0) return FP8Q_OK;
    if (!w || !q || !scale) return FP8Q_ERR_NULL;
    if (q_t && !scale_t) return FP8Q_ERR_NULL;
    if (n % 128 != 0 || k % 128 != 0 || ld_w < k || ld_q < k || ld_s < k / 128) return FP8Q_ERR_SHAPE;
    if (q_t && (ld_qt < n || ld_st < n / 128)) return FP8Q_ERR_SHAPE;
    if (stride_w < 0) return FP8Q_ERR_SHAPE;  // inputs are only read: they may overlap
    // outputs of different groups must not overlap
    if (groups > 1 && (stride_q < n * ld_q || stride_s < (n / 128) * ld_s)) return FP8Q_ERR_SHAPE;
    if (groups > 1 && q_t && (stride_qt < k * ld_qt || stride_st < (k / 128) * ld_st)) return FP8Q_ERR_SHAPE;
    if (!aligned(w, 16) || !aligned(q, 16) || !aligned(scale, 4) || ld_w % 8 != 0 || ld_q % 16 != 0 ||
        stride_w % 8 != 0 || stride_q % 16 != 0)
        return FP8Q_ERR_ALIGN;
    if (q_t && (!aligned(q_t, 16) || !aligned(scale_t, 4) || ld_qt % 16 != 0 || stride_qt % 16 != 0))
        return FP8Q_ERR_ALIGN;
    if (!grid_ok((int64_t)groups * (n / 128) * (k / 128))) return FP8Q_ERR_SHAPE;
    return hip_status(fp8q::launch_quant_weight(groups, w, n, k, ld_w, stride_w, q, ld_q, stride_q, scale,
                                                ld_s, stride_s, q_t, ld_qt, stride_qt, scale_t, ld_st,
                                                stride_st, stream));
}

int fp8_quantize_act_weight(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q,
                            int64_t ld_q, float* scale, int64_t ld_s, const uint16_t* w, int64_t n, int64_t k,
                            int64_t ld_w, uint8_t* wq, int64_t ld_wq, float* wscale, int64_t ld_ws,
                            uint8_t* wq_t, int64_t ld_wqt, float* wscale_t, int64_t ld_wst, hipStream_t stream) {
    // the checks of fp8_quantize_act (1x128) and fp8_quantize_weight, both
    if (rows < 0 || cols < 0 || n < 0 || k < 0) return FP8Q_ERR_SHAPE;
    const bool act = rows > 0 && cols > 0, wgt = n > 0 && k > 0;
    if (act) {
        if (!x || !q || !scale) return FP8Q_ERR_NULL;
        if (ld_x < cols || cols % 128 != 0 || ld_q < cols || ld_s < rows) return FP8Q_ERR_SHAPE;
        if (!aligned(x, 16) || !aligned(q, 16) || !aligned(scale, 4) || ld_x % 8 != 0 || ld_q % 16 != 0)
            return FP8Q_ERR_ALIGN;
    }
    if (wgt) {
        if (!w || !wq || !wscale) return FP8Q_ERR_NULL;
        if (wq_t && !wscale_t) return FP8Q_ERR_NULL;
        if (n % 128 != 0 || k % 128 != 0 || ld_w < k || ld_wq < k || ld_ws < k / 128) return FP8Q_ERR_SHAPE;
        if (wq_t && (ld_wqt < n || ld_wst < n / 128)) return FP8Q_ERR_SHAPE;
        if (!aligned(w, 16) || !aligned(wq, 16) || !aligned(wscale, 4) || ld_w % 8 != 0 || ld_wq % 16 != 0)
            return FP8Q_ERR_ALIGN;
        if (wq_t && (!aligned(wq_t, 16) || !aligned(wscale_t, 4) || ld_wqt % 16 != 0)) return FP8Q_ERR_ALIGN;
    }
    if (!act && !wgt) return FP8Q_OK;
    if (act && wgt) {
        // the two halves of the launch run concurrently: no output of one may
        // share a byte with an output of the other
        const Span a_out[2] = {span(q, rows, cols, ld_q, 1), span(scale, cols / 128, rows, ld_s, 4)};
        const Span w_out[4] = {span(wq, n, k, ld_wq, 1), span(wscale, n / 128, k / 128, ld_ws, 4),
                               wq_t ? span(wq_t, k, n, ld_wqt, 1) : Span{0, 0},
                               wq_t ? span(wscale_t, k / 128, n / 128, ld_wst, 4) : Span{0, 0}};
        for (const Span& x : a_out)
            for (const Span& y : w_out)
                if (overlap(x, y)) return FP8Q_ERR_SHAPE;
    }
    const int64_t act_blocks = act ? (rows + 15) / 16 * (cols / 128) / 4 + 1 : 0;
    if (!grid_ok(act_blocks + (wgt ? n / 128 * (k / 128) : 0))) return FP8Q_ERR_SHAPE;
    // an empty operand is skipped: its block range is empty
    return hip_status(fp8q::launch_quant_act_weight(
        x, act ? rows : 0, act ? cols : 0, ld_x, q, ld_q, scale, ld_s, w, wgt ? n : 0, wgt ? k : 0, ld_w, wq,
        ld_wq, wscale, ld_ws, wq_t, ld_wqt, wscale_t, ld_wst, stream));
}

int fp8_quantize_act_128x1_pair(int64_t tokens, const uint16_t* x0, int64_t cols0, int64_t ld_x0, uint8_t* q0,
                                int64_t ld_q0, float* scale0, int64_t ld_s0, const uint16_t* x1, int64_t cols1,
                                int64_t ld_x1, uint8_t* q1, int64_t ld_q1, float* scale1, int64_t ld_s1,
                                hipStream_t stream) {
    // the checks of fp8_quantize_act (128x1) on each operand
    if (tokens < 0 || cols0 < 0 || cols1 < 0) return FP8Q_ERR_SHAPE;
    const bool op0 = tokens > 0 && cols0 > 0, op1 = tokens > 0 && cols1 > 0;
    const uint16_t* xs[2] = {x0, x1};
    uint8_t* qs[2] = {q0, q1};
    float* ss[2] = {scale0, scale1};
    const int64_t cols[2] = {cols0, cols1}, ld_x[2] = {ld_x0, ld_x1}, ld_q[2] = {ld_q0, ld_q1},
                  ld_s[2] = {ld_s0, ld_s1};
    const bool on[2] = {op0, op1};
    for (int i = 0; i < 2; ++i) {
        if (!on[i]) continue;
        if (!xs[i] || !qs[i] || !ss[i]) return FP8Q_ERR_NULL;
        if (ld_x[i] < cols[i] || tokens % 128 != 0 || cols[i] % 8 != 0 || ld_q[i] < tokens || ld_s[i] < cols[i])
            return FP8Q_ERR_SHAPE;
        if (!aligned(xs[i], 16) || !aligned(qs[i], 16) || !aligned(ss[i], 4) || ld_x[i] % 8 != 0 ||
            ld_q[i] % 16 != 0)
            return FP8Q_ERR_ALIGN;
    }
    if (!op0 && !op1) return FP8Q_OK;
    if (op0 && op1) {
        // the two halves of the launch run concurrently: their outputs must be disjoint
        const Span o0[2] = {span(q0, cols0, tokens, ld_q0, 1), span(scale0, tokens / 128, cols0, ld_s0, 4)};
        const Span o1[2] = {span(q1, cols1, tokens, ld_q1, 1), span(scale1, tokens / 128, cols1, ld_s1, 4)};
        for (const Span& a : o0)
            for (const Span& b : o1)
                if (overlap(a, b)) return FP8Q_ERR_SHAPE;
    }
    const int64_t blocks = tokens / 128 * ((op0 ? (cols0 + 127) / 128 : 0) + (op1 ? (cols1 + 127) / 128 : 0));
    if (!grid_ok(blocks)) return FP8Q_ERR_SHAPE;
    // an empty operand is skipped: its block range is empty
    return hip_status(fp8q::launch_quant_act_128x1_pair(tokens, x0, op0 ? cols0 : 0, ld_x0, q0, ld_q0, scale0,
                                                        ld_s0, x1, op1 ? cols1 : 0, ld_x1, q1, ld_q1, scale1,
                                                        ld_s1, stream));
}

int fp8_quantize_act_128x1_retile(int64_t tokens, const uint16_t* x0, int64_t cols0, int64_t ld_x0, uint8_t* q0,
                                  int64_t ld_q0, float* scale0, int64_t ld_s0, const uint8_t* xq, int64_t cols1,
                                  int64_t ld_xq, const float* xs, int64_t ld_xs, uint8_t* q1, int64_t ld_q1,
                                  float* scale1, int64_t ld_s1, hipStream_t stream) {
    // the checks of fp8_quantize_act (128x1) on x0 and of fp8_retile_act_128x1 on the cache
    if (tokens < 0 || cols0 < 0 || cols1 < 0) return FP8Q_ERR_SHAPE;
    const bool op0 = tokens > 0 && cols0 > 0, op1 = tokens > 0 && cols1 > 0;
    if (op0) {
        if (!x0 || !q0 || !scale0) return FP8Q_ERR_NULL;
        if (ld_x0 < cols0 || tokens % 128 != 0 || cols0 % 8 != 0 || ld_q0 < tokens || ld_s0 < cols0)
            return FP8Q_ERR_SHAPE;
        if (!aligned(x0, 16) || !aligned(q0, 16) || !aligned(scale0, 4) || ld_x0 % 8 != 0 || ld_q0 % 16 != 0)
            return FP8Q_ERR_ALIGN;
    }
    if (op1) {
        if (!xq || !xs || !q1 || !scale1) return FP8Q_ERR_NULL;
        if (tokens % 128 != 0 || cols1 % 128 != 0 || ld_xq < cols1 || ld_xs < tokens || ld_q1 < tokens ||
            ld_s1 < cols1)
            return FP8Q_ERR_SHAPE;
        if (!aligned(xq, 16) || !aligned(xs, 16) || !aligned(q1, 16) || !aligned(scale1, 4) || ld_xq % 16 != 0 ||
            ld_xs % 4 != 0 || ld_q1 % 16 != 0)
            return FP8Q_ERR_ALIGN;
    }
    if (!op0 && !op1) return FP8Q_OK;
    if (op0 && op1) {
        // the two halves of the launch run concurrently: their outputs must be disjoint
        const Span o0[2] = {span(q0, cols0, tokens, ld_q0, 1), span(scale0, tokens / 128, cols0, ld_s0, 4)};
        const Span o1[2] = {span(q1, cols1, tokens, ld_q1, 1), span(scale1, tokens / 128, cols1, ld_s1, 4)};
        for (const Span& a : o0)
            for (const Span& b : o1)
                if (overlap(a, b)) return FP8Q_ERR_SHAPE;
    }
    const int64_t blocks = tokens / 128 * ((op0 ? (cols0 + 127) / 128 : 0) + (op1 ? cols1 / 128 : 0));
    if (!grid_ok(blocks)) return FP8Q_ERR_SHAPE;
    // an empty operand is skipped: its block range is empty
    return hip_status(fp8q::launch_quant_retile_128x1(tokens, x0, op0 ? cols0 : 0, ld_x0, q0, ld_q0, scale0, ld_s0,
                                                      xq, op1 ? cols1 : 0, ld_xq, xs, ld_xs, q1, ld_q1, scale1,
                                                      ld_s1, stream));
}

int fp8_quantize_weight(const uint16_t* w, int64_t n, int64_t k, int64_t ld_w,
                        uint8_t* q, int64_t ld_q, float* scale, int64_t ld_s,
                        uint8_t* q_t, int64_t ld_qt, float* scale_t, int64_t ld_st,
                        hipStream_t stream) {
    return fp8_quantize_weight_grouped(1, w, n, k, ld_w, 0, q, ld_q, 0, scale, ld_s, 0, q_t, ld_qt, 0,
                                       scale_t, ld_st, 0, stream);
}

static int check_gemm_common(int64_t m, int64_t n, int64_t k, const uint8_t* a, int64_t lda,
                             const float* a_scale, int64_t ld_as, const uint8_t* b, int64_t ldb,
                             const float* b_scale, void* c, int64_t ldc, int out_dtype) {
    if (out_dtype != FP8Q_OUT_BF16 && out_dtype != FP8Q_OUT_F32) return FP8Q_ERR_ENUM;
    // k == 0: C is all zeros; A, B and their scales are not read (may be NULL)
    if (!c || (k > 0 && (!a || !b || !a_scale || !b_scale))) return FP8Q_ERR_NULL;
    if (k % 128 != 0 || ldc < n || (k > 0 && (lda < k || ldb < k || ld_as < m))) return FP8Q_ERR_SHAPE;
    // tiles and scales are addressed through 31-bit buffer ranges
    if (k > 0 && (lda > FP8Q_MAX_GEMM_LD || ldb > FP8Q_MAX_GEMM_LD || !scale_span_ok(k / 128, ld_as)))
        return FP8Q_ERR_SHAPE;
    if (!aligned(c, 16) || ldc % 8 != 0) return FP8Q_ERR_ALIGN;
    if (k > 0 && (!aligned(a, 16) || !aligned(b, 16) || !aligned(a_scale, 4) || !aligned(b_scale, 4) ||
                  lda % 16 != 0 || ldb % 16 != 0))
        return FP8Q_ERR_ALIGN;
    return FP8Q_OK;
}

int fp8_gemm(int64_t m, int64_t n, int64_t k,
             const uint8_t* a, int64_t lda, const float* a_scale, int64_t ld_as,
             const uint8_t* b, int64_t ldb, const float* b_scale, int64_t ld_bs, int b_scale_kind,
             void* c, int64_t ldc, int out_dtype, hipStream_t stream) {
    if (b_scale_kind != FP8Q_BSCALE_BLOCK128 && b_scale_kind != FP8Q_BSCALE_ROW128) return FP8Q_ERR_ENUM;
    if (m < 0 || n < 0 || k < 0) return FP8Q_ERR_SHAPE;
    if (m == 0 || n == 0) return FP8Q_OK;
    int st = check_gemm_common(m, n, k, a, lda, a_scale, ld_as, b, ldb, b_scale, c, ldc, out_dtype);
    if (st != FP8Q_OK) return st;
    if (k > 0 && b_scale_kind == FP8Q_BSCALE_BLOCK128 &&
        (ld_bs < k / 128 || !scale_span_ok((n + 127) / 128, ld_bs)))
        return FP8Q_ERR_SHAPE;
    if (k > 0 && b_scale_kind == FP8Q_BSCALE_ROW128 && (ld_bs < n || !scale_span_ok(k / 128, ld_bs)))
        return FP8Q_ERR_SHAPE;
    if (!grid_ok(((m + 255) / 256) * ((n + 223) / 224) + 8)) return FP8Q_ERR_SHAPE;
    fp8q::GemmProblem g = {};
    g.m = m; g.n = n; g.k = k;
    g.a = a; g.lda = lda; g.a_scale = a_scale; g.ld_as = ld_as;
    g.b = b; g.ldb = ldb; g.b_scale = b_scale; g.ld_bs = ld_bs;
    g.b_rowscale = b_scale_kind == FP8Q_BSCALE_ROW128;
    g.c = c; g.ldc = ldc; g.out_f32 = out_dtype == FP8Q_OUT_F32;
    return hip_status(fp8q::launch_gemm(g, stream));
}

// fp8_grouped_gemm with the caller's workspace, or (scratch) with the
// library's own.
static int grouped_gemm(int32_t groups, const int32_t* group_offsets, const int32_t* group_rows,
                        int64_t m_total, int64_t n, int64_t k,
                        const uint8_t* a, int64_t lda, const float* a_scale, int64_t ld_as,
                        const uint8_t* b, int64_t ldb, int64_t stride_b,
                        const float* b_scale, int64_t ld_bs, int64_t stride_bs,
                        void* c, int64_t ldc, int out_dtype,
                        void* workspace, int64_t workspace_bytes, bool scratch, hipStream_t stream) {
    if (groups < 0 || m_total < 0 || n < 0 || k < 0 || workspace_bytes < 0) return FP8Q_ERR_SHAPE;
    if (out_dtype != FP8Q_OUT_BF16 && out_dtype != FP8Q_OUT_F32) return FP8Q_ERR_ENUM;
    if (groups == 0 || m_total == 0 || n == 0) return FP8Q_OK;
    if (!group_offsets) return FP8Q_ERR_NULL;
    int st = check_gemm_common(m_total, n, k, a, lda, a_scale, ld_as, b, ldb, b_scale, c, ldc, out_dtype);
    if (st != FP8Q_OK) return st;
    if (m_total % 128 != 0 || n % 128 != 0 || m_total > 0x7FFFFFFFLL) return FP8Q_ERR_SHAPE;
    if (k > 0 && (ld_bs < k / 128 || !scale_span_ok(n / 128, ld_bs))) return FP8Q_ERR_SHAPE;
    // the experts' weights are only read: their rows may interleave
    if (stride_b < 0 || stride_bs < 0) return FP8Q_ERR_SHAPE;
    if (stride_b % 16 != 0) return FP8Q_ERR_ALIGN;
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return FP8Q_ERR_ALIGN;
    if (!grid_ok((m_total / 128) * ((n + 255) / 256) + 256)) return FP8Q_ERR_SHAPE;
    if (debug_checks()) {
        st = check_segments_on_host(groups, group_offsets, group_rows, m_total, stream);
        if (st != FP8Q_OK) return st;
    }
    fp8q::GemmProblem g = {};
    g.m = m_total; g.n = n; g.k = k;
    g.a = a; g.lda = lda; g.a_scale = a_scale; g.ld_as = ld_as;
    g.b = b; g.ldb = ldb; g.b_scale = b_scale; g.ld_bs = ld_bs;
    g.b_rowscale = false;
    g.c = c; g.ldc = ldc; g.out_f32 = out_dtype == FP8Q_OUT_F32;
    g.groups = groups; g.group_offsets = group_offsets; g.group_rows = group_rows;
    g.stride_b = stride_b; g.stride_bs = stride_bs;
    if (scratch) {
        const hipError_t e = fp8q::grouped_scratch(&workspace);
        if (e != hipSuccess) return hip_status(e);
        workspace_bytes = FP8Q_GROUPED_WORKSPACE_BYTES;
    }
    g.workspace = workspace; g.workspace_bytes = workspace ? workspace_bytes : 0;
    return hip_status(fp8q::launch_grouped_gemm(g, stream));
}

int fp8_grouped_gemm(int32_t groups, const int32_t* group_offsets, const int32_t* group_rows,
                     int64_t m_total, int64_t n, int64_t k,
                     const uint8_t* a, int64_t lda, const float* a_scale, int64_t ld_as,
                     const uint8_t* b, int64_t ldb, int64_t stride_b,
                     const float* b_scale, int64_t ld_bs, int64_t stride_bs,
                     void* c, int64_t ldc, int out_dtype,
                     void* workspace, int64_t workspace_bytes, hipStream_t stream) {
    return grouped_gemm(groups, group_offsets, group_rows, m_total, n, k, a, lda, a_scale, ld_as, b, ldb, stride_b,
                        b_scale, ld_bs, stride_bs, c, ldc, out_dtype, workspace, workspace_bytes, false, stream);
}

int fp8_grouped_gemm_noalloc(int32_t groups, const int32_t* group_offsets, const int32_t* group_rows,
                             int64_t m_total, int64_t n, int64_t k,
                             const uint8_t* a, int64_t lda, const float* a_scale, int64_t ld_as,
                             const uint8_t* b, int64_t ldb, int64_t stride_b,
                             const float* b_scale, int64_t ld_bs, int64_t stride_bs,
                             void* c, int64_t ldc, int out_dtype, hipStream_t stream) {
    return grouped_gemm(groups, group_offsets, group_rows, m_total, n, k, a, lda, a_scale, ld_as, b, ldb, stride_b,
                        b_scale, ld_bs, stride_bs, c, ldc, out_dtype, nullptr, 0, true, stream);
}

int fp8_grouped_gemm_wgrad(int32_t groups, const int32_t* group_offsets, int64_t k_total,
                           int64_t m, int64_t n,
                           const uint8_t* a, int64_t lda, const float* a_scale, int64_t ld_as,
                           const uint8_t* b, int64_t ldb, const float* b_scale, int64_t ld_bs,
                           void* c, int64_t ldc, int64_t stride_c, int out_dtype, hipStream_t stream) {
    if (groups < 0 || k_total < 0 || m < 0 || n < 0) return FP8Q_ERR_SHAPE;
    if (out_dtype != FP8Q_OUT_BF16 && out_dtype != FP8Q_OUT_F32) return FP8Q_ERR_ENUM;
    if (groups == 0 || m == 0 || n == 0) return FP8Q_OK;
    if (!group_offsets) return FP8Q_ERR_NULL;
    int st = check_gemm_common(m, n, k_total, a, lda, a_scale, ld_as, b, ldb, b_scale, c, ldc, out_dtype);
    if (st != FP8Q_OK) return st;
    if (k_total > 0x7FFFFFFFLL || (k_total > 0 && (ld_bs < n || !scale_span_ok(k_total / 128, ld_bs))) ||
        stride_c < m * ldc)
        return FP8Q_ERR_SHAPE;
    if (stride_c % 8 != 0) return FP8Q_ERR_ALIGN;
    if (!grid_ok(((m + 255) / 256) * ((n + 223) / 224) * groups + 256)) return FP8Q_ERR_SHAPE;
    if (debug_checks()) {
        st = check_segments_on_host(groups, group_offsets, nullptr, k_total, stream);
        if (st != FP8Q_OK) return st;
    }
    fp8q::GemmProblem g = {};
    g.m = m; g.n = n; g.k = k_total;
    g.a = a; g.lda = lda; g.a_scale = a_scale; g.ld_as = ld_as;
    g.b = b; g.ldb = ldb; g.b_scale = b_scale; g.ld_bs = ld_bs;
    g.b_rowscale = true;
    g.c = c; g.ldc = ldc; g.out_f32 = out_dtype == FP8Q_OUT_F32;
    g.groups = groups; g.group_offsets = group_offsets;
    g.stride_c = stride_c;
    return hip_status(fp8q::launch_grouped_k_gemm(g, stream));
}

int fp8_quantize_mx(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q,
                    int64_t ld_q, uint32_t* scale, int64_t ld_s, hipStream_t stream) {
    if (rows < 0 || cols < 0) return FP8Q_ERR_SHAPE;
    if (rows == 0 || cols == 0) return FP8Q_OK;
    if (!x || !q || !scale) return FP8Q_ERR_NULL;
    if (cols % 128 != 0 || ld_x < cols || ld_q < cols || ld_s < rows) return FP8Q_ERR_SHAPE;
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(scale, 4) || ld_x % 8 != 0 || ld_q % 16 != 0)
        return FP8Q_ERR_ALIGN;
    if (!grid_ok((rows + 15) / 16 * (cols / 128) / 4 + 1)) return FP8Q_ERR_SHAPE;
    return hip_status(fp8q::launch_quant_mx(x, rows, cols, ld_x, q, ld_q, scale, ld_s, stream));
}

int fp8_quantize_mx_pair(const uint16_t* x0, int64_t rows0, int64_t cols0, int64_t ld_x0, uint8_t* q0,
                         int64_t ld_q0, uint32_t* scale0, int64_t ld_s0, const uint16_t* x1, int64_t rows1,
                         int64_t cols1, int64_t ld_x1, uint8_t* q1, int64_t ld_q1, uint32_t* scale1,
                         int64_t ld_s1, hipStream_t stream) {
    // the checks of fp8_quantize_mx on each matrix
    if (rows0 < 0 || cols0 < 0 || rows1 < 0 || cols1 < 0) return FP8Q_ERR_SHAPE;
    const uint16_t* xs[2] = {x0, x1};
    uint8_t* qs[2] = {q0, q1};
    uint32_t* ss[2] = {scale0, scale1};
    const int64_t rows[2] = {rows0, rows1}, cols[2] = {cols0, cols1}, ld_x[2] = {ld_x0, ld_x1},
                  ld_q[2] = {ld_q0, ld_q1}, ld_s[2] = {ld_s0, ld_s1};
    const bool on[2] = {rows0 > 0 && cols0 > 0, rows1 > 0 && cols1 > 0};
    for (int i = 0; i < 2; ++i) {
        if (!on[i]) continue;
        if (!xs[i] || !qs[i] || !ss[i]) return FP8Q_ERR_NULL;
        if (cols[i] % 128 != 0 || ld_x[i] < cols[i] || ld_q[i] < cols[i] || ld_s[i] < rows[i])
            return FP8Q_ERR_SHAPE;
        if (!aligned(xs[i], 16) || !aligned(qs[i], 16) || !aligned(ss[i], 4) || ld_x[i] % 8 != 0 ||
            ld_q[i] % 16 != 0)
            return FP8Q_ERR_ALIGN;
    }
    if (!on[0] && !on[1]) return FP8Q_OK;
    if (on[0] && on[1]) {
        // the two halves of the launch run concurrently: their outputs must be disjoint
        const Span o0[2] = {span(q0, rows0, cols0, ld_q0, 1), span(scale0, cols0 / 128, rows0, ld_s0, 4)};
        const Span o1[2] = {span(q1, rows1, cols1, ld_q1, 1), span(scale1, cols1 / 128, rows1, ld_s1, 4)};
        for (const Span& a : o0)
            for (const Span& b : o1)
                if (overlap(a, b)) return FP8Q_ERR_SHAPE;
    }
    int64_t blocks = 0;
    for (int i = 0; i < 2; ++i)
        if (on[i]) blocks += (rows[i] + 15) / 16 * (cols[i] / 128) / 4 + 1;
    if (!grid_ok(blocks)) return FP8Q_ERR_SHAPE;
    // an empty matrix is skipped: its block range is empty
    return hip_status(fp8q::launch_quant_mx_pair(x0, on[0] ? rows0 : 0, on[0] ? cols0 : 0, ld_x0, q0, ld_q0, scale0,
                                                 ld_s0, x1, on[1] ? rows1 : 0, on[1] ? cols1 : 0, ld_x1, q1, ld_q1,
                                                 scale1, ld_s1, stream));
}

int fp8_gemm_mx(int64_t m, int64_t n, int64_t k,
                const uint8_t* a, int64_t lda, const uint32_t* a_scale, int64_t ld_as,
                const uint8_t* b, int64_t ldb, const uint32_t* b_scale, int64_t ld_bs,
                void* c, int64_t ldc, int out_dtype, hipStream_t stream) {
    if (m < 0 || n < 0 || k < 0) return FP8Q_ERR_SHAPE;
    if (out_dtype != FP8Q_OUT_BF16 && out_dtype != FP8Q_OUT_F32) return FP8Q_ERR_ENUM;
    if (m == 0 || n == 0) return FP8Q_OK;
    const float* as = reinterpret_cast<const float*>(a_scale);
    const float* bs = reinterpret_cast<const float*>(b_scale);
    int st = check_gemm_common(m, n, k, a, lda, as, ld_as, b, ldb, bs, c, ldc, out_dtype);
    if (st != FP8Q_OK) return st;
    if (k > 0 && (ld_bs < n || !scale_span_ok(k / 128, ld_bs))) return FP8Q_ERR_SHAPE;
    if (!grid_ok(((m + 255) / 256) * ((n + 223) / 224) + 8)) return FP8Q_ERR_SHAPE;
    fp8q::GemmProblem g = {};
    g.m = m; g.n = n; g.k = k;
    g.a = a; g.lda = lda; g.a_scale = as; g.ld_as = ld_as;
    g.b = b; g.ldb = ldb; g.b_scale = bs; g.ld_bs = ld_bs;
    g.b_rowscale = true;
    g.c = c; g.ldc = ldc; g.out_f32 = out_dtype == FP8Q_OUT_F32;
    return hip_status(fp8q::launch_gemm_mx(g, stream));
}

int fp8_retile_act_128x1(const uint8_t* q, int64_t tokens, int64_t cols, int64_t ld_q,
                         const float* scale, int64_t ld_s, uint8_t* q_t, int64_t ld_qt,
                         float* scale_t, int64_t ld_st, hipStream_t stream) {
    if (tokens < 0 || cols < 0) return FP8Q_ERR_SHAPE;
    if (tokens == 0 || cols == 0) return FP8Q_OK;
    if (!q || !scale || !q_t || !scale_t) return FP8Q_ERR_NULL;
    if (tokens % 128 != 0 || cols % 128 != 0 || ld_q < cols || ld_s < tokens || ld_qt < tokens ||
        ld_st < cols)
        return FP8Q_ERR_SHAPE;
    if (!aligned(q, 16) || !aligned(scale, 16) || !aligned(q_t, 16) || !aligned(scale_t, 4) ||
        ld_q % 16 != 0 || ld_s % 4 != 0 || ld_qt % 16 != 0)
        return FP8Q_ERR_ALIGN;
    if (!grid_ok(tokens / 128 * (cols / 128))) return FP8Q_ERR_SHAPE;
    return hip_status(fp8q::launch_retile_128x1(q, tokens, cols, ld_q, scale, ld_s, q_t, ld_qt, scale_t,
                                                ld_st, stream));
}

int fp8_gemm_tensor(int64_t m, int64_t n, int64_t k, const uint8_t* a, int64_t lda, const float* a_scale,
                    const uint8_t* b, int64_t ldb, const float* b_scale, void* c, int64_t ldc,
                    int out_dtype, hipStream_t stream) {
    if (m < 0 || n < 0 || k < 0) return FP8Q_ERR_SHAPE;
    if (out_dtype != FP8Q_OUT_BF16 && out_dtype != FP8Q_OUT_F32) return FP8Q_ERR_ENUM;
    if (m == 0 || n == 0) return FP8Q_OK;
    // one scale per operand: the slab-major scale checks see a leading dimension of m
    int st = check_gemm_common(m, n, k, a, lda, a_scale, m, b, ldb, b_scale, c, ldc, out_dtype);
    if (st != FP8Q_OK) return st;
    if (!grid_ok(((m + 255) / 256) * ((n + 223) / 224) + 8)) return FP8Q_ERR_SHAPE;
    fp8q::GemmProblem g = {};
    g.m = m; g.n = n; g.k = k;
    g.a = a; g.lda = lda; g.a_scale = a_scale; g.ld_as = 0;
    g.b = b; g.ldb = ldb; g.b_scale = b_scale; g.ld_bs = 0;
    g.b_rowscale = true;
    g.c = c; g.ldc = ldc; g.out_f32 = out_dtype == FP8Q_OUT_F32;
    return hip_status(fp8q::launch_gemm_tensor(g, stream));
}

}  // extern "C"
