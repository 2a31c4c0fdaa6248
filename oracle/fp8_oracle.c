/*
 * fp8_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, scalar CPU oracle for fine-grained FP8 quantization. Only the
 * tests, the smoke check and the benchmark's CPU-baseline leg may load it. It
 * shares no code, header, table or constant with the GPU library, and the GPU
 * library never calls it.
 *
 * What it computes (the fine-grained quantization of the DeepSeek-V3 FP8
 * framework as quoted on the pages):
 *   - every GEMM operand is E4M3 (4 exponent bits, 3 mantissa bits) -- page
 *     "Deepseek Ai News Expert Interview", passage adopting E4M3 on all tensors;
 *   - activations are scaled per 1x128 tile (one token, 128 channels) and
 *     weights per 128x128 block (128 input x 128 output channels) -- page
 *     dssusan.co.kr (Q&A board), passage on Figure 7(a);
 *   - each group shares one exponent through its scale -- page "Deepseek Ai
 *     News Expert Interview", passage on smaller element groups.
 * Readings where the pages are silent:
 *   - the E4M3 variant is OCP E4M3FN: bias 7, no infinities, 0x7F/0xFF are NaN,
 *     largest finite value 448;
 *   - scale s = fl32(amax / 448), an IEEE single-precision division;
 *   - q = E4M3(fl32(x / s)), an IEEE single division, then round to nearest,
 *     ties to the even code, saturating at +-448 (|v| >= 464 -> 448);
 *   - an all-zero tile stores s = 0 and encodes each element as signed zero;
 *   - the sign of the code is the sign of x (so -0 and negative values that
 *     round to zero give 0x80);
 *   - the Wgrad operands use 128x1 tiles along the token dimension.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC.
 * Float arithmetic here is IEEE binary32 (SSE, FLT_EVAL_METHOD == 0); no
 * flush-to-zero mode is set, so bf16/fp32 subnormals are honoured.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ---------------------------------------------------------------- formats */

/* bf16 bit pattern -> float: the 16 bits are the top half of a binary32. */
float oracle_bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* E4M3 (OCP E4M3FN) code -> value, from the format definition.
 * sign s = bit 7, exponent e = bits 6..3 (bias 7), mantissa m = bits 2..0.
 * e == 0: (-1)^s * m * 2^-9 (subnormal); e == 15 && m == 7: NaN;
 * otherwise (-1)^s * (1 + m/8) * 2^(e-7). */
double oracle_e4m3_decode(uint8_t code) {
    int s = code >> 7, e = (code >> 3) & 0xF, m = code & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -v : v;
}

/* Encoder 1: bit arithmetic on the binary32 fields.
 * Rounds |v| to a whole number of target ulps with round-half-even on the
 * dropped significand bits, then packs exponent and mantissa. */
uint8_t oracle_e4m3_encode_bits(float v) {
    uint32_t u;
    memcpy(&u, &v, sizeof u);
    uint8_t sign = (uint8_t)((u >> 31) << 7);
    uint32_t a = u & 0x7FFFFFFFu;
    if (a >= 0x43E80000u) /* |v| >= 464: past the last rounding midpoint */
        return sign | 0x7E;
    int biased = (int)(a >> 23);
    uint64_t sig = (a & 0x7FFFFFu) | (biased ? 0x800000u : 0u); /* |v| = sig * 2^(ue-23) */
    int ue = biased ? biased - 127 : -126;
    int target_ulp_exp = (ue >= -6 ? ue : -6) - 3; /* E4M3 normals hold 3 fraction bits */
    int shift = target_ulp_exp - (ue - 23);         /* >= 20 */
    uint64_t q;
    if (shift >= 40) {
        q = 0; /* far below half of the smallest subnormal */
    } else {
        uint64_t half = (uint64_t)1 << (shift - 1);
        uint64_t rem = sig & (((uint64_t)1 << shift) - 1);
        q = sig >> shift;
        if (rem > half || (rem == half && (q & 1))) q++;
    }
    if (ue >= -6) {           /* normal target: q in [8, 16] */
        int e = ue + 7;
        if (q == 16) { e++; q = 8; }
        return sign | (uint8_t)(e << 3) | (uint8_t)(q - 8);
    }
    return sign | (uint8_t)q; /* subnormal target: q in [0, 8]; 8 is 0x08 */
}

/* Encoder 2: nearest-value search over the sorted non-negative finite codes
 * 0x00..0x7E (their values increase with the code). Ties go to the even code;
 * anything above 448 is nearest to 448, which gives saturation for free. */
uint8_t oracle_e4m3_encode_search(float v) {
    double a = fabs((double)v);
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    int lo = 0, hi = 0x7E; /* find the last code with value <= a */
    if (a >= oracle_e4m3_decode(0x7E)) return sign | 0x7E;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (oracle_e4m3_decode((uint8_t)mid) <= a) lo = mid; else hi = mid - 1;
    }
    double dlo = a - oracle_e4m3_decode((uint8_t)lo);
    double dhi = oracle_e4m3_decode((uint8_t)(lo + 1)) - a;
    int best;
    if (dlo < dhi) best = lo;
    else if (dhi < dlo) best = lo + 1;
    else best = (lo % 2 == 0) ? lo : lo + 1;
    return sign | (uint8_t)best;
}

/* ------------------------------------------------------------ quantizers */

/* One group: amax = max |x|, s = fl32(amax / 448), q = E4M3(fl32(x / s)). */
static float group_scale(float amax) { return amax / 448.0f; }

static uint8_t quantize_value(float x, float amax, float s) {
    if (amax == 0.0f) return oracle_e4m3_encode_bits(x); /* x is +-0 */
    return oracle_e4m3_encode_bits(x / s);
}

/* 1x128 tiles (per token per 128 channels).
 * x[rows][ldx] bf16; q[rows][ldq]; scale[cols/128][lds] (slab-major).
 * cols must be a multiple of 128. */
void oracle_quant_act_1x128(const uint16_t *x, int64_t rows, int64_t cols, int64_t ldx,
                            uint8_t *q, int64_t ldq, float *scale, int64_t lds) {
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t j = 0; j < cols / 128; j++) {
            const uint16_t *tile = x + r * ldx + j * 128;
            float amax = 0.0f;
            for (int i = 0; i < 128; i++) {
                float a = fabsf(oracle_bf16_to_f32(tile[i]));
                if (a > amax) amax = a;
            }
            float s = group_scale(amax);
            scale[j * lds + r] = s;
            for (int i = 0; i < 128; i++)
                q[r * ldq + j * 128 + i] = quantize_value(oracle_bf16_to_f32(tile[i]), amax, s);
        }
    }
}

/* 128x1 tiles along tokens (Wgrad operands).
 * x[rows=tokens][ldx] bf16; output is token-contiguous: qt[cols][ldqt];
 * scale[rows/128][lds]. rows must be a multiple of 128. */
void oracle_quant_act_128x1(const uint16_t *x, int64_t rows, int64_t cols, int64_t ldx,
                            uint8_t *qt, int64_t ldqt, float *scale, int64_t lds) {
    #pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cols; c++) {
        for (int64_t j = 0; j < rows / 128; j++) {
            float amax = 0.0f;
            for (int i = 0; i < 128; i++) {
                float a = fabsf(oracle_bf16_to_f32(x[(j * 128 + i) * ldx + c]));
                if (a > amax) amax = a;
            }
            float s = group_scale(amax);
            scale[j * lds + c] = s;
            for (int i = 0; i < 128; i++)
                qt[c * ldqt + j * 128 + i] =
                    quantize_value(oracle_bf16_to_f32(x[(j * 128 + i) * ldx + c]), amax, s);
        }
    }
}

/* 128x128 blocks (per 128 output channels per 128 input channels).
 * w[n][ldw] bf16; q[n][ldq]; scale[n/128][lds]. n and k multiples of 128. */
void oracle_quant_weight_128x128(const uint16_t *w, int64_t n, int64_t k, int64_t ldw,
                                 uint8_t *q, int64_t ldq, float *scale, int64_t lds) {
    #pragma omp parallel for collapse(2) schedule(static)
    for (int64_t bn = 0; bn < n / 128; bn++) {
        for (int64_t bk = 0; bk < k / 128; bk++) {
            float amax = 0.0f;
            for (int i = 0; i < 128; i++)
                for (int jj = 0; jj < 128; jj++) {
                    float a = fabsf(oracle_bf16_to_f32(w[(bn * 128 + i) * ldw + bk * 128 + jj]));
                    if (a > amax) amax = a;
                }
            float s = group_scale(amax);
            scale[bn * lds + bk] = s;
            for (int i = 0; i < 128; i++)
                for (int jj = 0; jj < 128; jj++) {
                    int64_t idx = (bn * 128 + i) * ldw + bk * 128 + jj;
                    q[(bn * 128 + i) * ldq + bk * 128 + jj] =
                        quantize_value(oracle_bf16_to_f32(w[idx]), amax, s);
                }
        }
    }
}

/* ------------------------------------------------ FP8 activation cache */

/* A cached FP8 activation re-tiled for Wgrad. The FP8 Wgrad GEMM lets the
 * forward activations be kept in FP8 for the backward pass (page "Is aI
 * Hitting a Wall?", passage on storing activations in FP8 for the backward
 * pass), but Wgrad wants 128x1 tiles along tokens while the forward pass
 * made 1x128 tiles. Reading: each cached value is dequantized to binary32,
 * v = fl32(dec(q) * s), and the values are quantized again in 128x1 tiles
 * exactly as oracle_quant_act_128x1 quantizes bf16 input.
 * q[rows=tokens][ldq] with scale[cols/128][lds] (1x128, slab-major) ->
 * qt[cols][ldqt] (token-contiguous) with scale_t[rows/128][ldst].
 * rows and cols must be multiples of 128. */
void oracle_retile_128x1(const uint8_t *q, int64_t rows, int64_t cols, int64_t ldq,
                         const float *scale, int64_t lds, uint8_t *qt, int64_t ldqt,
                         float *scale_t, int64_t ldst) {
    #pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cols; c++) {
        float v[128];
        for (int64_t j = 0; j < rows / 128; j++) {
            float amax = 0.0f;
            for (int i = 0; i < 128; i++) {
                int64_t r = j * 128 + i;
                float d = (float)oracle_e4m3_decode(q[r * ldq + c]); /* exact in binary32 */
                v[i] = d * scale[(c / 128) * lds + r];
                float a = fabsf(v[i]);
                if (a > amax) amax = a;
            }
            float s = group_scale(amax);
            scale_t[j * ldst + c] = s;
            for (int i = 0; i < 128; i++) qt[c * ldqt + j * 128 + i] = quantize_value(v[i], amax, s);
        }
    }
}

/* ------------------------------------------------------- self-check helpers */

/* Agreement of the two encoders over the binary32 bit patterns lo_bits,
 * lo_bits + stride, ... <= hi_bits (both signs; stride 1 is exhaustive).
 * Returns the number of disagreements and the smallest disagreeing pattern in
 * *first_bad (or 0xFFFFFFFF). */
int64_t oracle_encoders_disagree(uint32_t lo_bits, uint32_t hi_bits, uint32_t stride,
                                 uint32_t *first_bad) {
    int64_t bad = 0;
    uint32_t first = 0xFFFFFFFFu;
    #pragma omp parallel for reduction(+ : bad) schedule(static, 4096)
    for (int64_t b = lo_bits; b <= (int64_t)hi_bits; b += stride) {
        for (int sgn = 0; sgn < 2; sgn++) {
            uint32_t u = (uint32_t)b | ((uint32_t)sgn << 31);
            float v;
            memcpy(&v, &u, sizeof v);
            if (oracle_e4m3_encode_bits(v) != oracle_e4m3_encode_search(v)) {
                bad++;
                #pragma omp critical
                { if (u < first) first = u; }
            }
        }
    }
    *first_bad = first;
    return bad;
}

/* Element-wise scalar quantization of given (x, amax) bf16 pairs, used by the
 * exhaustive (x, amax) sweep: q[i] = E4M3(fl32(x[i] / fl32(amax[i] / 448))). */
void oracle_quant_pairs(const uint16_t *x, const uint16_t *amax, int64_t count, uint8_t *q) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; i++) {
        float a = fabsf(oracle_bf16_to_f32(amax[i]));
        q[i] = quantize_value(oracle_bf16_to_f32(x[i]), a, group_scale(a));
    }
}

/* ------------------------------------------------------------ microscaling */

/* The microscaling variant (page "Deepseek Ai News Expert Interview", passage
 * likening the fine-grained groups to microscaling formats with smaller
 * quantization granularity): blocks of 32 consecutive elements along a row
 * share one power-of-two scale X = 2^e, stored as an E8M0 byte e + 127.
 * Readings (OCP MX, FP8 E4M3 elements): e = floor(log2(amax)) - 8, where 8
 * is the exponent of E4M3's largest normal (448 = 1.75 * 2^8), clamped to
 * [-127, 127]; an all-zero block takes e = -127. Each element is
 * E4M3_RNE_sat(x / X); the division by a power of two is done exactly (in
 * double) before the single rounding to E4M3. */
static int mx_exponent(float amax) {
    if (amax == 0.0f) return -127;
    int ex;
    (void)frexp((double)amax, &ex);   /* amax = m * 2^ex, m in [0.5, 1) */
    int e = (ex - 1) - 8;             /* floor(log2(amax)) - 8 */
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/* x[rows][ldx] bf16, cols % 32 == 0 -> q[rows][ldq], e8m0[rows][lde]
 * (byte b of row r is the exponent byte of columns [32b, 32b + 32)). */
void oracle_quant_mx_1x32(const uint16_t *x, int64_t rows, int64_t cols, int64_t ldx,
                          uint8_t *q, int64_t ldq, uint8_t *e8m0, int64_t lde) {
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t b = 0; b < cols / 32; b++) {
            const uint16_t *blk = x + r * ldx + b * 32;
            float amax = 0.0f;
            for (int i = 0; i < 32; i++) {
                float a = fabsf(oracle_bf16_to_f32(blk[i]));
                if (a > amax) amax = a;
            }
            int e = mx_exponent(amax);
            e8m0[r * lde + b] = (uint8_t)(e + 127);
            for (int i = 0; i < 32; i++) {
                float v = (float)ldexp((double)oracle_bf16_to_f32(blk[i]), -e);
                q[r * ldq + b * 32 + i] = oracle_e4m3_encode_bits(v);
            }
        }
    }
}
