// launch.h -- host-side kernel launchers of libfp8q (internal; arguments are
// already validated by the C ABI layer in api.cpp).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace fp8q {

hipError_t launch_quant_act_1x128(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                                  uint8_t* q, int64_t ld_q, float* scale, int64_t ld_s,
                                  hipStream_t stream);

hipError_t launch_quant_act_scatter(const uint16_t* x, int64_t tokens, int64_t cols, int64_t ld_x,
                                    int topk, const int32_t* dst_rows, int64_t m_total, uint8_t* q,
                                    int64_t ld_q, float* scale, int64_t ld_s, hipStream_t stream);

hipError_t launch_quant_mx(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q,
                           int64_t ld_q, uint32_t* scale, int64_t ld_s, hipStream_t stream);

hipError_t launch_quant_mx_pair(const uint16_t* x0, int64_t rows0, int64_t cols0, int64_t ld_x0, uint8_t* q0,
                                int64_t ld_q0, uint32_t* s0, int64_t ld_s0, const uint16_t* x1, int64_t rows1,
                                int64_t cols1, int64_t ld_x1, uint8_t* q1, int64_t ld_q1, uint32_t* s1,
                                int64_t ld_s1, hipStream_t stream);
hipError_t launch_quant_act_128x1(const uint16_t* x, int64_t tokens, int64_t cols, int64_t ld_x,
                                  uint8_t* qt, int64_t ld_q, float* scale, int64_t ld_s,
                                  hipStream_t stream);
hipError_t launch_quant_act_128x1_pair(int64_t tokens, const uint16_t* x0, int64_t cols0, int64_t ld_x0,
                                       uint8_t* q0, int64_t ld_q0, float* s0, int64_t ld_s0,
                                       const uint16_t* x1, int64_t cols1, int64_t ld_x1, uint8_t* q1,
                                       int64_t ld_q1, float* s1, int64_t ld_s1, hipStream_t stream);

hipError_t launch_quant_retile_128x1(int64_t tokens, const uint16_t* x0, int64_t cols0, int64_t ld_x0,
                                     uint8_t* q0, int64_t ld_q0, float* s0, int64_t ld_s0, const uint8_t* xq,
                                     int64_t cols1, int64_t ld_xq, const float* xs, int64_t ld_xs, uint8_t* q1,
                                     int64_t ld_q1, float* s1, int64_t ld_s1, hipStream_t stream);
hipError_t launch_retile_128x1(const uint8_t* q, int64_t tokens, int64_t cols, int64_t ld_q,
                               const float* scale, int64_t ld_s, uint8_t* qt, int64_t ld_qt,
                               float* scale_t, int64_t ld_st, hipStream_t stream);

// 1x128 activation quantization and 128x128 weight quantization (optional
// transposed copy) in one launch.
hipError_t launch_quant_act_weight(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q,
                                   int64_t ld_q, float* scale, int64_t ld_s, const uint16_t* w, int64_t n,
                                   int64_t k, int64_t ld_w, uint8_t* wq, int64_t ld_wq, float* ws, int64_t ld_ws,
                                   uint8_t* wq_t, int64_t ld_wqt, float* ws_t, int64_t ld_wst,
                                   hipStream_t stream);

// groups weight matrices, group e at each base pointer + e * its stride
// (elements); groups == 1 with zero strides is one matrix.
hipError_t launch_quant_weight(int64_t groups, const uint16_t* w, int64_t n, int64_t k, int64_t ld_w,
                               int64_t stride_w, uint8_t* q, int64_t ld_q, int64_t stride_q, float* scale,
                               int64_t ld_s, int64_t stride_s, uint8_t* q_t, int64_t ld_qt, int64_t stride_qt,
                               float* scale_t, int64_t ld_st, int64_t stride_st, hipStream_t stream);

struct GemmProblem {
    int64_t m, n, k;
    const uint8_t* a;
    int64_t lda;
    const float* a_scale;
    int64_t ld_as;
    const uint8_t* b;
    int64_t ldb;
    const float* b_scale;
    int64_t ld_bs;
    bool b_rowscale;  // false: 128x128 blocks, true: per (slab, row)
    void* c;
    int64_t ldc;
    bool out_f32;
    // grouped (MoE) problems only
    int32_t groups;
    const int32_t* group_offsets;
    const int32_t* group_rows;
    int64_t stride_b;
    int64_t stride_bs;
    int64_t stride_c;  // grouped over K: elements between expert outputs
    // grouped over M: the caller's workspace for a K-split last round of
    // tiles (NULL or too small: no split)
    void* workspace;
    int64_t workspace_bytes;
};

hipError_t launch_gemm(const GemmProblem& p, hipStream_t stream);
hipError_t launch_grouped_gemm(const GemmProblem& p, hipStream_t stream);
// Device address of the library's grouped-GEMM scratch on the current device
// (FP8Q_GROUPED_WORKSPACE_BYTES), looked up once per device.
hipError_t grouped_scratch(void** ptr);
hipError_t launch_grouped_k_gemm(const GemmProblem& p, hipStream_t stream);
hipError_t launch_gemm_mx(const GemmProblem& p, hipStream_t stream);
hipError_t launch_gemm_tensor(const GemmProblem& p, hipStream_t stream);

}  // namespace fp8q
