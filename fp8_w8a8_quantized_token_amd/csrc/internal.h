// Internal declarations shared by the HIP translation units of libfp8w8a8.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8w8a8.h"

namespace fp8w8a8 {

// Launch the per-row quantiser: q[r, :] = e4m3fn(x[r, :] / s[r]), s[r] = amax_r / 448.
// Arguments are already validated (cols % 16 == 0, 16-byte aligned pointers, rows > 0).
hipError_t launch_quant_rows(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* q, float* scale,
                             hipStream_t stream);

// Build the 65536-entry bf16 -> bf16 table of activation `act` (FP8W8A8_ACT_*).
hipError_t launch_act_table(int act, uint16_t* table, hipStream_t stream);

// y = table[x] elementwise over `elems` bf16 values (elems % 16 == 0, 16-byte aligned).
hipError_t launch_act_rows(const uint16_t* x, int64_t elems, const uint16_t* table, uint16_t* y, int cus,
                           hipStream_t stream);

// The fused producer: per-token quantisation of table[x] (same arguments as launch_quant_rows).
hipError_t launch_act_quant_rows(const uint16_t* x, int64_t rows, int64_t cols, const uint16_t* table, uint8_t* q,
                                 float* scale, int cus, hipStream_t stream);

// Per-tensor quantisation (per-workgroup maxima into `workspace`, then the codes and the
// scale) and fp32 dequantisation; numel % 16 == 0, 16-byte aligned buffers. form: one of
// kTensor* (FP8W8A8_TENSOR_FORM_*); a one-pass form on a tensor that does not fit gives
// hipErrorInvalidValue.
constexpr int kTensorAuto = 0, kTensorOnePass = 1, kTensorTwoPass = 2, kTensorOnePassNoWait = 3;
size_t quant_tensor_workspace_bytes();
bool quant_tensor_fits_one_pass(int64_t numel, int cus);
hipError_t launch_quant_tensor(const uint16_t* x, int64_t numel, int fmt, uint8_t* q, float* scale, float* workspace,
                               int cus, hipStream_t stream, int form = kTensorAuto);
hipError_t launch_dequant_tensor(const uint8_t* q, int64_t numel, int fmt, const float* scale, float* out, int cus,
                                 hipStream_t stream);

// One compiled GEMM kernel configuration.
struct GemmConfig {
  int id;
  int tile_m;   // block rows along m (activation rows)
  int tile_n;   // block columns along n (weight rows / output channels)
  int waves;    // 64-lane wavefronts per workgroup
  int stages;   // LDS pipeline depth (128 bytes of k per stage)
  const char* name;
};

int gemm_config_count();
const GemmConfig* gemm_config(int id);

// Workgroups a configuration launches for an m x n output, and threads per workgroup.
int64_t gemm_workgroups(int id, int64_t m, int64_t n);
int gemm_threads(int id);

// Launch configuration `id` for out[m, n] = epilogue(qa[m, k] x qw[n, k]^T). cus: the
// device's compute units (sizes the grid of the persistent configuration).
hipError_t launch_gemm(int id, int64_t m, int64_t n, int64_t k, const uint8_t* qa, const float* a_scale,
                       const uint8_t* qw, const float* w_scale, const uint16_t* bias, uint16_t* out, int cus,
                       hipStream_t stream);

// Configuration `id` (6, persistent; or 5, skinny) over up to FP8W8A8_MAX_GROUP problems
// that share the activation codes qa [m, k] and scales: problem p is out_p[m, n_p] =
// epilogue(qa x qw_p^T), all in one launch (the problems' column blocks side by side).
struct GroupProblem {
  const uint8_t* qw;
  const float* w_scale;
  const uint16_t* bias;
  uint16_t* out;
  int64_t n;
};
hipError_t launch_gemm_group(int id, int64_t m, int64_t k, const uint8_t* qa, const float* a_scale, int nprob,
                             const GroupProblem* probs, int cus, hipStream_t stream);

// Per-token quantisation and the FP8 GEMM (configuration 0) in one launch. qa_ws [m, k]
// and sa_ws [m] receive the codes and scales (as launch_quant_rows writes them); flags
// holds kQuantGemmMaxWorkgroups 64-bit words of any prior content; epoch must differ
// from every epoch used before with the same flags. cus: the device's compute units
// (one share of the tokens per workgroup of the first wave).
constexpr int kQuantGemmMaxWorkgroups = 1024;
hipError_t launch_quant_gemm(int64_t m, int64_t n, int64_t k, const uint16_t* a_bf16, uint8_t* qa_ws, float* sa_ws,
                             unsigned long long* flags, unsigned long long epoch, const uint8_t* qw,
                             const float* w_scale, const uint16_t* bias, uint16_t* out, int cus, hipStream_t stream);

// The FP8 weight-only (W8A16) GEMM: out[m, n] = bf16(sum_k a[m, k] dec(qw[n, k]) * w_scale[n] + bias[n]).
int w8a16_config_count();
const GemmConfig* w8a16_config(int id);
int64_t w8a16_workgroups(int id, int64_t m, int64_t n);
int w8a16_threads(int id);
// w_format: FP8W8A8_FMT_E4M3FN or FP8W8A8_FMT_E5M2 codes in qw.
hipError_t launch_w8a16(int id, int w_format, int64_t m, int64_t n, int64_t k, const uint16_t* a, const uint8_t* qw,
                        const float* w_scale, const uint16_t* bias, uint16_t* out, hipStream_t stream);

}  // namespace fp8w8a8
