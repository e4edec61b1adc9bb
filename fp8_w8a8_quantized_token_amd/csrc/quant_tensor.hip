// Per-tensor FP8 quantisation (e4m3fn or e5m2) and fp32 dequantisation for gfx950.
//
// The state-dict converter of the QuantizeFP8Format page (runcomfy.com, "Quantize
// Model to FP8 Format") turns each tensor into float8_e4m3fn or float8_e5m2 by
// scaling it (no formula given); the Stable Diffusion 3.5 FP8 page (dn008.com.cn, section
// on FP8, steps 1-4) spells the steps out: the largest magnitude, a scale, x / scale
// rounded to the 8-bit format, and x_q * scale back in fp32. One scale per tensor:
//
//   s  = fl32(amax / fmax)        fmax = 448 (e4m3fn) or 57344 (e5m2); 0 for a zero tensor
//   q  = rne_sat(fl32(x / s))     signed-zero codes when s == 0
//   x' = fl32(dec(q) * s)
//
// Two launches, no atomics and no memset (so a captured graph replays them as they
// are): amax_partials writes one maximum per workgroup into the caller's workspace;
// quant_tensor reduces those partials in every workgroup (at most 1024 values, one
// LDS pass), derives s, writes it once, and quantises its grid-stride share. e4m3fn
// quotients reuse the per-token quantiser's arithmetic (quant_row.h, including its
// divide-free fast path); e5m2 quotients take an IEEE division, since its subnormal
// range reaches quotients below the fast path's proven range. v_cvt_pk_bf8_f32 /
// v_cvt_pk_fp8_f32 round to nearest even into the OCP encodings; quotients never
// exceed fmax * (1 + 2^-23), which both round to fmax. Dequantisation converts codes
// exactly with v_cvt_pk_f32_{fp8,bf8} and multiplies once in fp32.
#include "internal.h"
#include "quant_row.h"

namespace fp8w8a8 {
namespace {

constexpr int kBlock = 256;
typedef unsigned v4u32 __attribute__((ext_vector_type(4)));
constexpr int kMaxPartials = 1024;

__device__ __forceinline__ uint32_t pack4_bf8(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
  return static_cast<uint32_t>(w);
}

// 16 bf16 (two uint4) -> 16 e5m2 codes: IEEE quotient (or the value itself when s == 0)
__device__ __forceinline__ uint4 quant16_e5m2(const uint4& a, const uint4& b, float s, bool zero) {
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t u0 = w[2 * i], u1 = w[2 * i + 1];
    const float x0 = qrow::bf16_lo(u0), x1 = qrow::bf16_hi(u0), x2 = qrow::bf16_lo(u1), x3 = qrow::bf16_hi(u1);
    o[i] = zero ? pack4_bf8(x0, x1, x2, x3) : pack4_bf8(x0 / s, x1 / s, x2 / s, x3 / s);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

__device__ __forceinline__ float block_max(float v, float* red) {
  v = qrow::wave_max(v);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < kBlock / 64; ++i) m = fmaxf(m, red[i]);
  return m;
}

// One maximum |x| per workgroup over a grid-stride share of 8-element groups.
__global__ __launch_bounds__(kBlock) void amax_partials(const uint4* __restrict__ x, int64_t n8,
                                                        float* __restrict__ partials) {
  __shared__ float red[kBlock / 64];
  float m = 0.0f;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < n8; i += stride) {
    const uint4 v = x[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) m = fmaxf(m, fmaxf(fabsf(qrow::bf16_lo(w[j])), fabsf(qrow::bf16_hi(w[j]))));
  }
  m = block_max(m, red);
  if (threadIdx.x == 0) partials[blockIdx.x] = m;
}

template <int FMT>
__global__ __launch_bounds__(kBlock) void quant_tensor_kernel(const uint4* __restrict__ x, int64_t n16,
                                                              const float* __restrict__ partials, int nparts,
                                                              uint4* __restrict__ q, float* __restrict__ scale_out) {
  __shared__ float red[kBlock / 64];
  float m = 0.0f;
  for (int i = threadIdx.x; i < nparts; i += kBlock) m = fmaxf(m, partials[i]);
  const float amax = block_max(m, red);
  const float s = amax / (FMT == FP8W8A8_FMT_E5M2 ? 57344.0f : 448.0f);
  if (blockIdx.x == 0 && threadIdx.x == 0) *scale_out = s;
  const float r = 1.0f / s;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < n16; i += stride) {
    const uint4 a = x[2 * i], b = x[2 * i + 1];
    uint4 o;
    if constexpr (FMT == FP8W8A8_FMT_E5M2) {
      o = quant16_e5m2(a, b, s, amax == 0.0f);
    } else {
      if (amax >= qrow::kTinyAmax)
        o = qrow::quant16<qrow::Mode::kFast>(a, b, s, r);
      else if (amax == 0.0f)
        o = qrow::quant16<qrow::Mode::kZero>(a, b, s, r);
      else
        o = qrow::quant16<qrow::Mode::kExact>(a, b, s, r);
    }
    // non-temporal: the codes are not read again here (8192 x 2048: 19.1 -> 18.2 us)
    __builtin_nontemporal_store((v4u32){o.x, o.y, o.z, o.w}, reinterpret_cast<v4u32*>(q + i));
  }
}

// 4 codes (one dword) -> 4 fp32 values, exactly
template <int FMT>
__device__ __forceinline__ float4 decode4(uint32_t w) {
  if constexpr (FMT == FP8W8A8_FMT_E5M2) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_bf8(static_cast<int>(w), false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_bf8(static_cast<int>(w), true);
    return make_float4(lo[0], lo[1], hi[0], hi[1]);
  } else {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
    return make_float4(lo[0], lo[1], hi[0], hi[1]);
  }
}

template <int FMT>
__global__ __launch_bounds__(kBlock) void dequant_tensor_kernel(const uint4* __restrict__ q, int64_t n16,
                                                                const float* __restrict__ scale,
                                                                float4* __restrict__ out) {
  const float s = *scale;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < n16; i += stride) {
    const uint4 v = q[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 d = decode4<FMT>(w[j]);
      out[4 * i + j] = make_float4(d.x * s, d.y * s, d.z * s, d.w * s);
    }
  }
}

int grid_for(int64_t items, int cap) {
  const int64_t need = (items + kBlock - 1) / kBlock;
  return static_cast<int>(need < cap ? (need > 0 ? need : 1) : cap);
}

}  // namespace

size_t quant_tensor_workspace_bytes() { return kMaxPartials * sizeof(float); }

hipError_t launch_quant_tensor(const uint16_t* x, int64_t numel, int fmt, uint8_t* q, float* scale, float* workspace,
                               int cus, hipStream_t stream) {
  const int64_t n8 = numel / 8, n16 = numel / 16;
  const int nparts = grid_for((n8 + 3) / 4, kMaxPartials);  // at least 4 groups per thread
  amax_partials<<<nparts, kBlock, 0, stream>>>(reinterpret_cast<const uint4*>(x), n8, workspace);
  const int nq = grid_for(n16, 8 * cus);
  if (fmt == FP8W8A8_FMT_E5M2)
    quant_tensor_kernel<FP8W8A8_FMT_E5M2><<<nq, kBlock, 0, stream>>>(reinterpret_cast<const uint4*>(x), n16, workspace,
                                                                     nparts, reinterpret_cast<uint4*>(q), scale);
  else
    quant_tensor_kernel<FP8W8A8_FMT_E4M3FN><<<nq, kBlock, 0, stream>>>(reinterpret_cast<const uint4*>(x), n16,
                                                                       workspace, nparts, reinterpret_cast<uint4*>(q),
                                                                       scale);
  return hipGetLastError();
}

hipError_t launch_dequant_tensor(const uint8_t* q, int64_t numel, int fmt, const float* scale, float* out, int cus,
                                 hipStream_t stream) {
  const int64_t n16 = numel / 16;
  const int nb = grid_for(n16, 8 * cus);
  if (fmt == FP8W8A8_FMT_E5M2)
    dequant_tensor_kernel<FP8W8A8_FMT_E5M2><<<nb, kBlock, 0, stream>>>(reinterpret_cast<const uint4*>(q), n16, scale,
                                                                       reinterpret_cast<float4*>(out));
  else
    dequant_tensor_kernel<FP8W8A8_FMT_E4M3FN><<<nb, kBlock, 0, stream>>>(reinterpret_cast<const uint4*>(q), n16,
                                                                         scale, reinterpret_cast<float4*>(out));
  return hipGetLastError();
}

}  // namespace fp8w8a8
