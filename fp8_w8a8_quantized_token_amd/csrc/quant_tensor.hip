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
// Two forms, each two launches with no memset (so a captured graph replays them as they
// are):
//   * One pass, for e4m3fn tensors that fit in the registers of one 1024-thread
//     workgroup per CU (up to 4 groups of 16 elements per thread: 32 MiB of bf16 on 256
//     CUs). A tiny
//     kernel marks the per-workgroup maxima unwritten; then every workgroup loads its
//     share into registers and publishes its maximum, workgroup 0 waits for all of them
//     (all workgroups are resident at once: one per CU) and publishes the largest, and
//     every workgroup quantises the values it holds with that. The input is read from HBM once (3 bytes per
//     element in all, against 5 for two passes).
//   * Two passes, for larger tensors: amax_partials writes one maximum per workgroup
//     into the caller's workspace; quant_tensor reduces those partials in every
//     workgroup (at most 1024 values, one LDS pass), derives s, writes it once, and
//     quantises its grid-stride share, reading the input again. Both formats form
// their quotients with the per-token quantiser's arithmetic (quant_row.h): divide-free
// from amax >= 2^-80, an IEEE division below. For the e5m2 scale fl32(amax / 57344), over
// every pair of finite bf16 values (x, amax >= 2^-80) with |x| <= amax, the divide-free
// quotient differs from fl32(x / s) only where both lie below 2^-17.03 in magnitude with
// the same sign, and every such value encodes to the same signed zero (e5m2's smallest
// subnormal is 2^-16). v_cvt_pk_bf8_f32 / v_cvt_pk_fp8_f32 round to nearest even into the
// OCP encodings and do not saturate.
// e4m3fn quotients stay below 464 (the midpoint above 448) for every bf16 pair
// (x, amax), fp32-subnormal scales included. e5m2 quotients do not: for a bf16 amax of
// 1..3 x 2^-133 the scale fl32(amax / 57344) is an fp32 subnormal of 1..3 units that
// rounded down, and amax / s = 65536 would convert to infinity; they are clamped to
// +-57344 first (which keeps the sign of -0). Dequantisation converts codes exactly
// with v_cvt_pk_f32_{fp8,bf8} and multiplies once in fp32.
#include <algorithm>

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

// Clamp a quotient to the largest finite e5m2 magnitude (57344), sign kept.
__device__ __forceinline__ float sat_e5m2(float q) { return fminf(fmaxf(q, -57344.0f), 57344.0f); }

// 16 bf16 (two uint4) -> 16 e5m2 codes, quotients formed as quant_row.h's mode M forms them
template <qrow::Mode M>
__device__ __forceinline__ uint4 quant16_e5m2(const uint4& a, const uint4& b, float s, float r) {
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t u0 = w[2 * i], u1 = w[2 * i + 1];
    o[i] = pack4_bf8(sat_e5m2(qrow::quotient<M>(qrow::bf16_lo(u0), s, r)),
                     sat_e5m2(qrow::quotient<M>(qrow::bf16_hi(u0), s, r)),
                     sat_e5m2(qrow::quotient<M>(qrow::bf16_lo(u1), s, r)),
                     sat_e5m2(qrow::quotient<M>(qrow::bf16_hi(u1), s, r)));
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

template <int NT = kBlock>
__device__ __forceinline__ float block_max(float v, float* red) {
  v = qrow::wave_max(v);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) m = fmaxf(m, red[i]);
  return m;
}

// max |x| over the 16 bf16 values of two uint4
__device__ __forceinline__ float abs_max16(const uint4& a, const uint4& b, float m) {
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int j = 0; j < 8; ++j) m = fmaxf(m, fmaxf(fabsf(qrow::bf16_lo(w[j])), fabsf(qrow::bf16_hi(w[j]))));
  return m;
}

// 16 bf16 -> 16 codes of format FMT with scale s = amax / fmax (r = 1 / s)
template <int FMT>
__device__ __forceinline__ uint4 quant16_fmt(const uint4& a, const uint4& b, float amax, float s, float r) {
  if constexpr (FMT == FP8W8A8_FMT_E5M2) {
    if (amax >= qrow::kTinyAmax) return quant16_e5m2<qrow::Mode::kFast>(a, b, s, r);
    if (amax == 0.0f) return quant16_e5m2<qrow::Mode::kZero>(a, b, s, r);
    return quant16_e5m2<qrow::Mode::kExact>(a, b, s, r);
  } else {
    if (amax >= qrow::kTinyAmax) return qrow::quant16<qrow::Mode::kFast>(a, b, s, r);
    if (amax == 0.0f) return qrow::quant16<qrow::Mode::kZero>(a, b, s, r);
    return qrow::quant16<qrow::Mode::kExact>(a, b, s, r);
  }
}

// One maximum |x| per workgroup over a grid-stride share of 8-element groups.
__global__ __launch_bounds__(kBlock) void amax_partials(const uint4* __restrict__ x, int64_t n8,
                                                        float* __restrict__ partials) {
  __shared__ float red[kBlock / 64];
  float m = 0.0f;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
  int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  // four independent loads in flight per thread (one at a time left HBM idle: 32 MiB took
  // 8.2 us)
  for (; i + 3 * stride < n8; i += 4 * stride) {
    const uint4 v0 = x[i], v1 = x[i + stride], v2 = x[i + 2 * stride], v3 = x[i + 3 * stride];
    m = abs_max16(v0, v1, m);
    m = abs_max16(v2, v3, m);
  }
  for (; i < n8; i += stride) m = abs_max16(x[i], make_uint4(0, 0, 0, 0), m);
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
  // back to front: the maxima pass read the tensor front to back, so its last part is the
  // likeliest to still sit in the memory-side cache
  for (int64_t j = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; j < n16; j += stride) {
    const int64_t i = n16 - 1 - j;
    const uint4 a = x[2 * i], b = x[2 * i + 1];
    const uint4 o = quant16_fmt<FMT>(a, b, amax, s, r);
    // non-temporal: the codes are not read again here (8192 x 2048: 19.1 -> 18.2 us)
    __builtin_nontemporal_store((v4u32){o.x, o.y, o.z, o.w}, reinterpret_cast<v4u32*>(q + i));
  }
}

// ---- one pass ----------------------------------------------------------------------

constexpr int kOnePassBlock = 1024;      // threads per workgroup
constexpr int kOnePassMaxGroups = 1023;  // workgroups (one maximum each; the counter after them)
constexpr int kOnePassMaxNP = 4;         // 16-element groups held per thread (8 spills)
constexpr int kDoneWord = kMaxPartials - 1;
constexpr unsigned kUnset = 0xffffffffu;  // no finite |x| has these bits
constexpr uint64_t kBarrierGiveUpTicks = 100000;  // 1 ms of the 100 MHz real-time clock

// Marks every per-workgroup maximum, and the final one, as not yet written.
__global__ __launch_bounds__(kMaxPartials) void onepass_reset(unsigned* ws) {
  __hip_atomic_store(ws + threadIdx.x, kUnset, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroup b holds 16-element groups b * NP * 1024 + j * 1024 + t (j < NP) in thread t:
// each load instruction of a wavefront reads 2 KiB of contiguous input. Each workgroup
// writes its maximum to its own word; workgroup 0 waits until every word is written,
// takes the maximum and writes it to one more word, which the others wait for. Every
// word is written once and read by agent-scope atomics, which go to the device
// coherence point, whatever XCD the reader runs on; no read-modify-write is involved
// (with one counter that every workgroup incremented the kernel took 19.0 us, against 14.4). A workgroup still
// waiting after kBarrierGiveUpTicks (some workgroup not resident, e.g. while another
// stream's kernel holds CUs) reads the whole input itself for the maximum instead: the
// same value, so the wait always ends and the result does not change. give_up_ticks == 0
// sends every workgroup down that path at once (a test of it).
template <int FMT, int NP>
__global__ __launch_bounds__(kOnePassBlock) void quant_tensor_onepass(const uint4* __restrict__ x, int64_t n16,
                                                                     unsigned* __restrict__ ws,
                                                                     uint4* __restrict__ q,
                                                                     float* __restrict__ scale_out,
                                                                     uint64_t give_up_ticks) {
  __shared__ float red[kOnePassBlock / 64];
  __shared__ unsigned amax_bits;
  __shared__ int gave_up;
  const int64_t g0 = (int64_t)blockIdx.x * (NP * kOnePassBlock) + threadIdx.x;
  uint4 va[NP], vb[NP];
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int64_t g = g0 + (int64_t)j * kOnePassBlock;
    if (g < n16) {
      va[j] = x[2 * g];
      vb[j] = x[2 * g + 1];
    } else {
      va[j] = make_uint4(0, 0, 0, 0);
      vb[j] = make_uint4(0, 0, 0, 0);
    }
  }
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < NP; ++j) m = abs_max16(va[j], vb[j], m);
  m = block_max<kOnePassBlock>(m, red);
  if (threadIdx.x < 64) {  // wavefront 0
    const int lane = threadIdx.x;
    if (lane == 0) __hip_atomic_store(ws + blockIdx.x, __float_as_uint(m), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    bool ok = give_up_ticks > 0;
    unsigned result = kUnset;
    if (blockIdx.x == 0) {
      float mx = 0.0f;
      for (int i0 = 0; ok && i0 < (int)gridDim.x; i0 += 64) {
        const int i = i0 + lane;
        while (true) {
          const unsigned v =
              i < (int)gridDim.x ? __hip_atomic_load(ws + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
          if (__ballot(v == kUnset) == 0) {
            mx = fmaxf(mx, __uint_as_float(v));
            break;
          }
          if (__builtin_amdgcn_s_memrealtime() - t0 > give_up_ticks) {
            ok = false;
            break;
          }
          __builtin_amdgcn_s_sleep(2);
        }
      }
      mx = qrow::wave_max(mx);
      if (ok) {
        result = __float_as_uint(mx);
        if (lane == 0) __hip_atomic_store(ws + kDoneWord, result, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    } else {
      while (ok) {
        const unsigned v = __builtin_amdgcn_readfirstlane(
            __hip_atomic_load(ws + kDoneWord, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        if (v != kUnset) {
          result = v;
          break;
        }
        if (__builtin_amdgcn_s_memrealtime() - t0 > give_up_ticks) ok = false;
        else __builtin_amdgcn_s_sleep(8);
      }
    }
    if (lane == 0) {
      amax_bits = result;
      gave_up = !ok;
    }
  }
  __syncthreads();
  float amax;
  if (!gave_up) {
    amax = __uint_as_float(amax_bits);
  } else {
    float mm = 0.0f;
    for (int64_t g = threadIdx.x; g < n16; g += kOnePassBlock) mm = abs_max16(x[2 * g], x[2 * g + 1], mm);
    amax = block_max<kOnePassBlock>(mm, red);
  }
  const float s = amax / (FMT == FP8W8A8_FMT_E5M2 ? 57344.0f : 448.0f);
  const float r = 1.0f / s;
  if (blockIdx.x == 0 && threadIdx.x == 0) *scale_out = s;
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int64_t g = g0 + (int64_t)j * kOnePassBlock;
    if (g < n16) {
      const uint4 o = quant16_fmt<FMT>(va[j], vb[j], amax, s, r);
      __builtin_nontemporal_store((v4u32){o.x, o.y, o.z, o.w}, reinterpret_cast<v4u32*>(q + g));
    }
  }
}

template <int FMT>
hipError_t launch_onepass(const uint4* x, int64_t n16, int np, int groups, unsigned* ws, uint4* q, float* scale,
                          uint64_t give_up, hipStream_t stream) {
  onepass_reset<<<1, kMaxPartials, 0, stream>>>(ws);
  switch (np) {
    case 1: quant_tensor_onepass<FMT, 1><<<groups, kOnePassBlock, 0, stream>>>(x, n16, ws, q, scale, give_up); break;
    case 2: quant_tensor_onepass<FMT, 2><<<groups, kOnePassBlock, 0, stream>>>(x, n16, ws, q, scale, give_up); break;
    default: quant_tensor_onepass<FMT, 4><<<groups, kOnePassBlock, 0, stream>>>(x, n16, ws, q, scale, give_up); break;
  }
  return hipGetLastError();
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

bool quant_tensor_fits_one_pass(int64_t numel, int cus) {
  const int64_t groups_max = std::min<int64_t>(std::max(cus, 1), kOnePassMaxGroups);
  return numel / 16 <= groups_max * kOnePassBlock * kOnePassMaxNP;
}

hipError_t launch_quant_tensor(const uint16_t* x, int64_t numel, int fmt, uint8_t* q, float* scale, float* workspace,
                               int cus, hipStream_t stream, int form) {
  const int64_t n8 = numel / 8, n16 = numel / 16;
  // one pass when the tensor fits in the registers of one workgroup per CU
  const int64_t groups_max = std::min<int64_t>(std::max(cus, 1), kOnePassMaxGroups);
  int np = 1;
  while (np <= kOnePassMaxNP && groups_max * kOnePassBlock * np < n16) np *= 2;
  if (form == kTensorOnePass || form == kTensorOnePassNoWait) {
    if (np > kOnePassMaxNP) return hipErrorInvalidValue;
  } else if (form == kTensorTwoPass) {
    np = kOnePassMaxNP + 1;
  }
  if (np <= kOnePassMaxNP) {
    const int groups = (int)std::min<int64_t>(groups_max, (n16 + (int64_t)kOnePassBlock * np - 1) /
                                                                ((int64_t)kOnePassBlock * np));
    unsigned* ws = reinterpret_cast<unsigned*>(workspace);
    const uint4* xv = reinterpret_cast<const uint4*>(x);
    uint4* qv = reinterpret_cast<uint4*>(q);
    const uint64_t give_up = form == kTensorOnePassNoWait ? 0 : kBarrierGiveUpTicks;
    return fmt == FP8W8A8_FMT_E5M2
               ? launch_onepass<FP8W8A8_FMT_E5M2>(xv, n16, np, groups, ws, qv, scale, give_up, stream)
               : launch_onepass<FP8W8A8_FMT_E4M3FN>(xv, n16, np, groups, ws, qv, scale, give_up, stream);
  }
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
