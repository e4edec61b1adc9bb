// Dynamic per-token (per-row) FP8 E4M3 quantisation for gfx950.
//
// The step the HunyuanVideo1.5 BF16->FP8 retrospective (aigcage.com, section 3.1)
// puts between the bf16 activation and the FP8 GEMM: one scale per token,
// s = amax / 448, and every element rounded to the nearest e4m3fn value of x / s
// (ties to even, saturating). Section 2 of that page notes that this run-time
// quantisation weighs heavily on the whole FP8 path, so it runs at HBM speed:
//
//   * one wavefront per row, the row held in registers between the amax and the
//     quantise passes (one HBM read of the bf16 row, one write of the codes);
//   * each lane owns 16 consecutive elements per chunk: two 16-byte loads, one
//     16-byte store, so every wave-wide access is a contiguous run of memory;
//   * the row maximum is a wavefront butterfly reduction, no LDS, no barrier;
//   * x / s is the correctly rounded fp32 quotient, obtained without a divide per
//     element: r = 1/s once per row, q0 = x*r, e = q0*s - x (exact, FMA), and
//     q = q0 - e*r. For every bf16 pair (x, amax) with amax >= 2^-80 this equals
//     fl32(x / s) whenever |fl32(x / s)| >= 2^-12; smaller quotients all round to
//     a signed zero code either way, and the sign of q always follows x. Rows with
//     0 < amax < 2^-80 (never seen in practice) take an IEEE division per element;
//   * gfx950's v_cvt_pk_fp8_f32 rounds to nearest even into the OCP e4m3fn
//     encoding; the quotient never exceeds 448 * (1 + 2^-23), which it rounds to
//     448, so no clamp is needed.
#include "internal.h"

#pragma clang fp contract(off)

namespace fp8w8a8 {
namespace {

constexpr int kRowsPerBlock = 4;  // one 64-lane wavefront per row
constexpr int kBlock = 64 * kRowsPerBlock;
constexpr float kTinyAmax = 0x1p-80f;

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ __forceinline__ uint32_t pack4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return static_cast<uint32_t>(w);
}

// The three ways a row's quotients are formed.
enum class Mode { kZero, kFast, kExact };

template <Mode M>
__device__ __forceinline__ float quotient(float x, float s, float r) {
  if constexpr (M == Mode::kZero) {
    return x;  // every element is +-0; the convert keeps the sign
  } else if constexpr (M == Mode::kFast) {
    const float q0 = x * r;
    const float e = __builtin_fmaf(q0, s, -x);
    return __builtin_fmaf(-e, r, q0);
  } else {
    return x / s;
  }
}

// 16 bf16 (two uint4) -> 16 codes (one uint4)
template <Mode M>
__device__ __forceinline__ uint4 quant16(const uint4& a, const uint4& b, float s, float r) {
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t u0 = w[2 * i], u1 = w[2 * i + 1];
    o[i] = pack4(quotient<M>(bf16_lo(u0), s, r), quotient<M>(bf16_hi(u0), s, r),
                 quotient<M>(bf16_lo(u1), s, r), quotient<M>(bf16_hi(u1), s, r));
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

__device__ __forceinline__ float absmax16(float m, const uint4& a, const uint4& b) {
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fmaxf(fabsf(bf16_lo(w[i])), fabsf(bf16_hi(w[i]))));
  return m;
}

// NC = number of 16-element chunks each lane keeps in registers (NC * 1024 >= cols).
template <int NC>
__global__ __launch_bounds__(kBlock) void quant_rows_regs(const uint16_t* __restrict__ x, int64_t rows,
                                                         int cols, uint8_t* __restrict__ q,
                                                         float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;  // uniform across the wavefront
  const uint16_t* xr = x + row * cols;
  uint8_t* qr = q + row * cols;
  const int nchunks = cols >> 4;

  uint4 va[NC], vb[NC];
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int c = j * 64 + lane;
    if (c < nchunks) {
      const uint4* p = reinterpret_cast<const uint4*>(xr + static_cast<int64_t>(c) * 16);
      va[j] = p[0];
      vb[j] = p[1];
    } else {
      va[j] = make_uint4(0, 0, 0, 0);
      vb[j] = make_uint4(0, 0, 0, 0);
    }
  }
#pragma unroll
  for (int j = 0; j < NC; ++j) amax = absmax16(amax, va[j], vb[j]);
  amax = wave_max(amax);

  const float s = amax / 448.0f;
  if (lane == 0) scale[row] = s;

#define FP8W8A8_QUANT_STORE(MODE, R)                                                     \
  _Pragma("unroll") for (int j = 0; j < NC; ++j) {                                       \
    const int c = j * 64 + lane;                                                         \
    if (c < nchunks)                                                                     \
      *reinterpret_cast<uint4*>(qr + static_cast<int64_t>(c) * 16) =                     \
          quant16<MODE>(va[j], vb[j], s, R);                                             \
  }
  if (amax >= kTinyAmax) {
    const float r = 1.0f / s;
    FP8W8A8_QUANT_STORE(Mode::kFast, r)
  } else if (amax == 0.0f) {
    FP8W8A8_QUANT_STORE(Mode::kZero, 0.0f)
  } else {
    FP8W8A8_QUANT_STORE(Mode::kExact, 0.0f)
  }
#undef FP8W8A8_QUANT_STORE
}

// Rows longer than the register-resident variants: the row is read twice (the
// second read is served by L2), same arithmetic.
__global__ __launch_bounds__(kBlock) void quant_rows_loop(const uint16_t* __restrict__ x, int64_t rows,
                                                         int cols, uint8_t* __restrict__ q,
                                                         float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint16_t* xr = x + row * cols;
  uint8_t* qr = q + row * cols;
  const int nchunks = cols >> 4;

  float amax = 0.0f;
  for (int c = lane; c < nchunks; c += 64) {
    const uint4* p = reinterpret_cast<const uint4*>(xr + static_cast<int64_t>(c) * 16);
    amax = absmax16(amax, p[0], p[1]);
  }
  amax = wave_max(amax);
  const float s = amax / 448.0f;
  if (lane == 0) scale[row] = s;
  const float r = 1.0f / s;
  for (int c = lane; c < nchunks; c += 64) {
    const uint4* p = reinterpret_cast<const uint4*>(xr + static_cast<int64_t>(c) * 16);
    const uint4 a = p[0], b = p[1];
    uint4 o;
    if (amax >= kTinyAmax)
      o = quant16<Mode::kFast>(a, b, s, r);
    else if (amax == 0.0f)
      o = quant16<Mode::kZero>(a, b, s, r);
    else
      o = quant16<Mode::kExact>(a, b, s, r);
    *reinterpret_cast<uint4*>(qr + static_cast<int64_t>(c) * 16) = o;
  }
}

}  // namespace

hipError_t launch_quant_rows(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* q, float* scale,
                             hipStream_t stream) {
  const int64_t blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  const int chunks_per_lane = static_cast<int>((cols / 16 + 63) / 64);
  const dim3 grid(static_cast<unsigned>(blocks)), block(kBlock);
  const int c = static_cast<int>(cols);
  if (chunks_per_lane <= 1)
    quant_rows_regs<1><<<grid, block, 0, stream>>>(x, rows, c, q, scale);
  else if (chunks_per_lane <= 2)
    quant_rows_regs<2><<<grid, block, 0, stream>>>(x, rows, c, q, scale);
  else if (chunks_per_lane <= 4)
    quant_rows_regs<4><<<grid, block, 0, stream>>>(x, rows, c, q, scale);
  else if (chunks_per_lane <= 8)
    quant_rows_regs<8><<<grid, block, 0, stream>>>(x, rows, c, q, scale);
  else
    quant_rows_loop<<<grid, block, 0, stream>>>(x, rows, c, q, scale);
  return hipGetLastError();
}

}  // namespace fp8w8a8
