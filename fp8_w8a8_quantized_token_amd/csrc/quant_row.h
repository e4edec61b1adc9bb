// Per-row e4m3fn quantisation of bf16 values held in registers, shared by the plain
// per-token quantiser and the activation producers that emit FP8.
//
// One 64-lane wavefront owns a row (or a share of it, when a workgroup splits long rows
// over several wavefronts); each lane holds 16 consecutive bf16 per chunk (two uint4).
// The row maximum is a butterfly over the wavefront (and across the wavefronts of a
// split row, an exchange the caller does), the scale is
// s = fl32(amax / 448), and each element becomes the e4m3fn code of the correctly
// rounded fp32 quotient x / s (HunyuanVideo1.5 BF16->FP8 retrospective,
// aigcage.com, section 3.1; the 448 denominator is the largest finite e4m3fn).
//
//   * x / s without a divide per element: r = 1/s once per row, q0 = x*r,
//     e = q0*s - x (exact, FMA), q = q0 - e*r. For every bf16 pair (x, amax) with
//     amax >= 2^-80 this equals fl32(x / s) whenever |fl32(x / s)| >= 2^-12;
//     smaller quotients all round to a signed zero code either way, and the sign of
//     q always follows x. Rows with 0 < amax < 2^-80 take an IEEE division per
//     element; all-zero rows convert x itself (signed zeros).
//   * v_cvt_pk_fp8_f32 rounds to nearest even into the OCP e4m3fn encoding; the
//     quotient never exceeds 448 * (1 + 2^-23), which it rounds to 448, so no clamp
//     is needed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#pragma clang fp contract(off)

namespace fp8w8a8 {
namespace qrow {

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

// Load a row's chunks into registers: with the row split over WPR wavefronts, wavefront
// `part` holds chunks c = (j * WPR + part) * 64 + lane (j < NC); one wavefront per row
// (WPR = 1) holds c = j * 64 + lane. Chunks past the row read as zeros (they never raise
// the maximum and are never stored).
template <int NC, int WPR = 1>
__device__ __forceinline__ void load_row(const uint16_t* xr, int nchunks, int lane, uint4 (&va)[NC],
                                         uint4 (&vb)[NC], int part = 0) {
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int c = (j * WPR + part) * 64 + lane;
    if (c < nchunks) {
      const uint4* p = reinterpret_cast<const uint4*>(xr + static_cast<int64_t>(c) * 16);
      va[j] = p[0];
      vb[j] = p[1];
    } else {
      va[j] = make_uint4(0, 0, 0, 0);
      vb[j] = make_uint4(0, 0, 0, 0);
    }
  }
}

// How a row's results reach memory: plain stores (the default), or a policy with the
// same two members (the single-launch quantise + GEMM kernel writes through to the
// device coherence point). `qr` is the row's code pointer (uniform across the
// wavefront), `c` a 16-code chunk index. The codes are stored non-temporal: the next
// reader is another kernel, mostly on other XCDs, so they need not stay in this XCD's
// L2 (FFN-up quantise + GEMM 65.9 -> 65.1 us).
struct PlainStore {
  typedef unsigned v4u32 __attribute__((ext_vector_type(4)));
  __device__ __forceinline__ void codes(uint8_t* qr, int c, int, const uint4& v) const {
    __builtin_nontemporal_store((v4u32){v.x, v.y, v.z, v.w},
                                reinterpret_cast<v4u32*>(qr + static_cast<int64_t>(c) * 16));
  }
  __device__ __forceinline__ void scale(float* srow, float s) const { *srow = s; }
};

// Largest magnitude among the chunks this lane holds (0 for none).
template <int NC>
__device__ __forceinline__ float lane_absmax(const uint4 (&va)[NC], const uint4 (&vb)[NC]) {
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < NC; ++j) amax = absmax16(amax, va[j], vb[j]);
  return amax;
}

// Scale and codes of the chunks one wavefront holds (loaded by load_row<NC, WPR> as
// `part`), given the whole row's maximum `amax`. Wavefront 0's lane 0 stores the scale.
template <int NC, int WPR = 1, class Store = PlainStore>
__device__ __forceinline__ void quant_row_part(const uint4 (&va)[NC], const uint4 (&vb)[NC], int nchunks,
                                               int lane, int part, float amax, uint8_t* qr, float* srow,
                                               const Store& st = Store{}) {
  const float s = amax / 448.0f;
  if (lane == 0 && part == 0) st.scale(srow, s);

#define FP8W8A8_QUANT_STORE(MODE, R)                                                     \
  _Pragma("unroll") for (int j = 0; j < NC; ++j) {                                       \
    const int c = (j * WPR + part) * 64 + lane;                                          \
    if (c < nchunks) st.codes(qr, c, nchunks, quant16<MODE>(va[j], vb[j], s, R));        \
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

// Scale and codes of a register-resident row (every lane of the wavefront calls it).
template <int NC, class Store = PlainStore>
__device__ __forceinline__ void quant_row(const uint4 (&va)[NC], const uint4 (&vb)[NC], int nchunks, int lane,
                                          uint8_t* qr, float* srow, const Store& st = Store{}) {
  quant_row_part<NC, 1, Store>(va, vb, nchunks, lane, 0, wave_max(lane_absmax<NC>(va, vb)), qr, srow, st);
}

// Identity map of a chunk (the plain quantiser).
struct NoMap {
  __device__ __forceinline__ void operator()(uint4&) const {}
};

// Rows longer than the register-resident variants: the row is read twice (the
// second read is served by L2); `map` is applied to every chunk on both passes.
template <class Map, class Store = PlainStore>
__device__ __forceinline__ void quant_row_loop(const uint16_t* xr, int nchunks, int lane, uint8_t* qr,
                                               float* srow, const Map& map, const Store& st = Store{}) {
  float amax = 0.0f;
  for (int c = lane; c < nchunks; c += 64) {
    const uint4* p = reinterpret_cast<const uint4*>(xr + static_cast<int64_t>(c) * 16);
    uint4 a = p[0], b = p[1];
    map(a);
    map(b);
    amax = absmax16(amax, a, b);
  }
  amax = wave_max(amax);
  const float s = amax / 448.0f;
  if (lane == 0) st.scale(srow, s);
  const float r = 1.0f / s;
  for (int c = lane; c < nchunks; c += 64) {
    const uint4* p = reinterpret_cast<const uint4*>(xr + static_cast<int64_t>(c) * 16);
    uint4 a = p[0], b = p[1];
    map(a);
    map(b);
    uint4 o;
    if (amax >= kTinyAmax)
      o = quant16<Mode::kFast>(a, b, s, r);
    else if (amax == 0.0f)
      o = quant16<Mode::kZero>(a, b, s, r);
    else
      o = quant16<Mode::kExact>(a, b, s, r);
    st.codes(qr, c, nchunks, o);
  }
}

}  // namespace qrow
}  // namespace fp8w8a8
