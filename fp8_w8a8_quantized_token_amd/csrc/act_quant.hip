// Activation producers for gfx950: GELU / SiLU on bf16, rounded to bf16, and the
// fused variant that emits the per-token FP8 codes and scales directly.
//
// The HunyuanVideo1.5 BF16->FP8 retrospective (aigcage.com, section 3, item 5,
// producer fusion) has the activation upstream of the FFN-down linear hand the FP8
// linear its (codes, per-token scale) pair instead of a bf16 tensor that a separate
// pass would quantise. The fused result is defined as the plain path's:
// y = bf16_rne(act(x)) for each bf16 x, then the per-token quantiser on y.
//
// A bf16 -> bf16 function has only 2^16 inputs, so it is a table:
//
//   * act_table_kernel evaluates act once per input pattern in fp64 and rounds the
//     fp64 value directly to bf16 (no fp32 step, so no double rounding). Every
//     finite input's value lies more than 1e-9 (relative) away from a bf16 rounding
//     midpoint, far outside fp64's error here, with one exception: for
//     0 < |x| < 2^-125, x/2 can be exactly such a midpoint, and act(x) = x/2 + c x^2
//     + ... with c > 0 for all three functions, so those ties go toward +inf (the
//     x^2 term is far below fp64's resolution at that size).
//   * the producers stage the 128 KiB table in LDS (one workgroup of 16 wavefronts
//     per CU, persistent over rows); each element costs one LDS lookup instead of
//     an erfc / exp evaluation, and the exact rounding comes for free. The row's
//     HBM loads are issued before the table barrier, so the table fill overlaps
//     the first row's latency.
//   * the fused producer keeps the mapped row in registers for the amax and
//     quantise passes (quant_row.h): HBM traffic is 2 bytes read + 1 byte written
//     per element, against 2 + 2 (act) + 2 + 1 (quant) for the plain path.
#include "internal.h"
#include "quant_row.h"

namespace fp8w8a8 {
namespace {

constexpr int kTableEntries = 1 << 16;
constexpr int kWaves = 16;  // per workgroup; one workgroup per CU (the table fills LDS)
constexpr int kBlock = 64 * kWaves;

// ---- table construction --------------------------------------------------------

// Round a finite fp64 value to bf16, ties to even, except that an exact tie is
// broken toward +inf when tie_up is set (the caller knows the true value lies just
// above y). Handles the bf16 subnormal range (quantum 2^-133).
__device__ uint16_t f64_to_bf16(double y, bool tie_up) {
  const bool neg = signbit(y);
  const double a = fabs(y);
  if (a == 0.0) return neg ? 0x8000 : 0;
  const int e = ilogb(a);                 // a in [2^e, 2^(e+1))
  const int qe = e - 7 > -133 ? e - 7 : -133;  // quantum exponent: 8 significant bits
  const double t = ldexp(a, -qe);         // exact: a power-of-two scaling
  const double f = floor(t);
  const double d = t - f;                 // exact
  double r = f;
  // |value| = t exactly, or just above it by a magnitude of sign (tie_up ? +1 : -1) * (neg ? -1 : 1)
  const bool mag_up_at_tie = tie_up ? !neg : false;
  if (d > 0.5) {
    r = f + 1.0;
  } else if (d == 0.5) {
    if (tie_up)
      r = mag_up_at_tie ? f + 1.0 : f;
    else
      r = (fmod(f, 2.0) != 0.0) ? f + 1.0 : f;
  }
  // r in [0, 256]; value = r * 2^qe, biased exponent of r in [128, 256) is qe + 7 + 127
  const int ri = static_cast<int>(r);
  const uint32_t bits = static_cast<uint32_t>(((qe + 134) << 7) + (ri - 128));
  return static_cast<uint16_t>(bits | (neg ? 0x8000u : 0u));
}

__device__ double act_f64(int act, double x) {
  switch (act) {
    case FP8W8A8_ACT_GELU_ERF:
      return 0.5 * x * erfc(-x * 0.70710678118654752440);  // x * Phi(x)
    case FP8W8A8_ACT_GELU_TANH: {
      const double u = 0.79788456080286535588 * (x + 0.044715 * x * x * x);  // sqrt(2/pi) (x + 0.044715 x^3)
      return x / (1.0 + exp(-2.0 * u));  // x/2 (1 + tanh u), no cancellation for u << 0
    }
    default:
      return x / (1.0 + exp(-x));  // SiLU
  }
}

// Exact value of a bf16 bit pattern as fp64 (integer arithmetic: independent of
// the fp32 denormal mode).
__device__ double bf16_bits_to_f64(uint32_t bits) {
  const int e = static_cast<int>((bits >> 7) & 0xFF);
  const int m = static_cast<int>(bits & 0x7F);
  const double mag = e == 0 ? ldexp(static_cast<double>(m), -133) : ldexp(static_cast<double>(128 + m), e - 134);
  return (bits & 0x8000) ? -mag : mag;
}

__global__ __launch_bounds__(256) void act_table_kernel(int act, uint16_t* __restrict__ table) {
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p >= kTableEntries) return;
  const uint32_t bits = static_cast<uint32_t>(p);
  const uint32_t mag = bits & 0x7FFF;
  uint16_t out;
  if (mag >= 0x7F80) {
    // outside the contract; defined as the limits: NaN -> NaN, +inf -> +inf, -inf -> -0
    out = mag > 0x7F80 ? 0x7FC0 : ((bits & 0x8000) ? 0x8000 : 0x7F80);
  } else if (mag == 0) {
    out = static_cast<uint16_t>(bits);  // act(+-0) = +-0
  } else if (mag < 0x0100) {
    out = f64_to_bf16(0.5 * bf16_bits_to_f64(bits), true);  // |x| < 2^-125
  } else {
    out = f64_to_bf16(act_f64(act, bf16_bits_to_f64(bits)), false);
  }
  table[p] = out;
}

// ---- producers -------------------------------------------------------------------

// Copy the table into the workgroup's LDS copy (16 bytes per thread per step).
template <int THREADS = kBlock>
__device__ __forceinline__ void stage_table(const uint16_t* __restrict__ table, uint16_t* lut) {
  const uint4* src = reinterpret_cast<const uint4*>(table);
  uint4* dst = reinterpret_cast<uint4*>(lut);
#pragma unroll
  for (int i = 0; i < kTableEntries / 8 / THREADS; ++i) dst[i * THREADS + threadIdx.x] = src[i * THREADS + threadIdx.x];
}

struct LutMap {
  const uint16_t* lut;
  __device__ __forceinline__ uint32_t word(uint32_t w) const {
    return static_cast<uint32_t>(lut[w & 0xFFFFu]) | (static_cast<uint32_t>(lut[w >> 16]) << 16);
  }
  __device__ __forceinline__ void operator()(uint4& v) const {
    v.x = word(v.x);
    v.y = word(v.y);
    v.z = word(v.z);
    v.w = word(v.w);
  }
};

__device__ __forceinline__ uint16_t* shared_table() {
  __shared__ __attribute__((aligned(16))) uint16_t lut[kTableEntries];
  return lut;
}

// Fused producer, rows held in registers (NC chunks of 16 per lane), WAVES rows in
// flight per workgroup.
template <int NC, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void act_quant_rows_regs(const uint16_t* __restrict__ x, int64_t rows,
                                                                 int cols, const uint16_t* __restrict__ table,
                                                                 uint8_t* __restrict__ q, float* __restrict__ scale) {
  uint16_t* lut = shared_table();
  const int lane = threadIdx.x & 63;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * WAVES;
  int64_t row = static_cast<int64_t>(blockIdx.x) * WAVES + (threadIdx.x >> 6);
  const int nchunks = cols >> 4;
  uint4 va[NC], vb[NC];
  if (row < rows) qrow::load_row<NC>(x + row * cols, nchunks, lane, va, vb);  // in flight across the fill
  stage_table<64 * WAVES>(table, lut);
  __syncthreads();
  const LutMap map{lut};
  for (; row < rows; row += stride) {
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      map(va[j]);
      map(vb[j]);
    }
    qrow::quant_row<NC>(va, vb, nchunks, lane, q + row * cols, scale + row);
    if (row + stride < rows) qrow::load_row<NC>(x + (row + stride) * cols, nchunks, lane, va, vb);
  }
}

// Fused producer for rows of 4097..8192 elements: each row split over 4 wavefronts (NC
// chunks per lane), 4 rows in flight per 16-wavefront workgroup, and the next row's
// loads issued before the current row is mapped, so every wavefront keeps a row in
// flight while it works through the table lookups. The 4 wavefront maxima of a row meet
// in LDS (double-buffered by iteration, one barrier per iteration); every wavefront of
// the workgroup runs the same iterations, so the barrier count matches.
constexpr int kSplit = 4;                  // wavefronts per row
constexpr int kSlots = kWaves / kSplit;    // rows in flight per workgroup
template <int NC>
__global__ __launch_bounds__(kBlock) void act_quant_rows_split(const uint16_t* __restrict__ x, int64_t rows,
                                                              int cols, const uint16_t* __restrict__ table,
                                                              uint8_t* __restrict__ q, float* __restrict__ scale) {
  uint16_t* lut = shared_table();
  __shared__ float wave_amax[2][kWaves];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int slot = wave / kSplit, part = wave % kSplit;
  const int nchunks = cols >> 4;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kSlots;
  int64_t base = static_cast<int64_t>(blockIdx.x) * kSlots;
  uint4 va[NC], vb[NC], na[NC] = {}, nb[NC] = {};
  if (base + slot < rows) qrow::load_row<NC, kSplit>(x + (base + slot) * cols, nchunks, lane, va, vb, part);
  stage_table(table, lut);
  __syncthreads();
  const LutMap map{lut};
  for (int it = 0; base < rows; base += stride, ++it) {
    const int64_t row = base + slot, next = row + stride;
    if (next < rows) qrow::load_row<NC, kSplit>(x + next * cols, nchunks, lane, na, nb, part);
    float m = 0.0f;
    if (row < rows) {
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        map(va[j]);
        map(vb[j]);
      }
      m = qrow::wave_max(qrow::lane_absmax<NC>(va, vb));
    }
    if (lane == 0) wave_amax[it & 1][wave] = m;
    __syncthreads();
    if (row < rows) {
      float amax = wave_amax[it & 1][slot * kSplit];
#pragma unroll
      for (int i = 1; i < kSplit; ++i) amax = fmaxf(amax, wave_amax[it & 1][slot * kSplit + i]);
      qrow::quant_row_part<NC, kSplit>(va, vb, nchunks, lane, part, amax, q + row * cols, scale + row);
    }
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      va[j] = na[j];
      vb[j] = nb[j];
    }
  }
}

__global__ __launch_bounds__(kBlock) void act_quant_rows_loop(const uint16_t* __restrict__ x, int64_t rows, int cols,
                                                             const uint16_t* __restrict__ table,
                                                             uint8_t* __restrict__ q, float* __restrict__ scale) {
  uint16_t* lut = shared_table();
  stage_table(table, lut);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kWaves;
  for (int64_t row = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6); row < rows; row += stride)
    qrow::quant_row_loop(x + row * cols, cols >> 4, lane, q + row * cols, scale + row, LutMap{lut});
}

// Plain producer: y = table[x] elementwise over n16 16-byte groups (8 bf16 each);
// each thread keeps kUnroll loads in flight.
constexpr int kUnroll = 4;

__global__ __launch_bounds__(kBlock) void act_map_kernel(const uint4* __restrict__ x, int64_t n16,
                                                        const uint16_t* __restrict__ table, uint4* __restrict__ y) {
  uint16_t* lut = shared_table();
  const int64_t step = static_cast<int64_t>(gridDim.x) * kBlock;
  const int64_t first = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  uint4 v[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t i = first + u * step;
    v[u] = i < n16 ? x[i] : make_uint4(0, 0, 0, 0);
  }
  stage_table(table, lut);
  __syncthreads();
  const LutMap map{lut};
  for (int64_t base = first; base < n16; base += kUnroll * step) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + u * step;
      if (i < n16) {
        map(v[u]);
        y[i] = v[u];
      }
      const int64_t nxt = i + kUnroll * step;
      v[u] = nxt < n16 ? x[nxt] : make_uint4(0, 0, 0, 0);
    }
  }
}

int64_t producer_grid(int64_t work_items, int64_t per_block, int cus) {
  const int64_t need = (work_items + per_block - 1) / per_block;
  return need < cus ? need : cus;
}

}  // namespace

hipError_t launch_act_table(int act, uint16_t* table, hipStream_t stream) {
  act_table_kernel<<<dim3(kTableEntries / 256), dim3(256), 0, stream>>>(act, table);
  return hipGetLastError();
}

hipError_t launch_act_quant_rows(const uint16_t* x, int64_t rows, int64_t cols, const uint16_t* table, uint8_t* q,
                                 float* scale, int cus, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(producer_grid(rows, kWaves, cus))), block(kBlock);
  const int chunks_per_lane = static_cast<int>((cols / 16 + 63) / 64);
  const int c = static_cast<int>(cols);
  if (chunks_per_lane <= 1) {
    act_quant_rows_regs<1, kWaves><<<grid, block, 0, stream>>>(x, rows, c, table, q, scale);
  } else if (chunks_per_lane <= 2) {
    act_quant_rows_regs<2, kWaves><<<grid, block, 0, stream>>>(x, rows, c, table, q, scale);
  } else if (chunks_per_lane <= 4) {
    act_quant_rows_regs<4, kWaves><<<grid, block, 0, stream>>>(x, rows, c, table, q, scale);
  } else if (chunks_per_lane <= 8) {
    const dim3 gs(static_cast<unsigned>(producer_grid(rows, kSlots, cus)));
    act_quant_rows_split<2><<<gs, block, 0, stream>>>(x, rows, c, table, q, scale);
  } else {
    act_quant_rows_loop<<<grid, block, 0, stream>>>(x, rows, c, table, q, scale);
  }
  return hipGetLastError();
}

hipError_t launch_act_rows(const uint16_t* x, int64_t elems, const uint16_t* table, uint16_t* y, int cus,
                           hipStream_t stream) {
  const int64_t n16 = elems / 8;
  const dim3 grid(static_cast<unsigned>(producer_grid(n16, static_cast<int64_t>(kBlock) * kUnroll, cus))),
      block(kBlock);
  act_map_kernel<<<grid, block, 0, stream>>>(reinterpret_cast<const uint4*>(x), n16, table,
                                             reinterpret_cast<uint4*>(y));
  return hipGetLastError();
}

}  // namespace fp8w8a8
