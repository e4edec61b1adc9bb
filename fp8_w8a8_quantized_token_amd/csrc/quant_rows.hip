// Dynamic per-token (per-row) FP8 E4M3 quantisation for gfx950.
//
// The step the HunyuanVideo1.5 BF16->FP8 retrospective (aigcage.com, section 3.1)
// puts between the bf16 activation and the FP8 GEMM: one scale per token,
// s = amax / 448, and every element rounded to the nearest e4m3fn value of x / s
// (ties to even, saturating). Section 2 of that page notes that this run-time
// quantisation weighs heavily on the whole FP8 path, so it runs at HBM speed: one
// wavefront per row, the row held in registers between the amax and the quantise
// passes (one HBM read of the bf16 row, one write of the codes), 16-byte accesses
// that make every wave-wide load and store one contiguous run of memory, and no
// LDS or barrier (the arithmetic is in quant_row.h).
#include "internal.h"
#include "quant_row.h"

namespace fp8w8a8 {
namespace {

constexpr int kRowsPerBlock = 4;  // one 64-lane wavefront per row
constexpr int kBlock = 64 * kRowsPerBlock;

// Rows per workgroup of the register-resident kernel: one wavefront per row; rows of
// 8192 and more go one per workgroup (measured 5-6% faster at [4096 | 32760, 8192] than
// four per workgroup, equal for shorter rows).
template <int NC>
constexpr int rows_per_block() { return NC >= 8 ? 1 : kRowsPerBlock; }
static_assert(rows_per_block<8>() == 1, "the NC = 8 launch below assumes one row per workgroup");

// NC = number of 16-element chunks each lane keeps in registers (NC * 1024 >= cols).
template <int NC>
__global__ __launch_bounds__(64 * rows_per_block<NC>()) void quant_rows_regs(const uint16_t* __restrict__ x,
                                                                           int64_t rows, int cols,
                                                                           uint8_t* __restrict__ q,
                                                                           float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * rows_per_block<NC>() + (threadIdx.x >> 6);
  if (row >= rows) return;  // uniform across the wavefront
  const int nchunks = cols >> 4;
  uint4 va[NC], vb[NC];
  qrow::load_row<NC>(x + row * cols, nchunks, lane, va, vb);
  qrow::quant_row<NC>(va, vb, nchunks, lane, q + row * cols, scale + row);
}

__global__ __launch_bounds__(kBlock) void quant_rows_loop(const uint16_t* __restrict__ x, int64_t rows,
                                                         int cols, uint8_t* __restrict__ q,
                                                         float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  qrow::quant_row_loop(x + row * cols, cols >> 4, lane, q + row * cols, scale + row, qrow::NoMap{});
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
    quant_rows_regs<8><<<dim3(static_cast<unsigned>(rows)), dim3(64 * rows_per_block<8>()), 0, stream>>>(
        x, rows, c, q, scale);
  else
    quant_rows_loop<<<grid, block, 0, stream>>>(x, rows, c, q, scale);
  return hipGetLastError();
}

}  // namespace fp8w8a8
