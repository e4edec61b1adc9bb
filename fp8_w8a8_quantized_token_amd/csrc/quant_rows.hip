// Dynamic per-token (per-row) FP8 E4M3 quantisation for gfx950.
//
// The step the HunyuanVideo1.5 BF16->FP8 retrospective (aigcage.com, section 3.1)
// puts between the bf16 activation and the FP8 GEMM: one scale per token,
// s = amax / 448, and every element rounded to the nearest e4m3fn value of x / s
// (ties to even, saturating). Section 2 of that page notes that this run-time
// quantisation weighs heavily on the whole FP8 path, so it runs at HBM speed: the row
// held in registers between the amax and the quantise passes (one HBM read of the
// bf16 row, one write of the codes), 16-byte accesses that make every wave-wide load
// and store one contiguous run of memory. Rows of up to 2048 elements take one
// wavefront each, with no LDS or barrier; rows of up to 8192 are split over the 4
// wavefronts of a workgroup, whose maxima meet in LDS; longer rows are read twice
// (the arithmetic is in quant_row.h).
#include "internal.h"
#include "quant_row.h"

namespace fp8w8a8 {
namespace {

constexpr int kRowsPerBlock = 4;  // one 64-lane wavefront per row
constexpr int kBlock = 64 * kRowsPerBlock;

// NC = number of 16-element chunks each lane keeps in registers (NC * 1024 >= cols).
template <int NC>
__global__ __launch_bounds__(kBlock) void quant_rows_regs(const uint16_t* __restrict__ x, int64_t rows, int cols,
                                                         uint8_t* __restrict__ q, float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;  // uniform across the wavefront
  const int nchunks = cols >> 4;
  uint4 va[NC], vb[NC];
  qrow::load_row<NC>(x + row * cols, nchunks, lane, va, vb);
  qrow::quant_row<NC>(va, vb, nchunks, lane, q + row * cols, scale + row);
}

// Rows of more than 2048 elements: one row per workgroup, split over its WPR wavefronts
// (NC chunks per lane, WPR * NC * 1024 >= cols); the wavefront maxima meet in LDS. Against
// one wavefront per row, 4 wavefronts: [4096, 8192] 22.4 -> 20.2 us, [32760, 8192] 143.1 ->
// 139.9 us, [32760, 4096] 72.4 -> 69.6 us, [4096, 4096] unchanged (same codes and scales).
// Many rows of 4097..8192 elements take 8 wavefronts per row (one chunk per lane): at
// [32760, 8192] 131.7 against 137.6 us, while at [4096, 8192] 4 stay ahead (18.8 against
// 19.6 us), so 8 are used from kSplit8Rows rows on.
constexpr int kSplitWaves = 4;
constexpr int64_t kSplit8Rows = 16384;
template <int NC, int WPR>
__global__ __launch_bounds__(64 * WPR) void quant_rows_split(const uint16_t* __restrict__ x, int cols,
                                                            uint8_t* __restrict__ q, float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int part = threadIdx.x >> 6;
  const int64_t row = blockIdx.x;  // the grid is exactly one workgroup per row
  const int nchunks = cols >> 4;
  uint4 va[NC], vb[NC];
  qrow::load_row<NC, WPR>(x + row * cols, nchunks, lane, va, vb, part);
  __shared__ float wave_amax[WPR];
  const float m = qrow::wave_max(qrow::lane_absmax<NC>(va, vb));
  if (lane == 0) wave_amax[part] = m;
  __syncthreads();
  float amax = wave_amax[0];
#pragma unroll
  for (int i = 1; i < WPR; ++i) amax = fmaxf(amax, wave_amax[i]);
  qrow::quant_row_part<NC, WPR>(va, vb, nchunks, lane, part, amax, q + row * cols, scale + row);
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
  const dim3 split_grid(static_cast<unsigned>(rows)), split_block(64 * kSplitWaves);
  if (chunks_per_lane <= 1)
    quant_rows_regs<1><<<grid, block, 0, stream>>>(x, rows, c, q, scale);
  else if (chunks_per_lane <= 2)
    quant_rows_regs<2><<<grid, block, 0, stream>>>(x, rows, c, q, scale);
  else if (chunks_per_lane <= 4)
    quant_rows_split<1, kSplitWaves><<<split_grid, split_block, 0, stream>>>(x, c, q, scale);
  else if (chunks_per_lane <= 8 && rows >= kSplit8Rows)
    quant_rows_split<1, 2 * kSplitWaves><<<split_grid, dim3(128 * kSplitWaves), 0, stream>>>(x, c, q, scale);
  else if (chunks_per_lane <= 8)
    quant_rows_split<2, kSplitWaves><<<split_grid, split_block, 0, stream>>>(x, c, q, scale);
  else
    quant_rows_loop<<<grid, block, 0, stream>>>(x, rows, c, q, scale);
  return hipGetLastError();
}

}  // namespace fp8w8a8
