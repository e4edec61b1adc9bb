// Building blocks shared by the GEMM kernels (FP8 x FP8 and bf16 x FP8) for gfx950:
// buffer descriptors, global -> LDS DMA, bf16 packing, the output-tile store, the XCD-aware tile order,
// per-stage LDS objects, precise waits, the MFMA / LDS-read interleave and the LDS
// chunk swizzle. Each translation unit that includes it gets its own copy.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8w8a8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kXcds = 8;          // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kBufferConfig = 0x00020000;  // gfx9 raw buffer descriptor, word 3
constexpr int kCpolNt = 2;                 // cache-policy operand of buffer stores: nt


// Raw buffer descriptor in SGPRs: 48-bit base, stride 0, num_records bytes.
__device__ __forceinline__ v4i make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  v4i r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xffff);
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = kBufferConfig;
  return r;
}

// buffer_load_dwordx4 ... lds: lane i's 16 bytes land at LDS address lds + 16 i. Issued
// from inline asm so the compiler does not make every later LDS read wait for all
// fills in flight; the kernel waits for exactly the fills it needs (vmcnt) and
// synchronises the workgroup itself. The instruction has no register result. The LDS
// address goes in through M0 as an operand bound to that register ("{m0}"), so the
// compiler writes M0 itself and knows its contents, rather than having it changed
// behind its back inside the asm.
__device__ __forceinline__ void dma16(v4i rsrc, uint32_t lds, uint32_t voffset) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voffset), "s"(rsrc), "{m0}"(lds)
               : "memory");
}

// The same for 4 bytes per lane: lane i's dword lands at LDS address lds + 4 i.
__device__ __forceinline__ void dma4(v4i rsrc, uint32_t lds, uint32_t voffset) {
  asm volatile("buffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(voffset), "s"(rsrc), "{m0}"(lds)
               : "memory");
}

typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf16 __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16 (round to nearest even), lo in bits 0..15. Converted as one
// two-element vector so that a single v_cvt_pk_bf16_f32 does both: converting the two
// values one by one costs two converts plus a shift and an OR.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){lo, hi}, v2bf16));
}

// Store a wave's bf16 output tile, staged in LDS at `wout` (WTM rows of RC 16-byte chunks,
// chunk c of row r at position c ^ (r % RC)), to out[row0 + r][col0 + 8 c ...] of an
// m x n row-major bf16 matrix. Each store writes 64 / RC whole rows of the wave tile, 16
// bytes per lane. The buffer descriptor covers exactly the tile's valid rows, so rows
// past m fall outside it and are dropped, and lanes whose 8 columns lie past n are
// pointed out of range: no per-store bounds test. The stores are non-temporal: the output
// is not read again by this kernel, and marking its lines for early eviction keeps the
// operand panels other tiles still read in the XCD's L2 (FFN-up 68.5 -> 66.1 us,
// 32760 x 2048 x 2048 138.3 -> 129.5 us, bit-identical output).
// ALWAYS_ISSUE: a piece wholly past m still issues its stores (an empty descriptor drops
// them), so a caller that counts its outstanding memory operations knows the number.
template <int WTM, int RC, bool ALWAYS_ISSUE = false>
__device__ __forceinline__ void store_wave_tile(const uint8_t* wout, int lane, uint16_t* out, int m, int n,
                                                int row0, int col0) {
  constexpr int kRowsPerStore = 64 / RC;
  static_assert(64 % RC == 0 && WTM % kRowsPerStore == 0, "row segments tile the wavefront");
  const int rows_valid = max(0, min(WTM, m - row0));
  if (!ALWAYS_ISSUE && rows_valid == 0) return;
  const uint32_t row_bytes = (uint32_t)n * 2u;
  // base and size are uniform; readfirstlane keeps the descriptor in SGPRs even where the
  // compiler cannot tell (no waterfall loop around the stores)
  const uint64_t base = reinterpret_cast<uint64_t>(out + (int64_t)row0 * n);
  const uint64_t ubase = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)base) |
                         ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(base >> 32)) << 32);
  const uint32_t nrec = (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)rows_valid * row_bytes));
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(ubase), 0, nrec, kBufferConfig);
  const int c = lane % RC;
  const int ncol = col0 + c * 8;
  const uint32_t voff = ncol < n ? (uint32_t)(lane / RC) * row_bytes + (uint32_t)ncol * 2u : kOutOfRange;
#pragma unroll
  for (int t = 0; t < WTM / kRowsPerStore; ++t) {
    const int r = t * kRowsPerStore + lane / RC;
    const uint4 v = *reinterpret_cast<const uint4*>(wout + r * (RC * 16) + ((c ^ (r % RC)) << 4));
    const v4u data = {v.x, v.y, v.z, v.w};
    __builtin_amdgcn_raw_buffer_store_b128(data, rsrc, voff + (uint32_t)(t * kRowsPerStore) * row_bytes, 0,
                                           kCpolNt);
  }
}

// Workgroup id -> (tile_m, tile_n). Hardware deals ids to XCDs round-robin (id % 8);
// renumber so XCD x owns a contiguous range of logical tiles, then walk that range in
// groups of GROUP_M tile rows so concurrent tiles share operand panels in L2.
// tile_coords_at: the same for logical tile `id` of `nwg` (a persistent workgroup's id plus
// a multiple of its grid, which keeps id % 8 its own XCD when the grid is a multiple of 8).
template <int GROUP_M>
__device__ __forceinline__ void tile_coords_at(int id, int nwg, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int q = nwg / kXcds, r = nwg % kXcds;
  const int xcd = id % kXcds, local = id / kXcds;
  const int logical = xcd * q + min(xcd, r) + local;
  const int group_size = GROUP_M * tiles_n;
  const int group = logical / group_size;
  const int first_m = group * GROUP_M;
  const int gm = min(tiles_m - first_m, GROUP_M);
  const int in_group = logical - group * group_size;
  tm = first_m + in_group % gm;
  tn = in_group / gm;
}

template <int GROUP_M>
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int& tm, int& tn) {
  tile_coords_at<GROUP_M>(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
}

// Distinct LDS objects per (kernel, stage).
template <typename Tag, int I, int BYTES>
__device__ __forceinline__ uint8_t* stage_buf() {
  __shared__ __attribute__((aligned(1024))) uint8_t buf[BYTES];
  return buf;
}

// s_waitcnt with vmcnt = N (0..63) and lgkmcnt = 0 (gfx9 encoding, expcnt untouched).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | (((N >> 4) & 3) << 14));
}

// Wait until the fills of the stage about to be read have landed, allowing the
// `pending` younger stages (F fills each) to stay in flight; also drains this wave's
// LDS reads (lgkmcnt(0)) so the workgroup barrier that follows may recycle a buffer.
template <int F, int S>
__device__ __forceinline__ void wait_stage(int pending) {
  if constexpr (S >= 6) {
    if (pending >= 5) { wait_vm_lgkm0<5 * F>(); return; }
  }
  if constexpr (S >= 5) {
    if (pending >= 4) { wait_vm_lgkm0<4 * F>(); return; }
  }
  if constexpr (S >= 4) {
    if (pending >= 3) { wait_vm_lgkm0<3 * F>(); return; }
  }
  if constexpr (S >= 3) {
    if (pending >= 2) { wait_vm_lgkm0<2 * F>(); return; }
  }
  if (pending >= 1) { wait_vm_lgkm0<F>(); return; }
  wait_vm_lgkm0<0>();
}

// Interleave the MFMAs of the current sub-step with the LDS reads of the next one:
// after each MFMA, up to R ds_reads (the matrix pipe keeps running while they issue).
template <int MFMAS, int READS>
__device__ __forceinline__ void interleave_mfma_ds_read() {
  constexpr int R = (READS + MFMAS - 1) / MFMAS;
#pragma unroll
  for (int i = 0; i < MFMAS; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    if (R > 0 && (i + 1) * R <= READS) __builtin_amdgcn_sched_group_barrier(0x100, R, 0);  // DS reads
  }
}

__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// LDS swizzle of 16-byte chunks within a tile row of BK bytes: chunk c of row r sits at
// position c ^ swz(r). Chosen so that 16 consecutive rows read at one logical chunk hit
// 16 distinct 16-byte bank groups of a 256-byte LDS line, and any 8 consecutive rows 8
// distinct groups of a 128-byte line: the ds_read_b128 operand reads are conflict free.
template <int BK>
__device__ __forceinline__ int swz(int r) {
  if constexpr (BK == 64) return ((r >> 1) & 3) ^ ((r >> 3) & 1);
  else return ((r >> 1) & 7) ^ ((r & 1) << 2);
}

}  // namespace
}  // namespace fp8w8a8
