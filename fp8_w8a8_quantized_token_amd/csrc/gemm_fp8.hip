// FP8 (e4m3fn) x FP8 GEMM with the scale / bias / bf16 epilogue fused, for gfx950.
//
//   out[m, n] = bf16_rne( acc[m, n] * a_scale[m] * w_scale[n] + bias[n] ),
//   acc[m, n] = sum_k dec(qa[m, k]) * dec(qw[n, k])   (fp32 accumulation on the MFMA units)
//
// This is the FP8 GEMM step and the scale / bias / output-type step of the chain in the
// HunyuanVideo1.5 BF16->FP8 retrospective (aigcage.com, section 3.1). Both operands
// are k-contiguous: the activation codes [m, k] and the weight in nn.Linear's [n, k]
// layout (the page's column-major B, never transposed). Section 3.2 of the page finds
// that the tile shape, the memory pipeline and the full epilogue, not the bare GEMM,
// decide the speed. The design here is gfx950's own:
//
//   * V_MFMA_F32_32X32X64_F8F6F4. The weight rows feed the MFMA's first operand and
//     the activation rows its second, so a lane's results come in runs of four
//     consecutive output channels of one token: one 8-byte bf16 store each.
//   * Block tiles of BM tokens x BN channels, BK = 128 bytes of k per stage, STAGES
//     stage buffers in LDS (up to the 160 KiB of a CU). Stages are filled by
//     buffer_load_dwordx4 ... lds (HBM/L2 -> LDS with no VGPR staging) STAGES - 1
//     stages ahead of their use. Each wave waits with a precise vmcnt for its own fills
//     of the stage it is about to read, then the workgroup barrier publishes every
//     wave's fills.
//   * The buffer descriptors cover only the block's valid rows, and lanes past k are
//     pointed out of range: ragged m / n / k tails read zeros and no access leaves
//     the operands.
//   * 16-byte chunk c of LDS row r sits at position c ^ swz(r) (gemm_common.h), which
//     makes the fills and the ds_read_b128 operand reads free of bank conflicts.
//   * Two waves per SIMD (8-wave workgroups) for the large tiles, so one wave's
//     barrier or LDS wait is covered by the other's MFMAs. A wave stalls while it issues
//     a burst of fills, so with 8 waves only one wave per SIMD issues the refills; the
//     first stages, before any MFMA work exists, are filled by all of them.
//   * Workgroup ids are remapped so each of the 8 XCDs (own L2 each) walks a
//     contiguous, m-grouped range of tiles and concurrent tiles share panels in L2.
//   * The tile's scales and bias are requested at kernel start (one value per
//     thread), staged through LDS after the k loop, and applied in fp32 with a single
//     rounding to bf16. The bf16 tile is then staged through LDS as well, so the
//     output leaves in whole 128-byte lines (16 bytes per lane) instead of scattered
//     8-byte pieces.
//   * A single-launch form (FUSED, 256 x 256 tiles) takes the bf16 activation instead
//     of its codes: the option of one kernel for the run-time quantisation and the
//     GEMM that section 3.2 of the page points towards (quantisation and its memory
//     traffic as a cost of the FP8 path). Per-token scales need a token's whole row
//     before its first code and a tile needs all k of its tokens, so the first wave of
//     workgroups quantises the tokens in shares (the per-token quantiser's arithmetic,
//     bit for bit) and flags each share; every workgroup waits for the flags of the
//     shares holding its tile's tokens, then runs
//     its tile as above. The weight half of the first stages is requested before the
//     quantisation so it lands meanwhile.
#include <algorithm>

#include "internal.h"
#include "gemm_common.h"
#include "quant_row.h"

namespace fp8w8a8 {
namespace {

struct GemmArgs {
  const uint8_t* qa;
  const float* a_scale;
  const uint8_t* qw;
  const float* w_scale;
  const uint16_t* bias;  // may be null
  uint16_t* out;
  int m, n, k;
  int tiles_m, tiles_n;
  // single-launch form only: the bf16 activation, its per-token shares and their flags
  const uint16_t* a_bf16;
  uint8_t* qa_out;     // == qa
  float* a_scale_out;  // == a_scale
  unsigned long long* flags;
  unsigned long long epoch;
  int shares, rows_per_share;
};

constexpr int kScDevice = 16;  // cache-policy bit sc1: device-scope coherent access
constexpr uint64_t kStealAfterTicks = 10000;  // 100 us of the 100 MHz real-time clock

// Per-token results of the single-launch form are stored with device scope (sc1):
// written through the XCD's L2 to the device coherence point, and counted complete
// (vmcnt) only once visible there. A workgroup that has waited for its own stores can
// publish its flag without an L2 write-back (a release fence would write back the
// whole L2; issued by every workgroup at once that costs tens of microseconds).
struct DeviceScopeStore {
  __device__ __forceinline__ void codes(uint8_t* qr, int c, int nchunks, const uint4& v) const {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(qr, 0, nchunks * 16, kBufferConfig);
    const v4u data = {v.x, v.y, v.z, v.w};
    __builtin_amdgcn_raw_buffer_store_b128(data, r, c * 16, 0, kScDevice);
  }
  __device__ __forceinline__ void scale(float* srow, float s) const {
    __hip_atomic_store(reinterpret_cast<unsigned*>(srow), __float_as_uint(s), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
};

// Quantise the tokens of share `sh` (rows [sh * R, (sh + 1) * R) clipped to m), one
// wavefront per token, two tokens in flight per wavefront, then publish the share.
template <int NC, int WAVES>
__device__ __forceinline__ void quant_share_rows(const GemmArgs& args, int r_begin, int r_end, int wave, int lane) {
  const int K = args.k;
  const int nchunks = K >> 4;
  if constexpr (NC > 0) {
    for (int r = r_begin + wave; r < r_end; r += 2 * WAVES) {
      const int r2 = r + WAVES;
      uint4 va[NC], vb[NC], wa[NC], wb[NC];
      qrow::load_row<NC>(args.a_bf16 + (int64_t)r * K, nchunks, lane, va, vb);
      if (r2 < r_end) qrow::load_row<NC>(args.a_bf16 + (int64_t)r2 * K, nchunks, lane, wa, wb);
      qrow::quant_row<NC>(va, vb, nchunks, lane, args.qa_out + (int64_t)r * K, args.a_scale_out + r,
                          DeviceScopeStore{});
      if (r2 < r_end)
        qrow::quant_row<NC>(wa, wb, nchunks, lane, args.qa_out + (int64_t)r2 * K, args.a_scale_out + r2,
                            DeviceScopeStore{});
    }
  } else {
    for (int r = r_begin + wave; r < r_end; r += WAVES)
      qrow::quant_row_loop(args.a_bf16 + (int64_t)r * K, nchunks, lane, args.qa_out + (int64_t)r * K,
                           args.a_scale_out + r, qrow::NoMap{}, DeviceScopeStore{});
  }
}

template <int WAVES>
__device__ __forceinline__ void quant_share(const GemmArgs& args, int sh, int wave, int lane) {
  const int r_begin = min(sh * args.rows_per_share, args.m);
  const int r_end = min(r_begin + args.rows_per_share, args.m);
  const int nc = ((args.k >> 4) + 63) / 64;
  if (nc <= 1) quant_share_rows<1, WAVES>(args, r_begin, r_end, wave, lane);
  else if (nc <= 2) quant_share_rows<2, WAVES>(args, r_begin, r_end, wave, lane);
  else if (nc <= 4) quant_share_rows<4, WAVES>(args, r_begin, r_end, wave, lane);
  else if (nc <= 8) quant_share_rows<8, WAVES>(args, r_begin, r_end, wave, lane);
  else quant_share_rows<0, WAVES>(args, r_begin, r_end, wave, lane);
  wait_vm_lgkm0<0>();  // this wavefront's device-scope stores are complete
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(args.flags + sh, args.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until shares [sh_begin, sh_end) (those holding this tile's tokens) carry this
// launch's epoch. Wavefront 0 polls; a share still unpublished after kStealAfterTicks is
// quantised here as well (identical bytes, so a duplicate writer is harmless), so the
// wait ends even if the share's own workgroup is not resident. Ends with an agent-scope
// acquire so the GEMM reads see the shares.
template <int WAVES>
__device__ __forceinline__ void await_shares(const GemmArgs& args, int wave, int lane, int* slot, int sh_begin,
                                             int sh_end) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  while (true) {
    if (wave == 0) {
      int missing = -1;
      while (true) {
        int first = -1;
        for (int j0 = sh_begin; j0 < sh_end; j0 += 64) {
          const int j = j0 + lane;
          const bool miss =
              j < sh_end &&
              __hip_atomic_load(args.flags + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != args.epoch;
          const unsigned long long b = __ballot(miss);
          if (b != 0 && first < 0) first = j0 + __builtin_ctzll(b);
        }
        if (first < 0) break;
        if (__builtin_amdgcn_s_memrealtime() - t0 > kStealAfterTicks) {
          missing = first;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      if (lane == 0) *slot = missing;
    }
    __syncthreads();
    const int sh = __builtin_amdgcn_readfirstlane(*slot);
    __syncthreads();  // every wave has read the slot before wavefront 0 may rewrite it
    if (sh < 0) break;
    quant_share<WAVES>(args, sh, wave, lane);
  }
  if (wave == 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // L1 / L2 invalidate
  __syncthreads();
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, int BK, int GROUP_M, bool FUSED>
struct KernelTag {};

// FUSED: the single-launch form. The activation codes and scales do not exist yet at
// launch: the first `shares` workgroups quantise the bf16 activation into them
// (quant_share), every workgroup waits for the shares of its tile's tokens (await_shares), and the weight
// half of the first stages is requested before all that so it lands meanwhile.
template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, int BK, int GROUP_M, bool FUSED = false>
__global__ __launch_bounds__(WAVES_M* WAVES_N * 64) void gemm_fp8_kernel(GemmArgs args) {
  using Tag = KernelTag<BM, BN, WAVES_M, WAVES_N, STAGES, BK, GROUP_M, FUSED>;
  static_assert(BK == 64 || BK == 128, "stage depth in k bytes");
  constexpr int H = BK / 64;         // 32x32x64 MFMA k-steps per stage
  constexpr int CPR = BK / 16;       // 16-byte chunks per tile row
  constexpr int RPF = 64 / CPR;      // tile rows per wave-wide 1 KiB fill
  constexpr int kWaves = WAVES_M * WAVES_N;
  constexpr int WTM = BM / WAVES_M;  // wave tile along m (tokens)
  constexpr int WTN = BN / WAVES_N;  // wave tile along n (channels)
  constexpr int FM = WTM / 32;
  constexpr int FN = WTN / 32;
  constexpr int kStageBytes = (BM + BN) * BK;
  constexpr int kRowGroups = (BM + BN) / RPF;
  static_assert(BM % (32 * WAVES_M) == 0 && BN % (32 * WAVES_N) == 0, "tile / wave mismatch");
  static_assert(kRowGroups % kWaves == 0, "fill work must split evenly across waves");
  static_assert(STAGES >= 2 && STAGES <= 6, "stage count");
  constexpr int kEpiBytes = (BM + 2 * BN) * 4;  // the tile's a_scale, w_scale, bias (fp32)
  static_assert(STAGES * kStageBytes + kEpiBytes <= 160 * 1024, "LDS budget of a CU");
  // Which waves issue the DMA fills. A burst of fills stalls the issuing wave at issue
  // while the texture path drains them, and the matrix core idles if both waves of a
  // SIMD stall together. With 8 waves (two per SIMD) only waves 0..3, one per SIMD,
  // issue fills, so each SIMD keeps one wave free to feed its matrix core.
  constexpr int kFillWaves = kWaves == 8 ? kWaves / 2 : kWaves;
  constexpr int F = kRowGroups / kFillWaves;   // fills per filling wave per stage
  constexpr int FA = (BM / RPF) / kFillWaves;  // of which activation rows
  static_assert(kRowGroups % kFillWaves == 0, "fill work must split evenly across the filling waves");
  static_assert((BM / RPF) % kFillWaves == 0, "activation fills split evenly across the filling waves");
  static_assert((STAGES - 1) * F < 64, "vmcnt range");
  // With two stages of 128-byte k and half the waves filling, a stage's refill goes out
  // in two halves: the activation rows right after the stage barrier, the weight rows
  // one MFMA k-step later (they still land before the next barrier).
  constexpr bool kSplitRefill = STAGES == 2 && H == 2 && kFillWaves < kWaves;
  static_assert(BM <= kWaves * 64 && BN <= kWaves * 64, "one epilogue operand per thread");
  static_assert(!FUSED || STAGES == 2, "the single-launch prologue's fill order assumes two stages");

  auto buf = [](int s) -> uint8_t* {
    switch (s) {
      case 0: return stage_buf<Tag, 0, kStageBytes>();
      case 1: return stage_buf<Tag, 1, kStageBytes>();
      case 2: return stage_buf<Tag, 2 % STAGES, kStageBytes>();
      case 3: return stage_buf<Tag, 3 % STAGES, kStageBytes>();
      case 4: return stage_buf<Tag, 4 % STAGES, kStageBytes>();
      default: return stage_buf<Tag, 5 % STAGES, kStageBytes>();
    }
  };

  const int lane = threadIdx.x & 63;
  int tm, tn;
  tile_coords<GROUP_M>(args.tiles_m, args.tiles_n, tm, tn);
  tm = __builtin_amdgcn_readfirstlane(tm);  // uniform by construction; keep it in SGPRs
  tn = __builtin_amdgcn_readfirstlane(tn);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave % WAVES_M, wn = wave / WAVES_M;
  const int m0 = tm * BM, n0 = tn * BN;
  const int K = args.k;
  const int rows_a = min(BM, args.m - m0);
  const int rows_w = min(BN, args.n - n0);
  const v4i rsrc_a = make_rsrc(args.qa + (int64_t)m0 * K, (uint32_t)rows_a * (uint32_t)K);
  const v4i rsrc_w = make_rsrc(args.qw + (int64_t)n0 * K, (uint32_t)rows_w * (uint32_t)K);

  // Epilogue operands of this tile, one value per thread, requested now; they arrive
  // with the first stage and are parked in LDS, so they hold no registers during the
  // k loop.
  float* const epi_sa = reinterpret_cast<float*>(stage_buf<Tag, 7, kEpiBytes>());
  float* const epi_sw = epi_sa + BM;
  float* const epi_b = epi_sw + BN;
  const int tid = threadIdx.x;
  const bool filler = wave < kFillWaves;
  float pre_sa = 0.0f, pre_sw = 0.0f, pre_b = 0.0f;
  if constexpr (!FUSED)
    if (tid < BM && tid < rows_a) pre_sa = args.a_scale[m0 + tid];
  if (tid < BN && tid < rows_w) {
    pre_sw = args.w_scale[n0 + tid];
    if (args.bias) pre_b = __uint_as_float((uint32_t)args.bias[n0 + tid] << 16);
  }

  // Fill geometry: a wave-wide fill covers RPF rows x BK bytes = 1 KiB of a stage;
  // lane i writes bytes [16 i, 16 i + 16): row i / CPR of the group, position i % CPR,
  // which holds logical chunk (i % CPR) ^ swz(row). swz depends on row % 16, so with
  // 8-row fills (BK = 128) the chunk differs between even and odd row groups. Tile rows
  // 0..BM-1 are the activation, BM.. the weight; filling wave w fills row groups w,
  // w + kFillWaves, ...
  const int fr = lane / CPR;
  const int fchunk0_ = (lane % CPR) ^ swz<BK>(fr);            // row group with g * RPF % 16 == 0
  const int fchunk1_ = (lane % CPR) ^ swz<BK>(fr + RPF % 16);  // row group with g * RPF % 16 == 8
  const uint32_t foff0_ = (uint32_t)fr * (uint32_t)K + 16u * (uint32_t)fchunk0_;
  const uint32_t foff1_ = (uint32_t)fr * (uint32_t)K + 16u * (uint32_t)fchunk1_;

  // part: 0 = the whole stage, 1 = activation rows only, 2 = weight rows only
  auto issue = [&](uint8_t* base, int k0, int part = 0) {
    if (!filler) return;
    int fchunk0 = fchunk0_, fchunk1 = fchunk1_;
    uint32_t foff0 = foff0_, foff1 = foff1_;
    if constexpr (FUSED) {
      // formed here from a fresh lane id: kept live across the quantisation phase they
      // would be spilled, and every refill would wait for the reload
      int l;
      asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
      const int r = l / CPR;
      fchunk0 = (l % CPR) ^ swz<BK>(r);
      fchunk1 = (l % CPR) ^ swz<BK>(r + RPF % 16);
      foff0 = (uint32_t)r * (uint32_t)K + 16u * (uint32_t)fchunk0;
      foff1 = (uint32_t)r * (uint32_t)K + 16u * (uint32_t)fchunk1;
    }
    const bool kvalid0 = k0 + 16 * fchunk0 < K;
    const bool kvalid1 = k0 + 16 * fchunk1 < K;
#pragma unroll
    for (int j = 0; j < F; ++j) {
      if ((part == 1 && j >= FA) || (part == 2 && j < FA)) continue;
      const int g = wave + j * kFillWaves;
      const bool odd = ((g * RPF) & 15) != 0;
      const bool kvalid = odd ? kvalid1 : kvalid0;
      const uint32_t foff = odd ? foff1 : foff0;
      const uint32_t dst = (uint32_t)reinterpret_cast<uintptr_t>(base + g * 1024);
      if (j < FA) {
        const uint32_t vo = kvalid ? (uint32_t)(g * RPF) * (uint32_t)K + foff + (uint32_t)k0 : kOutOfRange;
        dma16(rsrc_a, dst, vo);
      } else {
        const uint32_t vo = kvalid ? (uint32_t)(g * RPF - BM) * (uint32_t)K + foff + (uint32_t)k0 : kOutOfRange;
        dma16(rsrc_w, dst, vo);
      }
    }
  };

  // The first stages' fills, before any wave has MFMA work to keep fed, come from every
  // wave: FW per wave per stage instead of F from each filling wave (so the first stage
  // boundary waits for FW-sized stages, every later one for F-sized refills).
  constexpr bool kPrologueAll = !FUSED && kFillWaves < kWaves;
  constexpr int FW = kRowGroups / kWaves;
  constexpr int FAW = (BM / RPF) / kWaves;
  static_assert(!kPrologueAll || (kRowGroups % kWaves == 0 && (BM / RPF) % kWaves == 0),
                "prologue fills split evenly");
  auto issue_all = [&](uint8_t* base, int k0) {
    const bool kvalid0 = k0 + 16 * fchunk0_ < K;
    const bool kvalid1 = k0 + 16 * fchunk1_ < K;
#pragma unroll
    for (int j = 0; j < FW; ++j) {
      const int g = wave + j * kWaves;
      const bool odd = ((g * RPF) & 15) != 0;
      const bool kvalid = odd ? kvalid1 : kvalid0;
      const uint32_t foff = odd ? foff1_ : foff0_;
      const uint32_t dst = (uint32_t)reinterpret_cast<uintptr_t>(base + g * 1024);
      if (j < FAW) {
        const uint32_t vo = kvalid ? (uint32_t)(g * RPF) * (uint32_t)K + foff + (uint32_t)k0 : kOutOfRange;
        dma16(rsrc_a, dst, vo);
      } else {
        const uint32_t vo = kvalid ? (uint32_t)(g * RPF - BM) * (uint32_t)K + foff + (uint32_t)k0 : kOutOfRange;
        dma16(rsrc_w, dst, vo);
      }
    }
  };

  // Operand reads for the 32x32x64 MFMA k-step h of a stage: lane l holds row l % 32 of
  // a 32-row fragment, k bytes 64 h + [32 (l/32), +32) = logical chunks
  // 4 h + 2 (l/32) and 4 h + 2 (l/32) + 1.
  const int rrow = lane & 31;
  const int rkq = lane >> 5;
  const int rf = swz<BK>(rrow);
  uint32_t rd0[H], rd1[H];
#pragma unroll
  for (int h = 0; h < H; ++h) {
    rd0[h] = (uint32_t)rrow * BK + 16u * (uint32_t)((4 * h + 2 * rkq) ^ rf);
    rd1[h] = (uint32_t)rrow * BK + 16u * (uint32_t)((4 * h + 2 * rkq + 1) ^ rf);
  }

  v16f acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // Operand fragments of one MFMA k-step: FM activation and FN weight fragments.
  struct Frags {
    v8i a[FM];
    v8i w[FN];
  };
  auto read_frags = [&](const uint8_t* base, int h, Frags& f) {
    const uint8_t* sa = base + (wm * WTM) * BK;
    const uint8_t* sw = base + (BM + wn * WTN) * BK;
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const uint4 lo = *reinterpret_cast<const uint4*>(sa + j * 32 * BK + rd0[h]);
      const uint4 hi = *reinterpret_cast<const uint4*>(sa + j * 32 * BK + rd1[h]);
      f.a[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const uint4 lo = *reinterpret_cast<const uint4*>(sw + i * 32 * BK + rd0[h]);
      const uint4 hi = *reinterpret_cast<const uint4*>(sw + i * 32 * BK + rd1[h]);
      f.w[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
  };
  auto mfma_all = [&](const Frags& f) {
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.w[i], f.a[j], acc[i][j], 0, 0, 0, 0, 0, 0);
  };

  // Software pipeline over MFMA k-steps u = H t + h (stage t, half h). Stage t lives in
  // buffer t % STAGES; all STAGES buffers are in flight from the start. Sub-step u
  // multiplies the fragments of u (already in registers) while it reads those of u + 1
  // from LDS, interleaved instruction by instruction. Before the read crosses into
  // stage t + 1, a wait + barrier publishes stage t + 1 and confirms every wave has
  // finished reading stage t, whose buffer is then refilled with stage t + STAGES.
  const int nst = (K + BK - 1) / BK;
  const int nsub = nst * H;
  Frags f0, f1;
  if constexpr (FUSED) {
    // weight fills first; the activation codes are produced in this launch
#pragma unroll
    for (int s = 0; s < STAGES; ++s)
      if (s < nst) issue(buf(s), s * BK, 2);
    __shared__ int steal_slot;
    if (blockIdx.x < (unsigned)args.shares) quant_share<kWaves>(args, blockIdx.x, wave, lane);
    // only the shares holding this tile's tokens: a tile whose rows are ready starts
    // without waiting for the slowest share elsewhere
    const int sh_begin = m0 / args.rows_per_share;
    const int sh_end = min(args.shares, (m0 + rows_a + args.rows_per_share - 1) / args.rows_per_share);
    await_shares<kWaves>(args, wave, lane, &steal_slot, sh_begin, sh_end);
    if (tid < BM && tid < rows_a) pre_sa = args.a_scale[m0 + tid];
#pragma unroll
    for (int s = 0; s < STAGES; ++s)
      if (s < nst) issue(buf(s), s * BK, 1);
    // stage 0 is complete once at most the younger stage's activation fills remain
    if (filler && nst > 1) wait_vm_lgkm0<FA>();
    else wait_vm_lgkm0<0>();
  } else if constexpr (kPrologueAll) {
#pragma unroll
    for (int s = 0; s < STAGES; ++s)
      if (s < nst) issue_all(buf(s), s * BK);
    wait_stage<FW, STAGES>(min(nst - 1, STAGES - 1));
  } else {
#pragma unroll
    for (int s = 0; s < STAGES; ++s)
      if (s < nst) issue(buf(s), s * BK);
    if (filler) wait_stage<F, STAGES>(min(nst - 1, STAGES - 1));
    else wait_vm_lgkm0<0>();
  }
  // the epilogue operands were requested before the fills: the wait covered them
  if (tid < BM) epi_sa[tid] = pre_sa;
  if (tid < BN) {
    epi_sw[tid] = pre_sw;
    epi_b[tid] = pre_b;
  }
  block_barrier();
  read_frags(buf(0), 0, f0);

  auto sub = [&](int u, int s, int h, Frags& cur, Frags& nxt) {
    // s = stage index of u modulo STAGES, h = half of u (compile-time after unrolling)
    const int t = u / H;
    if (h == H - 1) {
      if (t + 1 < nst) {
        // stage t + 1 complete: the first stages came from every wave (FW each), later
        // ones from the filling waves (F each)
        if (kPrologueAll && t == 0) wait_stage<FW, STAGES>(min(nst - 2, STAGES - 2));
        else if (filler) wait_stage<F, STAGES>(min(nst - 2 - t, STAGES - 2));
        else wait_vm_lgkm0<0>();
        block_barrier();
        if (t + STAGES < nst) issue(buf(s), (t + STAGES) * BK, kSplitRefill ? 1 : 0);
      }
      read_frags(buf((s + 1) % STAGES), 0, nxt);
    } else {
      // the second half of the refill issued at the previous stage barrier
      if (kSplitRefill && t >= 1 && t + 1 < nst) issue(buf((s + 1) % STAGES), (t + 1) * BK, 2);
      read_frags(buf(s), h + 1, nxt);
    }
    mfma_all(cur);
    interleave_mfma_ds_read<FM * FN, 2 * (FM + FN)>();
  };
  constexpr int kUnroll = 2 * STAGES * H;  // whole stage ring, even number of sub-steps
  for (int u0 = 0; u0 < nsub; u0 += kUnroll) {
#pragma unroll
    for (int v = 0; v < kUnroll; v += 2) {
      if (u0 + v < nsub) sub(u0 + v, (v / H) % STAGES, v % H, f0, f1);
      if (u0 + v + 1 < nsub) sub(u0 + v + 1, ((v + 1) / H) % STAGES, (v + 1) % H, f1, f0);
    }
  }

  // Epilogue. The stage buffers are free once every wave has passed this barrier.
  // 1. Pull each lane's share of the tile's scales and bias from LDS into registers
  //    (the operand fragments are dead by now).
  // 2. Each wave applies them to its accumulators in fp32, rounds once to bf16 and
  //    writes its WTM x WTN tile row-major into its own LDS region (16-byte chunk c of
  //    row r at chunk position c ^ (r % RC)).
  // 3. Each wave reads its region back a row segment per lane group and stores whole
  //    rows (16 bytes per lane, full 128-byte lines) to the output.
  constexpr int RC = WTN / 8;                     // 16-byte chunks in a wave-tile row
  constexpr int kWaveOutBytes = WTM * WTN * 2;
  constexpr int kWavesPerBuf = kStageBytes / kWaveOutBytes;
  static_assert(kWavesPerBuf >= 1 && (kWaves + kWavesPerBuf - 1) / kWavesPerBuf <= STAGES,
                "output staging fits in the stage buffers");
  static_assert(64 % RC == 0 && (WTM * RC) % 64 == 0, "row segments tile the wavefront");
  float r_sa[FM];
  float4 r_sw[FN][4], r_b[FN][4];
#pragma unroll
  for (int j = 0; j < FM; ++j) r_sa[j] = epi_sa[wm * WTM + j * 32 + (lane & 31)];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int nl = wn * WTN + i * 32 + 8 * q + 4 * (lane >> 5);
      r_sw[i][q] = *reinterpret_cast<const float4*>(epi_sw + nl);
      r_b[i][q] = *reinterpret_cast<const float4*>(epi_b + nl);
    }
  wait_vm_lgkm0<63>();
  block_barrier();

  uint8_t* wout = buf(wave / kWavesPerBuf) + (wave % kWavesPerBuf) * kWaveOutBytes;
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    const int r = j * 32 + (lane & 31);  // row within the wave tile
    const float sa = r_sa[j];
#pragma unroll
    for (int i = 0; i < FN; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c8 = i * 32 + 8 * q + 4 * (lane >> 5);  // column within the wave tile
        const float4 sw4 = r_sw[i][q];
        const float4 b4 = r_b[i][q];
        const v16f& a = acc[i][j];
        const float o0 = __builtin_fmaf(a[4 * q + 0] * sa, sw4.x, b4.x);
        const float o1 = __builtin_fmaf(a[4 * q + 1] * sa, sw4.y, b4.y);
        const float o2 = __builtin_fmaf(a[4 * q + 2] * sa, sw4.z, b4.z);
        const float o3 = __builtin_fmaf(a[4 * q + 3] * sa, sw4.w, b4.w);
        const int chunk = c8 >> 3, half = (c8 >> 2) & 1;
        *reinterpret_cast<uint2*>(wout + r * (RC * 16) + ((chunk ^ (r % RC)) << 4) + (half << 3)) =
            make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
      }
    }
  }
  // own region only: LDS executes one wave's accesses in order, no barrier needed
  store_wave_tile<WTM, RC>(wout, lane, args.out, args.m, args.n, m0 + wm * WTM, n0 + wn * WTN);
}

template <int BM, int BN, int WM, int WN, int S, int BK, int GM, bool FUSED = false>
hipError_t launch(const GemmArgs& a, hipStream_t stream) {
  GemmArgs args = a;
  args.tiles_m = (a.m + BM - 1) / BM;
  args.tiles_n = (a.n + BN - 1) / BN;
  const int64_t wgs = (int64_t)args.tiles_m * args.tiles_n;
  gemm_fp8_kernel<BM, BN, WM, WN, S, BK, GM, FUSED><<<dim3((unsigned)wgs), dim3(WM * WN * 64), 0, stream>>>(args);
  return hipGetLastError();
}

// id, tile_m, tile_n, waves, stages, name (every stage holds 128 bytes of k)
const GemmConfig kConfigs[] = {
    {0, 256, 256, 8, 2, "bm256_bn256_w2x4_s2"},
    {1, 256, 128, 8, 3, "bm256_bn128_w4x2_s3"},
    {2, 128, 256, 8, 3, "bm128_bn256_w2x4_s3"},
    {3, 128, 128, 4, 2, "bm128_bn128_w2x2_s2"},
    {4, 64, 64, 4, 3, "bm64_bn64_w2x2_s3"},
};
constexpr int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);

}  // namespace

int gemm_config_count() { return kNumConfigs; }

const GemmConfig* gemm_config(int id) { return (id >= 0 && id < kNumConfigs) ? &kConfigs[id] : nullptr; }

int64_t gemm_workgroups(int id, int64_t m, int64_t n) {
  const GemmConfig* c = gemm_config(id);
  if (!c) return 0;
  return ((m + c->tile_m - 1) / c->tile_m) * ((n + c->tile_n - 1) / c->tile_n);
}

int gemm_threads(int id) {
  const GemmConfig* c = gemm_config(id);
  return c ? c->waves * 64 : 0;
}

hipError_t launch_gemm(int id, int64_t m, int64_t n, int64_t k, const uint8_t* qa, const float* a_scale,
                       const uint8_t* qw, const float* w_scale, const uint16_t* bias, uint16_t* out,
                       hipStream_t stream) {
  GemmArgs a{qa, a_scale, qw, w_scale, bias, out, (int)m, (int)n, (int)k, 0, 0};
  switch (id) {
    case 0: return launch<256, 256, 2, 4, 2, 128, 4>(a, stream);
    case 1: return launch<256, 128, 4, 2, 3, 128, 4>(a, stream);
    case 2: return launch<128, 256, 2, 4, 3, 128, 8>(a, stream);  // groups of 8: FFN-down 64.3 -> 63.4 us
    case 3: return launch<128, 128, 2, 2, 2, 128, 8>(a, stream);
    case 4: return launch<64, 64, 2, 2, 3, 128, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_quant_gemm(int64_t m, int64_t n, int64_t k, const uint16_t* a_bf16, uint8_t* qa_ws, float* sa_ws,
                             unsigned long long* flags, unsigned long long epoch, const uint8_t* qw,
                             const float* w_scale, const uint16_t* bias, uint16_t* out, int cus, hipStream_t stream) {
  GemmArgs a{qa_ws, sa_ws, qw, w_scale, bias, out, (int)m, (int)n, (int)k, 0, 0};
  a.a_bf16 = a_bf16;
  a.qa_out = qa_ws;
  a.a_scale_out = sa_ws;
  a.flags = flags;
  a.epoch = epoch;
  // one share per workgroup of the first wave (one 256 x 256 workgroup per CU)
  const int64_t tiles = gemm_workgroups(0, m, n);
  a.shares = (int)std::min<int64_t>({tiles, (int64_t)cus, (int64_t)kQuantGemmMaxWorkgroups});
  a.rows_per_share = (int)((m + a.shares - 1) / a.shares);
  return launch<256, 256, 2, 4, 2, 128, 4, true>(a, stream);
}

}  // namespace fp8w8a8
