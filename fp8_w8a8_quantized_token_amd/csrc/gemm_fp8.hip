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
//   * A skinny form for a few dozen tokens (the 26-row encoder input of the QKV
//     projections): a weight stream over many workgroups with k split across waves and
//     operands loaded straight into registers (gemm_fp8_skinny below).
//   * A persistent form of the 256 x 256 tiles (PERSIST): one workgroup per CU walks
//     its tiles and requests the next tile's first two stages as soon as the current
//     tile's k loop is done, so they land during its epilogue instead of after it. It
//     computes exactly what configuration 0 computes, in the same order.
//   * Groups (section 3.4 of the page: the hidden states feed the Q, K and V
//     projections): up to kMaxGroup problems that share the activation codes run as one
//     launch of the persistent or of the skinny form, their column blocks side by side;
//     each tile looks up its problem's weight, scales, bias, output and width. Each tile
//     computes what the problem's own launch computes, bit for bit.
#include <algorithm>

#include "internal.h"
#include "gemm_common.h"
#include "quant_row.h"

namespace fp8w8a8 {
namespace {

// The persistent form runs up to kMaxGroup problems in one launch (see gemm_fp8_kernel).
constexpr int kMaxGroup = FP8W8A8_MAX_GROUP;

// Kernel forms by how workgroups map to tiles: one tile each; persistent over one
// problem (the launch's own weight and output); persistent over a group of problems.
// The single-problem persistent form is its own instantiation: finding a tile's problem
// costs a dependent scalar load at every tile, measurable (about 1 %) on its own.
constexpr int kPersistNone = 0, kPersistOne = 1, kPersistGroup = 2;

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
  // grouped persistent form: problems 0 .. ngroup - 1 share qa, a_scale, m and k; problem p
  // has its own weight, w_scale, bias, output and n, and owns the global tile columns
  // [g_tn_end[p - 1], g_tn_end[p]) (from 0 for p = 0). Unused by the other forms.
  int ngroup;
  int g_tn_end[kMaxGroup];
  int g_n[kMaxGroup];
  const uint8_t* g_qw[kMaxGroup];
  const float* g_ws[kMaxGroup];
  const uint16_t* g_bias[kMaxGroup];
  uint16_t* g_out[kMaxGroup];
};

// The kernel's arguments read afresh from the kernel-argument segment. The address goes
// through an empty asm, so the compiler cannot reuse the values it loaded at the start:
// a persistent workgroup that needs them again only after its k loop does not hold them
// in scalar registers through it.
typedef const __attribute__((address_space(4))) GemmArgs* KernargGemmArgs;
__device__ __forceinline__ KernargGemmArgs kernarg_args() {
  uint64_t p = reinterpret_cast<uint64_t>(__builtin_amdgcn_kernarg_segment_ptr());
  asm volatile("" : "+s"(p));
  // (the compiler takes an asm result as divergent; the address is uniform)
  p = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p) |
      ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32)) << 32);
  return reinterpret_cast<KernargGemmArgs>(p);
}
__device__ __forceinline__ GemmArgs reload_args() {
  const KernargGemmArgs k = kernarg_args();
  GemmArgs r{};
  r.qa = k->qa;
  r.a_scale = k->a_scale;
  r.qw = k->qw;
  r.w_scale = k->w_scale;
  r.bias = k->bias;
  r.out = k->out;
  r.m = k->m;
  r.n = k->n;
  r.k = k->k;
  r.tiles_m = k->tiles_m;
  r.tiles_n = k->tiles_n;
  r.shares = k->shares;
  return r;
}

// The problem a global tile column belongs to (persistent form), and the tile's first
// column within that problem's output.
struct TileProblem {
  const uint8_t* qw;
  const float* ws;
  const uint16_t* bias;
  uint16_t* out;
  int n, n0;
};
template <int BN, bool GROUPED>
__device__ __forceinline__ TileProblem tile_problem(KernargGemmArgs k, int tn) {
  if constexpr (!GROUPED) return TileProblem{k->qw, k->w_scale, k->bias, k->out, k->n, tn * BN};
  int p = 0, first = 0;
#pragma unroll
  for (int i = 0; i + 1 < kMaxGroup; ++i)
    if (i + 1 < k->ngroup && tn >= k->g_tn_end[i]) {
      p = i + 1;
      first = k->g_tn_end[i];
    }
  TileProblem r;
  r.qw = k->g_qw[p];
  r.ws = k->g_ws[p];
  r.bias = k->g_bias[p];
  r.out = k->g_out[p];
  r.n = k->g_n[p];
  r.n0 = (tn - first) * BN;
  return r;
}

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

template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, int BK, int GROUP_M, bool FUSED, int PERSIST,
          bool W_FIRST>
struct KernelTag {};

// FUSED: the single-launch form. The activation codes and scales do not exist yet at
// launch: the first `shares` workgroups quantise the bf16 activation into them
// (quant_share), every workgroup waits for the shares of its tile's tokens (await_shares), and the weight
// half of the first stages is requested before all that so it lands meanwhile.
//
// PERSIST: one workgroup per CU walks tiles blockIdx.x, blockIdx.x + gridDim.x, ... . Once
// a tile's k loop has passed its last barrier the stage ring is free, so the next tile's
// first two stages are requested right then and land while this tile's epilogue runs.
// The epilogue therefore cannot stage its output in the ring: it goes through a region
// of its own (4 KiB per wave, which also holds the tile's epilogue operands between
// tiles), 32 token rows per wave at a time, and issues exactly kEpiStores stores per
// wave, so that the wait for the next tile's stages (older than the stores) is an exact
// count.
template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, int BK, int GROUP_M, bool FUSED = false,
          int PERSIST = kPersistNone, bool W_FIRST = false>
__global__ __launch_bounds__(WAVES_M* WAVES_N * 64) void gemm_fp8_kernel(GemmArgs args) {
  using Tag = KernelTag<BM, BN, WAVES_M, WAVES_N, STAGES, BK, GROUP_M, FUSED, PERSIST, W_FIRST>;
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
  // the tile's epilogue operands in LDS: a_scale [BM] and w_scale [BN] (fp32), bias [BN]
  // (bf16), each region a whole number of 256-byte DMA chunks
  constexpr int kEpiBiasBytes = (BN * 2 + 255) / 256 * 256;
  constexpr int kEpiBytes = (BM + BN) * 4 + kEpiBiasBytes;
  static_assert(BM % 64 == 0 && BN % 64 == 0, "whole DMA chunks of scales");
  // PERSIST's output staging: 32 token rows of the wave tile per wave; the epilogue
  // operands share the region (they are in registers while it holds output)
  constexpr int kPieceRows = 32;
  constexpr int kPieceBytes = kPieceRows * (BN / WAVES_N) * 2;
  constexpr int kStagingBytes = PERSIST ? kWaves * kPieceBytes : 0;
  static_assert(!PERSIST || kEpiBytes <= kStagingBytes, "epilogue operands fit in the staging region");
  static_assert(STAGES * kStageBytes + (PERSIST ? kStagingBytes : kEpiBytes) <= 160 * 1024, "LDS budget of a CU");
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
  // A fill's offset is its lane base plus its row offset (< max(BM, BN) * k <= 2^28 bytes);
  // from kOutOfRange (2^31) it stays below 2^32 and past every descriptor's end (<= 2^28).
  static_assert((int64_t)(BM > BN ? BM : BN) * FP8W8A8_MAX_DIM <= (int64_t)1 << 28 && kOutOfRange == 0x80000000u,
                "out-of-range offsets stay out of range");
  // With two stages of 128-byte k and half the waves filling, a stage's refill goes out
  // in two halves: the activation rows right after the stage barrier, the weight rows
  // one MFMA k-step later (they still land before the next barrier).
  constexpr bool kSplitRefill = STAGES == 2 && H == 2 && kFillWaves < kWaves;
  // W_FIRST: the weight rows of a split refill go out at the stage barrier and the
  // activation rows one k-step later (else the other way round). The launcher sends the
  // operand with more bytes in all first: its slices are the likelier L2 misses and need
  // the longer lead (FFN-up, n = 2 m: 65.8 -> 64.8 us; 32760 x 2048 x 2048 with the
  // weights first: 127.7 -> 132.0 us).
  constexpr int kRefillFirst = W_FIRST ? 2 : 1;
  static_assert(BM <= kWaves * 64 && BN <= kWaves * 64, "one epilogue operand per thread");
  static_assert(!FUSED || STAGES == 2, "the single-launch prologue's fill order assumes two stages");
  static_assert(!PERSIST || (!FUSED && STAGES == 2 && kWaves == 8),
                "the persistent form hands the two-stage ring of the 8-wave tile to the next tile");

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
  const int ntiles = args.tiles_m * args.tiles_n;
  int vtile = blockIdx.x;  // PERSIST: the logical tile this workgroup works on
  int tm, tn;
  if constexpr (PERSIST) tile_coords_at<GROUP_M>(vtile, ntiles, args.tiles_m, args.tiles_n, tm, tn);
  else tile_coords<GROUP_M>(args.tiles_m, args.tiles_n, tm, tn);
  tm = __builtin_amdgcn_readfirstlane(tm);  // uniform by construction; keep it in SGPRs
  tn = __builtin_amdgcn_readfirstlane(tn);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave % WAVES_M, wn = wave / WAVES_M;
  // the weight side of this tile: the launch's own, or (PERSIST) its problem's
  const uint8_t* w_base = args.qw;
  const float* ws_base = args.w_scale;
  const uint16_t* b_base = args.bias;
  int n_cur = args.n;
  int n0 = tn * BN;
  if constexpr (PERSIST) {
    const TileProblem pr = tile_problem<BN, PERSIST == kPersistGroup>(kernarg_args(), tn);
    w_base = pr.qw;
    ws_base = pr.ws;
    b_base = pr.bias;
    n_cur = pr.n;
    n0 = pr.n0;
  }
  int m0 = tm * BM;
  const int K = args.k;
  int rows_a = min(BM, args.m - m0);
  int rows_w = min(BN, n_cur - n0);
  v4i rsrc_a = make_rsrc(args.qa + (int64_t)m0 * K, (uint32_t)rows_a * (uint32_t)K);
  v4i rsrc_w = make_rsrc(w_base + (int64_t)n0 * K, (uint32_t)rows_w * (uint32_t)K);

  // Epilogue operands of this tile, parked in LDS so they hold no registers during the
  // k loop.
  uint8_t* epi_base;
  if constexpr (PERSIST) epi_base = stage_buf<Tag, 8, kStagingBytes>();
  else epi_base = stage_buf<Tag, 7, kEpiBytes>();
  float* const epi_sa = reinterpret_cast<float*>(epi_base);
  float* const epi_sw = epi_sa + BM;
  uint16_t* const epi_b16 = reinterpret_cast<uint16_t*>(epi_sw + BN);
  const int tid = threadIdx.x;
  const bool filler = wave < kFillWaves;
  // They come by 4-byte LDS DMA, issued by the filling waves before the tile's fills:
  // 256-byte chunks (one wave-wide load each), a_scale first, then w_scale, then the bias;
  // rows and channels past the tile's valid ones, and a missing bias, read zeros. Loaded
  // into registers instead, they would be the only memory reads the compiler counts, and
  // its wait for them (vmcnt(0): it cannot see the fills) would hold the first fills back
  // by a whole memory round trip and then wait for every fill of the prologue.
  constexpr int kEpiChunksA = BM / 64, kEpiChunksW = BN / 64;
  constexpr int kEpiChunks = kEpiChunksA + kEpiChunksW + kEpiBiasBytes / 256;
  auto issue_epi = [&](const float* a_scale, const float* w_scale, const uint16_t* bias, int em0, int en0,
                       int erows_a, int erows_w) {
    if (!filler) return;
    const v4i rs_a = make_rsrc(a_scale + em0, (uint32_t)erows_a * 4u);
    const v4i rs_w = make_rsrc(w_scale + en0, (uint32_t)erows_w * 4u);
    const v4i rs_b = make_rsrc(bias ? bias + en0 : nullptr, bias ? (uint32_t)erows_w * 2u : 0u);
    const uint32_t vo = 4u * (uint32_t)lane;
#pragma unroll
    for (int c0 = 0; c0 < kEpiChunks; c0 += kFillWaves) {
      const int c = c0 + wave;  // uniform
      if (c >= kEpiChunks) break;
      const uint32_t dst = (uint32_t)reinterpret_cast<uintptr_t>(epi_base + 256 * c);
      if (c < kEpiChunksA) dma4(rs_a, dst, vo + 256u * (uint32_t)c);
      else if (c < kEpiChunksA + kEpiChunksW) dma4(rs_w, dst, vo + 256u * (uint32_t)(c - kEpiChunksA));
      else dma4(rs_b, dst, vo + 256u * (uint32_t)(c - kEpiChunksA - kEpiChunksW));
    }
  };
  // (the single-launch form loads them into registers: its a_scale exists only after
  // the quantisation phase, and it waits for everything before its k loop anyway)
  float pre_sa = 0.0f, pre_sw = 0.0f;
  uint32_t pre_b = 0;
  if constexpr (FUSED)
    if (tid < BN && tid < rows_w) {
      pre_sw = args.w_scale[n0 + tid];
      if (args.bias) pre_b = args.bias[n0 + tid];
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
  // (PERSIST passes these, and the wave index and k the fills use, through an empty asm
  // at each tile so the compiler does not keep the per-fill offsets and LDS addresses
  // derived from them alive across the epilogue)
  uint32_t foff0_ = (uint32_t)fr * (uint32_t)K + 16u * (uint32_t)fchunk0_;
  uint32_t foff1_ = (uint32_t)fr * (uint32_t)K + 16u * (uint32_t)fchunk1_;
  int fwave = wave, fK = K;  // the fills' copies (same laundering)

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
    const bool kvalid0 = k0 + 16 * fchunk0 < fK;
    const bool kvalid1 = k0 + 16 * fchunk1 < fK;
    if constexpr (PERSIST) {
      // Every fill of this wave has the same row parity (its row groups step by
      // kFillWaves * RPF rows, a multiple of 16) and the activation and weight halves
      // start at the same row offset, so one base per stage plus a multiple of a scalar
      // stride gives every fill's offset: one register, where one per fill held through
      // the k loop leaves the loop short of registers once it sits inside the tile loop.
      static_assert((kFillWaves * RPF) % 16 == 0 && FA * kFillWaves * RPF == BM, "one offset chain");
      const bool odd = ((fwave * RPF) & 15) != 0;
      const bool kvalid = odd ? kvalid1 : kvalid0;
      // (a lane past k starts from kOutOfRange; every fill's offset stays past the end)
      const uint32_t v0 =
          kvalid ? (uint32_t)(fwave * RPF) * (uint32_t)fK + (odd ? foff1 : foff0) + (uint32_t)k0 : kOutOfRange;
      uint32_t kk = (uint32_t)fK;
      asm volatile("" : "+s"(kk));
      kk = (uint32_t)__builtin_amdgcn_readfirstlane((int)kk);
      // Fill j's first row lies (j mod FA) * kFillWaves * RPF rows (< 2^8) past the base,
      // and k < 2^24, so the row offset is an exact 24-bit product: a full-rate
      // multiply-add per fill (a 32-bit product becomes a quarter-rate 64-bit one; every
      // formulation with plain adds measured here tipped the loop into spilling).
      static_assert((FA - 1) * kFillWaves * RPF < (1 << 8) && FP8W8A8_MAX_DIM < (1 << 24), "24-bit row offsets");
#pragma unroll
      for (int j = 0; j < F; ++j) {
        if ((part == 1 && j >= FA) || (part == 2 && j < FA)) continue;
        const int g = fwave + j * kFillWaves;
        const uint32_t dst = (uint32_t)reinterpret_cast<uintptr_t>(base + g * 1024);
        const uint32_t vo = v0 + __umul24(kk, (uint32_t)((j < FA ? j : j - FA) * kFillWaves * RPF));
        dma16(j < FA ? rsrc_a : rsrc_w, dst, vo);
      }
      return;
    }
    if constexpr (kFillWaves < kWaves) {
      // One lane base per call: the fills' row groups step by kFillWaves * RPF rows, a
      // multiple of 16, so all of them share the first one's row parity (swizzle) and k
      // validity; each fill adds its uniform row offset. A lane past k starts from
      // kOutOfRange, and every offset then stays past the descriptor's end. (Half the
      // waves fill here, and the select per fill it saves sits on their path to the stage
      // barrier: FFN-down on 128 x 256 tiles 63.5 -> 62.4 us. With every wave filling, the
      // 128 x 128 tiles measured 4% slower this way, so they keep the select per fill.)
      static_assert((kFillWaves * RPF) % 16 == 0, "one row parity per filling wave");
      const bool odd = ((fwave * RPF) & 15) != 0;
      const uint32_t vbase = (odd ? kvalid1 : kvalid0) ? (odd ? foff1 : foff0) + (uint32_t)k0 : kOutOfRange;
#pragma unroll
      for (int j = 0; j < F; ++j) {
        if ((part == 1 && j >= FA) || (part == 2 && j < FA)) continue;
        const int g = fwave + j * kFillWaves;
        const uint32_t dst = (uint32_t)reinterpret_cast<uintptr_t>(base + g * 1024);
        if (j < FA) dma16(rsrc_a, dst, vbase + (uint32_t)(g * RPF) * (uint32_t)fK);
        else dma16(rsrc_w, dst, vbase + (uint32_t)(g * RPF - BM) * (uint32_t)fK);
      }
    } else {
#pragma unroll
      for (int j = 0; j < F; ++j) {
        if ((part == 1 && j >= FA) || (part == 2 && j < FA)) continue;
        const int g = fwave + j * kFillWaves;
        const bool odd = ((g * RPF) & 15) != 0;
        const bool kvalid = odd ? kvalid1 : kvalid0;
        const uint32_t foff = odd ? foff1 : foff0;
        const uint32_t dst = (uint32_t)reinterpret_cast<uintptr_t>(base + g * 1024);
        if (j < FA) {
          const uint32_t vo = kvalid ? (uint32_t)(g * RPF) * (uint32_t)fK + foff + (uint32_t)k0 : kOutOfRange;
          dma16(rsrc_a, dst, vo);
        } else {
          const uint32_t vo = kvalid ? (uint32_t)(g * RPF - BM) * (uint32_t)fK + foff + (uint32_t)k0 : kOutOfRange;
          dma16(rsrc_w, dst, vo);
        }
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
    // (one lane base per call, as in issue)
    static_assert((kWaves * RPF) % 16 == 0, "one row parity per wave");
    const bool odd = ((fwave * RPF) & 15) != 0;
    const bool kvalid = k0 + 16 * (odd ? fchunk1_ : fchunk0_) < fK;
    const uint32_t vbase = kvalid ? (odd ? foff1_ : foff0_) + (uint32_t)k0 : kOutOfRange;
#pragma unroll
    for (int j = 0; j < FW; ++j) {
      const int g = fwave + j * kWaves;
      const uint32_t dst = (uint32_t)reinterpret_cast<uintptr_t>(base + g * 1024);
      if (j < FAW) dma16(rsrc_a, dst, vbase + (uint32_t)(g * RPF) * (uint32_t)fK);
      else dma16(rsrc_w, dst, vbase + (uint32_t)(g * RPF - BM) * (uint32_t)fK);
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
    issue_epi(args.a_scale, ws_base, b_base, m0, n0, rows_a, rows_w);
#pragma unroll
    for (int s = 0; s < STAGES; ++s)
      if (s < nst) issue_all(buf(s), s * BK);
    // stage 0 complete (and the epilogue operands, requested before it)
    wait_stage<FW, STAGES>(min(nst - 1, STAGES - 1));
  } else {
    issue_epi(args.a_scale, ws_base, b_base, m0, n0, rows_a, rows_w);
#pragma unroll
    for (int s = 0; s < STAGES; ++s)
      if (s < nst) issue(buf(s), s * BK);
    if (filler) wait_stage<F, STAGES>(min(nst - 1, STAGES - 1));
    else wait_vm_lgkm0<0>();
  }
  if constexpr (FUSED) {
    // the wait above covered these loads
    if (tid < BM) epi_sa[tid] = pre_sa;
    if (tid < BN) {
      epi_sw[tid] = pre_sw;
      epi_b16[tid] = (uint16_t)pre_b;
    }
  }
  block_barrier();
  bool first_tile = true;  // PERSIST: the first tile's prologue left its second stage in flight

  auto sub = [&](int u, int s, int h, Frags& cur, Frags& nxt) {
    // s = stage index of u modulo STAGES, h = half of u (compile-time after unrolling)
    const int t = u / H;
    if (h == H - 1) {
      if (t + 1 < nst) {
        // stage t + 1 complete: the first stages came from every wave (FW each), later
        // ones from the filling waves (F each). PERSIST, after the first tile: both first
        // stages were waited for before the loop, and the previous tile's output stores
        // may still be in flight; a wave that issues no refills has nothing else it waits for.
        if (PERSIST && t == 0 && !first_tile) wait_vm_lgkm0<63>();
        else if (kPrologueAll && t == 0) wait_stage<FW, STAGES>(min(nst - 2, STAGES - 2));
        else if (filler) wait_stage<F, STAGES>(min(nst - 2 - t, STAGES - 2));
        else if (PERSIST) wait_vm_lgkm0<63>();
        else wait_vm_lgkm0<0>();
        block_barrier();
        if (t + STAGES < nst) issue(buf(s), (t + STAGES) * BK, kSplitRefill ? kRefillFirst : 0);
      }
      read_frags(buf((s + 1) % STAGES), 0, nxt);
    } else {
      // the second half of the refill issued at the previous stage barrier
      if (kSplitRefill && t >= 1 && t + 1 < nst) issue(buf((s + 1) % STAGES), (t + 1) * BK, 3 - kRefillFirst);
      read_frags(buf(s), h + 1, nxt);
    }
    mfma_all(cur);
    interleave_mfma_ds_read<FM * FN, 2 * (FM + FN)>();
  };
  constexpr int kUnroll = 2 * STAGES * H;  // whole stage ring, even number of sub-steps
  for (;;) {  // one pass per tile (PERSIST), else exactly one
  if constexpr (PERSIST) {
    asm volatile("" : "+v"(foff0_), "+v"(foff1_), "+s"(fwave), "+s"(fK));
    fwave = __builtin_amdgcn_readfirstlane(fwave);
    fK = __builtin_amdgcn_readfirstlane(fK);
  }
  read_frags(buf(0), 0, f0);
  int u0 = 0;
  if constexpr (!PERSIST) {
    // whole rings without a bound check per sub-step (FFN-down on 128 x 256 tiles 63.2 ->
    // 62.5 us, 32760 x 2048 x 8192 on 256 x 256 422 -> 418); the rest goes through the
    // checked loop below. (Inside the persistent form's tile loop the second copy of the
    // ring cost registers: spills, 3-5% slower.)
    for (; u0 + kUnroll <= nsub; u0 += kUnroll) {
#pragma unroll
      for (int v = 0; v < kUnroll; v += 2) {
        sub(u0 + v, (v / H) % STAGES, v % H, f0, f1);
        sub(u0 + v + 1, ((v + 1) / H) % STAGES, (v + 1) % H, f1, f0);
      }
    }
  }
  for (; u0 < nsub; u0 += kUnroll) {
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
  // (PERSIST: the lane id goes through an empty asm so that the epilogue's per-lane
  // addresses are formed here, not hoisted above the k loop and held through it)
  int elane = lane;
  if constexpr (PERSIST) {
    asm volatile("" : "+v"(elane));
    // this tile's epilogue operands were requested by the filling waves after the
    // previous tile's output; the second stage barrier of the loop (nst >= 3) came after
    // their vmcnt(0), otherwise wait for them here
    if (!first_tile && nst < 3) {
      wait_vm_lgkm0<0>();
      block_barrier();
    }
  }
  float r_sa[FM];
  float4 r_sw[FN][4], r_b[FN][4];
#pragma unroll
  for (int j = 0; j < FM; ++j) r_sa[j] = epi_sa[wm * WTM + j * 32 + (elane & 31)];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int nl = wn * WTN + i * 32 + 8 * q + 4 * (elane >> 5);
      r_sw[i][q] = *reinterpret_cast<const float4*>(epi_sw + nl);
      const uint2 b2 = *reinterpret_cast<const uint2*>(epi_b16 + nl);  // four bf16 -> fp32 exactly
      r_b[i][q] = make_float4(__uint_as_float(b2.x << 16), __uint_as_float(b2.x & 0xffff0000u),
                              __uint_as_float(b2.y << 16), __uint_as_float(b2.y & 0xffff0000u));
    }
  wait_vm_lgkm0<63>();
  block_barrier();

  if constexpr (!PERSIST) {
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
  break;
  } else {
    // Every wave has read the ring and this tile's epilogue operands (barrier above).
    // (args.shares holds the persistent grid size)
    const GemmArgs ra = reload_args();
    const TileProblem cur = tile_problem<BN, PERSIST == kPersistGroup>(kernarg_args(), tn);  // this tile's output
    const int er0 = m0 + wm * WTM, ec0 = cur.n0 + wn * WTN;
    const int nt = ra.tiles_m * ra.tiles_n;
    vtile += ra.shares;
    const bool more = vtile < nt;
    if (more) {
      tile_coords_at<GROUP_M>(vtile, nt, ra.tiles_m, ra.tiles_n, tm, tn);
      tm = __builtin_amdgcn_readfirstlane(tm);
      tn = __builtin_amdgcn_readfirstlane(tn);
      const TileProblem nx = tile_problem<BN, PERSIST == kPersistGroup>(kernarg_args(), tn);
      m0 = tm * BM;
      n0 = nx.n0;
      rows_a = min(BM, ra.m - m0);
      rows_w = min(BN, nx.n - n0);
      rsrc_a = make_rsrc(ra.qa + (int64_t)m0 * ra.k, (uint32_t)rows_a * (uint32_t)ra.k);
      rsrc_w = make_rsrc(nx.qw + (int64_t)n0 * ra.k, (uint32_t)rows_w * (uint32_t)ra.k);
      asm volatile("" : "+v"(foff0_), "+v"(foff1_), "+s"(fwave), "+s"(fK));
      fwave = __builtin_amdgcn_readfirstlane(fwave);
      fK = __builtin_amdgcn_readfirstlane(fK);
#pragma unroll
      for (int st = 0; st < STAGES; ++st)
        if (st < nst) issue_all(buf(st), st * BK);
    }
    // Output in pieces of 32 token rows (MFMA fragment j): the wave writes its values
    // to its piece (chunk c of row r at position c ^ (r % RC)), which goes out as whole
    // 128-byte lines. LDS executes one wave's accesses in order, so the next piece may
    // overwrite the region right after the previous one's reads.
    constexpr int kEpiStores = FM * (kPieceRows / (64 / RC));
    static_assert(kPieceRows == 32 && kPieceBytes == kPieceRows * RC * 16, "piece geometry");
    uint8_t* const piece = epi_base + wave * kPieceBytes;
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int r = elane & 31;
      const float sa = r_sa[j];
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c8 = i * 32 + 8 * q + 4 * (elane >> 5);
          const float4 sw4 = r_sw[i][q];
          const float4 b4 = r_b[i][q];
          const v16f& a = acc[i][j];
          const float o0 = __builtin_fmaf(a[4 * q + 0] * sa, sw4.x, b4.x);
          const float o1 = __builtin_fmaf(a[4 * q + 1] * sa, sw4.y, b4.y);
          const float o2 = __builtin_fmaf(a[4 * q + 2] * sa, sw4.z, b4.z);
          const float o3 = __builtin_fmaf(a[4 * q + 3] * sa, sw4.w, b4.w);
          const int chunk = c8 >> 3, half = (c8 >> 2) & 1;
          *reinterpret_cast<uint2*>(piece + r * (RC * 16) + ((chunk ^ (r % RC)) << 4) + (half << 3)) =
              make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
        }
      store_wave_tile<kPieceRows, RC, true>(piece, elane, cur.out, ra.m, cur.n, er0 + j * 32, ec0);
    }
    if (!more) break;
    // the next tile's fills are older than this wave's kEpiStores stores; every wave
    // has read its last piece before the next epilogue operands overwrite the region
    static_assert(kEpiStores < 64, "vmcnt range");
    wait_vm_lgkm0<kEpiStores>();
    block_barrier();
    {
      const KernargGemmArgs kb = kernarg_args();
      const TileProblem nx = tile_problem<BN, PERSIST == kPersistGroup>(kb, tn);
      issue_epi(kb->a_scale, nx.ws, nx.bias, m0, n0, rows_a, rows_w);
    }
    first_tile = false;
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  }
  }
}

// PERSIST: one workgroup per CU (the LDS of a 256 x 256 tile admits no second), the
// count rounded down to a multiple of the XCD count so that each workgroup's later tiles
// stay on its own XCD; never more workgroups than tiles.
template <int BM, int BN, int WM, int WN, int S, int BK, int GM, bool FUSED = false, int PERSIST = kPersistNone>
hipError_t launch(const GemmArgs& a, hipStream_t stream, int cus = 0) {
  GemmArgs args = a;
  args.tiles_m = (a.m + BM - 1) / BM;
  args.tiles_n = (a.n + BN - 1) / BN;
  if (PERSIST == kPersistGroup) {
    if (a.ngroup < 1 || a.ngroup > kMaxGroup) return hipErrorInvalidValue;
    args.tiles_n = a.g_tn_end[a.ngroup - 1];  // the problems' tiles side by side
  }
  const int64_t tiles = (int64_t)args.tiles_m * args.tiles_n;
  int64_t wgs = tiles;
  if (PERSIST) {
    wgs = std::min<int64_t>(tiles, cus >= kXcds ? (int64_t)(cus / kXcds) * kXcds : std::max(cus, 1));
    args.shares = (int)wgs;  // the persistent form's stride over the tiles
  }
  const bool w_first = (int64_t)args.tiles_n * BN > (int64_t)args.tiles_m * BM;
  if constexpr (S == 2 && WM * WN == 8) {  // the forms whose refills are split in halves
    if (w_first) {
      gemm_fp8_kernel<BM, BN, WM, WN, S, BK, GM, FUSED, PERSIST, true>
          <<<dim3((unsigned)wgs), dim3(WM * WN * 64), 0, stream>>>(args);
      return hipGetLastError();
    }
  }
  gemm_fp8_kernel<BM, BN, WM, WN, S, BK, GM, FUSED, PERSIST, false>
      <<<dim3((unsigned)wgs), dim3(WM * WN * 64), 0, stream>>>(args);
  return hipGetLastError();
}

// ---- skinny form: few tokens (the 26-row encoder input of the QKV projections) ----------
//
// With m of a few dozen the product is a stream of the weight through the chip: 2 m n k
// flop against n k bytes of weight, far below any matrix-core limit. What bounds it is
// how many CUs pull weight bytes at once and how much else each of them must load. The
// tiled kernel's smallest tile (64 x 64) gives one workgroup per 64 channels (32 for
// n = 2048) that walks k through a three-stage LDS pipeline, so most CUs idle and each
// active one waits on a chain of dependent stages. Here a workgroup owns NW = 16 NF channels
// and 16 * MT tokens (grid: ceil(n / NW) x ceil(m / (16 MT)) workgroups; with NF = 1, 128
// for the encoder GEMM, and NF = 2 halves the grid where it would exceed the CUs, so that
// the activation, which every workgroup loads in full, is loaded once per 32 channels
// rather than 16), and its WAVES waves split k between them: wave w takes the 128-byte
// k-steps w, w + WAVES, ... . Each wave loads its operand fragments straight from
// memory into registers (no LDS staging, no barrier in the loop), two k-steps per batch
// with the next batch requested before the current one is multiplied, and runs
// V_MFMA_F32_16X16X128_F8F6F4 on them. The waves' partial sums meet in LDS once; the
// sum over waves is taken in a fixed order and the epilogue (fp32, one rounding to bf16)
// follows the tiled kernel's. Out-of-range rows and k-chunks read zeros through the
// buffer descriptors, as in the tiled kernel.
//
// Operand layout of the 16x16x128 MFMA: lane l holds row l % 16 of the 16-row operand
// and 32 bytes of its k; the two operands must agree on which k those are. Here lane
// l holds k bytes [16 q, 16 q + 16) and [64 + 16 q, 64 + 16 q + 16) of the step, q = l / 16,
// so each of the two 16-byte loads of a fragment reads the first or second half of
// every row's 128-byte line. Results: lane l holds column l % 16 (token) and rows
// 4 (l / 16) + i (channels), i = 0..3.
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kSkinnyWaves = 8;   // waves per workgroup, splitting k
constexpr int kSkinnyBatch = 2;   // 128-byte k-steps per load batch

template <int MT, int NF>
struct SkinnyFrags {
  v8i w[kSkinnyBatch][NF];
  v8i a[kSkinnyBatch][MT];
};

// NF: 16-channel weight fragments per wave (the workgroup owns 16 NF channels). Each
// fragment's sum runs exactly as with NF = 1 (same k-steps per wave, same order, same
// fixed-order sum over the waves), so every output is bit-identical whatever NF is; a
// larger NF loads the activation once for more weight bytes.
// GROUPED: column block blockIdx.x of problem blockIdx.y of GemmArgs' group, token block
// blockIdx.z (a 3-D grid, as many column blocks as the widest problem has; a workgroup
// past its problem's width exits at once). The problem's fields are read straight from
// the kernel arguments at that index, with no search over the group, and all the
// arguments are in registers before the width test, so they cost one round trip, as a
// single problem's do.
template <int MT, int NF, bool GROUPED = false>
__global__ __launch_bounds__(kSkinnyWaves * 64) void gemm_fp8_skinny(GemmArgs args) {
  constexpr int WAVES = kSkinnyWaves;
  constexpr int NW = 16 * NF;  // channels per workgroup
  constexpr int TM = 16 * MT;  // tokens per workgroup
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int tn, tm;
  TileProblem pr;
  const uint8_t* qa = args.qa;
  const float* a_scale = args.a_scale;
  int K = args.k, M = args.m;
  if constexpr (GROUPED) {
    tn = blockIdx.x;
    tm = blockIdx.z;
    const int p = blockIdx.y;
    const KernargGemmArgs k = kernarg_args();
    pr = TileProblem{k->g_qw[p], k->g_ws[p], k->g_bias[p], k->g_out[p], k->g_n[p], tn * NW};
    // every argument in registers here (one wait for all of them), not loaded after the test
    asm volatile("" ::"s"(pr.qw), "s"(pr.ws), "s"(pr.bias), "s"(pr.out), "s"(pr.n), "s"(qa), "s"(a_scale),
                 "s"(K), "s"(M));
    if (pr.n0 >= pr.n) return;  // the whole workgroup, before any barrier
  } else {
    tn = blockIdx.x % args.tiles_n;
    tm = blockIdx.x / args.tiles_n;
    pr = tile_problem<NW, false>(kernarg_args(), tn);
  }
  const int n = pr.n, n0 = pr.n0, m0 = tm * TM;
  const int rows_a = min(TM, M - m0);
  const int rows_w = min(NW, n - n0);
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(qa) + (int64_t)m0 * K, 0,
                                        (uint32_t)rows_a * (uint32_t)K, kBufferConfig);
  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(pr.qw) + (int64_t)n0 * K, 0,
                                        (uint32_t)rows_w * (uint32_t)K, kBufferConfig);

  // epilogue operands of this thread's NF outputs (output o = threadIdx.x + j WAVES 64 is
  // token o / NW, channel o % NW: every output of the workgroup's tile has one thread, since
  // TM * NW == NF * WAVES * 64), requested now and used only after the k loop. The loads
  // take no branch (indices clamped into the tile; outputs outside it are never stored, and
  // without a bias the weight scales stand in as an in-bounds source) and the bias stays
  // raw until the epilogue, so no wave waits for them before its operand loads go out.
  static_assert(TM * NW == NF * WAVES * 64, "NF outputs per thread");
  const uint16_t* bias_src = pr.bias ? pr.bias : reinterpret_cast<const uint16_t*>(pr.ws);
  float e_sa[NF], e_sw[NF];
  uint32_t e_b[NF];
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    const int o = threadIdx.x + j * WAVES * 64;
    const int ct = min(o / NW, rows_a - 1), cc = min(o % NW, rows_w - 1);
    e_sa[j] = a_scale[m0 + ct];
    e_sw[j] = pr.ws[n0 + cc];
    e_b[j] = bias_src[n0 + cc];
  }

  const int r = lane & 15, q = lane >> 4;
  const uint32_t row_off = (uint32_t)r * (uint32_t)K;
  const int steps = (K + 127) / 128;
  auto load = [&](int step, v8i* w, v8i* a) {
    // chunk c of the step's 128 bytes holds k bytes [16 c, 16 c + 16); lanes past k read zeros
    const int k0 = step * 128 + 16 * q, k1 = k0 + 64;
    const uint32_t o0 = k0 < K ? row_off + (uint32_t)k0 : kOutOfRange;
    const uint32_t o1 = k1 < K ? row_off + (uint32_t)k1 : kOutOfRange;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const uint32_t d = (uint32_t)(16 * f) * (uint32_t)K;
      const v4u w0 = __builtin_amdgcn_raw_buffer_load_b128(rw, o0 == kOutOfRange ? o0 : o0 + d, 0, 0);
      const v4u w1 = __builtin_amdgcn_raw_buffer_load_b128(rw, o1 == kOutOfRange ? o1 : o1 + d, 0, 0);
      w[f] = v8i{(int)w0[0], (int)w0[1], (int)w0[2], (int)w0[3], (int)w1[0], (int)w1[1], (int)w1[2], (int)w1[3]};
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const uint32_t d = (uint32_t)(16 * t) * (uint32_t)K;
      const v4u a0 = __builtin_amdgcn_raw_buffer_load_b128(ra, o0 == kOutOfRange ? o0 : o0 + d, 0, 0);
      const v4u a1 = __builtin_amdgcn_raw_buffer_load_b128(ra, o1 == kOutOfRange ? o1 : o1 + d, 0, 0);
      a[t] = v8i{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
    }
  };
  auto load_batch = [&](int first, SkinnyFrags<MT, NF>& fr) {
#pragma unroll
    for (int b = 0; b < kSkinnyBatch; ++b) {
      const int step = first + b * WAVES;
      if (step < steps) load(step, fr.w[b], fr.a[b]);
    }
  };

  v4f acc[NF][MT];
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[f][t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  auto mfma_batch = [&](int first, const SkinnyFrags<MT, NF>& fr) {
#pragma unroll
    for (int b = 0; b < kSkinnyBatch; ++b)
      if (first + b * WAVES < steps)
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
          for (int t = 0; t < MT; ++t)
            acc[f][t] =
                __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fr.w[b][f], fr.a[b][t], acc[f][t], 0, 0, 0, 0, 0, 0);
  };

  constexpr int kStride = kSkinnyBatch * WAVES;  // k-steps between a wave's batches
  SkinnyFrags<MT, NF> f0, f1;
  load_batch(wave, f0);
  for (int s = wave; s < steps; s += 2 * kStride) {
    load_batch(s + kStride, f1);
    mfma_batch(s, f0);
    if (s + kStride >= steps) break;
    load_batch(s + 2 * kStride, f0);
    mfma_batch(s + kStride, f1);
  }

  // partial sums of every wave -> LDS, then a fixed-order sum per output
  __shared__ v4f red[WAVES][NF][MT][64];
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int t = 0; t < MT; ++t) red[wave][f][t][lane] = acc[f][t];
  __syncthreads();
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    const int o = threadIdx.x + j * WAVES * 64, et = o / NW, ec = o % NW;
    // token et is column et % 16 of m-tile et / 16; channel ec is row ec % 16 of fragment ec / 16
    const int cf = ec >> 4, cr = ec & 15;
    const int src_lane = (et & 15) + 16 * (cr >> 2);
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) sum += red[w][cf][et >> 4][src_lane][cr & 3];
    if (et < rows_a && ec < rows_w) {
      const float b = pr.bias ? __uint_as_float(e_b[j] << 16) : 0.0f;
      const float v = __builtin_fmaf(sum * e_sa[j], e_sw[j], b);
      pr.out[(int64_t)(m0 + et) * n + n0 + ec] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xffffu);
    }
  }
}

template <int MT, int NF, bool GROUPED = false>
hipError_t launch_skinny(const GemmArgs& a, hipStream_t stream) {
  GemmArgs args = a;
  if (GROUPED && (a.ngroup < 1 || a.ngroup > kMaxGroup)) return hipErrorInvalidValue;
  int cols = (a.n + 16 * NF - 1) / (16 * NF);  // column blocks along x: the widest problem's
  if (GROUPED)
    for (int p = 0; p < a.ngroup; ++p) cols = std::max(cols, (a.g_n[p] + 16 * NF - 1) / (16 * NF));
  args.tiles_n = cols;
  args.tiles_m = (a.m + 16 * MT - 1) / (16 * MT);
  const dim3 grid = GROUPED ? dim3((unsigned)args.tiles_n, (unsigned)a.ngroup, (unsigned)args.tiles_m)
                            : dim3((unsigned)((int64_t)args.tiles_m * args.tiles_n));
  gemm_fp8_skinny<MT, NF, GROUPED><<<grid, dim3(kSkinnyWaves * 64), 0, stream>>>(args);
  return hipGetLastError();
}

// id, tile_m, tile_n, waves, stages, name (every stage holds 128 bytes of k)
const GemmConfig kConfigs[] = {
    {0, 256, 256, 8, 2, "bm256_bn256_w2x4_s2"},
    {1, 256, 128, 8, 3, "bm256_bn128_w4x2_s3"},
    {2, 128, 256, 8, 3, "bm128_bn256_w2x4_s3"},
    {3, 128, 128, 4, 2, "bm128_bn128_w2x2_s2"},
    {4, 64, 64, 4, 3, "bm64_bn64_w2x2_s3"},
    {5, 32, 16, 8, 0, "skinny_m32_n16_w8"},
    {6, 256, 256, 8, 2, "bm256_bn256_w2x4_s2_persistent"},
    {7, 32, 32, 8, 0, "skinny_m32_n32_w8"},
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
                       const uint8_t* qw, const float* w_scale, const uint16_t* bias, uint16_t* out, int cus,
                       hipStream_t stream) {
  GemmArgs a{qa, a_scale, qw, w_scale, bias, out, (int)m, (int)n, (int)k, 0, 0};
  switch (id) {
    case 0: return launch<256, 256, 2, 4, 2, 128, 4>(a, stream);
    case 1: return launch<256, 128, 4, 2, 3, 128, 4>(a, stream);
    case 2: return launch<128, 256, 2, 4, 3, 128, 8>(a, stream);  // groups of 8: FFN-down 64.3 -> 63.4 us
    case 3: return launch<128, 128, 2, 2, 2, 128, 8>(a, stream);
    case 4: return launch<64, 64, 2, 2, 3, 128, 8>(a, stream);
    case 5: return launch_skinny<2, 1>(a, stream);
    case 6: return launch<256, 256, 2, 4, 2, 128, 4, false, kPersistOne>(a, stream, cus);
    case 7: return launch_skinny<2, 2>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm_group(int id, int64_t m, int64_t k, const uint8_t* qa, const float* a_scale, int nprob,
                             const GroupProblem* probs, int cus, hipStream_t stream) {
  if (nprob < 1 || nprob > kMaxGroup) return hipErrorInvalidValue;
  if (id != 5 && id != 6 && id != 7) return hipErrorInvalidValue;
  GemmArgs a{qa, a_scale, probs[0].qw, probs[0].w_scale, probs[0].bias, probs[0].out, (int)m, (int)probs[0].n,
             (int)k, 0, 0};
  a.ngroup = nprob;
  const int cols = id == 6 ? 256 : id == 7 ? 32 : 16;  // the form's column block
  int tn = 0;
  for (int p = 0; p < nprob; ++p) {
    tn += (int)((probs[p].n + cols - 1) / cols);
    a.g_tn_end[p] = tn;
    a.g_n[p] = (int)probs[p].n;
    a.g_qw[p] = probs[p].qw;
    a.g_ws[p] = probs[p].w_scale;
    a.g_bias[p] = probs[p].bias;
    a.g_out[p] = probs[p].out;
  }
  if (id == 5) return launch_skinny<2, 1, true>(a, stream);
  if (id == 7) return launch_skinny<2, 2, true>(a, stream);
  return launch<256, 256, 2, 4, 2, 128, 4, false, kPersistGroup>(a, stream, cus);
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
