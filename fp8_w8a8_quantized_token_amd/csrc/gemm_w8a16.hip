// FP8 weight-only linear (W8A16) for gfx950: bf16 activation x e4m3fn (or e5m2) weight.
//
//   out[m, n] = bf16_rne( acc[m, n] * w_scale[n] + bias[n] ),
//   acc[m, n] = sum_k a[m, k] * dec(qw[n, k])   (fp32 accumulation on the MFMA units)
//
// The FP8 weight-only pipeline of the LongCat avatar comparison page
// (longcat-avatar-compare.pages.dev, speed overview table) keeps the weights in FP8
// with scales and the activations in 16-bit; the weight scale is per output channel
// as in the HunyuanVideo1.5 retrospective (aigcage.com, section 2), so it is constant
// along k and is applied once, after the sum. The weight stays in nn.Linear's [n, k]
// layout with k contiguous, read in place.
//
// The kernel is the FP8 GEMM's design with a bf16 left operand:
//   * V_MFMA_F32_32X32X16_BF16. Every e4m3fn value is exact in bf16 (3 mantissa bits,
//     exponents 2^-9 .. 2^8), and so is every finite e5m2 value (2 mantissa bits,
//     2^-16 .. 57344), so the weight fragments are converted in registers with
//     v_cvt_scalef32_pk_bf16_{fp8,bf8} at scale 1 (exact) right before the MFMAs; the
//     LDS holds the weight as FP8 (half the bytes of a bf16 copy). The e5m2 weights are
//     the QuantizeFP8Format page's default format (runcomfy.com, input parameters).
//   * A stage holds 64 k elements: 128-byte activation rows and 64-byte weight rows,
//     filled by buffer_load_dwordx4 ... lds, each row's 16-byte chunks swizzled so the
//     operand reads (ds_read_b128 for the activation, ds_read_b64 for the weight) and
//     the fills avoid bank conflicts. Three stages of a 256 x 256 tile use 144 KiB.
//   * Waits, barriers, the fragment double buffering, the XCD-aware tile order and
//     the LDS-staged epilogue are those of the FP8 GEMM (gemm_common.h).
#include "gemm_common.h"
#include "internal.h"

namespace fp8w8a8 {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

struct W16Args {
  const uint16_t* a;  // bf16 [m, k]
  const uint8_t* qw;  // e4m3fn [n, k]
  const float* w_scale;
  const uint16_t* bias;  // may be null
  uint16_t* out;
  int m, n, k;
  int tiles_m, tiles_n;
};

template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, int GROUP_M, int FMT>
struct W16Tag {};

// 2 codes (one 16-bit half of a dword) -> 2 bf16, exactly (scale 1; every e4m3fn and
// every finite e5m2 value is a bf16 value).
template <int FMT, bool HI>
__device__ __forceinline__ v2bf cvt2(uint32_t w) {
  if constexpr (FMT == FP8W8A8_FMT_E5M2)
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, HI);
  else
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
}

// 8 codes (two dwords) -> 8 bf16.
template <int FMT>
__device__ __forceinline__ v8bf fp8x8_to_bf16(uint2 w) {
  const v2bf p0 = cvt2<FMT, false>(w.x);
  const v2bf p1 = cvt2<FMT, true>(w.x);
  const v2bf p2 = cvt2<FMT, false>(w.y);
  const v2bf p3 = cvt2<FMT, true>(w.y);
  return v8bf{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, int GROUP_M, int FMT>
__global__ __launch_bounds__(WAVES_M* WAVES_N * 64) void gemm_w8a16_kernel(W16Args args) {
  using Tag = W16Tag<BM, BN, WAVES_M, WAVES_N, STAGES, GROUP_M, FMT>;
  constexpr int KE = 64;               // k elements per stage
  constexpr int kARow = 2 * KE;        // activation row bytes per stage (bf16)
  constexpr int kWRow = KE;            // weight row bytes per stage (e4m3fn)
  constexpr int H = KE / 16;           // 32x32x16 MFMA k-steps per stage
  constexpr int kARpf = 1024 / kARow;  // activation rows per wave-wide 1 KiB fill
  constexpr int kWRpf = 1024 / kWRow;  // weight rows per fill
  constexpr int kWaves = WAVES_M * WAVES_N;
  constexpr int WTM = BM / WAVES_M;
  constexpr int WTN = BN / WAVES_N;
  constexpr int FM = WTM / 32;
  constexpr int FN = WTN / 32;
  constexpr int kABytes = BM * kARow;
  constexpr int kStageBytes = BM * kARow + BN * kWRow;
  // As in the FP8 GEMM: with 8 waves only waves 0..3 (one per SIMD) issue the DMA
  // fills, so a wave stalled at fill issue always has a partner that can feed the SIMD's
  // matrix core.
  constexpr int kFillWaves = kWaves == 8 ? kWaves / 2 : kWaves;
  constexpr int FA = (BM / kARpf) / kFillWaves;  // activation fills per filling wave per stage
  constexpr int FW = (BN / kWRpf) / kFillWaves;  // weight fills per filling wave per stage
  constexpr int F = FA + FW;
  static_assert(BM % (32 * WAVES_M) == 0 && BN % (32 * WAVES_N) == 0, "tile / wave mismatch");
  static_assert(FA >= 1 && FW >= 1 && (BM / kARpf) % kFillWaves == 0 && (BN / kWRpf) % kFillWaves == 0,
                "fills split evenly across the filling waves");
  static_assert(STAGES >= 2 && STAGES <= 6, "stage count");
  // the tile's w_scale [BN] (fp32) and bias [BN] (bf16) in LDS, whole 256-byte DMA chunks
  constexpr int kEpiBiasBytes = (BN * 2 + 255) / 256 * 256;
  constexpr int kEpiBytes = BN * 4 + kEpiBiasBytes;
  static_assert(BN % 64 == 0, "whole DMA chunks of scales");
  static_assert(STAGES * kStageBytes + kEpiBytes <= 160 * 1024, "LDS budget of a CU");
  static_assert((STAGES - 1) * F < 64, "vmcnt range");
  static_assert(BM <= kWaves * 64 && BN <= kWaves * 64, "one epilogue operand per thread");

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
  tm = __builtin_amdgcn_readfirstlane(tm);
  tn = __builtin_amdgcn_readfirstlane(tn);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave % WAVES_M, wn = wave / WAVES_M;
  const int m0 = tm * BM, n0 = tn * BN;
  const int K = args.k;
  const int rows_a = min(BM, args.m - m0);
  const int rows_w = min(BN, args.n - n0);
  const v4i rsrc_a = make_rsrc(args.a + (int64_t)m0 * K, (uint32_t)rows_a * (uint32_t)K * 2u);
  const v4i rsrc_w = make_rsrc(args.qw + (int64_t)n0 * K, (uint32_t)rows_w * (uint32_t)K);

  // The epilogue operands come by 4-byte LDS DMA from the filling waves, before their
  // first fills (so the wait for stage 0 covers them): register loads would be the only
  // reads the compiler counts, and its vmcnt(0) for them would hold the first fills back
  // by a memory round trip. Channels past the tile and a missing bias read zeros.
  uint8_t* const epi_base = stage_buf<Tag, 7, kEpiBytes>();
  const float* const epi_sw = reinterpret_cast<const float*>(epi_base);
  const uint16_t* const epi_b16 = reinterpret_cast<const uint16_t*>(epi_base + BN * 4);

  // Fill geometry. Activation: lane i writes row i / 8 of an 8-row group, chunk
  // position i % 8 holding logical chunk (i % 8) ^ swz<128>(row); the swizzle period
  // is 16 rows, so even and odd groups differ. Weight: lane i writes row i / 4 of a
  // 16-row group (one swizzle period), position i % 4 = logical chunk ^ swz<64>(row).
  const int far = lane / 8;
  const int fac0 = (lane % 8) ^ swz<128>(far);
  const int fac1 = (lane % 8) ^ swz<128>(far + 8);
  const uint32_t faoff0 = (uint32_t)far * (uint32_t)K * 2u + 16u * (uint32_t)fac0;
  const uint32_t faoff1 = (uint32_t)far * (uint32_t)K * 2u + 16u * (uint32_t)fac1;
  const int fwr = lane / 4;
  const int fwc = (lane % 4) ^ swz<64>(fwr);
  const uint32_t fwoff = (uint32_t)fwr * (uint32_t)K + 16u * (uint32_t)fwc;

  const bool filler = wave < kFillWaves;
  constexpr int kEpiChunksW = BN / 64, kEpiChunks = kEpiChunksW + kEpiBiasBytes / 256;
  auto issue_epi = [&]() {
    if (!filler) return;
    const v4i rs_w = make_rsrc(args.w_scale + n0, (uint32_t)rows_w * 4u);
    const v4i rs_b = make_rsrc(args.bias ? args.bias + n0 : nullptr, args.bias ? (uint32_t)rows_w * 2u : 0u);
    const uint32_t vo = 4u * (uint32_t)lane;
#pragma unroll
    for (int c0 = 0; c0 < kEpiChunks; c0 += kFillWaves) {
      const int c = c0 + wave;  // uniform
      if (c >= kEpiChunks) break;
      const uint32_t dst = (uint32_t)reinterpret_cast<uintptr_t>(epi_base + 256 * c);
      if (c < kEpiChunksW) dma4(rs_w, dst, vo + 256u * (uint32_t)c);
      else dma4(rs_b, dst, vo + 256u * (uint32_t)(c - kEpiChunksW));
    }
  };
  auto issue = [&](uint8_t* base, int s) {
    if (!filler) return;
    const int ke0 = s * KE;  // first k element of the stage
    const bool va0 = ke0 + 8 * fac0 < K, va1 = ke0 + 8 * fac1 < K;
    if constexpr (kFillWaves < kWaves) {
      // As in the FP8 GEMM: one lane base per operand and call (every activation fill of
      // a wave has its first row's parity), each fill adding its uniform row offset; a
      // lane past k starts from kOutOfRange and stays past the descriptor's end.
      static_assert((kFillWaves * kARpf) % 16 == 0, "one row parity per filling wave");
      static_assert((int64_t)(BM > BN ? BM : BN) * 2 * FP8W8A8_MAX_DIM <= (int64_t)1 << 29 &&
                        kOutOfRange == 0x80000000u,
                    "out-of-range offsets stay out of range");
      const bool odd = ((wave * kARpf) & 15) != 0;
      const uint32_t ba = (odd ? va1 : va0) ? (odd ? faoff1 : faoff0) + (uint32_t)ke0 * 2u : kOutOfRange;
#pragma unroll
      for (int j = 0; j < FA; ++j) {
        const int g = wave + j * kFillWaves;
        dma16(rsrc_a, (uint32_t)reinterpret_cast<uintptr_t>(base + g * 1024),
              ba + (uint32_t)(g * kARpf) * (uint32_t)K * 2u);
      }
      const uint32_t bw = ke0 + 16 * fwc < K ? fwoff + (uint32_t)ke0 : kOutOfRange;
#pragma unroll
      for (int j = 0; j < FW; ++j) {
        const int g = wave + j * kFillWaves;
        dma16(rsrc_w, (uint32_t)reinterpret_cast<uintptr_t>(base + kABytes + g * 1024),
              bw + (uint32_t)(g * kWRpf) * (uint32_t)K);
      }
      return;
    }
#pragma unroll
    for (int j = 0; j < FA; ++j) {
      const int g = wave + j * kFillWaves;
      const bool odd = ((g * kARpf) & 15) != 0;
      const uint32_t vo = (odd ? va1 : va0)
                              ? (uint32_t)(g * kARpf) * (uint32_t)K * 2u + (odd ? faoff1 : faoff0) + (uint32_t)ke0 * 2u
                              : kOutOfRange;
      dma16(rsrc_a, (uint32_t)reinterpret_cast<uintptr_t>(base + g * 1024), vo);
    }
    const bool vw = ke0 + 16 * fwc < K;
#pragma unroll
    for (int j = 0; j < FW; ++j) {
      const int g = wave + j * kFillWaves;
      const uint32_t vo = vw ? (uint32_t)(g * kWRpf) * (uint32_t)K + fwoff + (uint32_t)ke0 : kOutOfRange;
      dma16(rsrc_w, (uint32_t)reinterpret_cast<uintptr_t>(base + kABytes + g * 1024), vo);
    }
  };

  // The first stages' fills, before any wave has MFMA work to keep fed, come from every
  // wave (FAA + FWA each per stage), the refills from the filling waves (F each): the
  // first stage boundary waits for the prologue's per-wave count.
  constexpr bool kPrologueAll = kFillWaves < kWaves;
  constexpr int FAA = (BM / kARpf) / kWaves;
  constexpr int FWA = (BN / kWRpf) / kWaves;
  static_assert(!kPrologueAll || ((BM / kARpf) % kWaves == 0 && (BN / kWRpf) % kWaves == 0 && FAA >= 1 && FWA >= 1),
                "prologue fills split evenly");
  auto issue_all = [&](uint8_t* base, int s) {
    const int ke0 = s * KE;
    const bool va0 = ke0 + 8 * fac0 < K, va1 = ke0 + 8 * fac1 < K;
#pragma unroll
    for (int j = 0; j < FAA; ++j) {
      const int g = wave + j * kWaves;
      const bool odd = ((g * kARpf) & 15) != 0;
      const uint32_t vo = (odd ? va1 : va0)
                              ? (uint32_t)(g * kARpf) * (uint32_t)K * 2u + (odd ? faoff1 : faoff0) + (uint32_t)ke0 * 2u
                              : kOutOfRange;
      dma16(rsrc_a, (uint32_t)reinterpret_cast<uintptr_t>(base + g * 1024), vo);
    }
    const bool vw = ke0 + 16 * fwc < K;
#pragma unroll
    for (int j = 0; j < FWA; ++j) {
      const int g = wave + j * kWaves;
      const uint32_t vo = vw ? (uint32_t)(g * kWRpf) * (uint32_t)K + fwoff + (uint32_t)ke0 : kOutOfRange;
      dma16(rsrc_w, (uint32_t)reinterpret_cast<uintptr_t>(base + kABytes + g * 1024), vo);
    }
  };

  // Operand reads of k-step h (16 k elements). Activation fragment: lane l holds row
  // l % 32, elements 8 (l / 32) .. +8 of the k-step = 16-byte chunk 2 h + l / 32.
  // Weight fragment: the same rows and elements, 8 bytes at chunk h, half l / 32.
  const int rrow = lane & 31;
  const int rkq = lane >> 5;
  const int rfa = swz<128>(rrow);
  const int rfw = swz<64>(rrow);
  uint32_t rda[H], rdw[H];
#pragma unroll
  for (int h = 0; h < H; ++h) {
    rda[h] = (uint32_t)rrow * kARow + 16u * (uint32_t)((2 * h + rkq) ^ rfa);
    rdw[h] = (uint32_t)rrow * kWRow + 16u * (uint32_t)(h ^ rfw) + 8u * (uint32_t)rkq;
  }

  v16f acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  struct Frags {
    v8bf a[FM];
    uint2 w[FN];  // e4m3fn codes, converted right before use
  };
  auto read_frags = [&](const uint8_t* base, int h, Frags& f) {
    const uint8_t* sa = base + (wm * WTM) * kARow;
    const uint8_t* sw = base + kABytes + (wn * WTN) * kWRow;
#pragma unroll
    for (int i = 0; i < FN; ++i) f.w[i] = *reinterpret_cast<const uint2*>(sw + i * 32 * kWRow + rdw[h]);
#pragma unroll
    for (int j = 0; j < FM; ++j) f.a[j] = *reinterpret_cast<const v8bf*>(sa + j * 32 * kARow + rda[h]);
  };
  auto mfma_all = [&](const Frags& f) {
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const v8bf w = fp8x8_to_bf16<FMT>(f.w[i]);
#pragma unroll
      for (int j = 0; j < FM; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w, f.a[j], acc[i][j], 0, 0, 0);
    }
  };

  // Software pipeline over MFMA k-steps u = H t + h, as in the FP8 GEMM: stage t lives
  // in buffer t % STAGES; sub-step u multiplies the fragments of u while reading those
  // of u + 1; before the reads cross into stage t + 1 a wait + barrier publishes it and
  // frees stage t's buffer, which is refilled with stage t + STAGES.
  const int nst = (K + KE - 1) / KE;
  const int nsub = nst * H;
  issue_epi();
  if constexpr (kPrologueAll) {
#pragma unroll
    for (int s = 0; s < STAGES; ++s)
      if (s < nst) issue_all(buf(s), s);
    wait_stage<FAA + FWA, STAGES>(min(nst - 1, STAGES - 1));
  } else {
#pragma unroll
    for (int s = 0; s < STAGES; ++s)
      if (s < nst) issue(buf(s), s);
    if (filler) wait_stage<F, STAGES>(min(nst - 1, STAGES - 1));
    else wait_vm_lgkm0<0>();
  }
  Frags f0, f1;
  block_barrier();
  read_frags(buf(0), 0, f0);

  auto sub = [&](int u, int s, int h, Frags& cur, Frags& nxt) {
    const int t = u / H;
    if (h == H - 1) {
      if (t + 1 < nst) {
        if (kPrologueAll && t == 0) wait_stage<FAA + FWA, STAGES>(min(nst - 2, STAGES - 2));
        else if (filler) wait_stage<F, STAGES>(min(nst - 2 - t, STAGES - 2));
        else wait_vm_lgkm0<0>();
        block_barrier();
        if (t + STAGES < nst) issue(buf(s), t + STAGES);
      }
      read_frags(buf((s + 1) % STAGES), 0, nxt);
    } else {
      read_frags(buf(s), h + 1, nxt);
    }
    mfma_all(cur);
    interleave_mfma_ds_read<FM * FN, FM + FN>();
  };
  constexpr int kUnroll = STAGES * H;  // whole stage ring; H is even, so is the unroll
  static_assert(kUnroll % 2 == 0, "cur / nxt alternate within the unrolled ring");
  // whole rings without a bound check per sub-step, then the rest with one
  int u0 = 0;
  for (; u0 + kUnroll <= nsub; u0 += kUnroll) {
#pragma unroll
    for (int v = 0; v < kUnroll; v += 2) {
      sub(u0 + v, (v / H) % STAGES, v % H, f0, f1);
      sub(u0 + v + 1, ((v + 1) / H) % STAGES, (v + 1) % H, f1, f0);
    }
  }
  for (; u0 < nsub; u0 += kUnroll) {
#pragma unroll
    for (int v = 0; v < kUnroll; v += 2) {
      if (u0 + v < nsub) sub(u0 + v, (v / H) % STAGES, v % H, f0, f1);
      if (u0 + v + 1 < nsub) sub(u0 + v + 1, ((v + 1) / H) % STAGES, (v + 1) % H, f1, f0);
    }
  }

  // Epilogue: the FP8 GEMM's (scale and bias from LDS into registers, one rounding to
  // bf16, the tile staged per wave in LDS and stored as whole rows), without an
  // activation scale.
  constexpr int RC = WTN / 8;
  constexpr int kWaveOutBytes = WTM * WTN * 2;
  constexpr int kWavesPerBuf = kStageBytes / kWaveOutBytes;
  static_assert(kWavesPerBuf >= 1 && (kWaves + kWavesPerBuf - 1) / kWavesPerBuf <= STAGES,
                "output staging fits in the stage buffers");
  static_assert(64 % RC == 0 && (WTM * RC) % 64 == 0, "row segments tile the wavefront");
  float4 r_sw[FN][4], r_b[FN][4];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int nl = wn * WTN + i * 32 + 8 * q + 4 * (lane >> 5);
      r_sw[i][q] = *reinterpret_cast<const float4*>(epi_sw + nl);
      const uint2 b2 = *reinterpret_cast<const uint2*>(epi_b16 + nl);  // four bf16 -> fp32 exactly
      r_b[i][q] = make_float4(__uint_as_float(b2.x << 16), __uint_as_float(b2.x & 0xffff0000u),
                              __uint_as_float(b2.y << 16), __uint_as_float(b2.y & 0xffff0000u));
    }
  wait_vm_lgkm0<63>();
  block_barrier();

  uint8_t* wout = buf(wave / kWavesPerBuf) + (wave % kWavesPerBuf) * kWaveOutBytes;
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    const int r = j * 32 + (lane & 31);
#pragma unroll
    for (int i = 0; i < FN; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c8 = i * 32 + 8 * q + 4 * (lane >> 5);
        const float4 sw4 = r_sw[i][q];
        const float4 b4 = r_b[i][q];
        const v16f& a = acc[i][j];
        const float o0 = __builtin_fmaf(a[4 * q + 0], sw4.x, b4.x);
        const float o1 = __builtin_fmaf(a[4 * q + 1], sw4.y, b4.y);
        const float o2 = __builtin_fmaf(a[4 * q + 2], sw4.z, b4.z);
        const float o3 = __builtin_fmaf(a[4 * q + 3], sw4.w, b4.w);
        const int chunk = c8 >> 3, half = (c8 >> 2) & 1;
        *reinterpret_cast<uint2*>(wout + r * (RC * 16) + ((chunk ^ (r % RC)) << 4) + (half << 3)) =
            make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
      }
    }
  }
  // own region only: LDS executes one wave's accesses in order, no barrier needed
  store_wave_tile<WTM, RC>(wout, lane, args.out, args.m, args.n, m0 + wm * WTM, n0 + wn * WTN);
}

template <int BM, int BN, int WM, int WN, int S, int GM, int FMT>
hipError_t launch(const W16Args& a, hipStream_t stream) {
  W16Args args = a;
  args.tiles_m = (a.m + BM - 1) / BM;
  args.tiles_n = (a.n + BN - 1) / BN;
  const int64_t wgs = (int64_t)args.tiles_m * args.tiles_n;
  gemm_w8a16_kernel<BM, BN, WM, WN, S, GM, FMT><<<dim3((unsigned)wgs), dim3(WM * WN * 64), 0, stream>>>(args);
  return hipGetLastError();
}

// id, tile_m, tile_n, waves, stages, name (every stage holds 64 k elements)
const GemmConfig kW16Configs[] = {
    {0, 256, 256, 8, 3, "w16_bm256_bn256_w2x4_s3"},
    {1, 256, 128, 8, 3, "w16_bm256_bn128_w4x2_s3"},
    {2, 128, 256, 8, 4, "w16_bm128_bn256_w2x4_s4"},
    {3, 128, 128, 4, 3, "w16_bm128_bn128_w2x2_s3"},
    {4, 64, 64, 4, 3, "w16_bm64_bn64_w2x2_s3"},
};
constexpr int kNumW16Configs = sizeof(kW16Configs) / sizeof(kW16Configs[0]);

}  // namespace

int w8a16_config_count() { return kNumW16Configs; }

const GemmConfig* w8a16_config(int id) { return (id >= 0 && id < kNumW16Configs) ? &kW16Configs[id] : nullptr; }

int64_t w8a16_workgroups(int id, int64_t m, int64_t n) {
  const GemmConfig* c = w8a16_config(id);
  if (!c) return 0;
  return ((m + c->tile_m - 1) / c->tile_m) * ((n + c->tile_n - 1) / c->tile_n);
}

int w8a16_threads(int id) {
  const GemmConfig* c = w8a16_config(id);
  return c ? 64 * c->waves : 0;
}

template <int FMT>
hipError_t launch_fmt(int id, const W16Args& args, hipStream_t stream) {
  switch (id) {
    case 0: return launch<256, 256, 2, 4, 3, 4, FMT>(args, stream);
    case 1: return launch<256, 128, 4, 2, 3, 4, FMT>(args, stream);
    case 2: return launch<128, 256, 2, 4, 4, 4, FMT>(args, stream);
    case 3: return launch<128, 128, 2, 2, 3, 8, FMT>(args, stream);
    case 4: return launch<64, 64, 2, 2, 3, 8, FMT>(args, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_w8a16(int id, int w_format, int64_t m, int64_t n, int64_t k, const uint16_t* a, const uint8_t* qw,
                        const float* w_scale, const uint16_t* bias, uint16_t* out, hipStream_t stream) {
  W16Args args{a, qw, w_scale, bias, out, (int)m, (int)n, (int)k, 0, 0};
  return w_format == FP8W8A8_FMT_E5M2 ? launch_fmt<FP8W8A8_FMT_E5M2>(id, args, stream)
                                      : launch_fmt<FP8W8A8_FMT_E4M3FN>(id, args, stream);
}

}  // namespace fp8w8a8
