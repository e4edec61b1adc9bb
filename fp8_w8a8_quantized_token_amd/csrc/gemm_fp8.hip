// FP8 (e4m3fn) x FP8 GEMM with the scale / bias / bf16 epilogue fused, for gfx950.
//
//   out[m, n] = bf16_rne( acc[m, n] * a_scale[m] * w_scale[n] + bias[n] ),
//   acc[m, n] = sum_k dec(qa[m, k]) * dec(qw[n, k])   (fp32 accumulation on the MFMA units)
//
// This is the "FP8 GEMM" and "scale / bias / output dtype" part of the chain in the
// HunyuanVideo1.5 BF16->FP8 retrospective (aigcage.com, section 3.1). Both operands
// are k-contiguous: the activation codes [m, k] and the weight in nn.Linear's [n, k]
// layout (the page's column-major B, never transposed). Section 3.2 of the page finds
// that the tile shape, the memory pipeline and the full epilogue, not the bare GEMM,
// decide the speed. The design here is gfx950's own:
//
//   * V_MFMA_F32_32X32X64_F8F6F4. The weight rows feed the MFMA's first operand and
//     the activation rows its second, so a lane's results come in runs of four
//     consecutive output channels of one token: one 8-byte bf16 store each.
//   * Block tiles of BM tokens x BN channels, 64 bytes of k per stage, STAGES stage
//     buffers in LDS (up to the 160 KiB of a CU). Stages are filled by
//     buffer_load_dwordx4 ... lds (HBM/L2 -> LDS with no VGPR staging) STAGES - 1
//     sub-steps ahead of their use, so an L2 miss has several MFMA sub-steps to land.
//     Each wave waits with a precise vmcnt for its own fills of the stage it is about
//     to read, then the workgroup barrier publishes every wave's fills.
//   * The buffer descriptors cover only the block's valid rows, and lanes past k are
//     pointed out of range: ragged m / n / k tails read zeros and no access leaves
//     the operands.
//   * LDS rows are 64 bytes; 16-byte chunk c of row r sits at position
//     c ^ f(r), f(r) = ((r >> 1) & 3) ^ ((r >> 3) & 1), which makes the fills and the
//     ds_read_b128 operand reads free of bank conflicts.
//   * Two waves per SIMD (8-wave workgroups) for the large tiles, so one wave's
//     barrier or LDS wait is covered by the other's MFMAs.
//   * Workgroup ids are remapped so each of the 8 XCDs (own L2 each) walks a
//     contiguous, m-grouped range of tiles and concurrent tiles share panels in L2.
//   * The tile's scales and bias are requested at kernel start (one value per
//     thread), staged through LDS after the k loop, and applied in fp32 with a single
//     rounding to bf16. The bf16 tile is then staged through LDS as well, so the
//     output leaves in whole 128-byte lines (16 bytes per lane) instead of scattered
//     8-byte pieces.
#include "internal.h"
#include "gemm_common.h"

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
};

template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, int BK, int GROUP_M>
struct KernelTag {};

template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, int BK, int GROUP_M>
__global__ __launch_bounds__(WAVES_M* WAVES_N * 64) void gemm_fp8_kernel(GemmArgs args) {
  using Tag = KernelTag<BM, BN, WAVES_M, WAVES_N, STAGES, BK, GROUP_M>;
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
  static_assert(STAGES * kStageBytes <= 160 * 1024, "LDS budget of a CU");
  constexpr int F = kRowGroups / kWaves;  // fills per wave per stage
  static_assert((STAGES - 1) * F < 64, "vmcnt range");
  static_assert((BM / RPF) % kWaves == 0, "activation fills split evenly across waves");
  static_assert(BM <= kWaves * 64 && BN <= kWaves * 64, "one epilogue operand per thread");
  static_assert((BM + 2 * BN) * 4 <= kStageBytes, "epilogue staging fits in one stage");

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

  // Epilogue operands of this tile, one value per thread, requested now so their
  // latency hides behind the k loop.
  const int tid = threadIdx.x;
  float pre_sa = 0.0f, pre_sw = 0.0f, pre_b = 0.0f;
  if (tid < BM && tid < rows_a) pre_sa = args.a_scale[m0 + tid];
  if (tid < BN && tid < rows_w) {
    pre_sw = args.w_scale[n0 + tid];
    if (args.bias) pre_b = __uint_as_float((uint32_t)args.bias[n0 + tid] << 16);
  }

  // Fill geometry: a wave-wide fill covers RPF rows x BK bytes = 1 KiB of a stage;
  // lane i writes bytes [16 i, 16 i + 16): row i / CPR of the group, position i % CPR,
  // which holds logical chunk (i % CPR) ^ swz(row). swz depends on row % 16, so with
  // 8-row fills (BK = 128) the chunk differs between even and odd row groups. Tile rows
  // 0..BM-1 are the activation, BM.. the weight; wave w fills row groups w, w + kWaves, ...
  const int fr = lane / CPR;
  const int fchunk0 = (lane % CPR) ^ swz<BK>(fr);            // row group with g * RPF % 16 == 0
  const int fchunk1 = (lane % CPR) ^ swz<BK>(fr + RPF % 16);  // row group with g * RPF % 16 == 8
  const uint32_t foff0 = (uint32_t)fr * (uint32_t)K + 16u * (uint32_t)fchunk0;
  const uint32_t foff1 = (uint32_t)fr * (uint32_t)K + 16u * (uint32_t)fchunk1;

  auto issue = [&](uint8_t* base, int k0) {
    const bool kvalid0 = k0 + 16 * fchunk0 < K;
    const bool kvalid1 = k0 + 16 * fchunk1 < K;
#pragma unroll
    for (int j = 0; j < F; ++j) {
      const int g = wave + j * kWaves;
      const bool odd = ((g * RPF) & 15) != 0;
      const bool kvalid = odd ? kvalid1 : kvalid0;
      const uint32_t foff = odd ? foff1 : foff0;
      const uint32_t dst = (uint32_t)reinterpret_cast<uintptr_t>(base + g * 1024);
      if (j < (BM / RPF) / kWaves) {
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
#pragma unroll
  for (int s = 0; s < STAGES; ++s)
    if (s < nst) issue(buf(s), s * BK);
  Frags f0, f1;
  wait_stage<F, STAGES>(min(nst - 1, STAGES - 1));
  block_barrier();
  read_frags(buf(0), 0, f0);

  auto sub = [&](int u, int s, int h, Frags& cur, Frags& nxt) {
    // s = stage index of u modulo STAGES, h = half of u (compile-time after unrolling)
    const int t = u / H;
    if (h == H - 1) {
      if (t + 1 < nst) {
        wait_stage<F, STAGES>(min(nst - 2 - t, STAGES - 2));
        block_barrier();
        if (t + STAGES < nst) issue(buf(s), (t + STAGES) * BK);
      }
      read_frags(buf((s + 1) % STAGES), 0, nxt);
    } else {
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
  // 1. Stage the tile's scales and bias in LDS, then pull each lane's share into
  //    registers (the operand fragments are dead by now).
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
  float* epi_sa = reinterpret_cast<float*>(buf(0));
  float* epi_sw = epi_sa + BM;
  float* epi_b = epi_sw + BN;
  block_barrier();
  if (tid < BM) epi_sa[tid] = pre_sa;
  if (tid < BN) {
    epi_sw[tid] = pre_sw;
    epi_b[tid] = pre_b;
  }
  wait_vm_lgkm0<63>();  // lgkmcnt(0): the LDS writes are done
  block_barrier();
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
  const int64_t N = args.n;
  constexpr int kRowsPerStore = 64 / RC;
#pragma unroll
  for (int t = 0; t < WTM / kRowsPerStore; ++t) {
    const int r = t * kRowsPerStore + lane / RC;
    const int c = lane % RC;
    const uint4 v = *reinterpret_cast<const uint4*>(wout + r * (RC * 16) + ((c ^ (r % RC)) << 4));
    const int m = m0 + wm * WTM + r;
    const int n = n0 + wn * WTN + c * 8;
    if (m < args.m && n < args.n) *reinterpret_cast<uint4*>(args.out + (int64_t)m * N + n) = v;
  }
}

template <int BM, int BN, int WM, int WN, int S, int BK, int GM>
hipError_t launch(const GemmArgs& a, hipStream_t stream) {
  GemmArgs args = a;
  args.tiles_m = (a.m + BM - 1) / BM;
  args.tiles_n = (a.n + BN - 1) / BN;
  const int64_t wgs = (int64_t)args.tiles_m * args.tiles_n;
  gemm_fp8_kernel<BM, BN, WM, WN, S, BK, GM><<<dim3((unsigned)wgs), dim3(WM * WN * 64), 0, stream>>>(args);
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
    case 2: return launch<128, 256, 2, 4, 3, 128, 4>(a, stream);
    case 3: return launch<128, 128, 2, 2, 2, 128, 8>(a, stream);
    case 4: return launch<64, 64, 2, 2, 3, 128, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fp8w8a8
