// FP8 (e4m3fn) x FP8 GEMM with the scale / bias / bf16 epilogue fused, for gfx950.
//
//   out[m, n] = bf16_rne( acc[m, n] * a_scale[m] * w_scale[n] + bias[n] ),
//   acc[m, n] = sum_k dec(qa[m, k]) * dec(qw[n, k])   (fp32 accumulation on the MFMA units)
//
// This is the "FP8 GEMM" and "scale / bias / output dtype" part of the chain in
// the HunyuanVideo1.5 BF16->FP8 retrospective (aigcage.com, section 3.1). Both
// operands are k-contiguous: the activation codes [m, k] and the weight in
// nn.Linear's [n, k] layout (the page's column-major B, never transposed).
// Section 3.2 of the page finds that tile shape and the full epilogue, not the
// bare GEMM, decide the speed; the design here is gfx950's own:
//
//   * V_MFMA_F32_16X16X128_F8F6F4: the weight rows feed the MFMA's first operand
//     and the activation rows its second, so each lane's four fp32 results are
//     four consecutive output channels of one token and leave as one 8-byte store;
//   * block tiles of BM (tokens) x BN (channels) x 128 bytes of k, double-buffered
//     in LDS and filled by buffer_load_dwordx4 ... lds (global -> LDS with no VGPR
//     staging). The buffer descriptor covers only the valid rows of the block and
//     lanes past k are pointed out of range, so ragged m / n / k tails read zeros
//     and never touch memory outside the operands;
//   * a 16-byte-chunk XOR swizzle (chunk ^ (row & 7)) makes both the LDS fill and
//     the ds_read_b128 operand reads bank-conflict free;
//   * workgroup ids are remapped so each of the 8 XCDs (own L2 each) walks a
//     contiguous, m-grouped range of tiles, keeping shared operand panels in one L2.
#include "internal.h"

namespace fp8w8a8 {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kBK = 128;          // k bytes per stage (one MFMA k-step)
constexpr int kXcds = 8;          // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kBufferConfig = 0x00020000;  // gfx9 raw buffer: dword3 data format

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

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferConfig);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rsrc, lds_ptr_t dst, uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 16, voffset, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// Workgroup id -> (tile_m, tile_n). Hardware deals ids to XCDs round-robin
// (id % 8); renumber so XCD x owns a contiguous range of logical tiles, then walk
// that range in groups of GROUP_M tile rows so concurrent tiles share panels.
template <int GROUP_M>
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int& tm, int& tn) {
  const int nwg = gridDim.x;
  const int id = blockIdx.x;
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

template <int BM, int BN, int WAVES_M, int WAVES_N, int GROUP_M>
__global__ __launch_bounds__(WAVES_M* WAVES_N * 64) void gemm_fp8_kernel(GemmArgs args) {
  constexpr int kWaves = WAVES_M * WAVES_N;
  constexpr int WTM = BM / WAVES_M;  // wave tile along m (tokens)
  constexpr int WTN = BN / WAVES_N;  // wave tile along n (channels)
  constexpr int FM = WTM / 16;       // 16-token fragments per wave
  constexpr int FN = WTN / 16;       // 16-channel fragments per wave
  constexpr int kStageBytes = (BM + BN) * kBK;
  constexpr int kRowGroups = (BM + BN) / 8;  // one wave-wide LDS fill covers 8 rows x 128 B
  static_assert(BM % (16 * WAVES_M) == 0 && BN % (16 * WAVES_N) == 0, "tile / wave mismatch");
  static_assert(kRowGroups % kWaves == 0, "fill work must split evenly across waves");
  constexpr int kFillsPerWave = kRowGroups / kWaves;

  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kStageBytes];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave % WAVES_M, wn = wave / WAVES_M;

  int tm, tn;
  tile_coords<GROUP_M>(args.tiles_m, args.tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int K = args.k;
  const int rows_a = min(BM, args.m - m0);
  const int rows_w = min(BN, args.n - n0);

  const __amdgpu_buffer_rsrc_t rsrc_a =
      make_rsrc(args.qa + (int64_t)m0 * K, (uint32_t)rows_a * (uint32_t)K);
  const __amdgpu_buffer_rsrc_t rsrc_w =
      make_rsrc(args.qw + (int64_t)n0 * K, (uint32_t)rows_w * (uint32_t)K);

  // Fill geometry: in a wave-wide fill lane i writes LDS bytes [16 i, 16 i + 16) of
  // an 8-row group, i.e. row i/8, chunk position i%8, which holds logical chunk
  // (i%8) ^ (i/8) of that row.
  const int fill_row = lane >> 3;
  const int fill_chunk = (lane & 7) ^ fill_row;
  const uint32_t fill_off = (uint32_t)fill_row * (uint32_t)K + 16u * (uint32_t)fill_chunk;

  auto issue_stage = [&](int stage, int k0) {
    const bool kvalid = k0 + 16 * fill_chunk < K;
    uint8_t* base = smem + stage * kStageBytes;
#pragma unroll
    for (int j = 0; j < kFillsPerWave; ++j) {
      const int g = wave + j * kWaves;  // row group
      lds_ptr_t dst = (lds_ptr_t)(base + g * 1024);
      if (g * 8 < BM) {
        const uint32_t vo = kvalid ? (uint32_t)(g * 8) * (uint32_t)K + fill_off + (uint32_t)k0 : kOutOfRange;
        load_lds16(rsrc_a, dst, vo);
      } else {
        const uint32_t vo =
            kvalid ? (uint32_t)(g * 8 - BM) * (uint32_t)K + fill_off + (uint32_t)k0 : kOutOfRange;
        load_lds16(rsrc_w, dst, vo);
      }
    }
  };

  // Operand reads: lane l reads row (l % 16) of a 16-row fragment, k bytes
  // [32 (l/16), +32) = logical chunks 2 (l/16) and 2 (l/16) + 1, swizzled by row & 7 = l & 7.
  const int frag_row = lane & 15;
  const int kq = lane >> 4;
  const int sw = lane & 7;
  const uint32_t rd0 = (uint32_t)frag_row * kBK + 16u * (uint32_t)((2 * kq) ^ sw);
  const uint32_t rd1 = (uint32_t)frag_row * kBK + 16u * (uint32_t)((2 * kq + 1) ^ sw);

  v4f acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int ktiles = (K + kBK - 1) / kBK;
  issue_stage(0, 0);
  for (int kt = 0; kt < ktiles; ++kt) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (kt + 1 < ktiles) issue_stage((kt + 1) & 1, (kt + 1) * kBK);

    const uint8_t* sa = smem + (kt & 1) * kStageBytes + (wm * WTM) * kBK;
    const uint8_t* sw_ = smem + (kt & 1) * kStageBytes + (BM + wn * WTN) * kBK;
    v8i afrag[FM];
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const uint4 lo = *reinterpret_cast<const uint4*>(sa + j * 16 * kBK + rd0);
      const uint4 hi = *reinterpret_cast<const uint4*>(sa + j * 16 * kBK + rd1);
      afrag[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const uint4 lo = *reinterpret_cast<const uint4*>(sw_ + i * 16 * kBK + rd0);
      const uint4 hi = *reinterpret_cast<const uint4*>(sw_ + i * 16 * kBK + rd1);
      const v8i wfrag = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
#pragma unroll
      for (int j = 0; j < FM; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wfrag, afrag[j], acc[i][j], 0, 0, 0, 0, 0, 0);
    }
  }

  // Epilogue: lane holds, for fragment (i, j), channels n = .. + 4 (l/16) + 0..3 of token
  // m = .. + (l % 16). One fp32 expression, one rounding to bf16, one 8-byte store.
  const int64_t N = args.n;
#pragma unroll
  for (int j = 0; j < FM; ++j) {
    const int m = m0 + wm * WTM + j * 16 + (lane & 15);
    if (m >= args.m) continue;
    const float sa = args.a_scale[m];
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const int n = n0 + wn * WTN + i * 16 + 4 * (lane >> 4);
      if (n >= args.n) continue;
      const float4 sw4 = *reinterpret_cast<const float4*>(args.w_scale + n);
      float b[4] = {0.f, 0.f, 0.f, 0.f};
      if (args.bias) {
        const uint2 braw = *reinterpret_cast<const uint2*>(args.bias + n);
        b[0] = __uint_as_float(braw.x << 16);
        b[1] = __uint_as_float(braw.x & 0xffff0000u);
        b[2] = __uint_as_float(braw.y << 16);
        b[3] = __uint_as_float(braw.y & 0xffff0000u);
      }
      const v4f a = acc[i][j];
      const float o0 = __builtin_fmaf(a[0] * sa, sw4.x, b[0]);
      const float o1 = __builtin_fmaf(a[1] * sa, sw4.y, b[1]);
      const float o2 = __builtin_fmaf(a[2] * sa, sw4.z, b[2]);
      const float o3 = __builtin_fmaf(a[3] * sa, sw4.w, b[3]);
      *reinterpret_cast<uint2*>(args.out + (int64_t)m * N + n) = make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
    }
  }
}

template <int BM, int BN, int WM, int WN, int GM>
hipError_t launch(const GemmArgs& a, hipStream_t stream) {
  GemmArgs args = a;
  args.tiles_m = (a.m + BM - 1) / BM;
  args.tiles_n = (a.n + BN - 1) / BN;
  const int64_t wgs = (int64_t)args.tiles_m * args.tiles_n;
  gemm_fp8_kernel<BM, BN, WM, WN, GM><<<dim3((unsigned)wgs), dim3(WM * WN * 64), 0, stream>>>(args);
  return hipGetLastError();
}

const GemmConfig kConfigs[] = {
    {0, 256, 256, "bm256_bn256_w2x2"},
    {1, 256, 128, "bm256_bn128_w2x2"},
    {2, 128, 256, "bm128_bn256_w2x2"},
    {3, 128, 128, "bm128_bn128_w2x2"},
    {4, 64, 64, "bm64_bn64_w2x2"},
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

hipError_t launch_gemm(int id, int64_t m, int64_t n, int64_t k, const uint8_t* qa, const float* a_scale,
                       const uint8_t* qw, const float* w_scale, const uint16_t* bias, uint16_t* out,
                       hipStream_t stream) {
  GemmArgs a{qa, a_scale, qw, w_scale, bias, out, (int)m, (int)n, (int)k, 0, 0};
  switch (id) {
    case 0: return launch<256, 256, 2, 2, 4>(a, stream);
    case 1: return launch<256, 128, 2, 2, 4>(a, stream);
    case 2: return launch<128, 256, 2, 2, 4>(a, stream);
    case 3: return launch<128, 128, 2, 2, 8>(a, stream);
    case 4: return launch<64, 64, 2, 2, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fp8w8a8
