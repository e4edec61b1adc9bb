// C ABI of libfp8w8a8: argument checks, the construction-time plan and its
// shape-keyed kernel selector, and the launch sequence of a forward.
//
// The HunyuanVideo1.5 BF16->FP8 retrospective (aigcage.com, section 3.3) moves
// every generic decision (input kind checks, "is the native op loaded", "which
// backend suits this shape", "fall back to torch?") out of the per-layer forward
// and into construction. Here: fp8_linear_create validates the weight, checks
// the device once and picks a GEMM configuration per activation-row bucket from
// (n, k, compute units); fp8_linear_run does O(1) argument checks, one bucket
// lookup and two launches. There is no fallback path of any kind.
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <mutex>
#include <random>

#include "internal.h"

using namespace fp8w8a8;

// Most activation-row buckets a plan keeps (see the bucket bounds below).
constexpr int kMaxBuckets = 10;

struct fp8_linear_plan {
  int device;
  int64_t n, k;
  const uint8_t* w;
  const float* w_scale;
  const uint16_t* bias;
  int cu_count;
  // m buckets: rows <= max_m[b] use config[b]; the last bucket is unbounded
  int64_t max_m[kMaxBuckets];
  int config[kMaxBuckets];
};

struct fp8_w8a16_plan {
  int device;
  int w_format;
  int64_t n, k;
  const uint8_t* w;
  const float* w_scale;
  const uint16_t* bias;
  int cu_count;
  int64_t max_m[kMaxBuckets];
  int config[kMaxBuckets];
};

namespace {

constexpr int64_t kMaxGridThreads = (int64_t)1 << 32;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Per-device "is gfx950" and compute-unit count, filled once per device ordinal.
constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other
std::atomic<int> g_dev_cus[kMaxDevices];

int query_device(int device, int* cus) {
  if (device < 0 || device >= kMaxDevices) return FP8W8A8_ERR_BAD_DEVICE;
  int st = g_dev_state[device].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) return FP8W8A8_ERR_HIP;
    st = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_dev_cus[device].store(prop.multiProcessorCount, std::memory_order_relaxed);
    g_dev_state[device].store(st, std::memory_order_release);
  }
  if (cus) *cus = g_dev_cus[device].load(std::memory_order_relaxed);
  return st == 1 ? FP8W8A8_OK : FP8W8A8_ERR_BAD_DEVICE;
}

int current_device_ok(int* cus = nullptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FP8W8A8_ERR_HIP;
  return query_device(dev, cus);
}

// A plan's weights live on the device it was created for; a run launches on the
// current device (or the stream's, which must be the same), so the two must agree.
int plan_device_current(int plan_device) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return FP8W8A8_ERR_HIP;
  return dev == plan_device ? FP8W8A8_OK : FP8W8A8_ERR_BAD_DEVICE;
}

bool valid_act(int act) {
  return act == FP8W8A8_ACT_GELU_ERF || act == FP8W8A8_ACT_GELU_TANH || act == FP8W8A8_ACT_SILU;
}

int check_quant_args(const void* x, int64_t rows, int64_t cols, const void* q, const float* scale) {
  if (!x || !q || !scale) return FP8W8A8_ERR_INVALID_ARG;
  if (rows < 0 || rows >= FP8W8A8_MAX_ROWS) return FP8W8A8_ERR_BAD_SHAPE;
  if (cols < 16 || cols > FP8W8A8_MAX_DIM || cols % 16 != 0) return FP8W8A8_ERR_BAD_SHAPE;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(scale, 4)) return FP8W8A8_ERR_MISALIGNED;
  return FP8W8A8_OK;
}

int check_weight_args(int64_t n, int64_t k, const void* w, const float* w_scale, const void* bias) {
  if (!w || !w_scale) return FP8W8A8_ERR_INVALID_ARG;
  if (n < 16 || k < 16 || n > FP8W8A8_MAX_DIM || k > FP8W8A8_MAX_DIM) return FP8W8A8_ERR_BAD_SHAPE;
  if (n % 16 != 0 || k % 16 != 0) return FP8W8A8_ERR_BAD_SHAPE;
  if (!aligned(w, 16) || !aligned(w_scale, 16) || (bias && !aligned(bias, 16))) return FP8W8A8_ERR_MISALIGNED;
  return FP8W8A8_OK;
}

// Relative k-loop throughput of one workgroup of each configuration, with one workgroup
// on a CU (eff1) and with two or more sharing it (eff2); how many of its workgroups can
// share a CU (LDS / register bound); and the per-tile fixed cost (prologue, epilogue,
// output stores) in units of k, alone on a CU (f1) and shared (f2: co-resident
// workgroups overlap one's fixed cost with the other's k loop). The two families order
// their configurations the same way: 256 x 256, 256 x 128, 128 x 256, 128 x 128
// (4 waves), 64 x 64 (4 waves).
struct TileModel {
  double eff1, eff2;
  int per_cu;
  double f1, f2;
};
// FP8 GEMM, fitted to MI355X timings (the configurations interleaved in one process, 17
// shapes from 26 x 2048 x 2048 to 32760 x 2048 x 8192, time per round of co-resident tiles
// at k = 2048 and 8192): one 256 x 256 tile per CU costs the time of ~580 k of loop in fixed
// work; the 256 x 128 and 128 x 256 tiles run their loop at ~0.84 of its rate per output
// (128 x 256 kept ahead on ties: it was up to 11% faster at mid sizes); two co-resident
// 4-wave 128 x 128 workgroups run at 0.75 but hide most of the fixed cost (~200 k), so they
// win at k = 2048 and lose at k = 8192; a lone one runs at about half rate.
TileModel w8a8_tile_model(int config) {
  switch (config) {
    case 0: return {1.00, 1.00, 1, 580, 580};
    case 1: return {0.84, 0.84, 1, 580, 580};
    case 2: return {0.845, 0.845, 1, 580, 580};
    case 3: return {0.48, 0.75, 2, 580, 200};
    default: return {0.44, 0.39, 3, 580, 240};
  }
}
// W8A16: 128 x 256 measured 4% faster than 256 x 128 at FFN-down (4096 x 2048 x 8192).
// (No fixed-cost term: its picks depend on m and n only.)
TileModel w8a16_tile_model(int config) {
  switch (config) {
    case 0: return {1.00, 1.00, 1, 0, 0};
    case 1: return {0.95, 0.95, 1, 0, 0};
    case 2: return {0.96, 0.96, 1, 0, 0};
    case 3: return {0.75, 0.75, 2, 0, 0};
    default: return {0.40, 0.40, 3, 0, 0};
  }
}

// A family of compiled GEMM configurations (the W8A8 GEMM, the W8A16 GEMM) as the
// selector sees it.
struct Family {
  const int64_t* bounds;  // m bucket bounds, ascending; the last is unbounded
  int buckets;
  int (*count)();
  const GemmConfig* (*config)(int);
  int64_t (*workgroups)(int, int64_t, int64_t);
  int (*threads)(int);
  TileModel (*model)(int);
  int skinny;           // configuration for m <= skinny_max_m (outside the tile model), or -1
  int64_t skinny_max_m;
  int skinny_wide;      // its form with more channels per workgroup, for grids wider than the CUs, or -1
  int persistent;       // persistent form of configuration 0 (outside the tile model), or -1
};
// m buckets: rows <= bound[b] use the configuration chosen at that bound; the last bucket
// is unbounded and chosen at 32768 rows. The W8A8 model picks the measured best on all 17
// timed shapes with these bounds; the W8A16 model, which has no fixed-cost term, needs the
// finer powers of two (with the coarse bounds it kept 128 x 256 tiles at 512 x 8192 x 2048
// and 2048 x 2048 x 8192, 13% and 11% slower than 128 x 128 there).
constexpr int64_t kW8A8Bounds[] = {32, 64, 256, 1024, 4096, 16384, FP8W8A8_MAX_ROWS};
constexpr int64_t kW8A16Bounds[] = {64, 128, 256, 512, 1024, 2048, 4096, 8192, 16384, FP8W8A8_MAX_ROWS};
static_assert(sizeof(kW8A8Bounds) / sizeof(int64_t) <= kMaxBuckets, "bucket count");
static_assert(sizeof(kW8A16Bounds) / sizeof(int64_t) <= kMaxBuckets, "bucket count");
// The skinny W8A8 configuration (one workgroup per 16 channels, k split across its waves)
// is a weight stream, not a tile of the model above. Timed against the 64 x 64 tiles
// (graph-replayed launches, random codes, rotating weights): m = 26 at n x k = 2048 x 2048
// 5.4 against 9.1 us, 8192 x 2048 7.9 against 9.3, 2048 x 8192 12.7 against 25.8; m = 1
// 4.0 against 9.0. Above 32 tokens it loads the weight once per 32 tokens and loses at
// wide n (m = 64, n = 8192: 14.8 against 9.6 us), so it serves m <= 32 only.
constexpr int kW8A8Skinny = 5;
// Configuration 7 is the same weight stream with 32 channels per workgroup: the activation
// is loaded once for twice the weight bytes, on half the workgroups; every output is
// bit-identical to configuration 5's. Timed against it (graph-replayed launches over
// > 256 MB of rotating weights, random codes, m = 26, k = 2048): 384 workgroups of
// configuration 5 (n = 6144, the grid of the Q/K/V encoder group) 8.00 -> 6.95 us, 512
// (n = 8192) 8.29 -> 7.31; at 256 or fewer it loses (n = 4096: 5.87 against 7.21 us, n =
// 2048: 5.16 against 6.57, k = 8192: 12.7 against 17.1), and the step is at the CU count:
// 256 workgroups of configuration 5 (n = 4096) 5.57 us, 272 (n = 4352) 7.77, against 6.6
// for configuration 7 at both. So it serves the skinny products whose configuration-5 grid
// exceeds the CU count.
constexpr int kW8A8SkinnyWide = 7;
// The persistent form of the 256 x 256 tiles (one workgroup per CU walking its tiles, the
// next tile's first stages requested before the current tile's epilogue) is output-for-
// output identical to configuration 0. Timed against it on 32 shapes (m 2048 .. 32760,
// n 2048 / 8192, k 1024 .. 8192, interleaved in one process) it was faster wherever each
// CU had two or more tiles and k was 2048 or 4096 (FFN-up 69.3 -> 67.4 us, 8192 x 8192 x
// 2048 122.8 -> 119.8, 32760 x 8192 x 2048 474 -> 465), within +-1% or slower elsewhere:
// its fill offsets cost a little per k step, so with one tile per CU, or at k = 8192, the
// saved prologue does not pay for them, and at k = 1024 the results went either way.
constexpr int kW8A8Persistent = 6;
const Family kW8A8{kW8A8Bounds, (int)(sizeof(kW8A8Bounds) / sizeof(int64_t)), gemm_config_count, gemm_config,
                   gemm_workgroups, gemm_threads, w8a8_tile_model, kW8A8Skinny, 32, kW8A8SkinnyWide,
                   kW8A8Persistent};
const Family kW8A16{kW8A16Bounds, (int)(sizeof(kW8A16Bounds) / sizeof(int64_t)), w8a16_config_count, w8a16_config,
                    w8a16_workgroups, w8a16_threads, w8a16_tile_model, -1, 0, -1, -1};

bool grid_fits(const Family& f, int config, int64_t m, int64_t n) {
  return f.workgroups(config, m, n) * f.threads(config) < kMaxGridThreads;
}
bool grid_fits(int config, int64_t m, int64_t n) { return grid_fits(kW8A8, config, m, n); }

// Estimated time (arbitrary units) of configuration c on an m x n x k product: rounds of
// co-resident tiles times the work of one round, its k loop plus its fixed cost.
double model_time(const Family& f, int c, int64_t m, int64_t n, int64_t k, int cus) {
  const GemmConfig* g = f.config(c);
  const TileModel t = f.model(c);
  const int64_t tiles = f.workgroups(c, m, n);
  const int64_t conc = std::min<int64_t>(t.per_cu, (tiles + cus - 1) / cus);
  const int64_t rounds = (tiles + cus * conc - 1) / (cus * conc);
  const bool shared = conc >= 2;
  return (double)rounds * conc * (double)g->tile_m * (double)g->tile_n * ((double)k + (shared ? t.f2 : t.f1)) /
         (shared ? t.eff2 : t.eff1);
}

int choose_config(const Family& f, int64_t m, int64_t n, int64_t k, int cus) {
  if (f.skinny >= 0 && m <= f.skinny_max_m) {
    if (f.skinny_wide >= 0 && f.workgroups(f.skinny, m, n) > cus && grid_fits(f, f.skinny_wide, m, n))
      return f.skinny_wide;
    if (grid_fits(f, f.skinny, m, n)) return f.skinny;
  }
  int best = -1;
  double best_t = 0;
  for (int c = 0; c < f.count(); ++c) {
    // the weight-stream forms (no LDS pipeline) are outside the tile model
    if (c == f.skinny || c == f.skinny_wide || c == f.persistent || f.config(c)->stages == 0 ||
        !grid_fits(f, c, m, n))
      continue;
    const double t = model_time(f, c, m, n, k, cus);
    if (best < 0 || t < best_t) {
      best = c;
      best_t = t;
    }
  }
  if (best < 0) best = 0;
  if (best == 0 && f.persistent >= 0 && k >= 2048 && k <= 4096 && f.workgroups(0, m, n) >= 2 * (int64_t)cus &&
      grid_fits(f, f.persistent, m, n))
    best = f.persistent;
  return best;
}


void fill_buckets(const Family& f, int64_t n, int64_t k, int cus, int64_t* max_m, int* config) {
  for (int b = 0; b < f.buckets; ++b) {
    max_m[b] = f.bounds[b];
    const int64_t rep = b + 1 < f.buckets ? f.bounds[b] : 32768;
    config[b] = choose_config(f, rep, n, k, cus);
  }
}

int bucket_config(const Family& f, const int64_t* max_m, const int* config, int64_t n, int64_t m) {
  int b = 0;
  while (b + 1 < f.buckets && m > max_m[b]) ++b;
  int c = config[b];
  if (!grid_fits(f, c, m, n)) c = 0;  // the largest tile launches the fewest workgroups
  return c;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The fixed scratch of fp8_linear_run_noalloc: a file-scope device array, one copy per
// GPU, held from the library's first use on that GPU until the process ends. In host
// code `scratch` is only a handle for the symbol lookup below, not a device address;
// kernels get the per-device address that hipGetSymbolAddress returns.
__device__ __align__(256) uint8_t scratch[FP8W8A8_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mutex;
std::atomic<uint8_t*> g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on `device`, which must be the current device; looked up
// once per device (no allocation). NULL on failure.
uint8_t* scratch_on(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  uint8_t* p = g_scratch_ptr[device].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  p = g_scratch_ptr[device].load(std::memory_order_relaxed);
  if (!p) {
    void* addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return nullptr;
    p = static_cast<uint8_t*>(addr);
    g_scratch_ptr[device].store(p, std::memory_order_release);
  }
  return p;
}

// Launch epochs of the single-launch quant + GEMM: unique within the process (a
// counter) and unlikely to repeat another process's (a random 64-bit start), so a
// workspace's flags from any earlier launch never match the current one.
unsigned long long next_epoch() {
  static std::atomic<unsigned long long> counter{[] {
    std::random_device rd;
    return ((unsigned long long)rd() << 32) ^ (unsigned long long)rd() ^
           (unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count();
  }()};
  return counter.fetch_add(1, std::memory_order_relaxed);
}

}  // namespace

extern "C" {

const char* fp8w8a8_status_string(int status) {
  switch (status) {
    case FP8W8A8_OK: return "ok";
    case FP8W8A8_ERR_INVALID_ARG: return "invalid argument: a required pointer is NULL or an enum value is unknown";
    case FP8W8A8_ERR_BAD_SHAPE: return "bad shape: a size is out of range, empty, or not a multiple of 16";
    case FP8W8A8_ERR_MISALIGNED: return "misaligned pointer: see the alignment rules in fp8w8a8.h";
    case FP8W8A8_ERR_BAD_DEVICE: return "bad device: not a gfx950 (MI355X-class) GPU";
    case FP8W8A8_ERR_WORKSPACE_TOO_SMALL: return "workspace too small: see fp8_linear_workspace_bytes";
    case FP8W8A8_ERR_HIP: return "HIP runtime error";
    case FP8W8A8_ERR_CAPTURE: return "not capturable: this call cannot be recorded into a HIP graph";
    case FP8W8A8_ERR_TOO_LARGE: return "too large: the input exceeds FP8W8A8_NOALLOC_SCRATCH_BYTES";
    default: return "unknown status";
  }
}

int fp8_quant_rows(const void* x_bf16, int64_t rows, int64_t cols, void* q_out, float* scale_out,
                   void* stream) {
  int st = check_quant_args(x_bf16, rows, cols, q_out, scale_out);
  if (st != FP8W8A8_OK) return st;
  if (rows == 0) return FP8W8A8_OK;
  st = current_device_ok();
  if (st != FP8W8A8_OK) return st;
  hipError_t e = launch_quant_rows(static_cast<const uint16_t*>(x_bf16), rows, cols,
                                   static_cast<uint8_t*>(q_out), scale_out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8W8A8_OK : FP8W8A8_ERR_HIP;
}

int fp8_act_table_build(int act, void* table, void* stream) {
  if (!table || !valid_act(act)) return FP8W8A8_ERR_INVALID_ARG;
  if (!aligned(table, 16)) return FP8W8A8_ERR_MISALIGNED;
  int st = current_device_ok();
  if (st != FP8W8A8_OK) return st;
  hipError_t e = launch_act_table(act, static_cast<uint16_t*>(table), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8W8A8_OK : FP8W8A8_ERR_HIP;
}

int fp8_act_rows(const void* x_bf16, int64_t rows, int64_t cols, const void* table, void* y_bf16, void* stream) {
  if (!x_bf16 || !table || !y_bf16) return FP8W8A8_ERR_INVALID_ARG;
  if (rows < 0 || rows >= FP8W8A8_MAX_ROWS) return FP8W8A8_ERR_BAD_SHAPE;
  if (cols < 16 || cols > FP8W8A8_MAX_DIM || cols % 16 != 0) return FP8W8A8_ERR_BAD_SHAPE;
  if (!aligned(x_bf16, 16) || !aligned(table, 16) || !aligned(y_bf16, 16)) return FP8W8A8_ERR_MISALIGNED;
  if (rows == 0) return FP8W8A8_OK;
  int cus = 0;
  int st = current_device_ok(&cus);
  if (st != FP8W8A8_OK) return st;
  hipError_t e = launch_act_rows(static_cast<const uint16_t*>(x_bf16), rows * cols, static_cast<const uint16_t*>(table),
                                 static_cast<uint16_t*>(y_bf16), cus, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8W8A8_OK : FP8W8A8_ERR_HIP;
}

int fp8_act_quant_rows(const void* x_bf16, int64_t rows, int64_t cols, const void* table, void* q_out,
                       float* scale_out, void* stream) {
  if (!table) return FP8W8A8_ERR_INVALID_ARG;
  int st = check_quant_args(x_bf16, rows, cols, q_out, scale_out);
  if (st != FP8W8A8_OK) return st;
  if (!aligned(table, 16)) return FP8W8A8_ERR_MISALIGNED;
  if (rows == 0) return FP8W8A8_OK;
  int cus = 0;
  st = current_device_ok(&cus);
  if (st != FP8W8A8_OK) return st;
  hipError_t e = launch_act_quant_rows(static_cast<const uint16_t*>(x_bf16), rows, cols,
                                       static_cast<const uint16_t*>(table), static_cast<uint8_t*>(q_out), scale_out,
                                       cus, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8W8A8_OK : FP8W8A8_ERR_HIP;
}

size_t fp8_quant_tensor_workspace_bytes(void) { return quant_tensor_workspace_bytes(); }

static int check_tensor_args(const void* x, int64_t numel, int format, const void* out) {
  if (!x || !out) return FP8W8A8_ERR_INVALID_ARG;
  if (format != FP8W8A8_FMT_E4M3FN && format != FP8W8A8_FMT_E5M2) return FP8W8A8_ERR_INVALID_ARG;
  if (numel < 0 || numel >= FP8W8A8_MAX_ROWS * FP8W8A8_MAX_DIM || numel % 16 != 0) return FP8W8A8_ERR_BAD_SHAPE;
  if (!aligned(x, 16) || !aligned(out, 16)) return FP8W8A8_ERR_MISALIGNED;
  return FP8W8A8_OK;
}

int fp8_quant_tensor_form(int form, const void* x_bf16, int64_t numel, int format, void* q_out, float* scale_out,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (form < FP8W8A8_TENSOR_FORM_AUTO || form > FP8W8A8_TENSOR_FORM_ONE_PASS_NO_WAIT) return FP8W8A8_ERR_INVALID_ARG;
  int st = check_tensor_args(x_bf16, numel, format, q_out);
  if (st != FP8W8A8_OK) return st;
  if (!scale_out || !workspace) return FP8W8A8_ERR_INVALID_ARG;
  if (!aligned(scale_out, 4) || !aligned(workspace, 16)) return FP8W8A8_ERR_MISALIGNED;
  if (workspace_bytes < quant_tensor_workspace_bytes()) return FP8W8A8_ERR_WORKSPACE_TOO_SMALL;
  if (numel == 0) return FP8W8A8_OK;
  int cus = 0;
  st = current_device_ok(&cus);
  if (st != FP8W8A8_OK) return st;
  if ((form == FP8W8A8_TENSOR_FORM_ONE_PASS || form == FP8W8A8_TENSOR_FORM_ONE_PASS_NO_WAIT) &&
      !quant_tensor_fits_one_pass(numel, cus))
    return FP8W8A8_ERR_BAD_SHAPE;
  static_assert(kTensorAuto == FP8W8A8_TENSOR_FORM_AUTO && kTensorOnePass == FP8W8A8_TENSOR_FORM_ONE_PASS &&
                    kTensorTwoPass == FP8W8A8_TENSOR_FORM_TWO_PASS &&
                    kTensorOnePassNoWait == FP8W8A8_TENSOR_FORM_ONE_PASS_NO_WAIT,
                "form numbering");
  hipError_t e = launch_quant_tensor(static_cast<const uint16_t*>(x_bf16), numel, format, static_cast<uint8_t*>(q_out),
                                     scale_out, static_cast<float*>(workspace), cus, static_cast<hipStream_t>(stream),
                                     form);
  return e == hipSuccess ? FP8W8A8_OK : FP8W8A8_ERR_HIP;
}

int fp8_quant_tensor(const void* x_bf16, int64_t numel, int format, void* q_out, float* scale_out, void* workspace,
                     size_t workspace_bytes, void* stream) {
  return fp8_quant_tensor_form(FP8W8A8_TENSOR_FORM_AUTO, x_bf16, numel, format, q_out, scale_out, workspace,
                               workspace_bytes, stream);
}

int fp8_dequant_tensor(const void* q, int64_t numel, int format, const float* scale, float* out_f32, void* stream) {
  int st = check_tensor_args(q, numel, format, out_f32);
  if (st != FP8W8A8_OK) return st;
  if (!scale) return FP8W8A8_ERR_INVALID_ARG;
  if (!aligned(scale, 4)) return FP8W8A8_ERR_MISALIGNED;
  if (numel == 0) return FP8W8A8_OK;
  int cus = 0;
  st = current_device_ok(&cus);
  if (st != FP8W8A8_OK) return st;
  hipError_t e = launch_dequant_tensor(static_cast<const uint8_t*>(q), numel, format, scale, out_f32, cus,
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8W8A8_OK : FP8W8A8_ERR_HIP;
}

int fp8_quant_weights_per_channel(const void* w_bf16, int64_t n, int64_t k, void* w_fp8_out,
                                  float* w_scale_out, void* stream) {
  if (n == 0 || k == 0) return FP8W8A8_ERR_BAD_SHAPE;
  return fp8_quant_rows(w_bf16, n, k, w_fp8_out, w_scale_out, stream);
}

int fp8_linear_create(int device, int64_t n, int64_t k, const void* w_fp8, const float* w_scale,
                      const void* bias_bf16, fp8_linear_plan** out) {
  if (!out) return FP8W8A8_ERR_INVALID_ARG;
  int st = check_weight_args(n, k, w_fp8, w_scale, bias_bf16);
  if (st != FP8W8A8_OK) return st;
  int cus = 0;
  st = query_device(device, &cus);
  if (st != FP8W8A8_OK) return st;
  fp8_linear_plan* p = static_cast<fp8_linear_plan*>(calloc(1, sizeof(fp8_linear_plan)));
  if (!p) return FP8W8A8_ERR_HIP;
  p->device = device;
  p->n = n;
  p->k = k;
  p->w = static_cast<const uint8_t*>(w_fp8);
  p->w_scale = w_scale;
  p->bias = static_cast<const uint16_t*>(bias_bf16);
  p->cu_count = cus > 0 ? cus : 256;
  fill_buckets(kW8A8, n, k, p->cu_count, p->max_m, p->config);
  *out = p;
  return FP8W8A8_OK;
}

static int plan_bucket_config(const fp8_linear_plan* p, int64_t m) {
  return bucket_config(kW8A8, p->max_m, p->config, p->n, m);
}

size_t fp8_linear_workspace_bytes(const fp8_linear_plan* plan, int64_t m) {
  if (!plan || m <= 0) return 0;
  return align256((size_t)m * (size_t)plan->k) + align256((size_t)m * sizeof(float));
}

int fp8_linear_run(const fp8_linear_plan* plan, int64_t m, const void* a, int a_kind, const float* a_scale,
                   void* out_bf16, void* workspace, size_t workspace_bytes, void* stream) {
  if (!plan || !a || !out_bf16) return FP8W8A8_ERR_INVALID_ARG;
  if (a_kind != FP8W8A8_A_BF16 && a_kind != FP8W8A8_A_E4M3) return FP8W8A8_ERR_INVALID_ARG;
  if (m < 0 || m >= FP8W8A8_MAX_ROWS) return FP8W8A8_ERR_BAD_SHAPE;
  if (!aligned(a, 16) || !aligned(out_bf16, 16)) return FP8W8A8_ERR_MISALIGNED;
  if (a_kind == FP8W8A8_A_E4M3) {
    if (!a_scale) return FP8W8A8_ERR_INVALID_ARG;
    if (!aligned(a_scale, 4)) return FP8W8A8_ERR_MISALIGNED;
  } else {
    if (!workspace) return FP8W8A8_ERR_INVALID_ARG;
    if (!aligned(workspace, 256)) return FP8W8A8_ERR_MISALIGNED;
    if (workspace_bytes < fp8_linear_workspace_bytes(plan, m)) return FP8W8A8_ERR_WORKSPACE_TOO_SMALL;
  }
  if (m == 0) return FP8W8A8_OK;
  int st = plan_device_current(plan->device);
  if (st != FP8W8A8_OK) return st;
  const int config = plan_bucket_config(plan, m);
  if (!grid_fits(config, m, plan->n)) return FP8W8A8_ERR_BAD_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t* qa = static_cast<const uint8_t*>(a);
  const float* sa = a_scale;
  if (a_kind == FP8W8A8_A_BF16) {
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    float* ws_scale = reinterpret_cast<float*>(ws + align256((size_t)m * (size_t)plan->k));
    hipError_t e = launch_quant_rows(static_cast<const uint16_t*>(a), m, plan->k, ws, ws_scale, s);
    if (e != hipSuccess) return FP8W8A8_ERR_HIP;
    qa = ws;
    sa = ws_scale;
  }
  hipError_t e = launch_gemm(config, m, plan->n, plan->k, qa, sa, plan->w, plan->w_scale, plan->bias,
                             static_cast<uint16_t*>(out_bf16), plan->cu_count, s);
  return e == hipSuccess ? FP8W8A8_OK : FP8W8A8_ERR_HIP;
}

// The configuration of the single GEMM launch that fp8_linear_run_group makes for these
// plans at m (config[i]: plan i's own choice at m), or -1 when each plan runs its own GEMM.
static int group_launch_form(const fp8_linear_plan* const* plans, int nplans, int64_t m, const int* config) {
  const fp8_linear_plan* p0 = plans[0];
  // One launch for the group: when every plan takes a skinny form (in the wide one, 7, when
  // the problems' 16-channel blocks together outnumber the CUs); or when every plan
  // takes the 256 x 256 tiles (configuration 0, or its persistent form 6, which compute
  // every tile alike) at a k where a single plan may take the persistent form, and one
  // persistent launch needs fewer rounds of tiles over the CUs than the separate launches,
  // or as many, all of them full. (Q, K and V at 8192 tokens: 256 tiles each, one round
  // apiece, 768 together, three full rounds: 92.7 -> 84.9 us. At 6144 tokens, 192 tiles
  // each: three rounds either way, the joint third a quarter full: 75.8 -> 79.5 us.)
  int group_form = -1;  // the configuration of the one launch
  if (nplans > 1) {
    bool skinny = true, big_tiles = p0->k >= 2048 && p0->k <= 4096;
    for (int i = 0; i < nplans; ++i) {
      skinny = skinny && (config[i] == kW8A8Skinny || config[i] == kW8A8SkinnyWide);
      big_tiles = big_tiles && (config[i] == 0 || config[i] == kW8A8Persistent);
    }
    if (skinny) {
      // the joint grid takes the wide form when the 16-channel blocks of all the
      // problems together exceed the CU count (the rule of a single plan, above)
      int64_t blocks = 0;
      for (int i = 0; i < nplans; ++i) blocks += gemm_workgroups(kW8A8Skinny, m, plans[i]->n);
      group_form = blocks > p0->cu_count ? kW8A8SkinnyWide : kW8A8Skinny;
      // and the joint grid must fit as each plan's does
      int64_t wgs = 0;
      for (int i = 0; i < nplans; ++i) wgs += gemm_workgroups(group_form, m, plans[i]->n);
      if (wgs * gemm_threads(group_form) >= kMaxGridThreads) group_form = -1;
    } else if (big_tiles) {
      const int64_t c = std::max(8, p0->cu_count / 8 * 8);  // the persistent grid
      int64_t tiles = 0, rounds_apart = 0;
      for (int i = 0; i < nplans; ++i) {
        const int64_t t = gemm_workgroups(0, m, plans[i]->n);
        tiles += t;
        rounds_apart += (t + c - 1) / c;
      }
      const int64_t rounds_joint = (tiles + c - 1) / c;
      if (rounds_joint < rounds_apart || (rounds_joint == rounds_apart && tiles % c == 0))
        group_form = kW8A8Persistent;
    }
  }
  return group_form;
}

int fp8_linear_run_group(const fp8_linear_plan* const* plans, int nplans, int64_t m, const void* a, int a_kind,
                         const float* a_scale, void* const* outs_bf16, void* workspace, size_t workspace_bytes,
                         void* stream) {
  if (!plans || !outs_bf16 || !a) return FP8W8A8_ERR_INVALID_ARG;
  if (nplans < 1 || nplans > FP8W8A8_MAX_GROUP) return FP8W8A8_ERR_INVALID_ARG;
  for (int i = 0; i < nplans; ++i)
    if (!plans[i] || !outs_bf16[i]) return FP8W8A8_ERR_INVALID_ARG;
  const fp8_linear_plan* p0 = plans[0];
  for (int i = 1; i < nplans; ++i) {
    if (plans[i]->k != p0->k) return FP8W8A8_ERR_BAD_SHAPE;
    if (plans[i]->device != p0->device) return FP8W8A8_ERR_BAD_DEVICE;
  }
  if (a_kind != FP8W8A8_A_BF16 && a_kind != FP8W8A8_A_E4M3) return FP8W8A8_ERR_INVALID_ARG;
  if (m < 0 || m >= FP8W8A8_MAX_ROWS) return FP8W8A8_ERR_BAD_SHAPE;
  if (!aligned(a, 16)) return FP8W8A8_ERR_MISALIGNED;
  for (int i = 0; i < nplans; ++i)
    if (!aligned(outs_bf16[i], 16)) return FP8W8A8_ERR_MISALIGNED;
  if (a_kind == FP8W8A8_A_E4M3) {
    if (!a_scale) return FP8W8A8_ERR_INVALID_ARG;
    if (!aligned(a_scale, 4)) return FP8W8A8_ERR_MISALIGNED;
  } else {
    if (!workspace) return FP8W8A8_ERR_INVALID_ARG;
    if (!aligned(workspace, 256)) return FP8W8A8_ERR_MISALIGNED;
    if (workspace_bytes < fp8_linear_workspace_bytes(p0, m)) return FP8W8A8_ERR_WORKSPACE_TOO_SMALL;
  }
  if (m == 0) return FP8W8A8_OK;
  int st = plan_device_current(p0->device);
  if (st != FP8W8A8_OK) return st;
  // every plan's choice at this m; one launch when all of them take the persistent form,
  // or all the skinny one
  int config[FP8W8A8_MAX_GROUP];
  for (int i = 0; i < nplans; ++i) {
    config[i] = plan_bucket_config(plans[i], m);
    if (!grid_fits(config[i], m, plans[i]->n)) return FP8W8A8_ERR_BAD_SHAPE;
  }
  const int group_form = group_launch_form(plans, nplans, m, config);
  const bool grouped = group_form >= 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t* qa = static_cast<const uint8_t*>(a);
  const float* sa = a_scale;
  if (a_kind == FP8W8A8_A_BF16) {
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    float* ws_scale = reinterpret_cast<float*>(ws + align256((size_t)m * (size_t)p0->k));
    if (launch_quant_rows(static_cast<const uint16_t*>(a), m, p0->k, ws, ws_scale, s) != hipSuccess)
      return FP8W8A8_ERR_HIP;
    qa = ws;
    sa = ws_scale;
  }
  if (grouped) {
    GroupProblem probs[FP8W8A8_MAX_GROUP];
    for (int i = 0; i < nplans; ++i)
      probs[i] = GroupProblem{plans[i]->w, plans[i]->w_scale, plans[i]->bias, static_cast<uint16_t*>(outs_bf16[i]),
                              plans[i]->n};
    return launch_gemm_group(group_form, m, p0->k, qa, sa, nplans, probs, p0->cu_count, s) == hipSuccess
               ? FP8W8A8_OK
               : FP8W8A8_ERR_HIP;
  }
  for (int i = 0; i < nplans; ++i) {
    const fp8_linear_plan* p = plans[i];
    if (launch_gemm(config[i], m, p->n, p->k, qa, sa, p->w, p->w_scale, p->bias, static_cast<uint16_t*>(outs_bf16[i]),
                    p->cu_count, s) != hipSuccess)
      return FP8W8A8_ERR_HIP;
  }
  return FP8W8A8_OK;
}

int fp8_linear_group_config(const fp8_linear_plan* const* plans, int nplans, int64_t m, int* config_id) {
  if (!plans || !config_id) return FP8W8A8_ERR_INVALID_ARG;
  if (nplans < 1 || nplans > FP8W8A8_MAX_GROUP) return FP8W8A8_ERR_INVALID_ARG;
  for (int i = 0; i < nplans; ++i)
    if (!plans[i]) return FP8W8A8_ERR_INVALID_ARG;
  for (int i = 1; i < nplans; ++i) {
    if (plans[i]->k != plans[0]->k) return FP8W8A8_ERR_BAD_SHAPE;
    if (plans[i]->device != plans[0]->device) return FP8W8A8_ERR_BAD_DEVICE;
  }
  if (m < 0 || m >= FP8W8A8_MAX_ROWS) return FP8W8A8_ERR_BAD_SHAPE;
  int config[FP8W8A8_MAX_GROUP];
  for (int i = 0; i < nplans; ++i) config[i] = plan_bucket_config(plans[i], m);
  *config_id = m == 0 ? -1 : group_launch_form(plans, nplans, m, config);
  return FP8W8A8_OK;
}

int fp8_linear_run_noalloc(const fp8_linear_plan* plan, int64_t m, const void* a, int a_kind, const float* a_scale,
                           void* out_bf16, void* stream) {
  if (!plan || !a || !out_bf16) return FP8W8A8_ERR_INVALID_ARG;
  if (a_kind != FP8W8A8_A_BF16 && a_kind != FP8W8A8_A_E4M3) return FP8W8A8_ERR_INVALID_ARG;
  if (m < 0 || m >= FP8W8A8_MAX_ROWS) return FP8W8A8_ERR_BAD_SHAPE;
  if (a_kind == FP8W8A8_A_E4M3)  // no scratch involved: exactly fp8_linear_run
    return fp8_linear_run(plan, m, a, a_kind, a_scale, out_bf16, nullptr, 0, stream);
  const size_t need = fp8_linear_workspace_bytes(plan, m);
  if (need > FP8W8A8_NOALLOC_SCRATCH_BYTES) return FP8W8A8_ERR_TOO_LARGE;
  if (m == 0) return FP8W8A8_OK;
  int st = plan_device_current(plan->device);
  if (st != FP8W8A8_OK) return st;
  uint8_t* ws = scratch_on(plan->device);
  if (!ws) return FP8W8A8_ERR_HIP;
  return fp8_linear_run(plan, m, a, a_kind, a_scale, out_bf16, ws, need, stream);
}

void fp8_linear_destroy(fp8_linear_plan* plan) { free(plan); }

int fp8_linear(const void* a, int a_kind, const float* a_scale, int64_t m, int64_t n, int64_t k,
               const void* w_fp8, const float* w_scale, const void* bias_bf16, void* out_bf16,
               void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_weight_args(n, k, w_fp8, w_scale, bias_bf16);
  if (st != FP8W8A8_OK) return st;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FP8W8A8_ERR_HIP;
  fp8_linear_plan* p = nullptr;
  st = fp8_linear_create(dev, n, k, w_fp8, w_scale, bias_bf16, &p);
  if (st != FP8W8A8_OK) return st;
  st = fp8_linear_run(p, m, a, a_kind, a_scale, out_bf16, workspace, workspace_bytes, stream);
  fp8_linear_destroy(p);
  return st;
}

int fp8_linear_plan_config(const fp8_linear_plan* plan, int64_t m, int* config_id, int* tile_m, int* tile_n,
                           int64_t* workgroups) {
  if (!plan || !config_id || !tile_m || !tile_n || !workgroups) return FP8W8A8_ERR_INVALID_ARG;
  if (m < 0 || m >= FP8W8A8_MAX_ROWS) return FP8W8A8_ERR_BAD_SHAPE;
  const int c = plan_bucket_config(plan, m > 0 ? m : 1);
  const GemmConfig* g = gemm_config(c);
  *config_id = c;
  *tile_m = g->tile_m;
  *tile_n = g->tile_n;
  *workgroups = m > 0 ? gemm_workgroups(c, m, plan->n) : 0;
  return FP8W8A8_OK;
}

int fp8_gemm_config_count(void) { return gemm_config_count(); }

int fp8_gemm_run_config(int config_id, int64_t m, int64_t n, int64_t k, const void* qa, const float* a_scale,
                        const void* w_fp8, const float* w_scale, const void* bias_bf16, void* out_bf16,
                        void* stream) {
  if (config_id < 0 || config_id >= gemm_config_count()) return FP8W8A8_ERR_INVALID_ARG;
  if (!qa || !a_scale || !out_bf16) return FP8W8A8_ERR_INVALID_ARG;
  int st = check_weight_args(n, k, w_fp8, w_scale, bias_bf16);
  if (st != FP8W8A8_OK) return st;
  if (m < 0 || m >= FP8W8A8_MAX_ROWS) return FP8W8A8_ERR_BAD_SHAPE;
  if (!aligned(qa, 16) || !aligned(out_bf16, 16) || !aligned(a_scale, 4)) return FP8W8A8_ERR_MISALIGNED;
  if (m == 0) return FP8W8A8_OK;
  if (!grid_fits(config_id, m, n)) return FP8W8A8_ERR_BAD_SHAPE;
  int cus = 0;
  st = current_device_ok(&cus);
  if (st != FP8W8A8_OK) return st;
  hipError_t e = launch_gemm(config_id, m, n, k, static_cast<const uint8_t*>(qa), a_scale,
                             static_cast<const uint8_t*>(w_fp8), w_scale, static_cast<const uint16_t*>(bias_bf16),
                             static_cast<uint16_t*>(out_bf16), cus > 0 ? cus : 256,
                             static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8W8A8_OK : FP8W8A8_ERR_HIP;
}

size_t fp8_quant_gemm_workspace_bytes(int64_t m, int64_t k) {
  if (m <= 0 || k <= 0) return 0;
  return align256((size_t)m * (size_t)k) + align256((size_t)m * sizeof(float)) +
         (size_t)kQuantGemmMaxWorkgroups * sizeof(unsigned long long);
}

int fp8_quant_gemm(int64_t m, int64_t n, int64_t k, const void* a_bf16, const void* w_fp8, const float* w_scale,
                   const void* bias_bf16, void* out_bf16, void* workspace, size_t workspace_bytes, void* stream) {
  if (!a_bf16 || !out_bf16 || !workspace) return FP8W8A8_ERR_INVALID_ARG;
  int st = check_weight_args(n, k, w_fp8, w_scale, bias_bf16);
  if (st != FP8W8A8_OK) return st;
  if (m < 0 || m >= FP8W8A8_MAX_ROWS) return FP8W8A8_ERR_BAD_SHAPE;
  if (!aligned(a_bf16, 16) || !aligned(out_bf16, 16) || !aligned(workspace, 256)) return FP8W8A8_ERR_MISALIGNED;
  if (workspace_bytes < fp8_quant_gemm_workspace_bytes(m, k)) return FP8W8A8_ERR_WORKSPACE_TOO_SMALL;
  if (m == 0) return FP8W8A8_OK;
  int cus = 0;
  st = current_device_ok(&cus);
  if (st != FP8W8A8_OK) return st;
  // The launch's generation number is a kernel argument chosen here: a captured graph
  // would replay it, and its flags from the previous replay would already match.
  hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(static_cast<hipStream_t>(stream), &capture) != hipSuccess) return FP8W8A8_ERR_HIP;
  if (capture != hipStreamCaptureStatusNone) return FP8W8A8_ERR_CAPTURE;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* ws_scale = reinterpret_cast<float*>(ws + align256((size_t)m * (size_t)k));
  auto* flags = reinterpret_cast<unsigned long long*>(reinterpret_cast<uint8_t*>(ws_scale) +
                                                      align256((size_t)m * sizeof(float)));
  hipError_t e = launch_quant_gemm(m, n, k, static_cast<const uint16_t*>(a_bf16), ws, ws_scale, flags, next_epoch(),
                                   static_cast<const uint8_t*>(w_fp8), w_scale, static_cast<const uint16_t*>(bias_bf16),
                                   static_cast<uint16_t*>(out_bf16), cus, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8W8A8_OK : FP8W8A8_ERR_HIP;
}

int fp8_w8a16_create(int device, int64_t n, int64_t k, int w_format, const void* w_fp8, const float* w_scale,
                     const void* bias_bf16, fp8_w8a16_plan** out) {
  if (!out) return FP8W8A8_ERR_INVALID_ARG;
  if (w_format != FP8W8A8_FMT_E4M3FN && w_format != FP8W8A8_FMT_E5M2) return FP8W8A8_ERR_INVALID_ARG;
  int st = check_weight_args(n, k, w_fp8, w_scale, bias_bf16);
  if (st != FP8W8A8_OK) return st;
  int cus = 0;
  st = query_device(device, &cus);
  if (st != FP8W8A8_OK) return st;
  fp8_w8a16_plan* p = static_cast<fp8_w8a16_plan*>(calloc(1, sizeof(fp8_w8a16_plan)));
  if (!p) return FP8W8A8_ERR_HIP;
  p->device = device;
  p->w_format = w_format;
  p->n = n;
  p->k = k;
  p->w = static_cast<const uint8_t*>(w_fp8);
  p->w_scale = w_scale;
  p->bias = static_cast<const uint16_t*>(bias_bf16);
  p->cu_count = cus > 0 ? cus : 256;
  fill_buckets(kW8A16, n, k, p->cu_count, p->max_m, p->config);
  *out = p;
  return FP8W8A8_OK;
}

int fp8_w8a16_run(const fp8_w8a16_plan* plan, int64_t m, const void* a_bf16, void* out_bf16, void* stream) {
  if (!plan || !a_bf16 || !out_bf16) return FP8W8A8_ERR_INVALID_ARG;
  if (m < 0 || m >= FP8W8A8_MAX_ROWS) return FP8W8A8_ERR_BAD_SHAPE;
  if (!aligned(a_bf16, 16) || !aligned(out_bf16, 16)) return FP8W8A8_ERR_MISALIGNED;
  if (m == 0) return FP8W8A8_OK;
  int st = plan_device_current(plan->device);
  if (st != FP8W8A8_OK) return st;
  const int c = bucket_config(kW8A16, plan->max_m, plan->config, plan->n, m);
  if (!grid_fits(kW8A16, c, m, plan->n)) return FP8W8A8_ERR_BAD_SHAPE;
  hipError_t e = launch_w8a16(c, plan->w_format, m, plan->n, plan->k, static_cast<const uint16_t*>(a_bf16), plan->w,
                              plan->w_scale,
                              plan->bias, static_cast<uint16_t*>(out_bf16), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8W8A8_OK : FP8W8A8_ERR_HIP;
}

void fp8_w8a16_destroy(fp8_w8a16_plan* plan) { free(plan); }

int fp8_w8a16_plan_config(const fp8_w8a16_plan* plan, int64_t m, int* config_id, int* tile_m, int* tile_n,
                          int64_t* workgroups) {
  if (!plan || !config_id || !tile_m || !tile_n || !workgroups) return FP8W8A8_ERR_INVALID_ARG;
  if (m < 0 || m >= FP8W8A8_MAX_ROWS) return FP8W8A8_ERR_BAD_SHAPE;
  const int c = bucket_config(kW8A16, plan->max_m, plan->config, plan->n, m > 0 ? m : 1);
  const GemmConfig* g = w8a16_config(c);
  *config_id = c;
  *tile_m = g->tile_m;
  *tile_n = g->tile_n;
  *workgroups = m > 0 ? w8a16_workgroups(c, m, plan->n) : 0;
  return FP8W8A8_OK;
}

int fp8_w8a16_config_count(void) { return w8a16_config_count(); }

int fp8_w8a16_run_config(int config_id, int w_format, int64_t m, int64_t n, int64_t k, const void* a_bf16,
                         const void* w_fp8, const float* w_scale, const void* bias_bf16, void* out_bf16, void* stream) {
  if (config_id < 0 || config_id >= w8a16_config_count()) return FP8W8A8_ERR_INVALID_ARG;
  if (w_format != FP8W8A8_FMT_E4M3FN && w_format != FP8W8A8_FMT_E5M2) return FP8W8A8_ERR_INVALID_ARG;
  if (!a_bf16 || !out_bf16) return FP8W8A8_ERR_INVALID_ARG;
  int st = check_weight_args(n, k, w_fp8, w_scale, bias_bf16);
  if (st != FP8W8A8_OK) return st;
  if (m < 0 || m >= FP8W8A8_MAX_ROWS) return FP8W8A8_ERR_BAD_SHAPE;
  if (!aligned(a_bf16, 16) || !aligned(out_bf16, 16)) return FP8W8A8_ERR_MISALIGNED;
  if (m == 0) return FP8W8A8_OK;
  if (!grid_fits(kW8A16, config_id, m, n)) return FP8W8A8_ERR_BAD_SHAPE;
  st = current_device_ok();
  if (st != FP8W8A8_OK) return st;
  hipError_t e = launch_w8a16(config_id, w_format, m, n, k, static_cast<const uint16_t*>(a_bf16),
                              static_cast<const uint8_t*>(w_fp8), w_scale, static_cast<const uint16_t*>(bias_bf16),
                              static_cast<uint16_t*>(out_bf16), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8W8A8_OK : FP8W8A8_ERR_HIP;
}

}  // extern "C"
