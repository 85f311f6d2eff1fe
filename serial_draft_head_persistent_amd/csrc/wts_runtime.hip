// Host runtime of the walk-resident serial draft head: argument checks,
// residency planning, create-time repacking, walk launches, error latch.
//
// "Weights That Stay" (arXiv 2611.00506) keeps each compute unit's shard of
// the vocabulary projection on chip for the whole walk, fully or partially
// (abstract, Fig. 1, Fig. 10, Fig. 14).  Here a 16-row tile is the unit of
// residency: each wave keeps its first tiles in VGPRs, the next in LDS, and
// streams the rest from memory at every step.

#include <algorithm>
#include <mutex>
#include <new>

#include "wts.h"
#include "wts_internal.h"

using namespace wts;

struct wts_ctx {
  int device = 0;
  int V = 0, head = 0, wtype = 0, tiles = 0, grid = 0;
  int max_batch = 0, max_steps = 0;
  int reg_cap = -1, lds_cap = -1;
  bool cooperative = false;
  bool xcd_l1 = false;  // first exchange level inside one XCD's L2
  int4* Wp = nullptr;
  float* sw = nullptr;
  int8_t* Eq = nullptr;
  float* Es = nullptr;
  uint16_t* Eb = nullptr;
  const float* E = nullptr;
  const uint16_t* A = nullptr;
  const float* c = nullptr;
  Ctrl* ctrl = nullptr;
  float* lse_part = nullptr;  // (max, sum) pairs of every workgroup, per row and step
  long long timeout_ticks = 0;
};

// Fixed device scratch of wts_walk_noalloc: a control block (exchange lines,
// step-wise slots, error word) and room for the log-normaliser partials.
// One copy per GPU, held until the process ends.  Host code never passes the
// array's name to a kernel (in host code it is a stand-in, not a device
// address); it uses the per-device address from hipGetSymbolAddress.
constexpr size_t kNoAllocCtrlBytes = (sizeof(Ctrl) + 255) / 256 * 256;
constexpr size_t kNoAllocLseBytes = WTS_NOALLOC_LSE_BYTES;
constexpr size_t kNoAllocBytes = kNoAllocCtrlBytes + kNoAllocLseBytes;
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

namespace {

constexpr int kMaxDevices = 64;
struct DevScratch {
  char* ptr = nullptr;            // device address of `scratch` on that GPU
};
DevScratch g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

struct DeviceGuard {
  int prev = -1;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev) (void)hipSetDevice(dev);
  }
  ~DeviceGuard() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};

int batch_bucket(int B) {
  int bb = 1;
  while (bb < B) bb <<= 1;
  return bb;
}

int tile_bytes(int wtype) { return wtype == WTS_W_INT8 ? kTileBytesI8 : kTileBytesBF; }

// Workgroups of one step-wise launch (8 tiles each).
int step_grid(const wts_ctx* ctx) { return std::max(1, (ctx->tiles + 7) / 8); }


// Gumbel noise of a T=1 persistent Markov walk is computed one step ahead
// into LDS (BB rows x the workgroup's vocabulary rows, fp32).
int noise_floats(const wts_ctx* ctx, int BB, int temperature) {
  if (!temperature || ctx->head != WTS_HEAD_MARKOV) return 0;
  const int per_wg = (ctx->tiles + ctx->grid - 1) / ctx->grid;
  return per_wg * kTileRows;
}

// Tiles wave w of a workgroup with cnt tiles owns (every NW-th tile).
int wave_tiles(int cnt, int w, int NW) { return cnt > w ? (cnt - w + NW - 1) / NW : 0; }

// Residency plan for one batch bucket.  *full: the variant with more register
// tiles and LDS tiles allotted per wave, which holds the whole shard on chip,
// chosen when the other cannot hold it or holds fewer tiles in registers.
// Returns false if the kernel's LDS scratch (with the T=1 noise of one step)
// does not fit in LDS.
bool make_plan(const wts_ctx* ctx, int BB, int exec, int temperature, bool lse, wts_plan* p, int* lds_bytes,
               int* noise_off = nullptr, int* noise_stride = nullptr, int* full = nullptr,
               int* lds_extra = nullptr) {
  const int per_wg = (ctx->tiles + ctx->grid - 1) / ctx->grid;
  const int NW = waves_for(ctx->head, ctx->wtype);
  const int per_wave = (per_wg + NW - 1) / NW;
  int reg = std::min(reg_tiles_max(ctx->head, ctx->wtype, BB, temperature, lse), per_wave);
  if (ctx->reg_cap >= 0) reg = std::min(reg, ctx->reg_cap);
  const int tb = tile_bytes(ctx->wtype);
  const int stride = noise_floats(ctx, BB, temperature);
  const int noise_bytes = BB * stride * 4;
  const int scratch = lds_scratch_bytes(ctx->head, ctx->wtype, BB) + noise_bytes;
  if (noise_off) *noise_off = stride ? lds_scratch_bytes(ctx->head, ctx->wtype, BB) : 0;
  if (noise_stride) *noise_stride = stride;
  int lds = std::max(0, (kLdsMax - scratch) / (NW * tb));
  lds = std::min(lds, per_wave - reg);
  if (ctx->lds_cap >= 0) lds = std::min(lds, ctx->lds_cap);
  if (exec != WTS_EXEC_RESIDENT) reg = lds = 0;
  bool whole = false;
  int lds_need = NW * lds;  // LDS tiles of the fullest workgroup
  const int regf = std::min(reg_tiles_full(ctx->head, ctx->wtype, BB), per_wave);
  // the whole-shard variant when the other cannot hold the shard, or when it
  // holds more of it in registers (fewer LDS tiles; measured faster)
  if (regf > 0 && exec == WTS_EXEC_RESIDENT && ctx->reg_cap < 0 && ctx->lds_cap < 0 &&
      (reg + lds < per_wave || regf > reg)) {
    int need = 0, most = 0;
    for (int w = 0; w < NW; ++w) {
      const int rest = wave_tiles(per_wg, w, NW) - std::min(wave_tiles(per_wg, w, NW), regf);
      need += rest;
      most = std::max(most, rest);
    }
    if (need * tb <= kLdsMax - scratch && most <= kFullLdsMax) {
      whole = true;
      reg = regf;
      lds = most;
      lds_need = need;
    }
  }
  // a walk that streams: the whole tiles that still fit in LDS go one each to
  // the first waves (those with the most tiles), so that fewer tiles stream
  int extra = 0;
  if (!whole && exec == WTS_EXEC_RESIDENT && ctx->lds_cap < 0 && reg + lds < per_wave)
    extra = std::max(0, std::min(NW - 1, (kLdsMax - scratch) / tb - NW * lds));
  lds_need += extra;
  if (lds_extra) *lds_extra = extra;
  if (full) *full = whole ? 1 : 0;
  p->grid = ctx->grid;
  p->waves = NW;
  p->tiles = ctx->tiles;
  p->tiles_per_wave = per_wave;
  p->reg_tiles = reg;
  p->lds_tiles = lds;
  p->stream_tiles = whole ? 0 : per_wave - reg - lds - (extra > 0 ? 1 : 0);
  // exact on-chip bytes: count each wave's tiles
  long long res_tiles = 0;
  for (int g = 0; g < ctx->grid; ++g) {
    const int cnt = (int)((long long)(g + 1) * ctx->tiles / ctx->grid) - (int)((long long)g * ctx->tiles / ctx->grid);
    for (int w = 0; w < NW; ++w)
      res_tiles += whole ? wave_tiles(cnt, w, NW) : std::min(wave_tiles(cnt, w, NW), reg + lds + (w < extra ? 1 : 0));
  }
  const long long esz = ctx->wtype == WTS_W_INT8 ? 1 : 2;
  p->w_bytes = (long long)ctx->V * kR * esz;
  p->resident_bytes = res_tiles * tb;
  p->streamed_bytes = (long long)ctx->tiles * tb - p->resident_bytes;
  p->exchange = ctx->xcd_l1 ? 0 : 1;
  *lds_bytes = std::min(kLdsMax, std::max(scratch + lds_need * tb, 96 * 1024));
  return scratch <= kLdsMax;
}

// Whether workgroup g of a grid of `grid` runs on the same XCD as workgroup
// g % kGroups (the first level of the exchange keeps each group inside one
// XCD's L2).  Reads every workgroup's XCC_ID once.
wts_status check_xcd_groups(int grid, bool* same) {
  *same = false;
  unsigned* d = nullptr;
  if (hipMalloc((void**)&d, kMaxGrid * sizeof(unsigned)) != hipSuccess) return WTS_ERR_NO_MEMORY;
  unsigned h[kMaxGrid];
  wts_status st = WTS_OK;
  if (launch_xcc_ids(d, grid, 0) != hipSuccess ||
      hipMemcpy(h, d, grid * sizeof(unsigned), hipMemcpyDeviceToHost) != hipSuccess)
    st = WTS_ERR_DEVICE;
  (void)hipFree(d);
  if (st != WTS_OK) return st;
  bool ok = true;
  for (int g = 0; g < grid; ++g) ok = ok && h[g] == h[g % kGroups];
  *same = ok;
  return WTS_OK;
}

template <class T>
wts_status dmalloc(T** p, size_t bytes) {
  *p = nullptr;
  if (hipMalloc((void**)p, bytes) != hipSuccess) {
    *p = nullptr;
    return WTS_ERR_NO_MEMORY;
  }
  return WTS_OK;
}

void free_ctx(wts_ctx* ctx) {
  (void)hipFree(ctx->Wp);
  (void)hipFree(ctx->sw);
  (void)hipFree(ctx->Eq);
  (void)hipFree(ctx->Es);
  (void)hipFree(ctx->Eb);
  (void)hipFree(ctx->ctrl);
  (void)hipFree(ctx->lse_part);
  delete ctx;
}

// Once per device, with that device current: the address of its copy of
// `scratch`, cleared with a fill kernel (a walk needs its control block at
// zero before the first call).
wts_status scratch_init(int device) {
  if (device >= kMaxDevices) return WTS_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch[device].ptr) return WTS_OK;
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return WTS_ERR_DEVICE;
  if (launch_fill_zero(ptr, kNoAllocBytes, 0) != hipSuccess || hipDeviceSynchronize() != hipSuccess)
    return WTS_ERR_DEVICE;
  g_scratch[device].ptr = (char*)ptr;
  return WTS_OK;
}

// Reads (and with clear resets) the error word of one control block.
wts_status read_ctrl_error(Ctrl* ctrl, bool clear) {
  unsigned err = 0;
  if (hipMemcpy(&err, &ctrl->err, sizeof(err), hipMemcpyDeviceToHost) != hipSuccess) return WTS_ERR_DEVICE;
  if (clear && err) {
    // A failed walk can leave its slots and counters in any state: start over.
    if (hipMemset(ctrl, 0, sizeof(Ctrl)) != hipSuccess || hipDeviceSynchronize() != hipSuccess)
      return WTS_ERR_DEVICE;
  }
  return (wts_status)err;
}

// One walk with the given control block and log-normaliser partials
// (lse_cap bytes of room; the context's own, or the device scratch).
wts_status walk_impl(wts_ctx* ctx, const wts_walk_params* p, Ctrl* ctrl, float* lse_part, size_t lse_cap);

}  // namespace

extern "C" {

const char* wts_status_string(wts_status s) {
  switch (s) {
    case WTS_OK: return "ok";
    case WTS_ERR_INVALID_ARG: return "invalid argument";
    case WTS_ERR_UNSUPPORTED: return "unsupported configuration";
    case WTS_ERR_NO_MEMORY: return "device allocation failed";
    case WTS_ERR_DEVICE: return "HIP runtime or launch error";
    case WTS_ERR_TIMEOUT: return "grid barrier watchdog expired";
    case WTS_ERR_TOKEN_RANGE: return "initial token outside [0, V)";
  }
  return "unknown status";
}

// The kernels address the base logits (2 B gamma V bytes) with 32-bit byte
// offsets; the limits on V (18-bit token field of the selection key), B and
// gamma keep them far below 2^32.
static_assert(2ull * kMaxB * kMaxSteps * 262143ull < (1ull << 32), "base logits within 32-bit offsets");

wts_status wts_create(const wts_create_params* p, wts_ctx** out) {
  if (!p || !out) return WTS_ERR_INVALID_ARG;
  *out = nullptr;
  if (p->V < 1 || p->V > 262143 || p->r < 1) return WTS_ERR_INVALID_ARG;
  if (p->r != kR) return WTS_ERR_UNSUPPORTED;
  if (p->head != WTS_HEAD_MARKOV && p->head != WTS_HEAD_RECURRENT) return WTS_ERR_INVALID_ARG;
  if (p->wtype != WTS_W_INT8 && p->wtype != WTS_W_BF16) return WTS_ERR_INVALID_ARG;
  if (!p->W || !p->E) return WTS_ERR_INVALID_ARG;
  if (p->wtype == WTS_W_INT8 && !p->w_scale) return WTS_ERR_INVALID_ARG;
  if (p->head == WTS_HEAD_RECURRENT && (!p->A || !p->c)) return WTS_ERR_INVALID_ARG;
  if (p->max_batch < 1 || p->max_batch > kMaxB) return WTS_ERR_INVALID_ARG;
  if (p->max_steps < 1 || p->max_steps > kMaxSteps) return WTS_ERR_INVALID_ARG;
  if (p->resident_tiles < -1 || p->lds_tiles < -1) return WTS_ERR_INVALID_ARG;
  if (((uintptr_t)p->W & 15) || ((uintptr_t)p->E & 15) || ((uintptr_t)p->A & 15) || ((uintptr_t)p->c & 3))
    return WTS_ERR_INVALID_ARG;
  if (p->grid < 0 || p->grid > kMaxGrid || (p->exchange != 0 && p->exchange != 1)) return WTS_ERR_INVALID_ARG;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || p->device < 0 || p->device >= ndev) return WTS_ERR_INVALID_ARG;
  DeviceGuard guard(p->device);

  int cus = 0, coop = 0, clock_khz = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, p->device) != hipSuccess ||
      hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, p->device) != hipSuccess ||
      hipDeviceGetAttribute(&clock_khz, hipDeviceAttributeWallClockRate, p->device) != hipSuccess)
    return WTS_ERR_DEVICE;
  if (cus < 1 || (p->cooperative && !coop)) return WTS_ERR_UNSUPPORTED;
  if (p->cooperative != 0 && p->cooperative != 1) return WTS_ERR_INVALID_ARG;
  if (p->watchdog_us < 0) return WTS_ERR_INVALID_ARG;
  if (p->grid > cus) return WTS_ERR_INVALID_ARG;
  {
    // the workgroup-local selection key holds a 16-bit row (V / grid rows at most)
    const int g = p->grid ? p->grid : std::min(cus, kMaxGrid);
    const long long tiles = (p->V + kTileRows - 1) / kTileRows;
    if ((tiles + g - 1) / g * kTileRows > 65535) return WTS_ERR_UNSUPPORTED;
  }
  const wts_status sst = scratch_init(p->device);
  if (sst != WTS_OK) return sst;

  wts_ctx* ctx = new (std::nothrow) wts_ctx();
  if (!ctx) return WTS_ERR_NO_MEMORY;
  ctx->device = p->device;
  ctx->V = p->V;
  ctx->head = p->head;
  ctx->wtype = p->wtype;
  ctx->tiles = (p->V + kTileRows - 1) / kTileRows;
  ctx->grid = p->grid ? p->grid : std::min(cus, kMaxGrid);
  ctx->cooperative = p->cooperative != 0;
  ctx->max_batch = p->max_batch;
  ctx->max_steps = p->max_steps;
  ctx->reg_cap = p->resident_tiles;
  ctx->lds_cap = p->lds_tiles;
  ctx->E = p->E;
  ctx->A = p->A;
  ctx->c = p->c;
  // per wait: 2 s, or the caller's limit (the wall clock runs at clock_khz kHz)
  ctx->timeout_ticks = p->watchdog_us ? std::max(1LL, (long long)clock_khz * p->watchdog_us / 1000LL)
                                      : (long long)clock_khz * 1000LL * 2;

  const size_t tb = tile_bytes(p->wtype);
  wts_status st = dmalloc(&ctx->Wp, (size_t)ctx->tiles * tb);
  if (st == WTS_OK) st = dmalloc(&ctx->ctrl, sizeof(Ctrl));
  if (st == WTS_OK && p->wtype == WTS_W_INT8) st = dmalloc(&ctx->sw, (size_t)ctx->tiles * kTileRows * 4);
  if (st == WTS_OK && p->head == WTS_HEAD_MARKOV && p->wtype == WTS_W_INT8) {
    st = dmalloc(&ctx->Eq, (size_t)p->V * 512);
    if (st == WTS_OK) st = dmalloc(&ctx->Es, (size_t)p->V * 4);
  }
  if (st == WTS_OK && p->head == WTS_HEAD_MARKOV && p->wtype == WTS_W_BF16)
    st = dmalloc(&ctx->Eb, (size_t)p->V * kR * 2);
  if (st == WTS_OK) {
    const size_t groups = (size_t)std::max(ctx->grid, step_grid(ctx));
    st = dmalloc(&ctx->lse_part, (size_t)p->max_batch * p->max_steps * groups * 2 * sizeof(float));
  }
  if (st != WTS_OK) {
    free_ctx(ctx);
    return st;
  }
  hipError_t e = hipMemset(ctx->ctrl, 0, sizeof(Ctrl));
  if (e == hipSuccess) e = prepare_kernels(kLdsMax);
  if (e == hipSuccess) {
    if (p->wtype == WTS_W_INT8)
      e = launch_repack_i8((const int8_t*)p->W, p->w_scale, p->V, ctx->tiles, ctx->Wp, ctx->sw, 0);
    else
      e = launch_repack_bf16((const uint16_t*)p->W, p->V, ctx->tiles, ctx->Wp, 0);
  }
  if (e == hipSuccess && ctx->Eq) e = launch_quant_rows(p->E, p->V, ctx->Eq, ctx->Es, 0);
  if (e == hipSuccess && ctx->Eb) e = launch_bf16_rows(p->E, p->V, ctx->Eb, 0);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    free_ctx(ctx);
    return WTS_ERR_DEVICE;
  }
  if (p->exchange == 0) {
    bool same = false;
    const wts_status xs = check_xcd_groups(ctx->grid, &same);
    if (xs != WTS_OK) {
      free_ctx(ctx);
      return xs;
    }
    ctx->xcd_l1 = same;
  }
  *out = ctx;
  return WTS_OK;
}

wts_status wts_get_plan(const wts_ctx* ctx, int32_t B, int32_t exec, int32_t temperature, wts_plan* out) {
  if (!ctx || !out || B < 1 || B > ctx->max_batch) return WTS_ERR_INVALID_ARG;
  if (exec < WTS_EXEC_RESIDENT || exec > WTS_EXEC_STEPWISE) return WTS_ERR_INVALID_ARG;
  if (temperature != 0 && temperature != 1) return WTS_ERR_INVALID_ARG;
  int lds_bytes = 0;
  return make_plan(ctx, batch_bucket(B), exec, temperature, false, out, &lds_bytes) ? WTS_OK
                                                                                     : WTS_ERR_UNSUPPORTED;
}

wts_status wts_walk(wts_ctx* ctx, const wts_walk_params* p) {
  if (!ctx || !p) return WTS_ERR_INVALID_ARG;
  const size_t groups = (size_t)std::max(ctx->grid, step_grid(ctx));
  return walk_impl(ctx, p, ctx->ctrl, ctx->lse_part, (size_t)ctx->max_batch * ctx->max_steps * groups * 8);
}

wts_status wts_walk_noalloc(wts_ctx* ctx, const wts_walk_params* p) {
  if (!ctx || !p) return WTS_ERR_INVALID_ARG;
  DevScratch& ds = g_scratch[ctx->device];   // set up by wts_create on this device
  if (!ds.ptr) return WTS_ERR_DEVICE;
  return walk_impl(ctx, p, (Ctrl*)ds.ptr, (float*)(ds.ptr + kNoAllocCtrlBytes), kNoAllocLseBytes);
}

}  // extern "C"

namespace {

wts_status walk_impl(wts_ctx* ctx, const wts_walk_params* p, Ctrl* ctrl, float* lse_part, size_t lse_cap) {
  if (p->B < 1 || p->B > ctx->max_batch || p->gamma < 1 || p->gamma > ctx->max_steps) return WTS_ERR_INVALID_ARG;
  if (p->temperature != 0 && p->temperature != 1) return WTS_ERR_INVALID_ARG;
  if (p->step_offset < 0 || (p->flags & ~(WTS_WALK_FIXED_LATENT | WTS_WALK_STRESS)) != 0) return WTS_ERR_INVALID_ARG;
  if (p->exec < WTS_EXEC_RESIDENT || p->exec > WTS_EXEC_STEPWISE) return WTS_ERR_INVALID_ARG;
  if (!p->base || !p->x0 || !p->tokens_out) return WTS_ERR_INVALID_ARG;
  if (ctx->head == WTS_HEAD_RECURRENT && !p->h0) return WTS_ERR_INVALID_ARG;
  if (((uintptr_t)p->base & 1) || ((uintptr_t)p->x0 & 3) || ((uintptr_t)p->tokens_out & 3) ||
      ((uintptr_t)p->logits_out & 1) || ((uintptr_t)p->h0 & 3) || ((uintptr_t)p->state_out & 3) ||
      ((uintptr_t)p->trace_out & 7) || ((uintptr_t)p->lse_out & 3) || ((uintptr_t)p->winners_out & 7))
    return WTS_ERR_INVALID_ARG;
  if (p->exec == WTS_EXEC_STEPWISE && ctx->head != WTS_HEAD_MARKOV) return WTS_ERR_UNSUPPORTED;
  // the forced delays and the winner record belong to the persistent kernel's exchange
  if (p->exec == WTS_EXEC_STEPWISE && ((p->flags & WTS_WALK_STRESS) || p->winners_out)) return WTS_ERR_UNSUPPORTED;
  {
    // room for the (max, sum) pair of every workgroup, row and step
    const size_t groups = (size_t)(p->exec == WTS_EXEC_STEPWISE ? step_grid(ctx) : ctx->grid);
    if (p->lse_out && (size_t)p->B * p->gamma * groups * 8 > lse_cap) return WTS_ERR_UNSUPPORTED;
  }
  DeviceGuard guard(ctx->device);
  const int BB = batch_bucket(p->B);
  wts_plan plan;
  int lds_bytes = 0;
  int noise_off = 0, noise_stride = 0, full = 0, lds_extra = 0;
  if (!make_plan(ctx, BB, p->exec, p->temperature, p->lse_out != nullptr, &plan, &lds_bytes, &noise_off,
                 &noise_stride, &full, &lds_extra))
    return WTS_ERR_UNSUPPORTED;

  WalkArgs a{};
  a.Wp = ctx->Wp;
  a.sw = ctx->sw;
  a.Eq = ctx->Eq;
  a.Es = ctx->Es;
  a.Eb = ctx->Eb;
  a.E = ctx->E;
  a.A = ctx->A;
  a.c = ctx->c;
  a.ctrl = ctrl;
  a.V = ctx->V;
  a.tiles = ctx->tiles;
  a.head = ctx->head;
  a.reg_tiles = plan.reg_tiles;
  a.lds_tiles = plan.lds_tiles;
  a.lds_extra = lds_extra;
  a.noise_off = noise_off;
  a.noise_stride = noise_stride;
  a.B = p->B;
  a.gamma = p->gamma;
  a.step_offset = p->step_offset;
  a.temperature = p->temperature;
  a.seed_lo = (unsigned)(p->seed & 0xFFFFFFFFull);
  a.seed_hi = (unsigned)(p->seed >> 32);
  a.base = p->base;
  a.base_bytes = (unsigned)(2ull * p->B * p->gamma * ctx->V);
  a.x0 = p->x0;
  a.h0 = p->h0;
  a.tokens = p->tokens_out;
  a.logits = p->logits_out;
  a.state = p->state_out;
  a.trace = (long long*)p->trace_out;
  a.timeout_ticks = ctx->timeout_ticks;
  a.fixed_latent = (p->flags & WTS_WALK_FIXED_LATENT) != 0;
  a.full = full;
  a.lse = p->lse_out;
  a.lse_part = lse_part;
  a.xcd_l1 = ctx->xcd_l1 ? 1 : 0;
  a.stress = (p->flags & WTS_WALK_STRESS) != 0;
  a.winners = (unsigned long long*)p->winners_out;
  hipStream_t s = (hipStream_t)p->stream;

  hipError_t e;
  if (p->exec == WTS_EXEC_STEPWISE) {
    const int grid = step_grid(ctx);
    e = hipSuccess;
    for (int t = 0; t < p->gamma && e == hipSuccess; ++t) {
      a.step = t;
      e = launch_step(ctx->wtype, BB, a, grid, s);
    }
    if (e == hipSuccess) e = launch_finish(a, s);
    if (e == hipSuccess && a.lse) e = launch_lse(a, grid, s);
  } else {
    e = launch_walk(ctx->wtype, BB, a, ctx->grid, lds_bytes, ctx->cooperative, s);
    if (e == hipSuccess && a.lse) e = launch_lse(a, ctx->grid, s);
  }
  if (e != hipSuccess) return WTS_ERR_DEVICE;
  return WTS_OK;
}

}  // namespace

extern "C" {

wts_status wts_get_error(wts_ctx* ctx, int clear) {
  if (!ctx) return WTS_ERR_INVALID_ARG;
  DeviceGuard guard(ctx->device);
  if (hipDeviceSynchronize() != hipSuccess) return WTS_ERR_DEVICE;
  wts_status st = read_ctrl_error(ctx->ctrl, clear != 0);
  // walks through wts_walk_noalloc latch into the device scratch
  DevScratch& ds = g_scratch[ctx->device];
  if (ds.ptr) {
    const wts_status s2 = read_ctrl_error((Ctrl*)ds.ptr, clear != 0);
    if (st == WTS_OK) st = s2;
  }
  return st;
}

wts_status wts_check_log_ratio(int32_t device, int64_t* mismatches) {
  if (!mismatches || device < 0) return WTS_ERR_INVALID_ARG;
  DeviceGuard guard(device);
  unsigned long long* d = nullptr;
  if (hipMalloc((void**)&d, sizeof(*d)) != hipSuccess) return WTS_ERR_NO_MEMORY;
  unsigned long long h = 0;
  wts_status st = WTS_OK;
  if (hipMemset(d, 0, sizeof(*d)) != hipSuccess || launch_check_log_ratio(d, nullptr) != hipSuccess ||
      hipMemcpy(&h, d, sizeof(h), hipMemcpyDeviceToHost) != hipSuccess)
    st = WTS_ERR_DEVICE;
  (void)hipFree(d);
  *mismatches = (int64_t)h;
  return st;
}

void wts_destroy(wts_ctx* ctx) {
  if (!ctx) return;
  DeviceGuard guard(ctx->device);
  (void)hipDeviceSynchronize();
  free_ctx(ctx);
}

}  // extern "C"
