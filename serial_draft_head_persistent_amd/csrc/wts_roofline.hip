// Host driver of the roofline microbenchmarks (include/wts_roofline.h): runs
// each small kernel of wts_kernels.hip on the walk's device and turns its
// timing into a rate.  Bandwidth kernels are timed with HIP events (best of
// several launches); the exchange, hop and clock kernels time themselves
// with the device's 100 MHz wall clock.

#include <algorithm>
#include <vector>

#include "wts.h"
#include "wts_internal.h"
#include "wts_roofline.h"

using namespace wts;

namespace {

constexpr double kWallMHz = 100.0;   // s_memrealtime rate (hipDeviceAttributeWallClockRate on MI355X)
constexpr long long kTimeoutTicks = 200000000LL;  // 2 s per wait

struct Bufs {
  std::vector<void*> p;
  ~Bufs() {
    for (void* q : p) (void)hipFree(q);
  }
  template <class T>
  T* get(size_t bytes) {
    void* q = nullptr;
    if (hipMalloc(&q, bytes) != hipSuccess) return nullptr;
    p.push_back(q);
    return (T*)q;
  }
};

// Best time (ms) of `reps` launches of f() after one warm-up launch.
template <class F>
bool best_ms(F f, int reps, float* ms) {
  hipEvent_t a, b;
  if (hipEventCreate(&a) != hipSuccess) return false;
  if (hipEventCreate(&b) != hipSuccess) {
    (void)hipEventDestroy(a);
    return false;
  }
  bool ok = f() == hipSuccess && hipDeviceSynchronize() == hipSuccess;
  float best = 1e30f;
  for (int i = 0; ok && i < reps; ++i) {
    float t = 0.0f;
    ok = hipEventRecord(a, 0) == hipSuccess && f() == hipSuccess && hipEventRecord(b, 0) == hipSuccess &&
         hipEventSynchronize(b) == hipSuccess && hipEventElapsedTime(&t, a, b) == hipSuccess;
    best = std::min(best, t);
  }
  (void)hipEventDestroy(a);
  (void)hipEventDestroy(b);
  *ms = best;
  return ok;
}

}  // namespace

extern "C" wts_status wts_roofline(int32_t device, wts_roofline_result* out) {
  if (!out || device < 0) return WTS_ERR_INVALID_ARG;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || device >= ndev) return WTS_ERR_INVALID_ARG;
  int prev = -1;
  (void)hipGetDevice(&prev);
  if (hipSetDevice(device) != hipSuccess) return WTS_ERR_DEVICE;
  struct Restore {
    int d;
    ~Restore() {
      if (d >= 0) (void)hipSetDevice(d);
    }
  } restore{prev};
  *out = wts_roofline_result{};
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) return WTS_ERR_DEVICE;
  const int G = std::min(cus, kMaxGrid);
  out->grid = G;

  Bufs bufs;
  unsigned* sink = bufs.get<unsigned>(65536 * sizeof(unsigned));
  long long* clk = bufs.get<long long>(2 * kMaxGrid * sizeof(long long));
  if (!sink || !clk) return WTS_ERR_NO_MEMORY;
  float ms = 0.0f;

  // LDS read: G workgroups x 512 lanes x 8 reads x 16 bytes per round
  {
    const int rounds = 4096;
    if (!best_ms([&] { return launch_rf_lds(G, rounds, sink, 0); }, 3, &ms)) return WTS_ERR_DEVICE;
    out->lds_read_GBps = (double)G * 512 * 8 * 16 * rounds / (ms * 1e-3) / 1e9;
  }
  // MFMA issue: G x 8 waves x 8 chains per round; 16x16x64 (int8) or 16x16x32 (bf16) MACs each
  {
    const int rounds = 4096;
    const double mf = (double)G * 8 * 8 * rounds;
    if (!best_ms([&] { return launch_rf_mfma(0, G, rounds, sink, clk, 0); }, 3, &ms)) return WTS_ERR_DEVICE;
    out->mfma_i8_TOPs = mf * 16 * 16 * 64 * 2 / (ms * 1e-3) / 1e12;
    std::vector<long long> h(2 * G);
    if (hipMemcpy(h.data(), clk, 2 * G * sizeof(long long), hipMemcpyDeviceToHost) != hipSuccess)
      return WTS_ERR_DEVICE;
    double cyc = 0.0, wall = 0.0;
    for (int g = 0; g < G; ++g) {
      cyc += (double)h[2 * g];
      wall += (double)h[2 * g + 1];
    }
    out->clock_MHz = wall > 0.0 ? cyc / wall * kWallMHz : -1.0;
    if (!best_ms([&] { return launch_rf_mfma(1, G, rounds, sink, clk, 0); }, 3, &ms)) return WTS_ERR_DEVICE;
    out->mfma_bf16_TFLOPs = mf * 16 * 16 * 32 * 2 / (ms * 1e-3) / 1e12;
  }
  // stream reads: 2 GiB (HBM) and 128 MiB (memory-side cache, after a warm-up read)
  {
    const size_t hbm = size_t(2) << 30, mall = size_t(128) << 20;
    char* big = bufs.get<char>(hbm);
    if (!big) return WTS_ERR_NO_MEMORY;
    if (hipMemset(big, 1, hbm) != hipSuccess || hipDeviceSynchronize() != hipSuccess) return WTS_ERR_DEVICE;
    const int sg = G * 16;
    if (!best_ms([&] { return launch_rf_stream(big, (long long)(hbm / 16), 1, sg, sink, 0); }, 3, &ms))
      return WTS_ERR_DEVICE;
    out->hbm_read_GBps = (double)hbm / (ms * 1e-3) / 1e9;
    // ten passes over 128 MiB in one launch (the warm-up launch brings it into the cache)
    const int passes = 10;
    if (!best_ms([&] { return launch_rf_stream(big, (long long)(mall / 16), passes, sg, sink, 0); }, 3, &ms))
      return WTS_ERR_DEVICE;
    out->mall_read_GBps = (double)mall * passes / (ms * 1e-3) / 1e9;
  }
  // exchange rounds
  {
    const int rounds = 100;   // step tags hold up to 127
    Ctrl* ctrl = bufs.get<Ctrl>(sizeof(Ctrl));
    unsigned long long* flat = bufs.get<unsigned long long>(2 * kCopies * kMaxGrid * 8);
    unsigned* cnt = bufs.get<unsigned>(rounds * 4);
    unsigned* wrong = bufs.get<unsigned>(2 * kMaxGrid * 4);
    unsigned* xcc = bufs.get<unsigned>(kMaxGrid * 4);
    if (!ctrl || !flat || !cnt || !wrong || !xcc) return WTS_ERR_NO_MEMORY;
    std::vector<unsigned> hx(G);
    if (launch_xcc_ids(xcc, G, 0) != hipSuccess ||
        hipMemcpy(hx.data(), xcc, G * 4, hipMemcpyDeviceToHost) != hipSuccess)
      return WTS_ERR_DEVICE;
    bool groups_on_one_xcd = true;
    for (int g = 0; g < G; ++g) groups_on_one_xcd = groups_on_one_xcd && hx[g] == hx[g % kGroups];
    for (int v = 0; v < 6; ++v) {
      out->exchange_us[v] = -1.0;
      if ((v == 0 || v == 4) && !groups_on_one_xcd) continue;
      if (hipMemset(ctrl, 0, sizeof(Ctrl)) != hipSuccess || hipMemset(flat, 0, 2 * kCopies * kMaxGrid * 8) != hipSuccess ||
          hipMemset(cnt, 0, rounds * 4) != hipSuccess || hipMemset(wrong, 0, 2 * kMaxGrid * 4) != hipSuccess ||
          launch_rf_exchange(v, G, rounds, ctrl, flat, cnt, kTimeoutTicks, clk, wrong, 0) != hipSuccess ||
          hipDeviceSynchronize() != hipSuccess)
        return WTS_ERR_DEVICE;
      std::vector<long long> hc(G);
      std::vector<unsigned> hw(2 * G);
      if (hipMemcpy(hc.data(), clk, G * sizeof(long long), hipMemcpyDeviceToHost) != hipSuccess ||
          hipMemcpy(hw.data(), wrong, 2 * G * 4, hipMemcpyDeviceToHost) != hipSuccess)
        return WTS_ERR_DEVICE;
      long long most = 0, bad = 0;
      for (int g = 0; g < G; ++g) {
        most = std::max(most, hc[g]);
        bad += hw[2 * g] + hw[2 * g + 1];
      }
      out->exchange_bad[v] = bad;
      out->exchange_us[v] = (double)most / kWallMHz / rounds;
    }
    // one-way hops: workgroup 0 with a workgroup on its XCD, then on another XCD
    int same = -1, other = -1;
    for (int g = 1; g < G; ++g) {
      if (same < 0 && hx[g] == hx[0]) same = g;
      if (other < 0 && hx[g] != hx[0]) other = g;
    }
    const int hops = 2000;
    auto hop = [&](int peer, int xcd, double* res) -> wts_status {
      *res = -1.0;
      if (peer < 0) return WTS_OK;
      if (hipMemset(flat, 0, 256) != hipSuccess || hipMemset(clk, 0xFF, 2 * sizeof(long long)) != hipSuccess ||
          launch_rf_pingpong(G, peer, xcd, hops, flat, kTimeoutTicks, clk, 0) != hipSuccess ||
          hipDeviceSynchronize() != hipSuccess)
        return WTS_ERR_DEVICE;
      long long hc[2];
      if (hipMemcpy(hc, clk, sizeof(hc), hipMemcpyDeviceToHost) != hipSuccess) return WTS_ERR_DEVICE;
      if (hc[0] > 0 && hc[1] > 0) *res = (double)hc[0] / kWallMHz / (2.0 * hops);
      return WTS_OK;
    };
    wts_status st = hop(same, 1, &out->hop_xcd_us);
    if (st == WTS_OK) st = hop(other, 0, &out->hop_device_us);
    if (st != WTS_OK) return st;
  }
  // VALU issue: one wave, then eight and sixteen waves (two and four per SIMD)
  // of one workgroup; then v_dot4_i32_i8 at two waves per SIMD
  {
    const int n = 1 << 20;
    float* fo = bufs.get<float>(1024 * sizeof(float));
    if (!fo) return WTS_ERR_NO_MEMORY;
    auto run = [&](int mode, int waves, double* res) -> wts_status {
      std::vector<long long> hc(waves);
      if (launch_rf_valu(mode, waves, n, fo, clk, 0) != hipSuccess || hipDeviceSynchronize() != hipSuccess ||
          launch_rf_valu(mode, waves, n, fo, clk, 0) != hipSuccess || hipDeviceSynchronize() != hipSuccess ||
          hipMemcpy(hc.data(), clk, waves * sizeof(long long), hipMemcpyDeviceToHost) != hipSuccess)
        return WTS_ERR_DEVICE;
      double m = 0.0;
      for (long long c : hc) m = std::max(m, (double)c);
      *res = m / n;
      return WTS_OK;
    };
    wts_status st = run(0, 1, &out->valu_dep_cycles);
    if (st == WTS_OK) st = run(1, 1, &out->valu_indep_cycles);
    if (st == WTS_OK) st = run(1, 8, &out->valu_indep_2w_cycles);
    if (st == WTS_OK) st = run(1, 16, &out->valu_indep_4w_cycles);
    if (st == WTS_OK) st = run(2, 8, &out->dot4_2w_cycles);
    if (st != WTS_OK) return st;
  }
  return hipDeviceSynchronize() == hipSuccess ? WTS_OK : WTS_ERR_DEVICE;
}
