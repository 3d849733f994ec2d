// Host-side runtime pieces of libkvc: status strings, size helpers and the
// optional per-kernel event timing used by the benchmark.
#include <math.h>
#include <string.h>

#include <atomic>
#include <map>
#include <string>
#include <vector>

#include "common.h"

namespace kvc {

int device_cu_count() {
  static std::atomic<int> cache[64];   // per device id; 0 = not queried yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 0;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

namespace {

struct Record {
  const char* name;
  hipEvent_t start, stop;
};

bool g_timing = false;
std::vector<Record> g_records;

struct Summary {
  std::string name;
  int32_t launches;
  double total_ms;
};
std::vector<Summary> g_summary;
bool g_summary_valid = false;

void clear_records() {
  for (auto& r : g_records) {
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  g_records.clear();
  g_summary.clear();
  g_summary_valid = false;
}

kvc_status build_summary() {
  if (g_summary_valid) return KVC_OK;
  std::map<std::string, size_t> pos;
  g_summary.clear();
  for (auto& r : g_records) {
    if (hipEventSynchronize(r.stop) != hipSuccess) return KVC_E_DEVICE;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) return KVC_E_DEVICE;
    auto it = pos.find(r.name);
    if (it == pos.end()) {
      pos[r.name] = g_summary.size();
      g_summary.push_back({r.name, 1, (double)ms});
    } else {
      g_summary[it->second].launches += 1;
      g_summary[it->second].total_ms += ms;
    }
  }
  g_summary_valid = true;
  return KVC_OK;
}

}  // namespace

int launch_begin(const char* name, hipStream_t s) {
  (void)hipGetLastError();  // start from a clean error state
  if (!g_timing) return -1;
  Record r{name, nullptr, nullptr};
  // timing-only events: no system-scope fence (an L2 writeback and
  // invalidate) when they signal, which would slow the launch being timed
  // and the one after it
  if (hipEventCreateWithFlags(&r.start, hipEventDisableSystemFence) != hipSuccess) return -1;
  if (hipEventCreateWithFlags(&r.stop, hipEventDisableSystemFence) != hipSuccess) {
    (void)hipEventDestroy(r.start);
    return -1;
  }
  (void)hipEventRecord(r.start, s);
  g_records.push_back(r);
  g_summary_valid = false;
  return (int)g_records.size() - 1;
}

kvc_status launch_end(int slot, hipStream_t s) {
  hipError_t e = hipGetLastError();
  if (slot >= 0) (void)hipEventRecord(g_records[slot].stop, s);
  return e == hipSuccess ? KVC_OK : KVC_E_DEVICE;
}

}  // namespace kvc

extern "C" {

const char* kvc_status_str(int status) {
  switch (status) {
    case KVC_OK: return "KVC_OK: success";
    case KVC_E_ARG: return "KVC_E_ARG: invalid argument";
    case KVC_E_SHAPE: return "KVC_E_SHAPE: inconsistent sizes";
    case KVC_E_WORKSPACE: return "KVC_E_WORKSPACE: workspace missing or too small";
    case KVC_E_DEVICE: return "KVC_E_DEVICE: HIP call or kernel launch failed";
    case KVC_E_UNSUPPORTED: return "KVC_E_UNSUPPORTED: not implemented for these sizes";
    default: return "KVC: unknown status";
  }
}

int kvc_abi_version(void) { return 1; }

int64_t kvc_cache_bytes(int64_t B, int64_t S, int64_t L, int64_t N, int64_t D, int64_t elem_bytes) {
  int64_t f[6] = {2, B, S, L, N, D};
  int64_t r = elem_bytes;
  if (elem_bytes < 0) return -1;
  for (int i = 0; i < 6; ++i) {
    if (f[i] < 0) return -1;
    if (f[i] != 0 && r > INT64_MAX / f[i]) return -1;
    r *= f[i];
  }
  return r;
}

int kvc_think_channels(int D, double lambda) {
  if (D <= 0 || !(lambda >= 0.0) || !(lambda < 1.0)) return -1;
  return (int)floor((1.0 - lambda) * (double)D);
}

kvc_status kvc_timing_enable(int32_t enable) {
  kvc::clear_records();
  kvc::g_timing = enable != 0;
  return KVC_OK;
}

int32_t kvc_timing_count(void) {
  if (kvc::build_summary() != KVC_OK) return -1;
  return (int32_t)kvc::g_summary.size();
}

kvc_status kvc_timing_read(int32_t idx, char* name_buf, int32_t name_len, int32_t* launches,
                           double* total_ms) {
  kvc_status st = kvc::build_summary();
  if (st != KVC_OK) return st;
  if (idx < 0 || idx >= (int32_t)kvc::g_summary.size()) return KVC_E_ARG;
  const auto& s = kvc::g_summary[idx];
  if (name_buf && name_len > 0) {
    strncpy(name_buf, s.name.c_str(), (size_t)name_len - 1);
    name_buf[name_len - 1] = '\0';
  }
  if (launches) *launches = s.launches;
  if (total_ms) *total_ms = s.total_ms;
  return KVC_OK;
}

}  // extern "C"
