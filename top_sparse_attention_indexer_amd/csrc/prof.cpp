// Stage timing of the library's own launches (dsa_profile_start / _stop):
// a pool of HIP events recorded on the launch stream around every kernel the
// entry points enqueue, summed per stage when the caller stops profiling.
// Off by default; when off, each mark costs one relaxed atomic load.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "launch.h"

namespace dsa {
namespace {

std::atomic<bool> g_on{false};
std::mutex g_mu;
// plain arrays (created by prof_start, released by prof_stop), so that no
// static object with a destructor is left for process exit
hipEvent_t* g_ev = nullptr;       // 2 per launch: begin, end
int* g_stage = nullptr;           // stage of each pair
char* g_closed = nullptr;         // end event recorded
size_t g_pairs = 0;               // capacity in pairs
size_t g_used = 0;                // pairs recorded
size_t g_dropped = 0;             // launches not recorded (pool full)
thread_local long long t_open = -1;  // pair opened by this thread's last prof_begin

}  // namespace

void prof_begin(hipStream_t s, int stage) {
  if (!g_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lock(g_mu);
  t_open = -1;
  if (!g_on.load(std::memory_order_relaxed)) return;
  if (g_used + 1 > g_pairs) {
    ++g_dropped;
    return;
  }
  if (hipEventRecord(g_ev[2 * g_used], s) != hipSuccess) return;
  g_stage[g_used] = stage;
  g_closed[g_used] = 0;
  t_open = (long long)g_used++;
}

void prof_end(hipStream_t s) {
  if (!g_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lock(g_mu);
  if (t_open < 0) return;
  if (hipEventRecord(g_ev[2 * t_open + 1], s) == hipSuccess) g_closed[t_open] = 1;
  t_open = -1;
}

void prof_release() {
  for (size_t k = 0; k < 2 * g_pairs; ++k)
    if (g_ev[k]) (void)hipEventDestroy(g_ev[k]);
  delete[] g_ev;
  delete[] g_stage;
  delete[] g_closed;
  g_ev = nullptr;
  g_stage = nullptr;
  g_closed = nullptr;
  g_pairs = g_used = g_dropped = 0;
}

hipError_t prof_start(int max_launches) {
  std::lock_guard<std::mutex> lock(g_mu);
  prof_release();
  g_ev = new hipEvent_t[2 * (size_t)max_launches]();
  g_stage = new int[max_launches]();
  g_closed = new char[max_launches]();
  g_pairs = (size_t)max_launches;
  for (size_t k = 0; k < 2 * g_pairs; ++k) {
    hipError_t err = hipEventCreate(&g_ev[k]);
    if (err != hipSuccess) {
      prof_release();
      return err;
    }
  }
  g_on.store(true, std::memory_order_relaxed);
  return hipSuccess;
}

hipError_t prof_stop(double* ms, int32_t* launches, int n_stages, long long* dropped) {
  std::lock_guard<std::mutex> lock(g_mu);
  g_on.store(false, std::memory_order_relaxed);
  for (int i = 0; i < n_stages; ++i) {
    if (ms) ms[i] = 0.0;
    if (launches) launches[i] = 0;
  }
  hipError_t err = hipSuccess;
  for (size_t k = 0; k < g_used && err == hipSuccess; ++k) {
    if (!g_closed[k]) continue;
    err = hipEventSynchronize(g_ev[2 * k + 1]);
    if (err != hipSuccess) break;
    float t = 0.f;
    err = hipEventElapsedTime(&t, g_ev[2 * k], g_ev[2 * k + 1]);
    const int st = g_stage[k];
    if (err == hipSuccess && st >= 0 && st < n_stages) {
      if (ms) ms[st] += t;
      if (launches) ++launches[st];
    }
  }
  if (dropped) *dropped = (long long)g_dropped;
  prof_release();
  return err;
}

}  // namespace dsa
