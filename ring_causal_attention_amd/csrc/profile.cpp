// Per-kernel timing registry behind lwm_profile_*: HIP event pairs recorded on the launch stream
// around each kernel, resolved (waited for) only when the caller asks for the totals.
#include "profile.hpp"

#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/lwm_attn.h"

namespace lwm {
namespace {

struct Kernel {
  std::string name;
  double total_ms = 0.0;
  int64_t launches = 0;
};
struct Pending {
  int kernel;
  hipEvent_t start, stop;
};

std::mutex g_mu;
bool g_on = false;
std::vector<Kernel> g_kernels;
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_free;

hipEvent_t take_event() {
  if (!g_free.empty()) {
    hipEvent_t e = g_free.back();
    g_free.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

int kernel_id(const char* name) {
  for (size_t i = 0; i < g_kernels.size(); ++i)
    if (g_kernels[i].name == name) return (int)i;
  g_kernels.push_back(Kernel{name});
  return (int)g_kernels.size() - 1;
}

// Waits for every pending pair and folds it into the totals (g_mu held).
int resolve() {
  int status = LWM_OK;
  for (const Pending& p : g_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(p.stop) != hipSuccess || hipEventElapsedTime(&ms, p.start, p.stop) != hipSuccess) {
      status = LWM_ERR_HIP;
    } else {
      g_kernels[p.kernel].total_ms += ms;
      g_kernels[p.kernel].launches += 1;
    }
    g_free.push_back(p.start);
    g_free.push_back(p.stop);
  }
  g_pending.clear();
  return status;
}

}  // namespace

int prof_begin(const char* kernel, hipStream_t stream) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on) return -1;
  Pending p{kernel_id(kernel), take_event(), take_event()};
  if (!p.start || !p.stop || hipEventRecord(p.start, stream) != hipSuccess) return -1;
  g_pending.push_back(p);
  return (int)g_pending.size() - 1;
}

void prof_end(int token, hipStream_t stream) {
  if (token < 0) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (token < (int)g_pending.size()) (void)hipEventRecord(g_pending[token].stop, stream);
}

}  // namespace lwm

extern "C" {

int lwm_profile_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(lwm::g_mu);
  lwm::g_on = on != 0;
  return LWM_OK;
}

int lwm_profile_reset(void) {
  std::lock_guard<std::mutex> lk(lwm::g_mu);
  const int s = lwm::resolve();
  lwm::g_kernels.clear();
  return s;
}

int lwm_profile_count(void) {
  std::lock_guard<std::mutex> lk(lwm::g_mu);
  lwm::resolve();
  return (int)lwm::g_kernels.size();
}

int lwm_profile_get(int32_t index, const char** name, double* total_ms, int64_t* launches) {
  std::lock_guard<std::mutex> lk(lwm::g_mu);
  const int s = lwm::resolve();
  if (index < 0 || index >= (int)lwm::g_kernels.size() || !name || !total_ms || !launches) return LWM_ERR_INVALID_ARG;
  *name = lwm::g_kernels[index].name.c_str();
  *total_ms = lwm::g_kernels[index].total_ms;
  *launches = lwm::g_kernels[index].launches;
  return s;
}

}  // extern "C"
