// Kernel timing hook: while enabled, every kernel launch of the library is
// bracketed by two hipEvents recorded on the launch stream; collect() waits
// for them and returns per-kernel launch counts and total GPU time.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "csa.h"
#include "kernels.h"

namespace csa {
namespace {

struct Pending {
  const char* name;
  hipEvent_t a, b;
};

std::atomic<int> g_on{0};
std::mutex g_mu;
std::vector<hipEvent_t> g_pool;
std::vector<Pending> g_pending;
std::map<std::string, std::pair<int64_t, double>> g_tot;

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

ProfScope::ProfScope(const char* name, hipStream_t s) : name_(name), s_(s), a_(nullptr) {
  if (!g_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_mu);
  a_ = take_event();
  if (a_) hipEventRecord((hipEvent_t)a_, s_);
}

ProfScope::~ProfScope() {
  if (!a_) return;
  std::lock_guard<std::mutex> lk(g_mu);
  hipEvent_t b = take_event();
  if (!b) return;
  hipEventRecord(b, s_);
  g_pending.push_back(Pending{name_, (hipEvent_t)a_, b});
}

}  // namespace csa

extern "C" {

csa_status csa_profile_enable(int on) {
  csa::g_on.store(on ? 1 : 0);
  return CSA_OK;
}

int csa_profile_collect(csa_kernel_time* out, int max_entries) {
  std::lock_guard<std::mutex> lk(csa::g_mu);
  for (auto& p : csa::g_pending) {
    float ms = 0.f;
    hipEventSynchronize(p.b);
    if (hipEventElapsedTime(&ms, p.a, p.b) == hipSuccess) {
      auto& t = csa::g_tot[p.name];
      t.first += 1;
      t.second += ms;
    }
    csa::g_pool.push_back(p.a);
    csa::g_pool.push_back(p.b);
  }
  csa::g_pending.clear();
  int n = 0;
  for (auto& kv : csa::g_tot) {
    if (out && n < max_entries) {
      std::memset(&out[n], 0, sizeof(out[n]));
      std::strncpy(out[n].name, kv.first.c_str(), sizeof(out[n].name) - 1);
      out[n].launches = kv.second.first;
      out[n].total_ms = kv.second.second;
    }
    ++n;
  }
  csa::g_tot.clear();
  return n;
}

}  // extern "C"
