// Host-side helpers shared by the C-ABI translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <string>

#include "kvev_internal.h"

namespace kvev {

inline kvev_status fail(kvev_ctx* c, kvev_status s, const std::string& msg) {
  if (c) c->err = msg;
  return s;
}

inline kvev_status hip_fail(kvev_ctx* c, hipError_t e, const char* where) {
  c->sticky = true;
  c->err = std::string(where) + ": " + hipGetErrorString(e);
  return KVEV_EHIP;
}

#define KVEV_HIP(c, expr)                                        \
  do {                                                           \
    hipError_t e_ = (expr);                                      \
    if (e_ != hipSuccess) return ::kvev::hip_fail((c), e_, #expr); \
  } while (0)

#define KVEV_LIVE(c)                                                          \
  do {                                                                        \
    if (!(c)) return KVEV_EINVAL;                                             \
    if ((c)->sticky) return KVEV_ESTATE;                                      \
  } while (0)

template <typename T>
hipError_t dalloc(T** p, size_t count) {
  *p = nullptr;
  if (count == 0) return hipSuccess;
  return hipMalloc(reinterpret_cast<void**>(p), count * sizeof(T));
}

// Profiling: events around named launches on the context's stream.
struct ProfScope {
  kvev_ctx* c;
  const char* name;
  hipEvent_t a = nullptr;
  ProfScope(kvev_ctx* c_, const char* n) : c(c_), name(n) {
    if (!c->prof.enabled || !name) return;
    a = take_event();
    if (a) hipEventRecord(a, c->stream);
  }
  hipEvent_t take_event() {
    if (!c->prof.pool.empty()) {
      hipEvent_t e = c->prof.pool.back();
      c->prof.pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
  ~ProfScope() {
    if (!c->prof.enabled || !name || !a) return;
    hipEvent_t b = take_event();
    if (!b) return;
    hipEventRecord(b, c->stream);
    c->prof.pending.push_back({name, a, b});
  }
};


}  // namespace kvev
