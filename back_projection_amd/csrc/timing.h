// Optional event pair around a kernel launch (host side).  The library's
// timing facility hands launchers a pair to record on the launch stream.
#pragma once

#include <hip/hip_runtime.h>

namespace tproj {

struct EvPair {
  hipEvent_t a = nullptr, b = nullptr;
};

inline void ev_begin(const EvPair* e, hipStream_t st) {
  if (e) (void)hipEventRecord(e->a, st);
}
inline void ev_end(const EvPair* e, hipStream_t st) {
  if (e) (void)hipEventRecord(e->b, st);
}

}  // namespace tproj
