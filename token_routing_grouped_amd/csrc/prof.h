// Optional per-kernel timing with HIP events, for benchmarks.  When enabled,
// selected launches are bracketed by events recorded on the launch stream;
// moe_prof_query() later waits on them and sums the elapsed times.  Off by
// default: then each bracket is a single relaxed load.
#pragma once

#include <hip/hip_runtime.h>

namespace trg {

bool prof_on();
void prof_begin(const char* name, hipStream_t s);
void prof_end(const char* name, hipStream_t s);

struct ProfScope {
  const char* name;
  hipStream_t s;
  ProfScope(const char* n, hipStream_t st) : name(n), s(st) {
    if (prof_on()) prof_begin(name, s);
  }
  ~ProfScope() {
    if (prof_on()) prof_end(name, s);
  }
};

}  // namespace trg
