// host_util.h -- host helpers shared by the entry points of libssmscan.so.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace ssm {

// Records a failed HIP call for ssm_last_hip_error() and returns SSM_ERR_HIP.
int hip_fail(hipError_t e);

// Compute units of the current device (queried once per device; 256 when the
// query fails).
int cu_count_cached();

// Workgroups of `block` threads of kernel f one compute unit holds at once
// (registers and LDS decide), or 0 when the runtime cannot say (no device);
// cached per kernel.
int blocks_per_cu(const void *f, int block);

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---------------------------------------------------------------------------
// Sequence split of the backward passes.  A grid of `blocks` workgroups, each
// walking `nck` chunks, runs on `units` workgroup slots (compute units times
// workgroups per unit).  Cutting the sequence into ns segments multiplies the
// workgroups by ns and divides each one's walk by ns, at the price of a carry
// pass over the segments after the first that costs `carry_cost` of the main
// pass per chunk.  Times are in units of one workgroup walking one chunk.
// ---------------------------------------------------------------------------

// The segment count (at most max_seg, each of at least min_chunks chunks)
// that minimises ceil(blocks ns / units) ceil(nck / ns) + carry_cost (ns - 1)
// / ns blocks nck / units; a split has to win by more than 1%.
inline int split_segments(int64_t blocks, int64_t nck, int64_t units, double carry_cost, int64_t max_seg,
                          int64_t min_chunks) {
  const int64_t most = nck / min_chunks < max_seg ? nck / min_chunks : max_seg;
  const double work = static_cast<double>(blocks) * static_cast<double>(nck) / units;
  int best = 1;
  double best_t = 1e300;
  for (int64_t k = 1; k <= (most > 1 ? most : 1); ++k) {
    const int64_t segc = (nck + k - 1) / k;
    const int64_t ns = (nck + segc - 1) / segc;
    const double rounds = static_cast<double>((blocks * ns + units - 1) / units);
    const double t = rounds * static_cast<double>(segc) + carry_cost * static_cast<double>(ns - 1) / ns * work;
    if (t < best_t * 0.99) {
      best_t = t;
      best = static_cast<int>(ns);
    }
  }
  return best;
}

// The time at which the last of n workgroups of la chunks and then n of lb
// chunks ends when each goes to the first slot free, in that order: the
// dispatch of a two-segment grid, segment 0 first.
inline int64_t two_class_makespan(int64_t n, int64_t la, int64_t lb, int64_t units) {
  struct Group { int64_t t, k; };   // k slots free from time t
  Group g[8];
  int ng = 1;
  g[0] = {0, units};
  int64_t end = 0;
  auto place = [&](int64_t cnt, int64_t len) -> bool {
    while (cnt > 0) {
      int i = 0;
      for (int j = 1; j < ng; ++j)
        if (g[j].t < g[i].t) i = j;
      const int64_t k = cnt < g[i].k ? cnt : g[i].k;
      const int64_t t = g[i].t + len;
      cnt -= k;
      g[i].k -= k;
      if (g[i].k == 0) g[i] = g[--ng];
      int m = -1;
      for (int j = 0; j < ng; ++j)
        if (g[j].t == t) m = j;
      if (m >= 0) {
        g[m].k += k;
      } else {
        if (ng == 8) return false;   // never reached: at most three free times coexist
        g[ng++] = {t, k};
      }
      if (t > end) end = t;
    }
    return true;
  };
  if (!place(n, la) || !place(n, lb)) return INT64_MAX;
  return end;
}

// The length of segment 0 when the library splits the sequence in two.
// Segment 0 (dispatched first) may be the longer one: the carry pass then
// covers only the short second segment, and the second segment's
// workgroups fill the slots the first segment's last round leaves free.  The
// length minimises two_class_makespan + carry_cost (chunks of segment 1)
// blocks / units, equal halves where a longer first segment does not pay
// (a grid of one round).
inline int split_first_segment(int64_t blocks, int64_t nck, int64_t units, double carry_cost) {
  const int64_t half = (nck + 1) / 2;
  int64_t best = half;
  double best_t = 1e300;
  for (int64_t l0 = half; l0 < nck; ++l0) {
    const double t = static_cast<double>(two_class_makespan(blocks, l0, nck - l0, units)) +
                     carry_cost * static_cast<double>(nck - l0) * static_cast<double>(blocks) / units;
    if (t < best_t * 0.99) {
      best_t = t;
      best = l0;
    }
  }
  return static_cast<int>(best);
}

}  // namespace ssm
