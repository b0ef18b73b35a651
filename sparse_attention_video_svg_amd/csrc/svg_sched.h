// Workgroup scheduling arithmetic shared by the host launchers and the
// kernels: the XCD-aware order of workgroup ids and the number of key slices
// of the sampled-row sweeps.  Plain C++ with no HIP dependency, so that the
// CPU tests can compile it on its own.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__) || defined(__HIP__)
#define SVG_HD __host__ __device__
#else
#define SVG_HD
#endif

namespace svg {

// The hardware deals workgroup ids round-robin to the XCDs (id w runs on XCD
// w mod nxcd).  xcd_logical maps id w to a logical work item so that every
// XCD receives runs of `run` consecutive logical items (which then share
// their K/V tiles in that XCD's L2).  On a grid of xcd_grid(total, nxcd, run)
// ids it is a bijection of [0, grid); callers skip items >= total.
SVG_HD inline int64_t xcd_grid(int64_t total, int32_t nxcd, int32_t run) {
  const int64_t per = (int64_t)nxcd * run;
  return (total + per - 1) / per * per;
}

SVG_HD inline int32_t xcd_logical(int32_t w, int32_t nxcd, int32_t run) {
  const int32_t xcd = w % nxcd, slot = w / nxcd;
  return ((slot / run) * nxcd + xcd) * run + slot % run;
}

// Key slices of each sampled-row sweep.  The full sweep runs one workgroup
// (rows chunk x head x slice) per CU at a time, so its time goes as
// ceil(workgroups / CUs) rounds of 1/ks of a chunk's keys each: take the ks in
// 1..min(16, key tiles, cap) that minimises rounds / ks; on ties the one
// whose workgroup count is nearest four per CU (enough to even out chunks of
// unequal size, few partials to merge).  wgs: chunks x heads.
inline int32_t choose_ksplit(int64_t wgs, int64_t nkt, int64_t cus, int32_t cap) {
  int64_t kmax = nkt < 16 ? nkt : 16;
  kmax = kmax < cap ? kmax : cap;
  if (cus < 1) cus = 1;
  int64_t best = 1;
  double best_t = 1e300;
  for (int64_t ks = 1; ks <= kmax; ++ks) {
    const double t = (double)((wgs * ks + cus - 1) / cus) / (double)ks;
    const int64_t dist = wgs * ks > 4 * cus ? wgs * ks - 4 * cus : 4 * cus - wgs * ks;
    const int64_t best_dist = wgs * best > 4 * cus ? wgs * best - 4 * cus : 4 * cus - wgs * best;
    if (t < best_t - 1e-12 || (t < best_t + 1e-12 && dist < best_dist)) {
      best_t = t;
      best = ks;
    }
  }
  return (int32_t)best;
}

}  // namespace svg
