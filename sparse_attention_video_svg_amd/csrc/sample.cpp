// svg_sample_rows: the query rows that online profiling samples.
//
// The rebuttal's answer on profiling puts the head-type decision at every
// diffusion step and layer, from a small set of query rows; the rows are
// drawn uniformly without replacement from the video rows [T, T + N*F),
// shared by all heads and sorted ascending (the order the profiling sweeps
// group rows by).  Host code: the list is small (1 % of the video rows of
// the pages' workloads) and the caller copies it to the device.
//
// Floyd's sampling (J. Bentley with R. Floyd, "Programming pearls: a sample
// of brilliance", CACM 30(9), 1987): for j = n - count .. n - 1 draw t
// uniform in [0, j]; keep t if it is new, else keep j.  Every count-subset
// of [0, n) comes out with the same probability, in O(count) draws whatever
// n is.  Random bits: SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast
// splittable pseudorandom number generators", OOPSLA 2014); integers in
// [0, j] by D. Lemire's multiply-and-reject ("Fast random integer generation
// in an interval", ACM TOMACS 29(1), 2019), which is exactly uniform.
#include <algorithm>
#include <cstdint>
#include <unordered_set>
#include <vector>

#include "svg.h"

namespace svg {

namespace {

struct SplitMix64 {
  uint64_t state;
  uint64_t next() {
    uint64_t z = (state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
  }
  // uniform in [0, range) for 0 < range <= 2^32
  uint32_t below(uint64_t range) {
    uint64_t x = next() >> 32;
    uint64_t m = x * range;
    if ((uint32_t)m < range) {
      const uint32_t t = (uint32_t)((0x100000000ull - range) % range);
      while ((uint32_t)m < t) {
        x = next() >> 32;
        m = x * range;
      }
    }
    return (uint32_t)(m >> 32);
  }
};

}  // namespace

// count distinct integers of [0, n), ascending, into out.  Membership of
// the drawn set is a hash set while the sample is sparse (count < n / 64),
// else a bitmap of n bits, which also yields the rows in order: host memory
// stays within about n bytes either way.
void sample_sorted(int64_t n, int32_t count, uint64_t seed, int32_t* out) {
  SplitMix64 rng{seed};
  if ((int64_t)count * 64 < n) {
    std::unordered_set<int32_t> seen;
    seen.reserve((size_t)count * 2);
    std::vector<int32_t> pick;
    pick.reserve(count);
    for (int64_t j = n - count; j < n; ++j) {
      const int32_t t = (int32_t)rng.below((uint64_t)j + 1);
      const int32_t keep = seen.insert(t).second ? t : (int32_t)j;
      if (keep != t) seen.insert(keep);
      pick.push_back(keep);
    }
    std::sort(pick.begin(), pick.end());
    std::copy(pick.begin(), pick.end(), out);
    return;
  }
  std::vector<uint64_t> bits((size_t)((n + 63) / 64), 0);
  auto test_set = [&](int64_t x) {  // sets bit x, returns whether it was clear
    uint64_t& w = bits[(size_t)(x >> 6)];
    const uint64_t m = 1ull << (x & 63);
    const bool was_clear = !(w & m);
    w |= m;
    return was_clear;
  };
  for (int64_t j = n - count; j < n; ++j) {
    const int64_t t = rng.below((uint64_t)j + 1);
    if (!test_set(t)) test_set(j);
  }
  int32_t k = 0;
  for (size_t wi = 0; wi < bits.size(); ++wi)
    for (uint64_t w = bits[wi]; w; w &= w - 1) out[k++] = (int32_t)(wi * 64 + __builtin_ctzll(w));
}

}  // namespace svg
