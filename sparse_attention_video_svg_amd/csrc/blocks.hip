// svg_build_blocks: per-(head, query tile) key-tile ranges and the
// longest-first head order.
//
// The spatial map is block-banded and, after the layout transformation, the
// temporal map is too (rebuttal answer to Weakness 1; abstract of "Sparse
// VideoGen").  Every mode's active keys for one row are [0, T) plus one
// contiguous run whose ends never decrease with the row, so the tiles a
// query tile touches are at most two ranges: the text tiles, and the tiles
// between the first row's run start and the last row's run end.
#include "svg_device.h"

namespace svg {

__global__ void k_build_ranges(KGeom g, const int32_t* __restrict__ modes, int32_t BM, int32_t BN,
                               int32_t nQT, int32_t* __restrict__ ranges) {
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)g.B * g.H * nQT;
  if (id >= total) return;
  const int bh = (int)(id / nQT), qt = (int)(id % nQT);
  const int mode = modes[bh];
  int4 r = make_int4(0, 0, 0, 0);
  const int nKT = (g.L + BN - 1) / BN;
  if (mode != SVG_SKIP) {
    const int r0 = qt * BM;
    const int r1 = min(g.L, r0 + BM);  // exclusive
    if (r0 < g.T) {
      r = make_int4(0, nKT, 0, 0);
    } else {
      int lo0, hi0, lo1, hi1;
      row_interval(g, mode, r0, lo0, hi0);
      row_interval(g, mode, r1 - 1, lo1, hi1);
      const int bs = lo0 / BN, be = (hi1 + BN - 1) / BN;
      const int te = (g.T + BN - 1) / BN;
      if (g.T == 0)
        r = make_int4(bs, be, 0, 0);
      else if (te >= bs)
        r = make_int4(0, max(be, te), 0, 0);
      else
        r = make_int4(0, te, bs, be);
    }
  }
  reinterpret_cast<int4*>(ranges)[id] = r;
}

// One workgroup: work of each head = listed tiles summed over its query
// tiles (one wave per head, integer sums); order = heads by descending work,
// ties by ascending index.
constexpr int kOrderThreads = 1024;

__global__ __launch_bounds__(kOrderThreads) void k_head_order(int32_t BH, int32_t nQT,
                                                              const int32_t* __restrict__ ranges,
                                                              int32_t* __restrict__ order) {
  extern __shared__ long long work[];  // BH entries
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  for (int h = wave; h < BH; h += kOrderThreads / 64) {
    long long s = 0;
    for (int qt = lane; qt < nQT; qt += 64) {
      const int4 r = reinterpret_cast<const int4*>(ranges)[(int64_t)h * nQT + qt];
      s += (r.y - r.x) + (r.w - r.z);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
    if (lane == 0) work[h] = s;
  }
  __syncthreads();
  for (int h = t; h < BH; h += kOrderThreads) {
    int rank = 0;
    const long long wh = work[h];
    for (int o = 0; o < BH; ++o) rank += (work[o] > wh) || (work[o] == wh && o < h);
    order[rank] = h;
  }
}

hipError_t launch_build_blocks(const KGeom& g, const int32_t* modes, int32_t BM, int32_t BN,
                               int32_t* ranges, int32_t* head_order, hipStream_t st) {
  const int32_t nQT = (g.L + BM - 1) / BM;
  const int64_t total = (int64_t)g.B * g.H * nQT;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  hipLaunchKernelGGL(k_build_ranges, dim3((unsigned)blocks), dim3(threads), 0, st, g, modes, BM, BN, nQT,
                     ranges);
  const int32_t BH = g.B * g.H;
  hipLaunchKernelGGL(k_head_order, dim3(1), dim3(kOrderThreads), sizeof(long long) * BH, st, BH, nQT, ranges,
                     head_order);
  return hipGetLastError();
}

}  // namespace svg
