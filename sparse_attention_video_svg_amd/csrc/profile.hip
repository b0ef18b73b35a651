// Profiling helpers: the position order of the sampled rows, and the merge of
// the profiling sweeps into per-head labels and statistics.
//
// Profiling (rebuttal: answer on when profiling happens; abstract: online
// prediction of each head's type) compares full attention with the spatial
// and the temporal mask on the sampled rows:
//   rel_m = sum (O_m - O_full)^2 / sum O_full^2   over rows x d,
//   label = SPATIAL if rel_s <= rel_t else TEMPORAL, FULL if min >= fallback.
// The sweeps leave per row and key slice three partial states (m in log2
// units, l, unnormalised acc): spatial, full and temporal.  Rows are merged in
// parallel, each row's three squared-error sums are written, and one
// workgroup per head adds them in a fixed order.
#include "svg_device.h"

namespace svg {

// Position order of the sampled rows (ascending, distinct video rows):
// rank = #rows with a smaller position j, plus #rows at the same position in
// earlier frames.  Each count is a binary search per frame.
__device__ __forceinline__ int lower_bound_rows(const int32_t* rows, int n, int key) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (rows[mid] < key)
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo;
}

__global__ void k_prof_rank(KGeom g, const int32_t* __restrict__ rows, int32_t n_rows, int32_t* __restrict__ ord_x,
                            int32_t* __restrict__ ord_r) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= n_rows) return;
  const int x = rows[r];
  const int u = x - g.T;
  const int i = fastdiv(u, g.divF_mul, g.divF_shift), j = u - i * g.F;
  int rank = 0;
  for (int f = 0; f < g.N; ++f) {
    const int fb = g.T + f * g.F;
    const int a = lower_bound_rows(rows, n_rows, fb);
    const int c = lower_bound_rows(rows, n_rows, fb + j);
    rank += c - a;
    if (f < i && c < n_rows && rows[c] == fb + j) ++rank;
  }
  ord_x[rank] = x;
  ord_r[rank] = r;
}

// One workgroup (D threads, one per dim) per (sampled row, head): each of
// the three states merged over the key slices, then normalised.
template <int D>
__global__ __launch_bounds__(D) void k_prof_merge_rows(int32_t n_rows, int32_t ksplit,
                                                       const float* __restrict__ part_acc,
                                                       const float* __restrict__ part_ml,
                                                       double* __restrict__ row_sums) {
  const int r = blockIdx.x, bh = blockIdx.y, c = threadIdx.x;
  const int64_t row = (int64_t)bh * n_rows + r;
  float o[3];
#pragma unroll
  for (int st = 0; st < 3; ++st) {
    float m = -INFINITY;
    for (int s = 0; s < ksplit; ++s) m = fmaxf(m, part_ml[((row * ksplit + s) * 3 + st) * 2]);
    float l = 0.f, a = 0.f;
    if (m != -INFINITY) {
      for (int s = 0; s < ksplit; ++s) {
        const int64_t slot = (row * ksplit + s) * 3 + st;
        const float w = exp2f(part_ml[slot * 2] - m);
        l += w * part_ml[slot * 2 + 1];
        a += w * part_acc[slot * D + c];
      }
    }
    o[st] = l > 0.f ? a / l : 0.f;
  }
  const float o_sp = o[0], o_f = o[1], o_tp = o[2];
  const double ds = (double)o_sp - (double)o_f, dt = (double)o_tp - (double)o_f;
  __shared__ double red[3][D];
  red[0][c] = ds * ds;
  red[1][c] = dt * dt;
  red[2][c] = (double)o_f * (double)o_f;
  __syncthreads();
  for (int w = D / 2; w > 0; w >>= 1) {
    if (c < w) {
#pragma unroll
      for (int k = 0; k < 3; ++k) red[k][c] += red[k][c + w];
    }
    __syncthreads();
  }
  if (c < 3) row_sums[row * 3 + c] = red[c][0];
}

__global__ __launch_bounds__(256) void k_prof_finalize(int32_t d, int32_t n_rows, const double* __restrict__ row_sums,
                                                       float fallback, int32_t* __restrict__ labels,
                                                       float* __restrict__ stats) {
  const int bh = blockIdx.x, t = threadIdx.x;
  double acc[3] = {0.0, 0.0, 0.0};
  for (int r = t; r < n_rows; r += 256)
#pragma unroll
    for (int k = 0; k < 3; ++k) acc[k] += row_sums[((int64_t)bh * n_rows + r) * 3 + k];
  __shared__ double red[3][256];
#pragma unroll
  for (int k = 0; k < 3; ++k) red[k][t] = acc[k];
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (t < w) {
#pragma unroll
      for (int k = 0; k < 3; ++k) red[k][t] += red[k][t + w];
    }
    __syncthreads();
  }
  if (t == 0) {
    const double den = red[2][0];
    const double rs = den > 0.0 ? red[0][0] / den : INFINITY;
    const double rt = den > 0.0 ? red[1][0] / den : INFINITY;
    const double best = rs <= rt ? rs : rt;
    labels[bh] = best >= (double)fallback ? SVG_FULL : (rs <= rt ? SVG_SPATIAL : SVG_TEMPORAL);
    stats[bh * 3 + 0] = (float)rs;
    stats[bh * 3 + 1] = (float)rt;
    stats[bh * 3 + 2] = (float)(den / ((double)n_rows * d));
  }
}

hipError_t launch_profile_rank(const KGeom& g, const int32_t* rows, int32_t n_rows, int32_t* ord_x, int32_t* ord_r,
                               hipStream_t st) {
  hipLaunchKernelGGL(k_prof_rank, dim3((unsigned)((n_rows + 255) / 256)), dim3(256), 0, st, g, rows, n_rows, ord_x,
                     ord_r);
  return hipGetLastError();
}

hipError_t launch_profile_merge(const KGeom& g, int32_t n_rows, int32_t ksplit, const float* part_acc,
                                const float* part_ml, double* row_sums, float fallback, int32_t* labels, float* stats,
                                hipStream_t st) {
  dim3 grid((unsigned)n_rows, (unsigned)(g.B * g.H));
  if (g.d == 64)
    hipLaunchKernelGGL(k_prof_merge_rows<64>, grid, dim3(64), 0, st, n_rows, ksplit, part_acc, part_ml, row_sums);
  else
    hipLaunchKernelGGL(k_prof_merge_rows<128>, grid, dim3(128), 0, st, n_rows, ksplit, part_acc, part_ml, row_sums);
  hipLaunchKernelGGL(k_prof_finalize, dim3((unsigned)(g.B * g.H)), dim3(256), 0, st, g.d, n_rows, row_sums, fallback,
                     labels, stats);
  return hipGetLastError();
}

}  // namespace svg
