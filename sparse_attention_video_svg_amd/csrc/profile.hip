// Profiling helpers: the position order of the sampled rows, and the merge of
// the profiling sweeps into per-head labels and statistics.
//
// Profiling (rebuttal: answer on when profiling happens; abstract: online
// prediction of each head's type) compares full attention with the spatial
// and the temporal mask on the sampled rows:
//   rel_m = sum (O_m - O_full)^2 / sum O_full^2   over rows x d,
//   label = SPATIAL if rel_s <= rel_t else TEMPORAL, FULL if min >= fallback.
// The mode search (Sparse-vDiT review: offline search scoring each candidate
// mode by its MSE against full attention plus a sparsity penalty, full
// attention kept when every candidate exceeds the threshold) reuses the same
// sweeps with the window, temporal-band and stripe masks.
// The sweeps leave per row and key slice one partial state per mask (m in
// log2 units, l, unnormalised acc): for profiling spatial, full and temporal,
// for the mode search full, window, temporal band and stripe.  Rows are merged
// in parallel, each row's squared-error sums are written, and one workgroup
// per head adds them in a fixed order.
#include "svg_device.h"

namespace svg {

// Position order of the sampled rows (ascending, distinct video rows): the
// key of row x = T + i*F + j is its token-major index j*N + i, and its rank
// is the number of rows with a smaller key (keys are distinct).  Rows are
// clamped into [T, L) as read, and ranks stay in [0, n_rows) whatever the
// list holds, so a list that breaks the contract is never a memory error.
// k_prof_rank_lds: all keys staged in LDS, four lanes per row each count
// over a quarter of them.
// k_prof_rank (more rows than fit): per frame, a binary search for the
// rows at smaller positions, plus the row at the same position if its
// frame comes earlier.
constexpr int kRankLdsRows = 8192;

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

__global__ __launch_bounds__(256) void k_prof_rank_lds(KGeom g, const int32_t* __restrict__ rows, int32_t n_rows,
                                                        int32_t* __restrict__ ord_x, int32_t* __restrict__ ord_r) {
  __shared__ __attribute__((aligned(16))) int32_t keys[kRankLdsRows];
  const int n4 = (n_rows + 3) & ~3;
  for (int r = threadIdx.x; r < n4; r += blockDim.x) {
    int key = INT_MAX;
    if (r < n_rows) {
      const int u = sampled_row(g, rows[r]) - g.T;
      const int i = fastdiv(u, g.divF_mul, g.divF_shift);
      key = (u - i * g.F) * g.N + i;
    }
    keys[r] = key;
  }
  __syncthreads();
  const int gt = blockIdx.x * blockDim.x + threadIdx.x;
  const int r = gt >> 2, q = gt & 3;  // row, quarter of the keys
  const bool ok = r < n_rows;
  const int own = ok ? keys[r] : 0;
  int rank = 0;
  // equal keys (a repeated row) are ranked by their index, so the ranks are
  // a permutation of [0, n_rows) for any list
  if (ok)
    for (int o = 4 * q; o < n4; o += 16) {
      const int4 k4 = *reinterpret_cast<const int4*>(keys + o);
      rank += (k4.x < own || (k4.x == own && o < r)) + (k4.y < own || (k4.y == own && o + 1 < r)) +
              (k4.z < own || (k4.z == own && o + 2 < r)) + (k4.w < own || (k4.w == own && o + 3 < r));
    }
  rank += __shfl_xor(rank, 1);
  rank += __shfl_xor(rank, 2);
  if (ok && q == 0) {
    ord_x[rank] = sampled_row(g, rows[r]);
    ord_r[rank] = r;
  }
}

__global__ void k_prof_rank(KGeom g, const int32_t* __restrict__ rows, int32_t n_rows, int32_t* __restrict__ ord_x,
                            int32_t* __restrict__ ord_r) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= n_rows) return;
  const int x = sampled_row(g, rows[r]);
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
  rank = min(max(rank, 0), n_rows - 1);  // (exact for a valid list)
  ord_x[rank] = x;
  ord_r[rank] = r;
}

// One wave per (sampled row, head), D/64 dims per lane: each of the nstates
// states merged over the key slices and normalised, then the row's sums
// over d: sum O_ref^2 at index ref, sum (O_s - O_ref)^2 at every other index
// s.  The (m, l) pairs are wave-uniform loads; each sum over d is the lane's
// dims in order, then a fixed butterfly over the lanes.
constexpr int kMaxStates = 4;
constexpr int kMergeWaves = 4;

template <int D>
__global__ __launch_bounds__(64 * kMergeWaves) void k_prof_merge_rows(int64_t total_rows, int32_t ksplit,
                                                                      int32_t nstates, int32_t ref,
                                                                      const float* __restrict__ part_acc,
                                                                      const float* __restrict__ part_ml,
                                                                      double* __restrict__ row_sums) {
  constexpr int kMaxSplit = 16;
  constexpr int PL = D / 64;  // dims per lane
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row = (int64_t)blockIdx.x * kMergeWaves + wave;  // bh * n_rows + r
  if (row >= total_rows) return;
  const float* ml = part_ml + row * ksplit * nstates * 2;
  float o[kMaxStates][PL];
#pragma unroll
  for (int st = 0; st < kMaxStates; ++st) {
#pragma unroll
    for (int p = 0; p < PL; ++p) o[st][p] = 0.f;
    if (st >= nstates) continue;
    float m = -INFINITY;
    for (int s = 0; s < ksplit; ++s) m = fmaxf(m, ml[(s * nstates + st) * 2]);
    if (m == -INFINITY) continue;
    // all slices' accumulator loads first (none for slices the row has no
    // key in: their acc is not written), then the sums in slice order
    float acc[kMaxSplit][PL];
#pragma unroll
    for (int s = 0; s < kMaxSplit; ++s) {
      const bool has = s < ksplit && ml[(s * nstates + st) * 2] != -INFINITY;
#pragma unroll
      for (int p = 0; p < PL; ++p)
        acc[s][p] = has ? part_acc[((row * ksplit + s) * nstates + st) * D + PL * lane + p] : 0.f;
    }
    float l = 0.f, a[PL];
#pragma unroll
    for (int p = 0; p < PL; ++p) a[p] = 0.f;
#pragma unroll
    for (int s = 0; s < kMaxSplit; ++s) {
      if (s < ksplit) {
        const float w = exp2f(ml[(s * nstates + st) * 2] - m);
        l += w * ml[(s * nstates + st) * 2 + 1];
#pragma unroll
        for (int p = 0; p < PL; ++p) a[p] += w * acc[s][p];
      }
    }
#pragma unroll
    for (int p = 0; p < PL; ++p) o[st][p] = l > 0.f ? a[p] / l : 0.f;
  }
  float o_ref[PL];
#pragma unroll
  for (int p = 0; p < PL; ++p) {
    o_ref[p] = o[0][p];
#pragma unroll
    for (int st = 1; st < kMaxStates; ++st) o_ref[p] = st == ref ? o[st][p] : o_ref[p];
  }
#pragma unroll
  for (int st = 0; st < kMaxStates; ++st) {
    if (st >= nstates) break;
    double sum = 0.0;
#pragma unroll
    for (int p = 0; p < PL; ++p) {
      const double dd = st == ref ? (double)o_ref[p] : (double)o[st][p] - (double)o_ref[p];
      sum += dd * dd;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
    if (lane == 0) row_sums[row * nstates + st] = sum;
  }
}

// Per-head fixed-order sums of the row sums (one workgroup per head).
template <int NS>
__device__ __forceinline__ void head_sums(int bh, int n_rows, const double* __restrict__ row_sums, double* out) {
  const int t = threadIdx.x;
  double acc[NS];
#pragma unroll
  for (int k = 0; k < NS; ++k) acc[k] = 0.0;
  for (int r = t; r < n_rows; r += 256)
#pragma unroll
    for (int k = 0; k < NS; ++k) acc[k] += row_sums[((int64_t)bh * n_rows + r) * NS + k];
  __shared__ double red[NS][256];
#pragma unroll
  for (int k = 0; k < NS; ++k) red[k][t] = acc[k];
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (t < w) {
#pragma unroll
      for (int k = 0; k < NS; ++k) red[k][t] += red[k][t + w];
    }
    __syncthreads();
  }
#pragma unroll
  for (int k = 0; k < NS; ++k) out[k] = red[k][0];
}

// Profiling labels: states 0 spatial, 1 full (reference), 2 temporal.
__global__ __launch_bounds__(256) void k_prof_finalize(int32_t d, int32_t n_rows, const double* __restrict__ row_sums,
                                                       float fallback, int32_t* __restrict__ labels,
                                                       float* __restrict__ stats) {
  const int bh = blockIdx.x;
  double sum[3];
  head_sums<3>(bh, n_rows, row_sums, sum);
  if (threadIdx.x == 0) {
    const double den = sum[1];
    const double rs = den > 0.0 ? sum[0] / den : INFINITY;
    const double rt = den > 0.0 ? sum[2] / den : INFINITY;
    const double best = rs <= rt ? rs : rt;
    labels[bh] = best >= (double)fallback ? SVG_FULL : (rs <= rt ? SVG_SPATIAL : SVG_TEMPORAL);
    stats[bh * 3 + 0] = (float)rs;
    stats[bh * 3 + 1] = (float)rt;
    stats[bh * 3 + 2] = (float)(den / ((double)n_rows * d));
  }
}

// Mode search: states 0 full (reference), 1 window, 2 temporal band, 3
// stripe; the skip candidate's error is the reference's own sum of squares.
// Candidates in the order skip, window, temporal, stripe (ties to the
// earlier); loss = mse + lam * (1 - S) or mse + lam * S; FULL when every
// loss exceeds eps.  stats[bh * 8]: mse[4] then loss[4].
__global__ __launch_bounds__(256) void k_search_finalize(int32_t d, int32_t n_rows, const double* __restrict__ row_sums,
                                                         SearchParams p, int32_t* __restrict__ modes,
                                                         float* __restrict__ stats) {
  const int bh = blockIdx.x;
  double sum[4];
  head_sums<4>(bh, n_rows, row_sums, sum);
  if (threadIdx.x == 0) {
    const double n = (double)n_rows * d;
    const int cand[4] = {SVG_SKIP, SVG_WINDOW, SVG_TEMPORAL, SVG_STRIPE};
    const double se[4] = {sum[0], sum[1], sum[2], sum[3]};
    int best = 0;
    double loss[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const double mse = se[c] / n;
      const double sp = (double)p.sparsity[c];
      loss[c] = mse + (p.penalty == 0 ? (double)p.lam * (1.0 - sp) : (double)p.lam * sp);
      if (loss[c] < loss[best]) best = c;
      stats[bh * 8 + c] = (float)mse;
      stats[bh * 8 + 4 + c] = (float)loss[c];
    }
    modes[bh] = loss[best] > (double)p.eps ? SVG_FULL : cand[best];
  }
}

hipError_t launch_profile_rank(const KGeom& g, const int32_t* rows, int32_t n_rows, int32_t* ord_x, int32_t* ord_r,
                               hipStream_t st) {
  if (n_rows <= kRankLdsRows)
    hipLaunchKernelGGL(k_prof_rank_lds, dim3((unsigned)((4 * n_rows + 255) / 256)), dim3(256), 0, st, g, rows, n_rows,
                       ord_x, ord_r);
  else
    hipLaunchKernelGGL(k_prof_rank, dim3((unsigned)((n_rows + 255) / 256)), dim3(256), 0, st, g, rows, n_rows, ord_x,
                       ord_r);
  return hipGetLastError();
}

hipError_t launch_prof_merge(const KGeom& g, int32_t n_rows, int32_t ksplit, int32_t nstates, int32_t ref,
                             const float* part_acc, const float* part_ml, double* row_sums, hipStream_t st) {
  if (nstates < 1 || nstates > kMaxStates) return hipErrorInvalidValue;
  if (ksplit < 1 || ksplit > 16) return hipErrorInvalidValue;
  const int64_t total = (int64_t)g.B * g.H * n_rows;
  const int64_t blocks = (total + kMergeWaves - 1) / kMergeWaves;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(64 * kMergeWaves);
  if (g.d == 64)
    hipLaunchKernelGGL(k_prof_merge_rows<64>, grid, block, 0, st, total, ksplit, nstates, ref, part_acc, part_ml,
                       row_sums);
  else
    hipLaunchKernelGGL(k_prof_merge_rows<128>, grid, block, 0, st, total, ksplit, nstates, ref, part_acc, part_ml,
                       row_sums);
  return hipGetLastError();
}

hipError_t launch_profile_merge(const KGeom& g, int32_t n_rows, int32_t ksplit, const float* part_acc,
                                const float* part_ml, double* row_sums, float fallback, int32_t* labels, float* stats,
                                hipStream_t st) {
  hipError_t e = launch_prof_merge(g, n_rows, ksplit, 3, 1, part_acc, part_ml, row_sums, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_prof_finalize, dim3((unsigned)(g.B * g.H)), dim3(256), 0, st, g.d, n_rows, row_sums, fallback,
                     labels, stats);
  return hipGetLastError();
}

hipError_t launch_search_merge(const KGeom& g, int32_t n_rows, int32_t ksplit, const float* part_acc,
                               const float* part_ml, double* row_sums, const SearchParams& p, int32_t* modes,
                               float* stats, hipStream_t st) {
  hipError_t e = launch_prof_merge(g, n_rows, ksplit, 4, 0, part_acc, part_ml, row_sums, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_search_finalize, dim3((unsigned)(g.B * g.H)), dim3(256), 0, st, g.d, n_rows, row_sums, p,
                     modes, stats);
  return hipGetLastError();
}

}  // namespace svg
