// Merge of the profiling sweeps into per-head labels and statistics.
//
// Profiling (rebuttal: answer on when profiling happens; abstract: online
// prediction of each head's type) compares full attention with the spatial
// and the temporal mask on the sampled rows:
//   rel_m = sum (O_m - O_full)^2 / sum O_full^2   over rows x d,
//   label = SPATIAL if rel_s <= rel_t else TEMPORAL, FULL if min >= fallback.
// One workgroup per head reduces the split partials (m in log2 units, l,
// unnormalised acc) of every sampled row, in a fixed order, in fp64.
#include "svg_device.h"

namespace svg {

__global__ __launch_bounds__(256) void k_profile_merge(int32_t d, int32_t n_rows, int32_t ksplit,
                                                       const float* __restrict__ part_acc,
                                                       const float* __restrict__ part_ml, float fallback,
                                                       int32_t* __restrict__ labels, float* __restrict__ stats) {
  const int bh = blockIdx.x;
  const int t = threadIdx.x;
  double ss = 0.0, st = 0.0, sf = 0.0;
  const int64_t n_el = (int64_t)n_rows * d;
  for (int64_t e = t; e < n_el; e += 256) {
    const int r = (int)(e / d), c = (int)(e % d);
    float o[3];
#pragma unroll
    for (int s3 = 0; s3 < 3; ++s3) {
      float mx = -INFINITY;
      for (int k = 0; k < ksplit; ++k) {
        const int64_t slot = (((int64_t)bh * n_rows + r) * ksplit + k) * 3 + s3;
        mx = fmaxf(mx, part_ml[slot * 2]);
      }
      float l = 0.f, acc = 0.f;
      if (mx != -INFINITY) {
        for (int k = 0; k < ksplit; ++k) {
          const int64_t slot = (((int64_t)bh * n_rows + r) * ksplit + k) * 3 + s3;
          const float w = exp2f(part_ml[slot * 2] - mx);
          l += w * part_ml[slot * 2 + 1];
          acc += w * part_acc[slot * d + c];
        }
      }
      o[s3] = l > 0.f ? acc / l : 0.f;
    }
    const double a = (double)o[1] - (double)o[0], b = (double)o[2] - (double)o[0];
    ss += a * a;
    st += b * b;
    sf += (double)o[0] * (double)o[0];
  }
  __shared__ double red[3][256];
  red[0][t] = ss;
  red[1][t] = st;
  red[2][t] = sf;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (t < w) {
      red[0][t] += red[0][t + w];
      red[1][t] += red[1][t + w];
      red[2][t] += red[2][t + w];
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
    stats[bh * 3 + 2] = (float)(den / (double)n_el);
  }
}

hipError_t launch_profile_merge(const KGeom& g, int32_t n_rows, int32_t ksplit, const float* part_acc,
                                const float* part_ml, float fallback, int32_t* labels, float* stats,
                                hipStream_t st) {
  hipLaunchKernelGGL(k_profile_merge, dim3((unsigned)(g.B * g.H)), dim3(256), 0, st, g.d, n_rows, ksplit,
                     part_acc, part_ml, fallback, labels, stats);
  return hipGetLastError();
}

}  // namespace svg
