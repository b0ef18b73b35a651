// fp32 path: masked attention and the profiling sweep for float32 inputs and
// outputs (the small exactness workload).  One wave per query row; lanes own
// one key each while scoring a 64-key tile and own dims c, c+64 while
// accumulating.  Dot products, the softmax and the accumulators are carried in
// double precision (cheap at this size on MI355X), so the float32 result is
// the exact softmax attention up to its final rounding.
#include "svg_device.h"

namespace svg {

__device__ __forceinline__ double wave_max_d(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmax(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Key active for query row x in the working layout: text key, or in [lo, hi).
__device__ __forceinline__ bool key_active(const KGeom& g, int key, int lo, int hi) {
  return key < g.L && (key < g.T || (key >= lo && key < hi));
}

template <int D>
__global__ __launch_bounds__(64) void k_attn_f32(KGeom g, AttnPtrs a, int32_t BM, int32_t BN, int32_t nQT) {
  static_assert(D == 64 || D == 128, "head dim");
  __shared__ float qs[D];
  __shared__ double ps[64];
  const int lane = threadIdx.x;
  const int bh = blockIdx.y;
  const int x = blockIdx.x;  // row in the head's working layout
  const int b = bh / g.H, h = bh % g.H;
  const int mode = a.modes[bh];
  const bool temporal = (mode == SVG_TEMPORAL);
  const bool virt = temporal && (a.flags & SVG_FLAG_VIRTUAL_PERMUTE);
  // temporal heads: K, V from their token-major copies (or through the index
  // map), Q and O from / to their copies when given, else through the map
  const bool use_p = temporal && !virt;
  const bool q_p = use_p && a.qp != nullptr, o_p = use_p && a.op != nullptr;
  const svg_strides skv = use_p ? a.sp : a.s, sq = q_p ? a.sp : a.s, sout = o_p ? a.sop : a.so;
  const float* Q = static_cast<const float*>(q_p ? a.qp : a.q) + (int64_t)b * sq.b + (int64_t)h * sq.h;
  const float* K = static_cast<const float*>(use_p ? a.kp : a.k) + (int64_t)b * skv.b + (int64_t)h * skv.h;
  const float* V = static_cast<const float*>(use_p ? a.vp : a.v) + (int64_t)b * skv.b + (int64_t)h * skv.h;
  float* O = static_cast<float*>(o_p ? a.op : a.o) + (int64_t)b * sout.b + (int64_t)h * sout.h;
  auto phys = [&](int r) { return virt ? perm_inv_row(g, r) : r; };                      // K, V rows
  auto qrow = [&](int r) { return temporal && !q_p ? perm_inv_row(g, r) : r; };
  const int64_t orow = (int64_t)(temporal && !o_p ? perm_inv_row(g, x) : x) * sout.x;
  if (mode == SVG_SKIP) {
    for (int c = lane; c < D; c += 64) O[orow + c] = 0.f;
    return;
  }
  for (int c = lane; c < D; c += 64) qs[c] = Q[(int64_t)qrow(x) * sq.x + c];
  __syncthreads();
  int lo, hi;
  row_interval(g, mode, x, lo, hi);
  const int qt = x / BM;
  const int4 rg = reinterpret_cast<const int4*>(a.ranges)[(int64_t)bh * nQT + qt];
  double m = -INFINITY, l = 0.0;
  double acc0 = 0.0, acc1 = 0.0;
  const int n1 = rg.y - rg.x, nt = n1 + (rg.w - rg.z);
  for (int t = 0; t < nt; ++t) {
    const int kt = t < n1 ? rg.x + t : rg.z + (t - n1);
    const int key = kt * BN + lane;
    const bool act = key_active(g, key, lo, hi);
    double s = -INFINITY;
    if (act) {
      const float* kr = K + (int64_t)phys(key) * skv.x;
      double dot = 0.0;
      for (int c = 0; c < D; ++c) dot = fma((double)qs[c], (double)kr[c], dot);
      s = dot * (double)g.scale;
    }
    const double mt = wave_max_d(s);
    const double mn = fmax(m, mt);
    if (mn == -INFINITY) continue;  // nothing active yet (wave-uniform)
    const double alpha = exp(m - mn);
    const double p = act ? exp(s - mn) : 0.0;
    l = l * alpha + wave_sum_d(p);
    m = mn;
    ps[lane] = p;
    __syncthreads();
    acc0 *= alpha;
    acc1 *= alpha;
    const int kb = kt * BN;
    for (int e = 0; e < 64; ++e) {
      const double pe = ps[e];
      if (pe != 0.0) {
        const float* vr = V + (int64_t)phys(kb + e) * skv.x;
        acc0 = fma(pe, (double)vr[lane], acc0);
        if (D == 128) acc1 = fma(pe, (double)vr[lane + 64], acc1);
      }
    }
    __syncthreads();
  }
  const double inv = l > 0.0 ? 1.0 / l : 0.0;
  O[orow + lane] = (float)(acc0 * inv);
  if (D == 128) O[orow + lane + 64] = (float)(acc1 * inv);
}

// Profiling sweep, fp32: one wave per (head, sampled row), three online
// softmax states (full, spatial, temporal mod form on frame-major indices)
// over every key; writes the partial (m, l, acc) of each state (one split).
template <int D>
__global__ __launch_bounds__(64) void k_profile_f32(KGeom g, const float* __restrict__ q,
                                                    const float* __restrict__ k, const float* __restrict__ v,
                                                    svg_strides s, const int32_t* __restrict__ rows,
                                                    int32_t n_rows, float* __restrict__ part_acc,
                                                    float* __restrict__ part_ml) {
  __shared__ float qs[D];
  __shared__ double ps[3][64];
  const int lane = threadIdx.x;
  const int bh = blockIdx.y, r = blockIdx.x;
  const int b = bh / g.H, h = bh % g.H;
  const int64_t base = (int64_t)b * s.b + (int64_t)h * s.h;
  const int x = sampled_row(g, rows[r]);
  for (int c = lane; c < D; c += 64) qs[c] = q[base + (int64_t)x * s.x + c];
  __syncthreads();
  // spatial run of frames and temporal band of positions of this row
  const int u = x - g.T;
  const int fi = u / g.F, fj = u % g.F;
  const int slo = g.T + max(0, fi - g.a1 + 1) * g.F, shi = g.T + min(g.N, fi + g.a1) * g.F;
  double m[3] = {-INFINITY, -INFINITY, -INFINITY}, l[3] = {0.0, 0.0, 0.0};
  double acc0[3] = {0.0, 0.0, 0.0}, acc1[3] = {0.0, 0.0, 0.0};
  const int nKT = (g.L + 63) / 64;
  for (int kt = 0; kt < nKT; ++kt) {
    const int key = kt * 64 + lane;
    const bool valid = key < g.L;
    double sc = -INFINITY;
    bool act[3] = {false, false, false};
    if (valid) {
      const float* kr = k + base + (int64_t)key * s.x;
      double dot = 0.0;
      for (int c = 0; c < D; ++c) dot = fma((double)qs[c], (double)kr[c], dot);
      sc = dot * (double)g.scale;
      const bool text = key < g.T;
      act[0] = true;
      act[1] = text || (key >= slo && key < shi);
      const int kj = text ? 0 : (key - g.T) % g.F;
      act[2] = text || abs(kj - fj) < g.a2;
    }
    double alpha[3];
#pragma unroll
    for (int st = 0; st < 3; ++st) {
      const double sv = act[st] ? sc : -INFINITY;
      const double mn = fmax(m[st], wave_max_d(sv));
      if (mn == -INFINITY) {
        alpha[st] = 1.0;
        ps[st][lane] = 0.0;
        continue;
      }
      alpha[st] = exp(m[st] - mn);
      const double p = act[st] ? exp(sv - mn) : 0.0;
      l[st] = l[st] * alpha[st] + wave_sum_d(p);
      m[st] = mn;
      ps[st][lane] = p;
    }
    __syncthreads();
#pragma unroll
    for (int st = 0; st < 3; ++st) {
      acc0[st] *= alpha[st];
      acc1[st] *= alpha[st];
    }
    for (int e = 0; e < 64; ++e) {
      const int kk = kt * 64 + e;
      if (kk >= g.L) break;
      const float* vr = v + base + (int64_t)kk * s.x;
      const double v0 = vr[lane], v1 = (D == 128) ? vr[lane + 64] : 0.0;
#pragma unroll
      for (int st = 0; st < 3; ++st) {
        const double pe = ps[st][e];
        acc0[st] = fma(pe, v0, acc0[st]);
        acc1[st] = fma(pe, v1, acc1[st]);
      }
    }
    __syncthreads();
  }
  // Outputs already normalised (l = 1, m = 0), one key slice: state 0 the
  // spatial, 1 the full, 2 the temporal output.
  const int64_t row = (int64_t)bh * n_rows + r;
  float* dst_acc[3] = {part_acc + (row * 3 + 0) * D, part_acc + (row * 3 + 1) * D, part_acc + (row * 3 + 2) * D};
  float* dst_ml[3] = {part_ml + (row * 3 + 0) * 2, part_ml + (row * 3 + 1) * 2, part_ml + (row * 3 + 2) * 2};
  const int which[3] = {1, 0, 2};  // destination of full, spatial, temporal
#pragma unroll
  for (int st = 0; st < 3; ++st) {
    const double inv = l[st] > 0.0 ? 1.0 / l[st] : 0.0;
    float* acc = dst_acc[which[st]];
    acc[lane] = (float)(acc0[st] * inv);
    if (D == 128) acc[lane + 64] = (float)(acc1[st] * inv);
    if (lane == 0) {
      dst_ml[which[st]][0] = 0.f;
      dst_ml[which[st]][1] = l[st] > 0.0 ? 1.f : 0.f;
    }
  }
}

hipError_t launch_attention_f32(const KGeom& g, const AttnPtrs& a, int32_t BM, int32_t BN, hipStream_t st) {
  const int32_t nQT = (g.L + BM - 1) / BM;
  dim3 grid((unsigned)g.L, (unsigned)(g.B * g.H));
  if (g.d == 64)
    hipLaunchKernelGGL(k_attn_f32<64>, grid, dim3(64), 0, st, g, a, BM, BN, nQT);
  else
    hipLaunchKernelGGL(k_attn_f32<128>, grid, dim3(64), 0, st, g, a, BM, BN, nQT);
  return hipGetLastError();
}

hipError_t launch_profile_f32(const KGeom& g, const void* q, const void* k, const void* v, svg_strides s,
                              const int32_t* rows, int32_t n_rows, float* part_acc, float* part_ml,
                              hipStream_t st) {
  dim3 grid((unsigned)n_rows, (unsigned)(g.B * g.H));
  const float *fq = static_cast<const float*>(q), *fk = static_cast<const float*>(k),
              *fv = static_cast<const float*>(v);
  if (g.d == 64)
    hipLaunchKernelGGL(k_profile_f32<64>, grid, dim3(64), 0, st, g, fq, fk, fv, s, rows, n_rows, part_acc,
                       part_ml);
  else
    hipLaunchKernelGGL(k_profile_f32<128>, grid, dim3(64), 0, st, g, fq, fk, fv, s, rows, n_rows, part_acc,
                       part_ml);
  return hipGetLastError();
}

}  // namespace svg
