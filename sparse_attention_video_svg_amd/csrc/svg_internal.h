// Internal declarations shared by the host-side API and the kernel files of
// libsvg.so.  Not part of the public ABI (that is include/svg.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "svg.h"
#include "svg_sched.h"
#include <atomic>

namespace svg {

// Geometry as the kernels see it (passed by value).
struct KGeom {
  int32_t B, H, d, N, F, T, a1, a2, window, stripe;
  int32_t L;          // T + N*F
  float scale;        // softmax scale
  float scale_log2;   // scale * log2(e)
  // invariant-divisor constants for x/N and x/F (see FastDiv)
  uint32_t divN_mul, divN_shift, divF_mul, divF_shift;
  int32_t nxcd;       // XCDs of the device the kernels run on (>= 1)
  int32_t ncu;        // its compute units
};

// Compute units and XCDs of the current device, read from the runtime once
// per device (a partitioned or CU-masked device reports its own share).
struct DevTopo {
  int32_t cus, xcds;
};
hipError_t device_topology(DevTopo* t);

// count distinct integers of [0, n), uniform without replacement, ascending
// (host; sample.cpp)
void sample_sorted(int64_t n, int32_t count, uint64_t seed, int32_t* out);

// Division of a non-negative int32 by an invariant positive divisor with one
// multiply-high, after Granlund and Montgomery, "Division by invariant
// integers using multiplication" (PLDI 1994): with s = ceil(log2 dv) and
// m = floor(2^32 (2^s - dv) / dv) + 1, n / dv = (mulhi(n, m) + n) >> s for
// 0 <= n < 2^31.
inline void fastdiv_init(uint32_t dv, uint32_t* mul, uint32_t* shift) {
  uint32_t s = 0;
  while ((1ull << s) < dv) ++s;
  uint64_t m = ((1ull << 32) * ((1ull << s) - dv)) / dv + 1;
  *mul = (uint32_t)m;
  *shift = s;
}

__device__ __forceinline__ int32_t fastdiv(int32_t n, uint32_t mul, uint32_t shift) {
  uint32_t hi = __umulhi((uint32_t)n, mul);
  return (int32_t)((hi + (uint32_t)n) >> shift);
}

// Workspace carve-up for svg_layer_forward / svg_profile_heads.
struct WsLayout {
  size_t part_acc, part_ml, row_sums, ord_x, ord_r;  // profiling
  size_t labels, ranges, order, perm, total;
  size_t q8, k8, sq, sk;     // fp8-score path: quantised Q, K and their scales
  size_t v8, svh;            // fp8 P.V: quantised V tiles and per-head scales
  size_t perm_tensor_bytes;  // one permuted tensor (all heads)
  int32_t ksplit;            // key slices the profiling partials are laid out for
};

// Launchers (each returns hipGetLastError() after its launches).
hipError_t launch_build_blocks(const KGeom& g, const int32_t* modes, int32_t BM, int32_t BN,
                               int32_t* ranges, int32_t* head_order, hipStream_t st);
hipError_t launch_permute(const KGeom& g, int elt_bytes, const void* src, svg_strides ss, void* dst,
                          svg_strides ds, const int32_t* modes, int inverse, hipStream_t st);

// Raises a kernel's dynamic-LDS limit on the current device the first time
// it is launched there.  The attribute is per device, so the caller keeps one
// flag word per kernel (bit = device id < 64); concurrent first calls just
// set the attribute twice.
inline hipError_t ensure_dynamic_lds(const void* kern, size_t bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t{1} << dev) : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
  return e;
}

struct AttnPtrs {
  const void *q, *k, *v, *qp, *kp, *vp;
  void *o, *op;
  svg_strides s, sp, so, sop;
  const int32_t *modes, *ranges, *order;
  int32_t flags;
};
hipError_t launch_attention_f32(const KGeom& g, const AttnPtrs& a, int32_t BM, int32_t BN, hipStream_t st);
hipError_t launch_attention_bf16(const KGeom& g, const AttnPtrs& a, bool out_bf16, hipStream_t st);

// FP8-score attention: quantisation of Q (per row) and K (per 64-key tile of
// the working layout) to E4M3 with power-of-two scales, and the attention
// kernel that takes them (TEMPORAL heads: Q8, V, O through the index map, K8
// already token-major).  q8 / k8: [B*H, L, d] bytes; sq: [B*H, L];
// sk: [B*H, ceil(L / 64)].
hipError_t launch_quant_qk(const KGeom& g, const void* q, const void* k, svg_strides s, const int32_t* modes,
                           uint8_t* q8, float* sq, uint8_t* k8, float* sk, hipStream_t st);
hipError_t launch_attention_fp8(const KGeom& g, const uint8_t* q8, const float* sq, const uint8_t* k8,
                                const float* sk, const void* v, svg_strides sv, void* o, svg_strides so,
                                bool out_bf16, const int32_t* modes, const int32_t* ranges, const int32_t* order,
                                hipStream_t st);
// FP8 P.V: V to E4M3 with one power-of-two scale per head, stored per 64-key
// tile of the working layout, transposed (v8: [B*H, ceil(L/64), d, 64]
// bytes in P-register key order; svh: [B*H] scales), and the attention kernel
// that takes Q8/K8 and V8 (scores and P.V on the FP8 matrix cores).
hipError_t launch_quant_v(const KGeom& g, const void* v, svg_strides s, const int32_t* modes, uint8_t* v8,
                          float* svh, hipStream_t st);
hipError_t launch_attention_fp8pv(const KGeom& g, const uint8_t* q8, const float* sq, const uint8_t* k8,
                                  const float* sk, const uint8_t* v8, const float* svh, void* o, svg_strides so,
                                  bool out_bf16, const int32_t* modes, const int32_t* ranges, const int32_t* order,
                                  hipStream_t st);

// SVG2 (semantic-aware permutation): k-means of one tensor per head
// (`iters` Lloyd iterations from the centroids in mu, which are updated in
// place), the stable cluster order (perm, start), the centroid-score top-p
// selection with tile lists, the gather of K / V into cluster order, and the
// attention over query clusters.  Scratch of the k-means:
struct Svg2Scratch {
  void *hi, *lo;          // bf16 [BH][C][d]: centroid and its residual
  float* hn;              // [BH][C]: 0.5 |mu|^2
  int32_t *hist, *base;   // [BH][ceil(L/256)][C]
  int32_t* rank;          // [BH][L]
};
constexpr int32_t kSvg2MaxClusters = 1024;
hipError_t launch_km_init(const KGeom& g, const void* x, svg_strides s, int32_t C, float* mu, hipStream_t st);
hipError_t launch_kmeans(const KGeom& g, const void* x, svg_strides s, int32_t C, int32_t iters, float* mu,
                         int32_t* labels, int32_t* perm, int32_t* start, const Svg2Scratch& w, hipStream_t st);
hipError_t launch_svg2_select(const KGeom& g, int32_t Cq, int32_t Ck, float p, const float* mu_q, const float* mu_k,
                              const int32_t* start_q, const int32_t* start_k, uint8_t* sel, void* segs,
                              int32_t* nseg, int32_t* nkeys, int32_t* ord, int32_t* rb_prefix, hipStream_t st);
hipError_t launch_gather_rows(const KGeom& g, const void* src, svg_strides s, const int32_t* perm, void* dst,
                              hipStream_t st);
hipError_t launch_svg2_attention(const KGeom& g, const void* q, svg_strides s, const void* kp, const void* vp, void* o,
                                 svg_strides so, bool out_bf16, const int32_t* perm_q, const int32_t* start_q,
                                 const int32_t* ord, const int32_t* rb_prefix, const void* segs, const int32_t* nseg,
                                 const int32_t* nkeys, int32_t Cq, int32_t Ck, hipStream_t st);

// Sampled-row sweeps (profiling, mode search): per (head, row, key slice)
// one partial online-softmax state (m in log2 units, l, unnormalised acc) per
// mask, at slot ((bh * n_rows + row) * ksplit + slice) * nstates + state.
// Profiling: nstates 3 = spatial, full, temporal.  Mode search: nstates 4 =
// full, window, temporal band, stripe.  The merges reduce them,
// deterministically, into labels / modes and stats.
struct SearchParams {
  float lam, eps;
  int32_t penalty;     // 0: lam * (1 - S), 1: lam * S
  float sparsity[4];   // S of skip, window, temporal, stripe
};
hipError_t launch_profile_rank(const KGeom& g, const int32_t* rows, int32_t n_rows, int32_t* ord_x, int32_t* ord_r,
                               hipStream_t st);
hipError_t launch_profile_f32(const KGeom& g, const void* q, const void* k, const void* v, svg_strides s,
                              const int32_t* rows, int32_t n_rows, float* part_acc, float* part_ml, hipStream_t st);
// bf16: one sweep per entry of modes[nstates] (state i = modes[i]; TEMPORAL
// is the band through the index map, rows in position order ord_x / ord_r).
hipError_t launch_sample_sweeps(const KGeom& g, const void* q, const void* k, const void* v, svg_strides s,
                                const int32_t* rows, int32_t n_rows, int32_t ksplit, const int32_t* ord_x,
                                const int32_t* ord_r, const int32_t* modes, int32_t nstates, float* part_acc,
                                float* part_ml, hipStream_t st);
hipError_t launch_profile_merge(const KGeom& g, int32_t n_rows, int32_t ksplit, const float* part_acc,
                                const float* part_ml, double* row_sums, float fallback, int32_t* labels, float* stats,
                                hipStream_t st);
hipError_t launch_search_merge(const KGeom& g, int32_t n_rows, int32_t ksplit, const float* part_acc,
                               const float* part_ml, double* row_sums, const SearchParams& p, int32_t* modes,
                               float* stats, hipStream_t st);

// Tile sizes of the bf16 MFMA attention kernel (32 query rows per wave, a
// ring of kAttnStages K/V tiles of 64 keys in LDS) and of the fp32 kernel.
constexpr int32_t kAttnWaves = 8, kAttnStages = 2;
constexpr int32_t kBM_bf16 = 32 * kAttnWaves, kBN_bf16 = 64;
constexpr int32_t kBM_f32 = 64, kBN_f32 = 64;
// Query rows per workgroup of the bf16 profiling sweeps.
constexpr int32_t kProfRows_bf16 = kBM_bf16;

// Fixed device scratch of svg_layer_forward_noalloc (one array per device,
// held until the process ends) and its device address on the current device
// (taken with hipGetSymbolAddress on the first call there).
constexpr size_t kStaticScratchBytes = size_t{64} << 20;
hipError_t static_scratch(void** ptr);

}  // namespace svg
