// C ABI of libsvg.so (declared in include/svg.h): argument validation,
// workspace layout and the order of launches of one attention layer.
//
// Every entry point validates all of its host-visible arguments before it
// makes any HIP call, so an invalid call enqueues nothing; this also makes the
// validation testable on a machine without a GPU.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <initializer_list>

#include "svg_internal.h"

using namespace svg;

namespace {

thread_local char g_err[512] = "";

svg_status fail(svg_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

svg_status hip_fail(hipError_t e, const char* where) {
  return fail(SVG_E_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr int64_t kMaxTokens = (int64_t)1 << 30;
constexpr int32_t kMaxHeads = 4096;

int elt_bytes(svg_dtype t) { return t == SVG_BF16 ? 2 : 4; }
bool dtype_ok(int t) { return t == SVG_F32 || t == SVG_BF16; }

svg_status check_geom(const svg_geom* geom, KGeom* out) {
  if (!geom) return fail(SVG_E_INVALID, "geom is NULL");
  const svg_geom& g = *geom;
  if (g.B < 1 || g.H < 1) return fail(SVG_E_INVALID, "B and H must be >= 1 (got %d, %d)", g.B, g.H);
  if ((int64_t)g.B * g.H > kMaxHeads) return fail(SVG_E_UNSUPPORTED, "B*H > %d", kMaxHeads);
  if (g.d != 64 && g.d != 128) return fail(SVG_E_UNSUPPORTED, "head dim d=%d (supported: 64, 128)", g.d);
  if (g.N < 1 || g.F < 1) return fail(SVG_E_INVALID, "N and F must be >= 1 (got %d, %d)", g.N, g.F);
  if (g.T < 0) return fail(SVG_E_INVALID, "T must be >= 0 (got %d)", g.T);
  if (g.a1 < 1 || g.a2 < 1) return fail(SVG_E_INVALID, "a1 and a2 must be >= 1 (got %d, %d)", g.a1, g.a2);
  if (g.window < 1 || g.stripe < 1)
    return fail(SVG_E_INVALID, "window and stripe must be >= 1 (got %d, %d)", g.window, g.stripe);
  const int64_t L = (int64_t)g.T + (int64_t)g.N * g.F;
  if (L > kMaxTokens) return fail(SVG_E_UNSUPPORTED, "T + N*F = %lld tokens exceeds 2^30", (long long)L);
  if (!(isfinite(g.scale) && g.scale >= 0.f)) return fail(SVG_E_INVALID, "scale must be finite and >= 0");
  if (out) {
    KGeom& k = *out;
    k.B = g.B;
    k.H = g.H;
    k.d = g.d;
    k.N = g.N;
    k.F = g.F;
    k.T = g.T;
    k.a1 = g.a1;
    k.a2 = g.a2;
    k.window = g.window;
    k.stripe = g.stripe;
    k.L = (int32_t)L;
    k.scale = g.scale > 0.f ? g.scale : (float)(1.0 / sqrt((double)g.d));
    k.scale_log2 = (float)((double)k.scale * 1.4426950408889634);
    fastdiv_init((uint32_t)g.N, &k.divN_mul, &k.divN_shift);
    fastdiv_init((uint32_t)g.F, &k.divF_mul, &k.divF_shift);
    k.nxcd = 8;  // until apply_topology reads the device's own
    k.ncu = 256;
  }
  return SVG_OK;
}

svg_status check_ptr(const void* p, const char* name, size_t align) {
  if (!p) return fail(SVG_E_INVALID, "%s is NULL", name);
  if (((uintptr_t)p) % align) return fail(SVG_E_INVALID, "%s is not %zu-byte aligned", name, align);
  return SVG_OK;
}

// An output starting where an input of the same call starts: the kernels
// read rows that other workgroups of the same launch overwrite.  (Any overlap
// is outside the contract; this catches the in-place call.)
svg_status check_distinct(const void* out, const char* name, std::initializer_list<const void*> ins) {
  if (!out) return SVG_OK;
  for (const void* p : ins)
    if (p == out) return fail(SVG_E_INVALID, "%s must not overlap an input of the call", name);
  return SVG_OK;
}

svg_status check_strides(const svg_strides& s, const KGeom& g, int elt, const char* name) {
  if (s.x < g.d) return fail(SVG_E_INVALID, "%s: token stride %lld < d", name, (long long)s.x);
  if (s.x > (1 << 24)) return fail(SVG_E_UNSUPPORTED, "%s: token stride %lld > 2^24", name, (long long)s.x);
  if (s.h < 0 || s.b < 0) return fail(SVG_E_INVALID, "%s: negative stride", name);
  if ((s.x * elt) % 16 || (s.h * elt) % 16 || (s.b * elt) % 16)
    return fail(SVG_E_INVALID, "%s: strides must be multiples of 16 bytes", name);
  return SVG_OK;
}

// Device topology, cached per device id (read once with that device current).
hipError_t query_topology(DevTopo* t) {
  static std::atomic<int64_t> cache[64];  // cus << 32 | xcds, 0 = not read yet
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64) {
    const int64_t c = cache[dev].load(std::memory_order_acquire);
    if (c != 0) {
      t->cus = (int32_t)(c >> 32);
      t->xcds = (int32_t)(c & 0xffffffff);
      return hipSuccess;
    }
  }
  int cus = 0, xcds = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&xcds, hipDeviceAttributeNumberOfXccs, dev);
  if (e != hipSuccess) return e;
  t->cus = cus > 0 ? cus : 1;
  t->xcds = xcds > 0 ? xcds : 1;
  if (dev >= 0 && dev < 64)
    cache[dev].store(((int64_t)t->cus << 32) | (int64_t)t->xcds, std::memory_order_release);
  return hipSuccess;
}

// The device's CU and XCD counts into g (after every argument has passed).
hipError_t apply_topology(KGeom* g) {
  DevTopo t;
  hipError_t e = query_topology(&t);
  if (e != hipSuccess) return e;
  g->ncu = t.cus;
  g->nxcd = t.xcds;
  return hipSuccess;
}

#define TRY(expr)                      \
  do {                                 \
    svg_status _st = (expr);           \
    if (_st != SVG_OK) return _st;     \
  } while (0)

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Key slices of the profiling sweeps for `cus` compute units (at most cap).
// The workspace is laid out for the slices chosen at kRefCUs, the MI355X's
// 256; a call then takes the slices chosen for the device's own CU count,
// at most as many as the layout holds.
constexpr int64_t kRefCUs = 256;

int32_t profile_ksplit(const KGeom& g, svg_dtype dtype, int32_t n_rows, int64_t cus, int32_t cap) {
  if (dtype != SVG_BF16) return 1;
  const int64_t chunks = (n_rows + kProfRows_bf16 - 1) / kProfRows_bf16;
  const int64_t nkt = (g.L + kBN_bf16 - 1) / kBN_bf16;
  return choose_ksplit(chunks * g.B * g.H, nkt, cus, cap);
}

// Layout: [profiling partials][labels][ranges][head order][permuted Q,K,V,O].
// ks_cap bounds the key slices of the profiling sweeps (fewer slices, fewer
// partials: the fixed scratch of svg_layer_forward_noalloc).
WsLayout ws_layout(const KGeom& g, svg_dtype dtype, int32_t n_rows, int32_t flags, int32_t ks_cap = 16) {
  WsLayout w{};
  const int64_t BH = (int64_t)g.B * g.H;
  const int32_t BM = dtype == SVG_BF16 ? kBM_bf16 : kBM_f32;
  const int64_t nQT = (g.L + BM - 1) / BM;
  size_t off = 0;
  w.ksplit = n_rows > 0 ? profile_ksplit(g, dtype, n_rows, kRefCUs, ks_cap) : 0;
  const size_t rows_bh = (size_t)BH * n_rows;
  const size_t nstates = (flags & SVG_FLAG_MODE_SEARCH) ? 4 : 3;  // masks swept per row
  w.part_acc = off;
  off = align256(off + sizeof(float) * rows_bh * w.ksplit * nstates * g.d);
  w.part_ml = off;
  off = align256(off + sizeof(float) * rows_bh * w.ksplit * nstates * 2);
  w.row_sums = off;
  off = align256(off + sizeof(double) * rows_bh * nstates);
  w.ord_x = off;
  off = align256(off + sizeof(int32_t) * (size_t)n_rows);
  w.ord_r = off;
  off = align256(off + sizeof(int32_t) * (size_t)n_rows);
  w.labels = off;
  off = align256(off + sizeof(int32_t) * (size_t)BH);
  w.ranges = off;
  off = align256(off + sizeof(int32_t) * 4 * (size_t)BH * nQT);
  w.order = off;
  off = align256(off + sizeof(int32_t) * (size_t)BH);
  w.perm = off;
  w.perm_tensor_bytes = 0;
  if (flags & SVG_FLAG_FP8_SCORES) {  // quantised Q, K and scales; no permuted copies
    const size_t n8 = align256((size_t)BH * g.L * g.d);
    const int64_t nKT = (g.L + kBN_bf16 - 1) / kBN_bf16;
    w.q8 = off;
    off += n8;
    w.k8 = off;
    off += n8;
    w.sq = off;
    off = align256(off + sizeof(float) * (size_t)BH * g.L);
    w.sk = off;
    off = align256(off + sizeof(float) * (size_t)BH * nKT);
    if (flags & SVG_FLAG_FP8_PV) {
      w.v8 = off;
      off = align256(off + (size_t)BH * nKT * g.d * 64);
      w.svh = off;
      off = align256(off + sizeof(float) * (size_t)BH);
    }
  } else if (!(flags & SVG_FLAG_VIRTUAL_PERMUTE)) {
    // token-major K and V in the input dtype
    w.perm_tensor_bytes = align256((size_t)BH * g.L * g.d * elt_bytes(dtype));
    off += 2 * w.perm_tensor_bytes;
  }
  w.total = off;
  return w;
}

size_t profile_ws_bytes(const WsLayout& w) { return w.labels; }

template <typename T>
T* ws_at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

svg_status tile_config_impl(svg_dtype dtype, int32_t d, int32_t* BM, int32_t* BN) {
  if (!dtype_ok(dtype)) return fail(SVG_E_INVALID, "unknown dtype %d", (int)dtype);
  if (d != 64 && d != 128) return fail(SVG_E_UNSUPPORTED, "head dim d=%d (supported: 64, 128)", d);
  if (dtype == SVG_BF16) {
    *BM = kBM_bf16;
    *BN = kBN_bf16;
  } else {
    *BM = kBM_f32;
    *BN = kBN_f32;
  }
  return SVG_OK;
}

svg_status validate_attention(const KGeom& g, svg_dtype in, svg_dtype out, const void* q, const void* k,
                              const void* v, svg_strides s, const void* qp, const void* kp, const void* vp,
                              svg_strides sp, const void* o, svg_strides so, const void* op, svg_strides sop,
                              const int32_t* modes, const int32_t* ranges, const int32_t* order, int32_t BM,
                              int32_t BN, int32_t flags, bool check_lists = true) {
  if (!dtype_ok(in) || !dtype_ok(out)) return fail(SVG_E_INVALID, "unknown dtype");
  if (in == SVG_F32 && out != SVG_F32) return fail(SVG_E_UNSUPPORTED, "f32 input requires f32 output");
  if (flags & ~SVG_FLAG_VIRTUAL_PERMUTE) return fail(SVG_E_INVALID, "unknown flags 0x%x", flags);
  int32_t bm, bn;
  TRY(tile_config_impl(in, g.d, &bm, &bn));
  if (BM != bm || BN != bn)
    return fail(SVG_E_UNSUPPORTED, "ranges built with %dx%d tiles; this kernel needs %dx%d", BM, BN, bm, bn);
  const int ei = elt_bytes(in), eo = elt_bytes(out);
  TRY(check_ptr(q, "q", 16));
  TRY(check_ptr(k, "k", 16));
  TRY(check_ptr(v, "v", 16));
  TRY(check_ptr(o, "o", 16));
  TRY(check_strides(s, g, ei, "q/k/v"));
  TRY(check_strides(so, g, eo, "o"));
  if (!(flags & SVG_FLAG_VIRTUAL_PERMUTE)) {
    // K and V copies are required; Q and O copies are optional (NULL: those
    // rows go through the index map)
    if (qp) TRY(check_ptr(qp, "qp", 16));
    TRY(check_ptr(kp, "kp", 16));
    TRY(check_ptr(vp, "vp", 16));
    if (op) TRY(check_ptr(op, "op", 16));
    TRY(check_strides(sp, g, ei, "qp/kp/vp"));
    if (op) TRY(check_strides(sop, g, eo, "op"));
  }
  TRY(check_distinct(o, "o", {q, k, v, qp, kp, vp}));
  TRY(check_distinct(op, "op", {q, k, v, qp, kp, vp, o}));
  TRY(check_ptr(modes, "modes", 4));
  if (check_lists) {  // svg_layer_forward places them in its own workspace
    TRY(check_ptr(ranges, "ranges", 16));
    TRY(check_ptr(order, "head_order", 4));
  }
  return SVG_OK;
}

hipError_t run_attention(const KGeom& g, svg_dtype in, svg_dtype out, const AttnPtrs& a, hipStream_t st) {
  if (in == SVG_BF16) return launch_attention_bf16(g, a, out == SVG_BF16, st);
  return launch_attention_f32(g, a, kBM_f32, kBN_f32, st);
}

svg_status validate_profile(const KGeom& g, svg_dtype dtype, const void* q, const void* k, const void* v,
                            svg_strides s, const int32_t* rows, int32_t n_rows, float fallback,
                            const int32_t* labels, const float* stats) {
  if (!dtype_ok(dtype)) return fail(SVG_E_INVALID, "unknown dtype %d", (int)dtype);
  const int e = elt_bytes(dtype);
  TRY(check_ptr(q, "q", 16));
  TRY(check_ptr(k, "k", 16));
  TRY(check_ptr(v, "v", 16));
  TRY(check_strides(s, g, e, "q/k/v"));
  TRY(check_ptr(rows, "rows", 4));
  if (n_rows < 1 || (int64_t)n_rows > (int64_t)g.N * g.F)
    return fail(SVG_E_INVALID, "n_rows=%d must be in [1, N*F]", n_rows);
  if (!(fallback > 0.f) || !isfinite(fallback)) return fail(SVG_E_INVALID, "fallback_rel_mse must be > 0");
  TRY(check_ptr(labels, "labels", 4));
  TRY(check_ptr(stats, "stats", 4));
  return SVG_OK;
}

hipError_t run_profile(const KGeom& g, svg_dtype dtype, const void* q, const void* k, const void* v,
                       svg_strides s, const int32_t* rows, int32_t n_rows, float fallback, int32_t* labels,
                       float* stats, void* ws, const WsLayout& w, hipStream_t st) {
  float* pa = ws_at<float>(ws, w.part_acc);
  float* pm = ws_at<float>(ws, w.part_ml);
  // key slices for this device's CUs, within the ones the partials hold
  const int32_t ks = dtype == SVG_BF16 ? profile_ksplit(g, dtype, n_rows, g.ncu, w.ksplit) : w.ksplit;
  hipError_t e;
  if (dtype == SVG_BF16) {
    int32_t* ox = ws_at<int32_t>(ws, w.ord_x);
    int32_t* orr = ws_at<int32_t>(ws, w.ord_r);
    e = launch_profile_rank(g, rows, n_rows, ox, orr, st);
    if (e != hipSuccess) return e;
    static const int32_t masks[3] = {SVG_SPATIAL, SVG_FULL, SVG_TEMPORAL};  // states 0, 1 (reference), 2
    e = launch_sample_sweeps(g, q, k, v, s, rows, n_rows, ks, ox, orr, masks, 3, pa, pm, st);
  } else {
    e = launch_profile_f32(g, q, k, v, s, rows, n_rows, pa, pm, st);
  }
  if (e != hipSuccess) return e;
  return launch_profile_merge(g, n_rows, ks, pa, pm, ws_at<double>(ws, w.row_sums), fallback, labels, stats, st);
}

// Active (query, key) pairs of a mode over the whole L x L map, from the
// closed forms of its masks: text rows and keys dense, video part per mode.
int64_t mode_nnz(const KGeom& g, int32_t mode) {
  if (mode == SVG_SKIP) return 0;
  const int64_t NF = (int64_t)g.N * g.F, Lt = g.T + NF;
  const int64_t text = Lt * Lt - NF * NF;
  int64_t video = 0;
  switch (mode) {
    case SVG_SPATIAL: {
      const int64_t a = g.a1 < g.N ? g.a1 : g.N;
      video = (int64_t)g.F * g.F * (g.N * (2 * a - 1) - a * (a - 1));
      break;
    }
    case SVG_TEMPORAL: {
      const int64_t a = g.a2 < g.F ? g.a2 : g.F;
      video = (int64_t)g.N * g.N * (g.F * (2 * a - 1) - a * (a - 1));
      break;
    }
    case SVG_WINDOW: {
      const int64_t w = g.window < NF ? g.window : NF;
      video = NF * (2 * w - 1) - w * (w - 1);
      break;
    }
    case SVG_STRIPE:
      video = NF * (g.stripe < NF ? g.stripe : NF);
      break;
    default:
      video = NF * NF;
  }
  return text + video;
}

// SVG2 workspace: k-means scratch, per-tensor clustering results, selection,
// K / V in cluster order.
struct Svg2Ws {
  size_t hi, lo, hn, hist, base, rank;
  size_t mu_q, mu_k, lab_q, lab_k, perm_q, perm_k, start_q, start_k;
  size_t sel, segs, nseg, nkeys, ord, rbp, kp, vp, total;
};

Svg2Ws svg2_ws_layout(const KGeom& g, int32_t Cq, int32_t Ck) {
  Svg2Ws w{};
  const size_t BH = (size_t)g.B * g.H, L = (size_t)g.L, d = (size_t)g.d;
  const size_t Cm = (size_t)(Cq > Ck ? Cq : Ck);
  const size_t nBlk = (L + 255) / 256;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  w.hi = take(BH * Cm * d * 2);
  w.lo = take(BH * Cm * d * 2);
  w.hn = take(BH * Cm * 4);
  w.hist = take(BH * nBlk * Cm * 4);
  w.base = take(BH * nBlk * Cm * 4);
  w.rank = take(BH * L * 4);
  w.mu_q = take(BH * (size_t)Cq * d * 4);
  w.mu_k = take(BH * (size_t)Ck * d * 4);
  w.lab_q = take(BH * L * 4);
  w.lab_k = take(BH * L * 4);
  w.perm_q = take(BH * L * 4);
  w.perm_k = take(BH * L * 4);
  w.start_q = take(BH * ((size_t)Cq + 1) * 4);
  w.start_k = take(BH * ((size_t)Ck + 1) * 4);
  w.sel = take(BH * (size_t)Cq * Ck);
  w.segs = take(BH * (size_t)Cq * Ck * 8);
  w.nseg = take(BH * (size_t)Cq * 4);
  w.nkeys = take(BH * (size_t)Cq * 4);
  w.ord = take(BH * (size_t)Cq * 4);
  w.rbp = take(BH * ((size_t)Cq + 1) * 4);
  w.kp = take(BH * L * d * 2);
  w.vp = take(BH * L * d * 2);
  w.total = off;
  return w;
}

Svg2Scratch svg2_scratch(void* ws, const Svg2Ws& w) {
  Svg2Scratch s;
  s.hi = ws_at<char>(ws, w.hi);
  s.lo = ws_at<char>(ws, w.lo);
  s.hn = ws_at<float>(ws, w.hn);
  s.hist = ws_at<int32_t>(ws, w.hist);
  s.base = ws_at<int32_t>(ws, w.base);
  s.rank = ws_at<int32_t>(ws, w.rank);
  return s;
}

svg_status check_svg2_params(const KGeom& g, const svg2_params* prm) {
  if (!prm) return fail(SVG_E_INVALID, "params is NULL");
  if (prm->C_q < 1 || prm->C_k < 1) return fail(SVG_E_INVALID, "cluster counts must be >= 1");
  if (prm->C_q > kSvg2MaxClusters || prm->C_k > kSvg2MaxClusters)
    return fail(SVG_E_UNSUPPORTED, "cluster counts must be in [1, %d] (got %d, %d)", kSvg2MaxClusters, prm->C_q,
                prm->C_k);
  if (prm->C_q > g.L || prm->C_k > g.L) return fail(SVG_E_INVALID, "more clusters than tokens");
  if (prm->iters < 1) return fail(SVG_E_INVALID, "iters must be >= 1");
  if (!(prm->p > 0.f) || !isfinite(prm->p)) return fail(SVG_E_INVALID, "p must be finite and > 0");
  return SVG_OK;
}

}  // namespace

namespace {

// svg_layer_forward, and with fixed_scratch its allocation-free variant: the
// workspace is then the device's fixed scratch (ws, ws_bytes unused), the
// layout transformation is always the index-map one (no permuted copies) and
// the profiling sweeps take as many key slices as fit in the scratch.
svg_status layer_forward_impl(const svg_geom* geom, svg_dtype in, svg_dtype out, const void* q, const void* k,
                              const void* v, svg_strides s, void* o, svg_strides so, const int32_t* rows,
                              int32_t n_rows, float fallback_rel_mse, const int32_t* modes_in, int32_t* labels_out,
                              float* stats_out, int32_t flags, void* ws, size_t ws_bytes, bool fixed_scratch,
                              void* stream) {
  KGeom g;
  TRY(check_geom(geom, &g));
  if (!dtype_ok(in) || !dtype_ok(out)) return fail(SVG_E_INVALID, "unknown dtype");
  if (flags & ~(SVG_FLAG_VIRTUAL_PERMUTE | SVG_FLAG_FP8_SCORES | SVG_FLAG_FP8_PV))
    return fail(SVG_E_INVALID, "unknown flags 0x%x", flags);
  if ((flags & SVG_FLAG_FP8_PV) && !(flags & SVG_FLAG_FP8_SCORES))
    return fail(SVG_E_INVALID, "SVG_FLAG_FP8_PV needs SVG_FLAG_FP8_SCORES");
  if (fixed_scratch) {
    if (flags & (SVG_FLAG_FP8_SCORES | SVG_FLAG_FP8_PV))
      return fail(SVG_E_UNSUPPORTED, "svg_layer_forward_noalloc: the fp8 paths need more scratch than it holds");
    flags |= SVG_FLAG_VIRTUAL_PERMUTE;
  }
  const bool fp8 = flags & SVG_FLAG_FP8_SCORES;
  const bool fp8pv = flags & SVG_FLAG_FP8_PV;
  if (fp8 && in != SVG_BF16) return fail(SVG_E_UNSUPPORTED, "fp8 scores take bf16 inputs");
  if (fp8) flags |= SVG_FLAG_VIRTUAL_PERMUTE;  // the fp8 path reads temporal heads through the index map
  TRY(check_distinct(o, "o", {q, k, v}));
  const bool profile = modes_in == nullptr;
  if (profile) {
    TRY(validate_profile(g, in, q, k, v, s, rows, n_rows, fallback_rel_mse, labels_out, stats_out));
  } else {
    TRY(check_ptr(modes_in, "modes_in", 4));
    if (labels_out) TRY(check_ptr(labels_out, "labels_out", 4));
  }
  WsLayout w = ws_layout(g, in, profile ? n_rows : 0, flags);
  if (fixed_scratch) {
    while (w.total > kStaticScratchBytes && w.ksplit > 1) w = ws_layout(g, in, n_rows, flags, w.ksplit - 1);
    // (only the profiling partials depend on the slice count)
    if (w.total > kStaticScratchBytes)
      return fail(SVG_E_WORKSPACE, "svg_layer_forward_noalloc: this layer needs %zu bytes of scratch, the fixed "
                  "scratch holds %zu", w.total, kStaticScratchBytes);
  } else {
    TRY(check_ptr(ws, "ws", 256));
    if (ws_bytes < w.total) return fail(SVG_E_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, w.total);
  }
  int32_t BM, BN;
  TRY(tile_config_impl(in, g.d, &BM, &BN));
  const bool virt = flags & SVG_FLAG_VIRTUAL_PERMUTE;
  const int ei = elt_bytes(in), eo = elt_bytes(out);
  const svg_strides sp{(int64_t)g.H * g.L * g.d, (int64_t)g.L * g.d, g.d};
  // workspace pointers (ws is the caller's, 256-byte aligned, or the fixed
  // scratch, whose address is only taken once every argument has passed)
  // explicit layout: token-major copies of K and V only (Q is read and O
  // written through the index map by the attention kernel)
  auto perm_at = [&](int t) -> void* { return virt ? nullptr : ws_at<char>(ws, w.perm) + t * w.perm_tensor_bytes; };
  TRY(validate_attention(g, in, out, q, k, v, s, nullptr, perm_at(0), perm_at(1), sp, o, so, nullptr, sp,
                         profile ? labels_out : modes_in, nullptr, nullptr, BM, BN, flags & SVG_FLAG_VIRTUAL_PERMUTE,
                         false));
  hipError_t e = apply_topology(&g);
  if (e != hipSuccess) return hip_fail(e, "svg_layer_forward (device topology)");
  if (fixed_scratch) {
    e = static_scratch(&ws);
    if (e != hipSuccess) return hip_fail(e, "svg_layer_forward_noalloc (scratch address)");
  }
  void *kp = perm_at(0), *vp = perm_at(1);
  int32_t* ranges = ws_at<int32_t>(ws, w.ranges);
  int32_t* order = ws_at<int32_t>(ws, w.order);
  hipStream_t st = (hipStream_t)stream;
  const int32_t* modes = modes_in;
  if (profile) {
    e = run_profile(g, in, q, k, v, s, rows, n_rows, fallback_rel_mse, labels_out, stats_out, ws, w, st);
    if (e != hipSuccess) return hip_fail(e, "svg_layer_forward (profiling)");
    modes = labels_out;
  } else if (labels_out && labels_out != modes_in) {
    e = hipMemcpyAsync(labels_out, modes_in, sizeof(int32_t) * g.B * g.H, hipMemcpyDeviceToDevice, st);
    if (e != hipSuccess) return hip_fail(e, "svg_layer_forward (labels copy)");
  }
  e = launch_build_blocks(g, modes, BM, BN, ranges, order, st);
  if (e != hipSuccess) return hip_fail(e, "svg_layer_forward (blocks)");
  if (fp8) {
    uint8_t* q8 = ws_at<uint8_t>(ws, w.q8);
    uint8_t* k8 = ws_at<uint8_t>(ws, w.k8);
    float* sq = ws_at<float>(ws, w.sq);
    float* sk = ws_at<float>(ws, w.sk);
    e = launch_quant_qk(g, q, k, s, modes, q8, sq, k8, sk, st);
    if (e != hipSuccess) return hip_fail(e, "svg_layer_forward (fp8 quantisation)");
    if (fp8pv) {
      uint8_t* v8 = ws_at<uint8_t>(ws, w.v8);
      float* svh = ws_at<float>(ws, w.svh);
      e = launch_quant_v(g, v, s, modes, v8, svh, st);
      if (e != hipSuccess) return hip_fail(e, "svg_layer_forward (fp8 V quantisation)");
      e = launch_attention_fp8pv(g, q8, sq, k8, sk, v8, svh, o, so, out == SVG_BF16, modes, ranges, order, st);
      return e == hipSuccess ? SVG_OK : hip_fail(e, "svg_layer_forward (fp8 attention)");
    }
    e = launch_attention_fp8(g, q8, sq, k8, sk, v, s, o, so, out == SVG_BF16, modes, ranges, order, st);
    return e == hipSuccess ? SVG_OK : hip_fail(e, "svg_layer_forward (fp8 attention)");
  }
  if (!virt) {
    const void* src[2] = {k, v};
    void* dst[2] = {kp, vp};
    for (int t = 0; t < 2; ++t) {
      e = launch_permute(g, ei, src[t], s, dst[t], sp, modes, 0, st);
      if (e != hipSuccess) return hip_fail(e, "svg_layer_forward (permute)");
    }
  }
  AttnPtrs a{q, k, v, nullptr, kp, vp, o, nullptr, s, sp, so, sp, modes, ranges, order, flags};
  e = run_attention(g, in, out, a, st);
  if (e != hipSuccess) return hip_fail(e, "svg_layer_forward (attention)");
  return SVG_OK;
}


}  // namespace

extern "C" {

int32_t svg_abi_version(void) { return SVG_ABI_VERSION; }

const char* svg_last_error(void) { return g_err; }

svg_status svg_tile_config(svg_dtype dtype, int32_t d, int32_t* BM, int32_t* BN) {
  if (!BM || !BN) return fail(SVG_E_INVALID, "BM/BN output pointer is NULL");
  return tile_config_impl(dtype, d, BM, BN);
}

svg_status svg_sample_rows(const svg_geom* geom, int32_t count, uint64_t seed, int32_t* rows) {
  KGeom g;
  TRY(check_geom(geom, &g));
  const int64_t n = (int64_t)g.N * g.F;
  if (count < 0 || count > n) return fail(SVG_E_INVALID, "count=%d must be in [0, N*F = %lld]", count, (long long)n);
  if (count == 0) return SVG_OK;
  if (!rows) return fail(SVG_E_INVALID, "rows is NULL");
  sample_sorted(n, count, seed, rows);
  for (int32_t r = 0; r < count; ++r) rows[r] += g.T;
  return SVG_OK;
}

svg_status svg_workspace_bytes(const svg_geom* geom, svg_dtype dtype, int32_t n_rows, int32_t flags,
                               size_t* bytes) {
  KGeom g;
  TRY(check_geom(geom, &g));
  if (!dtype_ok(dtype)) return fail(SVG_E_INVALID, "unknown dtype %d", (int)dtype);
  if (!bytes) return fail(SVG_E_INVALID, "bytes is NULL");
  if (n_rows < 0 || (int64_t)n_rows > (int64_t)g.N * g.F)
    return fail(SVG_E_INVALID, "n_rows=%d must be in [0, N*F]", n_rows);
  if (flags & ~(SVG_FLAG_VIRTUAL_PERMUTE | SVG_FLAG_MODE_SEARCH | SVG_FLAG_FP8_SCORES | SVG_FLAG_FP8_PV))
    return fail(SVG_E_INVALID, "unknown flags 0x%x", flags);
  if ((flags & SVG_FLAG_FP8_PV) && !(flags & SVG_FLAG_FP8_SCORES))
    return fail(SVG_E_INVALID, "SVG_FLAG_FP8_PV needs SVG_FLAG_FP8_SCORES");
  if ((flags & (SVG_FLAG_MODE_SEARCH | SVG_FLAG_FP8_SCORES)) && dtype != SVG_BF16)
    return fail(SVG_E_UNSUPPORTED, "the mode search and fp8 scores take bf16 inputs");
  *bytes = ws_layout(g, dtype, n_rows, flags).total;
  return SVG_OK;
}

svg_status svg_search_modes(const svg_geom* geom, svg_dtype dtype, const void* q, const void* k, const void* v,
                            svg_strides s, const int32_t* rows, int32_t n_rows, float lam, float eps,
                            int32_t penalty, int32_t* modes_out, float* stats_out, void* ws, size_t ws_bytes,
                            void* stream) {
  KGeom g;
  TRY(check_geom(geom, &g));
  if (dtype == SVG_F32) return fail(SVG_E_UNSUPPORTED, "the mode search takes bf16 inputs");
  TRY(validate_profile(g, dtype, q, k, v, s, rows, n_rows, 1.f, modes_out, stats_out));
  if (!isfinite(lam) || lam < 0.f) return fail(SVG_E_INVALID, "lambda must be finite and >= 0");
  if (!isfinite(eps)) return fail(SVG_E_INVALID, "epsilon must be finite");
  if (penalty != 0 && penalty != 1) return fail(SVG_E_INVALID, "penalty must be 0 (lam*(1-S)) or 1 (lam*S)");
  const WsLayout w = ws_layout(g, dtype, n_rows, SVG_FLAG_VIRTUAL_PERMUTE | SVG_FLAG_MODE_SEARCH);
  TRY(check_ptr(ws, "ws", 256));
  if (ws_bytes < profile_ws_bytes(w))
    return fail(SVG_E_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, profile_ws_bytes(w));
  SearchParams p;
  p.lam = lam;
  p.eps = eps;
  p.penalty = penalty;
  const double L2 = (double)g.L * (double)g.L;
  const int32_t cand[4] = {SVG_SKIP, SVG_WINDOW, SVG_TEMPORAL, SVG_STRIPE};
  for (int c = 0; c < 4; ++c) p.sparsity[c] = (float)(1.0 - (double)mode_nnz(g, cand[c]) / L2);
  hipStream_t st = (hipStream_t)stream;
  float* pa = ws_at<float>(ws, w.part_acc);
  float* pm = ws_at<float>(ws, w.part_ml);
  int32_t* ox = ws_at<int32_t>(ws, w.ord_x);
  int32_t* orr = ws_at<int32_t>(ws, w.ord_r);
  static const int32_t masks[4] = {SVG_FULL, SVG_WINDOW, SVG_TEMPORAL, SVG_STRIPE};  // state 0 = reference
  hipError_t e = apply_topology(&g);
  const int32_t ks = profile_ksplit(g, dtype, n_rows, g.ncu, w.ksplit);
  if (e == hipSuccess) e = launch_profile_rank(g, rows, n_rows, ox, orr, st);
  if (e == hipSuccess) e = launch_sample_sweeps(g, q, k, v, s, rows, n_rows, ks, ox, orr, masks, 4, pa, pm, st);
  if (e == hipSuccess)
    e = launch_search_merge(g, n_rows, ks, pa, pm, ws_at<double>(ws, w.row_sums), p, modes_out, stats_out, st);
  return e == hipSuccess ? SVG_OK : hip_fail(e, "svg_search_modes");
}

svg_status svg_profile_heads(const svg_geom* geom, svg_dtype dtype, const void* q, const void* k, const void* v,
                             svg_strides s, const int32_t* rows, int32_t n_rows, float fallback_rel_mse,
                             int32_t* labels, float* stats, void* ws, size_t ws_bytes, void* stream) {
  KGeom g;
  TRY(check_geom(geom, &g));
  TRY(validate_profile(g, dtype, q, k, v, s, rows, n_rows, fallback_rel_mse, labels, stats));
  const WsLayout w = ws_layout(g, dtype, n_rows, SVG_FLAG_VIRTUAL_PERMUTE);
  TRY(check_ptr(ws, "ws", 256));
  if (ws_bytes < profile_ws_bytes(w))
    return fail(SVG_E_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, profile_ws_bytes(w));
  hipError_t e = apply_topology(&g);
  if (e != hipSuccess) return hip_fail(e, "svg_profile_heads (device topology)");
  e = run_profile(g, dtype, q, k, v, s, rows, n_rows, fallback_rel_mse, labels, stats, ws, w,
                             (hipStream_t)stream);
  return e == hipSuccess ? SVG_OK : hip_fail(e, "svg_profile_heads");
}

svg_status svg_build_blocks(const svg_geom* geom, const int32_t* modes, int32_t BM, int32_t BN, int32_t* ranges,
                            int32_t* head_order, void* stream) {
  KGeom g;
  TRY(check_geom(geom, &g));
  if (BM < 16 || BN < 16 || BM > 1024 || BN > 1024 || BM % 16 || BN % 16)
    return fail(SVG_E_UNSUPPORTED, "tile sizes %dx%d must be multiples of 16 in [16, 1024]", BM, BN);
  TRY(check_ptr(modes, "modes", 4));
  TRY(check_ptr(ranges, "ranges", 16));
  TRY(check_ptr(head_order, "head_order", 4));
  hipError_t e = launch_build_blocks(g, modes, BM, BN, ranges, head_order, (hipStream_t)stream);
  return e == hipSuccess ? SVG_OK : hip_fail(e, "svg_build_blocks");
}

svg_status svg_layout_permute(const svg_geom* geom, svg_dtype dtype, const void* src, svg_strides ss, void* dst,
                              svg_strides ds, const int32_t* modes, int32_t inverse, void* stream) {
  KGeom g;
  TRY(check_geom(geom, &g));
  if (!dtype_ok(dtype)) return fail(SVG_E_INVALID, "unknown dtype %d", (int)dtype);
  const int e = elt_bytes(dtype);
  TRY(check_ptr(src, "src", 16));
  TRY(check_ptr(dst, "dst", 16));
  TRY(check_strides(ss, g, e, "src"));
  TRY(check_strides(ds, g, e, "dst"));
  if (src == dst) return fail(SVG_E_INVALID, "src and dst must not overlap");
  if (modes) TRY(check_ptr(modes, "modes", 4));
  hipError_t he = launch_permute(g, e, src, ss, dst, ds, modes, inverse ? 1 : 0, (hipStream_t)stream);
  return he == hipSuccess ? SVG_OK : hip_fail(he, "svg_layout_permute");
}

svg_status svg_sparse_attention(const svg_geom* geom, svg_dtype in, svg_dtype out, const void* q, const void* k,
                                const void* v, svg_strides s, const void* qp, const void* kp, const void* vp,
                                svg_strides sp, void* o, svg_strides so, void* op, svg_strides sop,
                                const int32_t* modes, const int32_t* ranges, const int32_t* head_order,
                                int32_t BM, int32_t BN, int32_t flags, void* stream) {
  KGeom g;
  TRY(check_geom(geom, &g));
  TRY(validate_attention(g, in, out, q, k, v, s, qp, kp, vp, sp, o, so, op, sop, modes, ranges, head_order, BM,
                         BN, flags));
  AttnPtrs a{q, k, v, qp, kp, vp, o, op, s, sp, so, sop, modes, ranges, head_order, flags};
  hipError_t e = apply_topology(&g);
  if (e == hipSuccess) e = run_attention(g, in, out, a, (hipStream_t)stream);
  return e == hipSuccess ? SVG_OK : hip_fail(e, "svg_sparse_attention");
}

svg_status svg_quantize_qk(const svg_geom* geom, svg_dtype dtype, const void* q, const void* k, svg_strides s,
                           const int32_t* modes, uint8_t* q8, float* sq, uint8_t* k8, float* sk, void* stream) {
  KGeom g;
  TRY(check_geom(geom, &g));
  if (dtype != SVG_BF16) return fail(dtype_ok(dtype) ? SVG_E_UNSUPPORTED : SVG_E_INVALID, "fp8 scores take bf16 inputs");
  TRY(check_ptr(q, "q", 16));
  TRY(check_ptr(k, "k", 16));
  TRY(check_strides(s, g, 2, "q/k"));
  TRY(check_ptr(modes, "modes", 4));
  TRY(check_ptr(q8, "q8", 16));
  TRY(check_ptr(k8, "k8", 16));
  TRY(check_distinct(q8, "q8", {q, k}));
  TRY(check_distinct(k8, "k8", {q, k, q8}));
  TRY(check_ptr(sq, "sq", 4));
  TRY(check_ptr(sk, "sk", 4));
  hipError_t e = launch_quant_qk(g, q, k, s, modes, q8, sq, k8, sk, (hipStream_t)stream);
  return e == hipSuccess ? SVG_OK : hip_fail(e, "svg_quantize_qk");
}

svg_status svg_sparse_attention_fp8(const svg_geom* geom, svg_dtype out, const uint8_t* q8, const float* sq,
                                    const uint8_t* k8, const float* sk, const void* v, svg_strides sv, void* o,
                                    svg_strides so, const int32_t* modes, const int32_t* ranges,
                                    const int32_t* head_order, int32_t BM, int32_t BN, void* stream) {
  KGeom g;
  TRY(check_geom(geom, &g));
  if (!dtype_ok(out)) return fail(SVG_E_INVALID, "unknown dtype");
  if (BM != kBM_bf16 || BN != kBN_bf16)
    return fail(SVG_E_UNSUPPORTED, "ranges built with %dx%d tiles; this kernel needs %dx%d", BM, BN, kBM_bf16,
                kBN_bf16);
  TRY(check_ptr(q8, "q8", 16));
  TRY(check_ptr(k8, "k8", 16));
  TRY(check_ptr(sq, "sq", 4));
  TRY(check_ptr(sk, "sk", 4));
  TRY(check_ptr(v, "v", 16));
  TRY(check_ptr(o, "o", 16));
  TRY(check_strides(sv, g, 2, "v"));
  TRY(check_strides(so, g, elt_bytes(out), "o"));
  TRY(check_distinct(o, "o", {q8, k8, v}));
  TRY(check_ptr(modes, "modes", 4));
  TRY(check_ptr(ranges, "ranges", 16));
  TRY(check_ptr(head_order, "head_order", 4));
  hipError_t e = apply_topology(&g);
  if (e == hipSuccess)
    e = launch_attention_fp8(g, q8, sq, k8, sk, v, sv, o, so, out == SVG_BF16, modes, ranges, head_order,
                                      (hipStream_t)stream);
  return e == hipSuccess ? SVG_OK : hip_fail(e, "svg_sparse_attention_fp8");
}

svg_status svg_quantize_v(const svg_geom* geom, svg_dtype dtype, const void* v, svg_strides s, const int32_t* modes,
                          uint8_t* v8, float* sv, void* stream) {
  KGeom g;
  TRY(check_geom(geom, &g));
  if (dtype != SVG_BF16) return fail(dtype_ok(dtype) ? SVG_E_UNSUPPORTED : SVG_E_INVALID, "fp8 V takes bf16 inputs");
  TRY(check_ptr(v, "v", 16));
  TRY(check_strides(s, g, 2, "v"));
  TRY(check_ptr(modes, "modes", 4));
  TRY(check_ptr(v8, "v8", 16));
  TRY(check_distinct(v8, "v8", {v}));
  TRY(check_ptr(sv, "sv", 4));
  hipError_t e = launch_quant_v(g, v, s, modes, v8, sv, (hipStream_t)stream);
  return e == hipSuccess ? SVG_OK : hip_fail(e, "svg_quantize_v");
}

svg_status svg_sparse_attention_fp8_pv(const svg_geom* geom, svg_dtype out, const uint8_t* q8, const float* sq,
                                       const uint8_t* k8, const float* sk, const uint8_t* v8, const float* sv,
                                       void* o, svg_strides so, const int32_t* modes, const int32_t* ranges,
                                       const int32_t* head_order, int32_t BM, int32_t BN, void* stream) {
  KGeom g;
  TRY(check_geom(geom, &g));
  if (!dtype_ok(out)) return fail(SVG_E_INVALID, "unknown dtype");
  if (BM != kBM_bf16 || BN != kBN_bf16)
    return fail(SVG_E_UNSUPPORTED, "ranges built with %dx%d tiles; this kernel needs %dx%d", BM, BN, kBM_bf16,
                kBN_bf16);
  TRY(check_ptr(q8, "q8", 16));
  TRY(check_ptr(k8, "k8", 16));
  TRY(check_ptr(sq, "sq", 4));
  TRY(check_ptr(sk, "sk", 4));
  TRY(check_ptr(v8, "v8", 16));
  TRY(check_ptr(sv, "sv", 4));
  TRY(check_ptr(o, "o", 16));
  TRY(check_strides(so, g, elt_bytes(out), "o"));
  TRY(check_distinct(o, "o", {q8, k8, v8}));
  TRY(check_ptr(modes, "modes", 4));
  TRY(check_ptr(ranges, "ranges", 16));
  TRY(check_ptr(head_order, "head_order", 4));
  hipError_t e = apply_topology(&g);
  if (e == hipSuccess)
    e = launch_attention_fp8pv(g, q8, sq, k8, sk, v8, sv, o, so, out == SVG_BF16, modes, ranges, head_order,
                                        (hipStream_t)stream);
  return e == hipSuccess ? SVG_OK : hip_fail(e, "svg_sparse_attention_fp8_pv");
}

svg_status svg2_workspace_bytes(const svg_geom* geom, const svg2_params* prm, size_t* bytes) {
  KGeom g;
  TRY(check_geom(geom, &g));
  TRY(check_svg2_params(g, prm));
  if (!bytes) return fail(SVG_E_INVALID, "bytes is NULL");
  *bytes = svg2_ws_layout(g, prm->C_q, prm->C_k).total;
  return SVG_OK;
}

svg_status svg2_kmeans(const svg_geom* geom, svg_dtype dtype, const void* x, svg_strides s, int32_t C, int32_t iters,
                       int32_t flags, float* mu, int32_t* labels, int32_t* perm, int32_t* start, void* ws,
                       size_t ws_bytes, void* stream) {
  KGeom g;
  TRY(check_geom(geom, &g));
  if (dtype != SVG_BF16) return fail(dtype_ok(dtype) ? SVG_E_UNSUPPORTED : SVG_E_INVALID, "bf16 inputs only");
  const svg2_params prm{C, C, iters, 1.f};
  TRY(check_svg2_params(g, &prm));
  if (flags & ~SVG2_FLAG_INIT_GIVEN) return fail(SVG_E_INVALID, "unknown flags 0x%x", flags);
  TRY(check_ptr(x, "x", 16));
  TRY(check_strides(s, g, 2, "x"));
  TRY(check_ptr(mu, "mu", 4));
  TRY(check_ptr(labels, "labels", 4));
  TRY(check_ptr(perm, "perm", 4));
  TRY(check_ptr(start, "start", 4));
  const Svg2Ws w = svg2_ws_layout(g, C, C);
  TRY(check_ptr(ws, "ws", 256));
  if (ws_bytes < w.mu_q) return fail(SVG_E_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, w.mu_q);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (!(flags & SVG2_FLAG_INIT_GIVEN)) e = launch_km_init(g, x, s, C, mu, st);
  if (e == hipSuccess) e = launch_kmeans(g, x, s, C, iters, mu, labels, perm, start, svg2_scratch(ws, w), st);
  return e == hipSuccess ? SVG_OK : hip_fail(e, "svg2_kmeans");
}

svg_status svg2_forward(const svg_geom* geom, const svg2_params* prm, svg_dtype in, svg_dtype out, const void* q,
                        const void* k, const void* v, svg_strides s, void* o, svg_strides so, int32_t flags, float* mu_q,
                        float* mu_k, uint8_t* sel, void* ws, size_t ws_bytes, void* stream) {
  KGeom g;
  TRY(check_geom(geom, &g));
  TRY(check_svg2_params(g, prm));
  if (in != SVG_BF16) return fail(dtype_ok(in) ? SVG_E_UNSUPPORTED : SVG_E_INVALID, "bf16 inputs only");
  if (!dtype_ok(out)) return fail(SVG_E_INVALID, "unknown output dtype");
  if (flags & ~SVG2_FLAG_INIT_GIVEN) return fail(SVG_E_INVALID, "unknown flags 0x%x", flags);
  TRY(check_ptr(q, "q", 16));
  TRY(check_ptr(k, "k", 16));
  TRY(check_ptr(v, "v", 16));
  TRY(check_ptr(o, "o", 16));
  TRY(check_strides(s, g, 2, "q/k/v"));
  TRY(check_strides(so, g, elt_bytes(out), "o"));
  TRY(check_distinct(o, "o", {q, k, v}));
  TRY(check_ptr(mu_q, "mu_q", 4));
  TRY(check_ptr(mu_k, "mu_k", 4));
  const Svg2Ws w = svg2_ws_layout(g, prm->C_q, prm->C_k);
  TRY(check_ptr(ws, "ws", 256));
  if (ws_bytes < w.total) return fail(SVG_E_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, w.total);
  hipStream_t st = (hipStream_t)stream;
  const Svg2Scratch sc = svg2_scratch(ws, w);
  int32_t* lab_q = ws_at<int32_t>(ws, w.lab_q);
  int32_t* lab_k = ws_at<int32_t>(ws, w.lab_k);
  int32_t* perm_q = ws_at<int32_t>(ws, w.perm_q);
  int32_t* perm_k = ws_at<int32_t>(ws, w.perm_k);
  int32_t* start_q = ws_at<int32_t>(ws, w.start_q);
  int32_t* start_k = ws_at<int32_t>(ws, w.start_k);
  uint8_t* sel_w = sel ? sel : ws_at<uint8_t>(ws, w.sel);
  hipError_t e = apply_topology(&g);
  if (e == hipSuccess && !(flags & SVG2_FLAG_INIT_GIVEN)) {
    e = launch_km_init(g, q, s, prm->C_q, mu_q, st);
    if (e == hipSuccess) e = launch_km_init(g, k, s, prm->C_k, mu_k, st);
  }
  if (e == hipSuccess) e = launch_kmeans(g, q, s, prm->C_q, prm->iters, mu_q, lab_q, perm_q, start_q, sc, st);
  if (e == hipSuccess) e = launch_kmeans(g, k, s, prm->C_k, prm->iters, mu_k, lab_k, perm_k, start_k, sc, st);
  if (e == hipSuccess)
    e = launch_svg2_select(g, prm->C_q, prm->C_k, prm->p, mu_q, mu_k, start_q, start_k, sel_w,
                           ws_at<char>(ws, w.segs), ws_at<int32_t>(ws, w.nseg), ws_at<int32_t>(ws, w.nkeys),
                           ws_at<int32_t>(ws, w.ord), ws_at<int32_t>(ws, w.rbp), st);
  if (e == hipSuccess) e = launch_gather_rows(g, k, s, perm_k, ws_at<char>(ws, w.kp), st);
  if (e == hipSuccess) e = launch_gather_rows(g, v, s, perm_k, ws_at<char>(ws, w.vp), st);
  if (e == hipSuccess)
    e = launch_svg2_attention(g, q, s, ws_at<char>(ws, w.kp), ws_at<char>(ws, w.vp), o, so, out == SVG_BF16, perm_q,
                              start_q, ws_at<int32_t>(ws, w.ord), ws_at<int32_t>(ws, w.rbp), ws_at<char>(ws, w.segs),
                              ws_at<int32_t>(ws, w.nseg), ws_at<int32_t>(ws, w.nkeys), prm->C_q, prm->C_k, st);
  return e == hipSuccess ? SVG_OK : hip_fail(e, "svg2_forward");
}

svg_status svg_layer_forward(const svg_geom* geom, svg_dtype in, svg_dtype out, const void* q, const void* k,
                             const void* v, svg_strides s, void* o, svg_strides so, const int32_t* rows,
                             int32_t n_rows, float fallback_rel_mse, const int32_t* modes_in, int32_t* labels_out,
                             float* stats_out, int32_t flags, void* ws, size_t ws_bytes, void* stream) {
  return layer_forward_impl(geom, in, out, q, k, v, s, o, so, rows, n_rows, fallback_rel_mse, modes_in, labels_out,
                            stats_out, flags, ws, ws_bytes, false, stream);
}

svg_status svg_layer_forward_noalloc(const svg_geom* geom, svg_dtype in, svg_dtype out, const void* q,
                                     const void* k, const void* v, svg_strides s, void* o, svg_strides so,
                                     const int32_t* rows, int32_t n_rows, float fallback_rel_mse,
                                     const int32_t* modes_in, int32_t* labels_out, float* stats_out, int32_t flags,
                                     void* stream) {
  return layer_forward_impl(geom, in, out, q, k, v, s, o, so, rows, n_rows, fallback_rel_mse, modes_in, labels_out,
                            stats_out, flags, nullptr, 0, true, stream);
}

size_t svg_noalloc_scratch_bytes(void) { return kStaticScratchBytes; }

}  // extern "C"
