/*
 * CPU oracle for the Sparse VideoGen spatial/temporal sparse-attention path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  The GPU library never
 * links, includes or calls it, and it shares no source with the GPU library.
 *
 * Plain and slow on purpose: every floating-point sum is accumulated in
 * double precision, inputs are float32 (the bf16-rounded values, widened
 * exactly), and masks are evaluated as the literal predicates of the
 * definitions.  The only "clever" routine is og_row_intervals(), which solves
 * each predicate for the key index in closed form so that the big shapes run
 * in minutes; tests pin it to the literal predicate by brute force.
 *
 * Sources (pages under their titles):
 *  - "Sparse Video-Gen: Accelerating Video Diffusion Transformers with
 *    Spatial-Temporal Sparsity", authors' rebuttal, answer to Weakness 1:
 *    token index x = i*F + j, spatial mask |floor(x1/F)-floor(x2/F)| < a1,
 *    temporal mask |(x1 mod F)-(x2 mod F)| < a2; profiling happens at every
 *    step and layer before attention (answer to the profiling question).
 *  - "Sparse VideoGen" abstract: heads are classified online as spatial or
 *    temporal; a layout transformation makes the temporal pattern
 *    hardware-friendly.
 *  - "Sparse-vDiT" review ("What carries the argument"): modes full, skip,
 *    diagonal (window), multi-diagonal (via token rearrangement), vertical
 *    stripe; skipped heads output zeros.
 * Readings where the pages are silent (text prefix, window/stripe geometry,
 * the relative-MSE fallback, tie-breaks) are the ones listed in the design
 * notes and restated at each function below.
 */
#include <math.h>
#include <stdio.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
  int32_t N;      /* frames */
  int32_t F;      /* tokens per frame */
  int32_t T;      /* text-prefix tokens, at indices [0, T) */
  int32_t a1;     /* spatial threshold, > 0 */
  int32_t a2;     /* temporal threshold, > 0 */
  int32_t window; /* diagonal (window) width W: |u1-u2| < W */
  int32_t stripe; /* vertical stripe: video keys u2 < stripe */
} og_geom;

enum {
  OG_SPATIAL = 0,
  OG_TEMPORAL = 1,
  OG_FULL = 2,
  OG_SKIP = 3,
  OG_WINDOW = 4,
  OG_STRIPE = 5,
  /* oracle-only: a temporal head expressed on permuted (token-major) indices */
  OG_TEMPORAL_PERMUTED = 6
};

static int64_t og_ltot(const og_geom* g) { return (int64_t)g->T + (int64_t)g->N * g->F; }
static int64_t iabs64(int64_t a) { return a < 0 ? -a : a; }

/* Layout transformation of the abstract: video token x = T + i*F + j (frame
 * i, position j) moves to x' = T + j*N + i; text tokens stay in place. */
int64_t og_perm(const og_geom* g, int64_t x) {
  if (x < g->T) return x;
  int64_t u = x - g->T;
  int64_t i = u / g->F, j = u % g->F;
  return g->T + j * g->N + i;
}

int64_t og_perm_inv(const og_geom* g, int64_t xp) {
  if (xp < g->T) return xp;
  int64_t up = xp - g->T;
  int64_t j = up / g->N, i = up % g->N;
  return g->T + i * g->F + j;
}

/* Mask predicate on natural (frame-major) indices, query x1, key x2.
 * Text rows and text columns are dense (reading of the text prefix).
 * Spatial: |floor(u1/F) - floor(u2/F)| < a1    (rebuttal, Weakness 1)
 * Temporal: |(u1 mod F) - (u2 mod F)| < a2     (rebuttal, Weakness 1)
 * Window (Sparse-vDiT "diagonal"): |u1 - u2| < W
 * Stripe (Sparse-vDiT "vertical stripe"): u2 < stripe
 * Skip: no key is active (the head outputs zeros).
 * OG_TEMPORAL_PERMUTED: x1, x2 are token-major indices; the predicate is the
 * temporal one evaluated on the inverse-permuted indices. */
int og_mask(const og_geom* g, int mode, int64_t x1, int64_t x2) {
  if (mode == OG_SKIP) return 0;
  if (mode == OG_TEMPORAL_PERMUTED) {
    x1 = og_perm_inv(g, x1);
    x2 = og_perm_inv(g, x2);
    mode = OG_TEMPORAL;
  }
  if (x1 < g->T || x2 < g->T) return 1;
  int64_t u1 = x1 - g->T, u2 = x2 - g->T;
  switch (mode) {
    case OG_SPATIAL: return iabs64(u1 / g->F - u2 / g->F) < g->a1;
    case OG_TEMPORAL: return iabs64(u1 % g->F - u2 % g->F) < g->a2;
    case OG_FULL: return 1;
    case OG_WINDOW: return iabs64(u1 - u2) < g->window;
    case OG_STRIPE: return u2 < g->stripe;
    default: return 0;
  }
}

/* Row copy under the layout transformation: forward writes dst[pi(x)] = src[x],
 * inverse writes dst[x] = src[pi(x)].  Rows are row_bytes long, packed. */
void og_permute_rows(const og_geom* g, int64_t row_bytes, const void* src, void* dst, int inverse) {
  const char* s = (const char*)src;
  char* d = (char*)dst;
  int64_t L = og_ltot(g);
  for (int64_t x = 0; x < L; ++x) {
    int64_t p = og_perm(g, x);
    if (!inverse)
      memcpy(d + p * row_bytes, s + x * row_bytes, (size_t)row_bytes);
    else
      memcpy(d + x * row_bytes, s + p * row_bytes, (size_t)row_bytes);
  }
}

static int64_t mini(int64_t a, int64_t b) { return a < b ? a : b; }
static int64_t maxi(int64_t a, int64_t b) { return a > b ? a : b; }

/* Largest number of intervals og_row_intervals() can return for this
 * geometry: the text columns plus one interval per frame (temporal rows). */
int og_max_intervals(const og_geom* g) { return g->N + 1; }

/* Appends the half-open interval [a, b) to (lo, hi, *n), merging it with the
 * previous one when they touch.  Returns -1 when the capacity max_n would be
 * exceeded (nothing is dropped silently). */
static int push_interval(int64_t a, int64_t b, int64_t* lo, int64_t* hi, int* n, int max_n) {
  if (b <= a) return 0;
  if (*n > 0 && hi[*n - 1] == a) {
    hi[*n - 1] = b;
    return 0;
  }
  if (*n >= max_n) return -1;
  lo[*n] = a;
  hi[*n] = b;
  ++*n;
  return 0;
}

/* Active keys of query row x1 as sorted, disjoint, half-open intervals,
 * obtained by solving each predicate of og_mask() for x2:
 *   spatial : floor(u2/F) in [i1-a1+1, i1+a1-1]  -> one interval of frames
 *   temporal: u2 mod F in [j1-a2+1, j1+a2-1]     -> one interval per frame
 *   window  : u2 in [u1-W+1, u1+W-1]
 *   stripe  : u2 in [0, stripe)
 *   temporal, token-major indices: u2' / N in [j1-a2+1, j1+a2-1]
 * plus the text columns [0, T); a text row sees every key.
 * Returns the number of intervals written, or -1 when more than max_n would
 * be needed (og_max_intervals() is always enough). */
int og_row_intervals(const og_geom* g, int mode, int64_t x1, int64_t* lo, int64_t* hi, int max_n) {
  int64_t T = g->T, N = g->N, F = g->F, L = og_ltot(g);
  int n = 0;
  if (mode == OG_SKIP) return 0;
  if (x1 < T) return push_interval(0, L, lo, hi, &n, max_n) < 0 ? -1 : n;
  if (push_interval(0, T, lo, hi, &n, max_n) < 0) return -1;
  int64_t u1 = x1 - T;
  int64_t a = 0, b = 0; /* one video interval in u coordinates, unless temporal */
  switch (mode) {
    case OG_SPATIAL: {
      int64_t i1 = u1 / F;
      a = maxi(0, i1 - g->a1 + 1) * F;
      b = mini(N, i1 + g->a1) * F;
      break;
    }
    case OG_TEMPORAL: {
      int64_t j1 = u1 % F;
      int64_t jl = maxi(0, j1 - g->a2 + 1), jh = mini(F, j1 + g->a2);
      for (int64_t i2 = 0; i2 < N; ++i2) /* whole frames merge into one interval */
        if (push_interval(T + i2 * F + jl, T + i2 * F + jh, lo, hi, &n, max_n) < 0) return -1;
      return n;
    }
    case OG_TEMPORAL_PERMUTED: {
      int64_t j1 = u1 / N; /* token-major: u' = j*N + i */
      a = maxi(0, j1 - g->a2 + 1) * N;
      b = mini(F, j1 + g->a2) * N;
      break;
    }
    case OG_FULL:
      a = 0;
      b = N * F;
      break;
    case OG_WINDOW:
      a = maxi(0, u1 - g->window + 1);
      b = mini(N * F, u1 + g->window);
      break;
    case OG_STRIPE:
      a = 0;
      b = mini(N * F, g->stripe);
      break;
    default:
      return 0;
  }
  if (push_interval(T + a, T + b, lo, hi, &n, max_n) < 0) return -1;
  return n;
}

/* og_row_intervals() for the internal callers, whose buffers hold
 * og_max_intervals() entries: an overflow there is a bug, so it aborts. */
static int row_intervals_checked(const og_geom* g, int mode, int64_t x1, int64_t* lo, int64_t* hi) {
  int n = og_row_intervals(g, mode, x1, lo, hi, og_max_intervals(g));
  if (n < 0) {
    fprintf(stderr, "svg oracle: interval capacity exceeded (mode %d, row %lld)\n", mode, (long long)x1);
    abort();
  }
  return n;
}

/* Softmax attention of one query row over an explicit key list (fp64).
 * s = (q . k) * scale; O = sum exp(s - max) v / sum exp(s - max).
 * No active key -> O = 0. */
static void attend_row(int32_t d, double scale, const float* qrow, const float* k, const float* v,
                       const int64_t* keys, int64_t nk, double* out, double* sbuf) {
  for (int32_t c = 0; c < d; ++c) out[c] = 0.0;
  if (nk == 0) return;
  double m = -INFINITY;
  for (int64_t t = 0; t < nk; ++t) {
    const float* kr = k + keys[t] * d;
    double s = 0.0;
    for (int32_t c = 0; c < d; ++c) s += (double)qrow[c] * (double)kr[c];
    s *= scale;
    sbuf[t] = s;
    if (s > m) m = s;
  }
  double l = 0.0;
  for (int64_t t = 0; t < nk; ++t) {
    double p = exp(sbuf[t] - m);
    l += p;
    const float* vr = v + keys[t] * d;
    for (int32_t c = 0; c < d; ++c) out[c] += p * (double)vr[c];
  }
  for (int32_t c = 0; c < d; ++c) out[c] /= l;
}

/* Masked attention for one head, every (row, key) pair through og_mask().
 * q, k, v: [L_tot][d] float32; out: [L_tot][d] fp64. Tiny shapes only. */
void og_attention_brute(const og_geom* g, int mode, int32_t d, double scale, const float* q,
                        const float* k, const float* v, double* out) {
  int64_t L = og_ltot(g);
  int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * (size_t)L);
  double* sbuf = (double*)malloc(sizeof(double) * (size_t)L);
  for (int64_t x1 = 0; x1 < L; ++x1) {
    int64_t nk = 0;
    for (int64_t x2 = 0; x2 < L; ++x2)
      if (og_mask(g, mode, x1, x2)) keys[nk++] = x2;
    attend_row(d, scale, q + x1 * d, k, v, keys, nk, out + x1 * d, sbuf);
  }
  free(keys);
  free(sbuf);
}

/* Masked attention for the listed query rows of one head, keys enumerated
 * from og_row_intervals().  out: [n_rows][d] fp64.  OpenMP over rows. */
void og_attention_rows(const og_geom* g, int mode, int32_t d, double scale, const float* q,
                       const float* k, const float* v, const int64_t* rows, int64_t n_rows,
                       double* out) {
  int64_t L = og_ltot(g);
#pragma omp parallel
  {
    int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * (size_t)L);
    double* sbuf = (double*)malloc(sizeof(double) * (size_t)L);
    int64_t* lo = (int64_t*)malloc(sizeof(int64_t) * (size_t)og_max_intervals(g));
    int64_t* hi = (int64_t*)malloc(sizeof(int64_t) * (size_t)og_max_intervals(g));
#pragma omp for schedule(dynamic, 4)
    for (int64_t r = 0; r < n_rows; ++r) {
      int64_t x1 = rows[r];
      int ni = row_intervals_checked(g, mode, x1, lo, hi);
      int64_t nk = 0;
      for (int t = 0; t < ni; ++t)
        for (int64_t x2 = lo[t]; x2 < hi[t]; ++x2) keys[nk++] = x2;
      attend_row(d, scale, q + x1 * d, k, v, keys, nk, out + r * d, sbuf);
    }
    free(keys);
    free(sbuf);
    free(lo);
    free(hi);
  }
}

/* Online profiling of one head on the sampled query rows (rebuttal: "online
 * profiling ... at every diffusion step and every layer"; abstract: the head
 * type is predicted from sampled rows).  Computes full, spatial and temporal
 * attention on the rows, then
 *   rel_m = sum (O_m - O_full)^2 / sum O_full^2   over rows x d,
 * label = SPATIAL if rel_s <= rel_t else TEMPORAL, and FULL when
 * min(rel_s, rel_t) >= fallback.  stats = {rel_s, rel_t, mean O_full^2}. */
void og_profile_head(const og_geom* g, int32_t d, double scale, const float* q, const float* k,
                     const float* v, const int64_t* rows, int64_t n_rows, double fallback,
                     double* stats, int32_t* label) {
  size_t n = (size_t)n_rows * (size_t)d;
  double* of = (double*)malloc(sizeof(double) * n);
  double* os = (double*)malloc(sizeof(double) * n);
  double* ot = (double*)malloc(sizeof(double) * n);
  og_attention_rows(g, OG_FULL, d, scale, q, k, v, rows, n_rows, of);
  og_attention_rows(g, OG_SPATIAL, d, scale, q, k, v, rows, n_rows, os);
  og_attention_rows(g, OG_TEMPORAL, d, scale, q, k, v, rows, n_rows, ot);
  double ss = 0.0, st = 0.0, sf = 0.0;
  for (size_t e = 0; e < n; ++e) {
    double a = os[e] - of[e], b = ot[e] - of[e];
    ss += a * a;
    st += b * b;
    sf += of[e] * of[e];
  }
  double rel_s = ss / sf, rel_t = st / sf;
  stats[0] = rel_s;
  stats[1] = rel_t;
  stats[2] = sf / (double)n;
  double best = rel_s <= rel_t ? rel_s : rel_t;
  if (best >= fallback)
    *label = OG_FULL;
  else
    *label = rel_s <= rel_t ? OG_SPATIAL : OG_TEMPORAL;
  free(of);
  free(os);
  free(ot);
}

/* Number of active (query, key) pairs of a mask over the whole L x L map,
 * summed from the per-row intervals (tests pin it to the literal predicate
 * counted pair by pair).  SKIP has none. */
int64_t og_mask_nnz(const og_geom* g, int mode) {
  int64_t L = og_ltot(g), total = 0;
#pragma omp parallel reduction(+ : total)
  {
    int64_t* lo = (int64_t*)malloc(sizeof(int64_t) * (size_t)og_max_intervals(g));
    int64_t* hi = (int64_t*)malloc(sizeof(int64_t) * (size_t)og_max_intervals(g));
#pragma omp for schedule(static)
    for (int64_t x1 = 0; x1 < L; ++x1) {
      int ni = row_intervals_checked(g, mode, x1, lo, hi);
      for (int t = 0; t < ni; ++t) total += hi[t] - lo[t];
    }
    free(lo);
    free(hi);
  }
  return total;
}

/* Offline mode search of one head ("Sparse-vDiT" review: the search scores
 * each candidate mode's output against full attention by mean squared error
 * plus a sparsity penalty, and keeps full attention when every candidate is
 * above the threshold; the referee report quotes Eq. (2) with the penalty
 * lam*(1 - S_i) and Algorithm 1 with lam*S_i).
 * Candidates, in this order (ties go to the earlier one): skip (O = 0,
 * S = 1), diagonal (WINDOW), multi-diagonal (TEMPORAL band), vertical stripe
 * (STRIPE).  S_i = 1 - nnz_i / L^2 is the fraction of the map a mode skips.
 *   mse_i  = mean over rows x d of (O_i - O_full)^2
 *   loss_i = mse_i + lam * (1 - S_i)   (penalty 0)   or   mse_i + lam * S_i   (penalty 1)
 * mode = the candidate with the lowest loss, or FULL if every loss > eps.
 * mse[4], loss[4], sparsity[4] in candidate order. */
void og_search_head(const og_geom* g, int32_t d, double scale, const float* q, const float* k,
                    const float* v, const int64_t* rows, int64_t n_rows, double lam, double eps,
                    int penalty, double* mse, double* loss, double* sparsity, int32_t* mode) {
  static const int cand[4] = {OG_SKIP, OG_WINDOW, OG_TEMPORAL, OG_STRIPE};
  size_t n = (size_t)n_rows * (size_t)d;
  double L = (double)og_ltot(g);
  double* of = (double*)malloc(sizeof(double) * n);
  double* om = (double*)malloc(sizeof(double) * n);
  og_attention_rows(g, OG_FULL, d, scale, q, k, v, rows, n_rows, of);
  int best = -1;
  for (int c = 0; c < 4; ++c) {
    double se = 0.0;
    if (cand[c] == OG_SKIP) {
      for (size_t e = 0; e < n; ++e) se += of[e] * of[e];
      sparsity[c] = 1.0;
    } else {
      og_attention_rows(g, cand[c], d, scale, q, k, v, rows, n_rows, om);
      for (size_t e = 0; e < n; ++e) {
        double dd = om[e] - of[e];
        se += dd * dd;
      }
      sparsity[c] = 1.0 - (double)og_mask_nnz(g, cand[c]) / (L * L);
    }
    mse[c] = se / (double)n;
    loss[c] = mse[c] + (penalty == 0 ? lam * (1.0 - sparsity[c]) : lam * sparsity[c]);
    if (best < 0 || loss[c] < loss[best]) best = c;
  }
  *mode = loss[best] > eps ? OG_FULL : cand[best];
  free(of);
  free(om);
}

/* Working layout of a head: temporal heads run on token-major indices. */
static int working_mode(int mode) { return mode == OG_TEMPORAL ? OG_TEMPORAL_PERMUTED : mode; }

/* Key-tile list of every query tile, by brute force over elements: tile
 * (qb, kb) is listed iff some (x1 in qb, x2 in kb) is active in the head's
 * working layout.  bitmap: [ceil(L/BM)][ceil(L/BN)] bytes. Tiny shapes. */
void og_blocks_brute(const og_geom* g, int mode, int32_t BM, int32_t BN, uint8_t* bitmap) {
  int64_t L = og_ltot(g);
  int64_t nq = (L + BM - 1) / BM, nkt = (L + BN - 1) / BN;
  int wm = working_mode(mode);
  memset(bitmap, 0, (size_t)(nq * nkt));
  for (int64_t x1 = 0; x1 < L; ++x1)
    for (int64_t x2 = 0; x2 < L; ++x2)
      if (og_mask(g, wm, x1, x2)) bitmap[(x1 / BM) * nkt + x2 / BN] = 1;
}

/* The same bitmap from the per-row intervals (for the large shapes). */
void og_blocks_rows(const og_geom* g, int mode, int32_t BM, int32_t BN, uint8_t* bitmap) {
  int64_t L = og_ltot(g);
  int64_t nq = (L + BM - 1) / BM, nkt = (L + BN - 1) / BN;
  int wm = working_mode(mode);
  memset(bitmap, 0, (size_t)(nq * nkt));
#pragma omp parallel
  {
    int64_t* lo = (int64_t*)malloc(sizeof(int64_t) * (size_t)og_max_intervals(g));
    int64_t* hi = (int64_t*)malloc(sizeof(int64_t) * (size_t)og_max_intervals(g));
#pragma omp for schedule(dynamic, 1)
    for (int64_t qb = 0; qb < nq; ++qb) {
      for (int64_t x1 = qb * BM; x1 < mini(L, (qb + 1) * BM); ++x1) {
        int ni = row_intervals_checked(g, wm, x1, lo, hi);
        for (int t = 0; t < ni; ++t)
          for (int64_t kb = lo[t] / BN; kb <= (hi[t] - 1) / BN; ++kb) bitmap[qb * nkt + kb] = 1;
      }
    }
    free(lo);
    free(hi);
  }
}

/* Longest-first head order: heads sorted by work (listed tiles) descending,
 * equal work by ascending head index. */
void og_head_order(int32_t n_heads, const int64_t* work, int32_t* order) {
  for (int32_t h = 0; h < n_heads; ++h) {
    int32_t rank = 0;
    for (int32_t o = 0; o < n_heads; ++o)
      if (work[o] > work[h] || (work[o] == work[h] && o < h)) ++rank;
    order[rank] = h;
  }
}

int og_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
