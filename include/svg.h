/*
 * svg.h - C ABI of libsvg.so: Sparse VideoGen spatial/temporal sparse 3D
 * attention for video diffusion transformers, native to MI355X (gfx950).
 *
 * The method (pages cited by title and section):
 *  - "Sparse Video-Gen ..." authors' rebuttal, answer to Weakness 1: a video
 *    of N frames with F tokens each is flattened as x = i*F + j.  A spatial
 *    head keeps pairs with |floor(x1/F) - floor(x2/F)| < a1 (a block band);
 *    a temporal head keeps pairs with |(x1 mod F) - (x2 mod F)| < a2
 *    (2N-1 slanted diagonals).  Answer on profiling: the head type is decided
 *    online at every diffusion step and layer, right before attention.
 *  - "Sparse VideoGen" abstract: online profiling predicts each head's type;
 *    a hardware-efficient layout transformation plus custom kernels turn the
 *    sparsity into speed.
 *  - "Sparse-vDiT" review, "What carries the argument": per-head modes full /
 *    skip / diagonal / multi-diagonal / vertical stripe, heads that share a
 *    mode fused into one operation, the multi-diagonal pattern rearranged into
 *    a diagonal one for a window kernel.
 *
 * Conventions for every entry point
 *  - Tensors are [B, H, L, d] with d contiguous, L = T + N*F tokens (a text
 *    prefix of T tokens first, then the video frame-major).  Element strides
 *    for b, h and token are given by svg_strides; rows must be 16-byte aligned
 *    (base pointer and every stride times the element size multiples of 16).
 *  - All pointers except `geom`, `BM`, `BN`, `bytes` are DEVICE pointers owned
 *    by the caller.  The library never allocates, frees or keeps a pointer;
 *    scratch memory is the caller's workspace, sized by svg_workspace_bytes.
 *  - No output of a call may share memory with an input of that call (the
 *    kernels read rows that other workgroups of the same launch write); an
 *    output starting at an input's address is rejected with SVG_E_INVALID.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every
 *    call only enqueues work on it and returns; nothing synchronises.
 *  - Return value: SVG_OK, or an error status.  On any error nothing has been
 *    enqueued and no output was touched (except SVG_E_HIP, which reports a
 *    failed launch); svg_last_error() then returns a message (thread-local).
 *  - Device-side contents are read on the device only; the library checks
 *    none of them.  Modes must be values of svg_mode: any other value is
 *    undefined behaviour.  A list of sampled rows must hold ascending
 *    distinct video rows in [T, L); every kernel clamps a row into [T, L) as
 *    it reads it, so a list that breaks this contract gives unspecified
 *    labels and statistics but never an access outside the caller's
 *    buffers.  The Python binding checks both on the host only in debug mode
 *    (SVG_DEBUG=1 in the environment).
 */
#ifndef SVG_H
#define SVG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SVG_ABI_VERSION 1

typedef enum {
  SVG_OK = 0,
  SVG_E_INVALID = 1,     /* bad argument (null pointer, bad size, misaligned, ...) */
  SVG_E_UNSUPPORTED = 2, /* valid but not implemented (head dim, dtype pair, tiles) */
  SVG_E_WORKSPACE = 3,   /* workspace missing or smaller than svg_workspace_bytes */
  SVG_E_HIP = 4          /* the HIP runtime reported an error */
} svg_status;

typedef enum { SVG_F32 = 0, SVG_BF16 = 1 } svg_dtype;

/* Per-head attention mode.  SPATIAL / TEMPORAL are the two head types of the
 * rebuttal's Weakness 1 answer; FULL is dense attention (the profiling
 * fallback, and Sparse-vDiT's "full"); SKIP outputs zeros; WINDOW keeps
 * |u1-u2| < window (Sparse-vDiT "diagonal"); STRIPE keeps video keys
 * u2 < stripe (Sparse-vDiT "vertical stripe").  u = x - T is the video index.
 * For every mode but SKIP, text rows (x1 < T) and text keys (x2 < T) are
 * dense. */
typedef enum {
  SVG_SPATIAL = 0,
  SVG_TEMPORAL = 1,
  SVG_FULL = 2,
  SVG_SKIP = 3,
  SVG_WINDOW = 4,
  SVG_STRIPE = 5
} svg_mode;

typedef struct {
  int32_t B, H;   /* batch, heads */
  int32_t d;      /* head dimension: 64 or 128 */
  int32_t N, F;   /* frames, tokens per frame (both >= 1) */
  int32_t T;      /* text-prefix tokens (>= 0) */
  int32_t a1, a2; /* spatial / temporal thresholds (>= 1) */
  int32_t window; /* WINDOW width (>= 1) */
  int32_t stripe; /* STRIPE key count (>= 1) */
  float scale;    /* softmax scale; 0 means 1/sqrt(d) */
} svg_geom;

typedef struct {
  int64_t b, h, x; /* element strides of batch, head and token; d is contiguous */
} svg_strides;

/* Flags of svg_sparse_attention / svg_layer_forward (and svg_workspace_bytes). */
#define SVG_FLAG_VIRTUAL_PERMUTE 1 /* temporal heads gather rows through the
                                      token-major index instead of reading
                                      explicitly permuted copies */
#define SVG_FLAG_MODE_SEARCH 2     /* svg_workspace_bytes only: size the
                                      workspace for svg_search_modes */
#define SVG_FLAG_FP8_SCORES 4      /* svg_layer_forward (and its workspace):
                                      scores on FP8 E4M3 Q and K, see
                                      svg_quantize_qk; implies the index-map
                                      reads of SVG_FLAG_VIRTUAL_PERMUTE */
#define SVG_FLAG_FP8_PV 8          /* with SVG_FLAG_FP8_SCORES: P.V on the
                                      FP8 matrix cores as well (V to E4M3 by
                                      svg_quantize_v) */

int32_t svg_abi_version(void);
const char* svg_last_error(void);

/* Query and key tile sizes (BM x BN) of the attention kernel for an input
 * dtype and head dim; key-tile ranges must be built with exactly these.
 * Errors: SVG_E_INVALID (null outputs), SVG_E_UNSUPPORTED (dtype/d). */
svg_status svg_tile_config(svg_dtype dtype, int32_t d, int32_t* BM, int32_t* BN);

/* Row sampling for online profiling (rebuttal: answer on profiling, the
 * head type decided at every diffusion step and layer from a few query
 * rows).  Writes `count` distinct video rows of the geometry, drawn
 * uniformly without replacement from [T, T + N*F) and sorted ascending, to
 * the HOST array rows[count] (the caller copies it to the device for
 * svg_profile_heads / svg_layer_forward).  The draw is a pure function of
 * (N*F, T, count, seed): Floyd's sampling (Bentley and Floyd, CACM 1987) on
 * SplitMix64 (Steele, Lea and Flood, OOPSLA 2014) started at `seed`; pass a
 * new seed per call for fresh rows.  Host only: no device work, no stream.
 * Errors: SVG_E_INVALID (geometry, count outside [0, N*F], rows NULL with
 * count > 0), SVG_E_UNSUPPORTED (geometry). */
svg_status svg_sample_rows(const svg_geom* geom, int32_t count, uint64_t seed, int32_t* rows);

/* Workspace needed by svg_layer_forward for this geometry, input dtype,
 * number of sampled rows (0 = no profiling) and flags.  Also covers
 * svg_profile_heads (which needs a subset).  With SVG_FLAG_MODE_SEARCH: the
 * workspace of svg_search_modes (bf16 only).  Writes *bytes.
 * Errors: SVG_E_INVALID (geometry, n_rows, flags), SVG_E_UNSUPPORTED. */
svg_status svg_workspace_bytes(const svg_geom* geom, svg_dtype dtype, int32_t n_rows, int32_t flags,
                               size_t* bytes);

/* Online profiling (rebuttal: answer on when profiling happens; abstract:
 * head types predicted online).  For every (b, h), on the n_rows sampled
 * query rows `rows` (device int32, ascending distinct video rows in [T, L),
 * shared by all heads, e.g. from svg_sample_rows; trusted, see the
 * conventions above), computes full, spatial and temporal attention,
 *   rel_m = sum (O_m - O_full)^2 / sum O_full^2   over rows x d,
 * and writes labels[b*H+h] = SPATIAL if rel_s <= rel_t else TEMPORAL, or FULL
 * when min(rel_s, rel_t) >= fallback_rel_mse; stats[(b*H+h)*3 + {0,1,2}] =
 * {rel_s, rel_t, mean O_full^2}.  Reductions are deterministic.
 * Errors: SVG_E_INVALID / SVG_E_UNSUPPORTED / SVG_E_WORKSPACE / SVG_E_HIP. */
svg_status svg_profile_heads(const svg_geom* geom, svg_dtype dtype, const void* q, const void* k,
                             const void* v, svg_strides s, const int32_t* rows, int32_t n_rows,
                             float fallback_rel_mse, int32_t* labels, float* stats, void* ws,
                             size_t ws_bytes, void* stream);

/* Offline mode search of Sparse-vDiT (review, "What carries the argument":
 * each candidate mode's output scored by its mean squared error against full
 * attention plus a sparsity penalty; full attention kept when every sparse
 * candidate exceeds the threshold; referee report, major comment 1: Eq. (2)
 * has the penalty lam*(1 - S_i), Algorithm 1 has lam*S_i, both offered).
 * For every (b, h), on the sampled query rows (as for svg_profile_heads)
 * computes full, WINDOW, TEMPORAL-band and STRIPE attention and scores the
 * candidates skip (O = 0), window, temporal, stripe:
 *   mse_c = mean over rows x d of (O_c - O_full)^2,  S_c = 1 - nnz_c / L^2
 *   loss_c = mse_c + lam * (1 - S_c)   (penalty 0)  or  mse_c + lam * S_c  (penalty 1)
 * (nnz_c: active pairs of the mode over the whole map, text dense; S = 1 for
 * skip).  modes_out[b*H+h] (device int32) = the candidate with the lowest
 * loss, ties to the earlier in that order, or FULL when every loss > eps.
 * stats_out (device float[B*H*8]): mse_c at +0..3, loss_c at +4..7.
 * Reductions are deterministic.  bf16 inputs only; ws: at least
 * svg_workspace_bytes(geom, SVG_BF16, n_rows, SVG_FLAG_MODE_SEARCH) bytes,
 * 256-byte aligned.  The resulting modes feed svg_layer_forward's modes_in.
 * Errors: SVG_E_INVALID (arguments, lam < 0, non-finite lam/eps, penalty not
 * 0/1), SVG_E_UNSUPPORTED (fp32), SVG_E_WORKSPACE, SVG_E_HIP. */
svg_status svg_search_modes(const svg_geom* geom, svg_dtype dtype, const void* q, const void* k,
                            const void* v, svg_strides s, const int32_t* rows, int32_t n_rows, float lam,
                            float eps, int32_t penalty, int32_t* modes_out, float* stats_out, void* ws,
                            size_t ws_bytes, void* stream);

/* Key-tile lists (rebuttal Weakness 1: block-banded structure; abstract:
 * layout transformation).  For each head (modes: device int32[B*H]) and each
 * query tile qb of BM rows of the head's working layout (token-major for
 * TEMPORAL heads, frame-major otherwise), writes
 * ranges[((b*H+h)*nQT + qb)*4 + {0,1,2,3}] = {s1, e1, s2, e2}: two sorted,
 * disjoint half-open ranges of key tiles of BN keys (empty when s == e) whose
 * union is exactly the tiles holding an active pair.  nQT = ceil(L/BM).
 * head_order (device int32[B*H]) lists heads by descending work (listed
 * tiles summed over query tiles), ties by ascending head index.
 * Errors: SVG_E_INVALID, SVG_E_UNSUPPORTED (BM/BN not multiples of 16), SVG_E_HIP. */
svg_status svg_build_blocks(const svg_geom* geom, const int32_t* modes, int32_t BM, int32_t BN,
                            int32_t* ranges, int32_t* head_order, void* stream);

/* Layout transformation (abstract: "hardware-efficient tensor layout
 * transformation"; Sparse-vDiT review: token rearrangement).  Forward:
 * dst row T + j*N + i = src row T + i*F + j, text rows copied unchanged.
 * Inverse (inverse != 0): dst row T + i*F + j = src row T + j*N + i.
 * Applied to every (b, h) whose mode is TEMPORAL (all heads if modes NULL);
 * other heads are left untouched.  src and dst must not overlap.
 * Errors: SVG_E_INVALID, SVG_E_UNSUPPORTED, SVG_E_HIP. */
svg_status svg_layout_permute(const svg_geom* geom, svg_dtype dtype, const void* src, svg_strides ss,
                              void* dst, svg_strides ds, const int32_t* modes, int32_t inverse,
                              void* stream);

/* Block-banded sparse attention (abstract: customised kernels; Sparse-vDiT:
 * pattern kernels with heads of one mode fused).  One launch runs every head:
 * O = softmax(Q K^T * scale over the head's active keys) V, fp32 accumulation
 * and softmax, bf16 (or fp32) inputs.  SKIP heads write zeros.  TEMPORAL heads
 * run in token-major order: they read kp/vp (the token-major copies of K and
 * V from svg_layout_permute, strides sp), and qp and op likewise when those
 * are given (strides sp for qp, sop for op); with qp NULL their query rows
 * are read from q, with op NULL their outputs written to o, through the
 * index map (each row once, so o then needs no inverse permute).  With
 * SVG_FLAG_VIRTUAL_PERMUTE they read q/k/v and write o through the index map
 * (qp, kp, vp, op may then all be NULL).  Every combination gives the same
 * outputs, bit for bit.  ranges / head_order come from svg_build_blocks
 * with the BM, BN of svg_tile_config(in, d), which are passed again here for
 * checking.  Supported (in, out): (F32, F32), (BF16, BF16), (BF16, F32).
 * Errors: SVG_E_INVALID, SVG_E_UNSUPPORTED, SVG_E_HIP. */
svg_status svg_sparse_attention(const svg_geom* geom, svg_dtype in, svg_dtype out, const void* q,
                                const void* k, const void* v, svg_strides s, const void* qp,
                                const void* kp, const void* vp, svg_strides sp, void* o,
                                svg_strides so, void* op, svg_strides sop, const int32_t* modes,
                                const int32_t* ranges, const int32_t* head_order, int32_t BM,
                                int32_t BN, int32_t flags, void* stream);

/* FP8 scores, step 1: quantisation of Q and K to FP8 E4M3 (OCP "fn"
 * encoding: bias 7, 3 mantissa bits, max 448, no infinities).  The pages
 * only report that Sparse-vDiT composes with FP8 (Sparse-vDiT review,
 * editorial extensions); the scheme is ours: every scale is the smallest
 * power of two s with 448*s >= max|x| of its group (1 for an all-zero
 * group), the values x/s are rounded to nearest E4M3, ties to even.
 * Q: one scale per token row, q8[(b*H+h)*L + x] row x in natural order,
 * sq[(b*H+h)*L + x].  K: one scale per tile of 64 rows of the head's working
 * layout (token-major, row T + j*N + i, for TEMPORAL heads per `modes`;
 * natural otherwise), k8 rows in that order, sk[(b*H+h)*ceil(L/64) + tile].
 * q8, k8: device uint8[B*H*L*d] (16-byte aligned); sq: float[B*H*L];
 * sk: float[B*H*ceil(L/64)].  bf16 inputs only.
 * Errors: SVG_E_INVALID, SVG_E_UNSUPPORTED (dtype), SVG_E_HIP. */
svg_status svg_quantize_qk(const svg_geom* geom, svg_dtype dtype, const void* q, const void* k, svg_strides s,
                           const int32_t* modes, uint8_t* q8, float* sq, uint8_t* k8, float* sk, void* stream);

/* FP8 scores, step 2: block-banded sparse attention as svg_sparse_attention,
 * with the scores s = (q8 . k8) * sq(row) * sk(tile) * scale from the FP8
 * matrix cores, fp32 softmax and bf16 P.V (V bf16, strides sv).  Inputs from
 * svg_quantize_qk with the same modes; TEMPORAL heads read Q8, V and write O
 * through the token-major index map (k8 is already token-major).  ranges /
 * head_order from svg_build_blocks with svg_tile_config(SVG_BF16, d).
 * out: SVG_BF16 or SVG_F32.
 * Errors: SVG_E_INVALID, SVG_E_UNSUPPORTED (tiles), SVG_E_HIP. */
svg_status svg_sparse_attention_fp8(const svg_geom* geom, svg_dtype out, const uint8_t* q8, const float* sq,
                                    const uint8_t* k8, const float* sk, const void* v, svg_strides sv, void* o,
                                    svg_strides so, const int32_t* modes, const int32_t* ranges,
                                    const int32_t* head_order, int32_t BM, int32_t BN, void* stream);

/* FP8 P.V, step 1b: V to FP8 E4M3 with one power-of-two scale per head
 * (Sparse-vDiT review, editorial extensions, as for svg_quantize_qk; the
 * scheme is ours): s_h = the smallest power of two with 448*s_h >= max|v|
 * over the head (1 if all zero), codes = E4M3(v / s_h), nearest, ties to
 * even.  Stored per tile of 64 rows of the head's working layout (as k8),
 * transposed: v8[((b*H+h)*ceil(L/64) + tile)*d*64 + dim*64 + p] is the code
 * of row tile*64 + key(p), dim `dim`, where for p = 32*g + j
 * key(p) = 32*(j/16) + 8*((j%16)/4) + 4*g + j%4 (the order in which the
 * score accumulators hold their keys); rows beyond L encode 0.
 * v8: device uint8[B*H*ceil(L/64)*d*64] (16-byte aligned); sv: float[B*H].
 * bf16 inputs only.  Errors: SVG_E_INVALID, SVG_E_UNSUPPORTED (dtype),
 * SVG_E_HIP. */
svg_status svg_quantize_v(const svg_geom* geom, svg_dtype dtype, const void* v, svg_strides s,
                          const int32_t* modes, uint8_t* v8, float* sv, void* stream);

/* FP8 scores and FP8 P.V, step 2: as svg_sparse_attention_fp8, with the
 * weights of each row taken as p = 2^(x - m + 6) in E4M3, x the score in
 * log2 units and m a running reference max that moves when a tile's max
 * exceeds it by more than 2, so p lies in [2^-9, 2^8] and a key is dropped
 * only below 2^-15 of the reference; P.V and the row sums both come from the
 * E4M3 weights (FP8 matrix cores), the output is scaled by sv[b*H+h] once.
 * Inputs from svg_quantize_qk and svg_quantize_v with the same modes.
 * Errors: SVG_E_INVALID, SVG_E_UNSUPPORTED (tiles), SVG_E_HIP. */
svg_status svg_sparse_attention_fp8_pv(const svg_geom* geom, svg_dtype out, const uint8_t* q8, const float* sq,
                                       const uint8_t* k8, const float* sk, const uint8_t* v8, const float* sv,
                                       void* o, svg_strides so, const int32_t* modes, const int32_t* ranges,
                                       const int32_t* head_order, int32_t BM, int32_t BN, void* stream);

/* SVG2: semantic-aware permutation ("Sparse VideoGen2 ..." explainer,
 * 2. Methodology, A-C).  Q and K rows of each head are clustered
 * independently by k-means into C_q / C_k clusters (Lloyd: `iters`
 * iterations of nearest-centroid assignment, squared Euclidean, ties to the
 * lower index, then the mean of each cluster's tokens, an empty cluster
 * keeping its centroid); tokens are reordered so that every cluster is
 * contiguous (stable inside a cluster); the share of query cluster a's
 * attention on key cluster b is estimated from the centroids as
 * n_b exp(scale * mu_a . mu_b) / sum_b' (...) (n_b: tokens of cluster b), and
 * key clusters are taken in descending estimate (ties to the lower index)
 * while the mass of those taken before is below p; every query token then
 * attends exactly to the keys of its cluster's selected key clusters.
 * Initial centroids: the tokens at floor(c * L / C), or the caller's with
 * SVG2_FLAG_INIT_GIVEN (e.g. the previous step's, the pages' centroid cache). */
typedef struct {
  int32_t C_q, C_k; /* clusters of Q and of K per head, 1 .. 1024 (and <= L) */
  int32_t iters;    /* Lloyd iterations, >= 1 */
  float p;          /* top-p threshold of the cumulative estimated attention, > 0 */
} svg2_params;

#define SVG2_FLAG_INIT_GIVEN 1 /* mu_q / mu_k hold the initial centroids */

/* Workspace of svg2_forward (also enough for svg2_kmeans with C <= max(C_q, C_k)). */
svg_status svg2_workspace_bytes(const svg_geom* geom, const svg2_params* params, size_t* bytes);

/* k-means of one tensor per head (bf16 x [B, H, L, d] with strides s):
 * mu (device float[B*H*C*d]): initial centroids with SVG2_FLAG_INIT_GIVEN,
 * always the final ones; labels (int32[B*H*L]) the last assignment;
 * perm (int32[B*H*L]): token at each position of the cluster order;
 * start (int32[B*H*(C+1)]): first position of each cluster, start[C] = L.
 * Errors: SVG_E_INVALID, SVG_E_UNSUPPORTED, SVG_E_WORKSPACE, SVG_E_HIP. */
svg_status svg2_kmeans(const svg_geom* geom, svg_dtype dtype, const void* x, svg_strides s, int32_t C,
                       int32_t iters, int32_t flags, float* mu, int32_t* labels, int32_t* perm, int32_t* start,
                       void* ws, size_t ws_bytes, void* stream);

/* The SVG2 attention step: k-means of Q and of K, selection, K / V gathered
 * into cluster order, attention over query clusters (queries read and
 * outputs written in the caller's token order).  mu_q / mu_k: device
 * float[B*H*C*d] (in with SVG2_FLAG_INIT_GIVEN, out always); sel (optional,
 * device uint8[B*H*C_q*C_k]): the selection.  Only geometry fields B, H, d,
 * N, F, T (L = T + N*F) and scale are used.
 * Errors: SVG_E_INVALID, SVG_E_UNSUPPORTED, SVG_E_WORKSPACE, SVG_E_HIP. */
svg_status svg2_forward(const svg_geom* geom, const svg2_params* params, svg_dtype in, svg_dtype out,
                        const void* q, const void* k, const void* v, svg_strides s, void* o, svg_strides so,
                        int32_t flags, float* mu_q, float* mu_k, uint8_t* sel, void* ws, size_t ws_bytes,
                        void* stream);

/* One attention layer of the method, as a diffusion step runs it:
 * (with SVG_FLAG_FP8_SCORES the attention is svg_quantize_qk followed by
 * svg_sparse_attention_fp8 and no permuted copies are made; with
 * SVG_FLAG_FP8_PV as well, svg_quantize_qk, svg_quantize_v and
 * svg_sparse_attention_fp8_pv)
 *   modes_in == NULL: profile on `rows` (writes labels_out, stats_out), else
 *   use modes_in (Sparse-vDiT's fixed per-head modes; no profiling, rows and
 *   stats_out unused, labels_out receives a copy of modes_in);
 *   build key-tile lists; permute K and V of TEMPORAL heads to token-major
 *   into the workspace (skipped with SVG_FLAG_VIRTUAL_PERMUTE); sparse
 *   attention, the TEMPORAL heads' query rows read from q and their outputs
 *   written to o through the index map (svg_sparse_attention with qp and op
 *   NULL), so no inverse permute is needed.
 * labels_out: device int32[B*H]; stats_out: device float[B*H*3] (may be NULL
 * when modes_in is given).  ws must hold svg_workspace_bytes(geom, in,
 * modes_in ? 0 : n_rows, flags) bytes, 256-byte aligned.
 * Errors: as the calls it makes. */
svg_status svg_layer_forward(const svg_geom* geom, svg_dtype in, svg_dtype out, const void* q,
                             const void* k, const void* v, svg_strides s, void* o, svg_strides so,
                             const int32_t* rows, int32_t n_rows, float fallback_rel_mse,
                             const int32_t* modes_in, int32_t* labels_out, float* stats_out,
                             int32_t flags, void* ws, size_t ws_bytes, void* stream);

/* svg_layer_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same layer, with the workspace taken from a fixed scratch
 * array that the library holds on each device it runs on (one per device,
 * svg_noalloc_scratch_bytes() = 64 MiB, kept until the process ends).  The
 * layout transformation is always the index-map one (as with
 * SVG_FLAG_VIRTUAL_PERMUTE; results are bit-identical to the explicit one);
 * the profiling sweeps use as many key slices as fit in the scratch, so the
 * statistics can differ from svg_layer_forward's in the last bits of their
 * fp32 sums, while labels and outputs are the same.  Calls no allocating
 * routine.  Every call on a device shares that device's scratch: calls that
 * overlap in time on one device (other streams, other host threads) race and
 * must be ordered by the caller.  flags: 0 or SVG_FLAG_VIRTUAL_PERMUTE.
 * Errors: as svg_layer_forward; SVG_E_UNSUPPORTED for the fp8 flags;
 * SVG_E_WORKSPACE when the layer needs more scratch than the array holds
 * (before anything is enqueued). */
svg_status svg_layer_forward_noalloc(const svg_geom* geom, svg_dtype in, svg_dtype out, const void* q,
                                     const void* k, const void* v, svg_strides s, void* o, svg_strides so,
                                     const int32_t* rows, int32_t n_rows, float fallback_rel_mse,
                                     const int32_t* modes_in, int32_t* labels_out, float* stats_out,
                                     int32_t flags, void* stream);

/* Size in bytes of the fixed scratch of svg_layer_forward_noalloc. */
size_t svg_noalloc_scratch_bytes(void);

#ifdef __cplusplus
}
#endif
#endif /* SVG_H */
