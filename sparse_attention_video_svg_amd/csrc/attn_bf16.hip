// bf16 block-banded flash attention (svg_sparse_attention) and the bf16
// profiling sweep (svg_profile_heads) for gfx950.
//
// What is computed: per head, O = softmax(Q K^T * scale over the head's
// active keys) V (rebuttal answer to Weakness 1 for the masks; "Sparse
// VideoGen" abstract for the customised kernels and layout transformation;
// Sparse-vDiT review for the per-mode kernels with heads of one mode fused).
//
// How (MI355X-first):
//  * A workgroup is 8 waves x 32 query rows (BM = 256) and walks its key-tile
//    ranges in tiles of BN = 64 keys.  K and V tiles are fetched straight
//    into LDS with global_load_lds_dwordx4 (no VGPR staging), double
//    buffered, one barrier per tile; two waves share each SIMD.
//  * Scores are formed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: Q stays in registers as the B operand, each
//    lane then owns one query and 16 keys per 32-key block, so the row max and
//    row sum need one v_permlane32_swap instead of a butterfly.
//  * O^T += V^T P^T reuses the score registers as the B operand directly (the
//    key order of the accumulator layout is matched on the V side); V^T
//    fragments come from ds_read_b64_tr_b16 transposing LDS reads, so V is
//    never transposed in memory.
//  * LDS rows are XOR-swizzled in 16-byte chunks (different patterns for K's
//    row reads and V's transposed reads) so neither read conflicts on banks.
//  * Online softmax in exp2 with the scale folded into one multiply; the
//    running max is only moved (and O rescaled) when a tile's max exceeds it
//    by more than 2^8, a wave-uniform branch that is almost never taken after
//    the first tile.  Element masks are evaluated only on tiles that are not
//    entirely inside every row's run; tiles no row of a wave needs are skipped
//    by that wave.
//  * Workgroup ids are remapped so that each XCD (ids are dealt round-robin
//    to the device's XCDs, eight on an MI355X) walks runs of consecutive query
//    tiles of one head, which share their K/V band in that XCD's L2; runs are
//    handed out in the longest-head-first order of svg_build_blocks.
#include "attn_common.h"

namespace svg {

// One query tile (32 * WAVES rows) of one head.  VIRT: a temporal head read
// and written through the token-major index map instead of explicitly
// permuted copies.
template <int D, bool OUT_BF16, bool VIRT, int WAVES, int STAGES>
__device__ __forceinline__ void attn_tile(const KGeom& g, const AttnPtrs& a, int bh, int qt, int mode, int nQT,
                                          __bf16 (*lds)[2][TileCfg<D>::TILE_ELEMS], int wave, int lane) {
  constexpr int BMW = 32 * WAVES;
  const int hh = lane >> 5;
  const int b = bh / g.H, h = bh % g.H;
  // temporal heads: K, V from their token-major copies (VIRT: through the
  // index map); Q and O from / to their copies when the caller gave them,
  // else through the index map (rows are then read and written once each)
  const bool temporal = mode == SVG_TEMPORAL;
  const bool use_p = temporal && !VIRT;
  const bool q_p = use_p && a.qp != nullptr, o_p = use_p && a.op != nullptr;
  const svg_strides skv = use_p ? a.sp : a.s, sq = q_p ? a.sp : a.s, sout = o_p ? a.sop : a.so;
  const int64_t ibase = (int64_t)b * skv.b + (int64_t)h * skv.h;
  const int64_t obase = (int64_t)b * sout.b + (int64_t)h * sout.h;
  const __bf16* Q = static_cast<const __bf16*>(q_p ? a.qp : a.q) + (int64_t)b * sq.b + (int64_t)h * sq.h;
  const __bf16* K = static_cast<const __bf16*>(use_p ? a.kp : a.k) + ibase;
  const __bf16* V = static_cast<const __bf16*>(use_p ? a.vp : a.v) + ibase;
  char* O = static_cast<char*>(o_p ? a.op : a.o);
  constexpr int OE = OUT_BF16 ? 2 : 4;  // output element bytes
  const bool q_map = temporal && !q_p, o_map = temporal && !o_p;
  auto qrow = [&g, q_map](int r) { return q_map ? perm_inv_row(g, r) : r; };
  auto orow_of = [&g, o_map](int r) { return o_map ? perm_inv_row(g, r) : r; };

  const int4 rg = reinterpret_cast<const int4*>(a.ranges)[(int64_t)bh * nQT + qt];

  // This lane's query row and its Q fragment (B operand of S^T = K Q^T).
  const int xq = qt * BMW + wave * 32 + (lane & 31);
  const bool valid = xq < g.L;
  const int xqc = valid ? xq : g.L - 1;
  bf16x8 qf[D / 16];
  load_q<D>(qf, Q + (int64_t)qrow(xqc) * sq.x, hh);
  int lo, hi;
  row_interval(g, mode, xqc, lo, hi);

  Flash<D> st;
  run_sweep<D, VIRT, WAVES, STAGES>(st, qf, K, V, skv.x, g, rg, lo, hi, valid, lds, wave, lane);

  // Epilogue: lane (query, h) holds dims 32*db + 8*(r/4) + 4*h + r%4.
  const float l_tot = half_sum(st.l_part);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  // the output row and column offset are formed anew from the lane id here
  // (read in asm so that it is not shared with the one taken before the
  // sweep), so that nothing of them stays live across the key loop
  int lid;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lid));
  const int xo = qt * BMW + wave * 32 + (lid & 31), ho = lid >> 5;
  if (xo < g.L) {
    char* orow = O + (obase + (int64_t)orow_of(xo) * sout.x) * OE;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = db * 32 + 8 * g4 + 4 * ho;
        f32x4 v4 = {st.o[db][4 * g4] * inv, st.o[db][4 * g4 + 1] * inv, st.o[db][4 * g4 + 2] * inv,
                    st.o[db][4 * g4 + 3] * inv};
        if (OUT_BF16) {
          bf16x4 b4 = __builtin_convertvector(v4, bf16x4);
          *reinterpret_cast<bf16x4*>(orow + d0 * 2) = b4;
        } else {
          *reinterpret_cast<f32x4*>(orow + d0 * 4) = v4;
        }
      }
    }
  }
}

// d 64: registers capped at 128 (four waves per SIMD), so that two
// workgroups share a CU and, not being in lock step, overlap one's softmax
// with the other's MFMAs (the softmax outweighs the MFMAs at d 64)
template <int D, bool OUT_BF16, int WAVES, int STAGES>
__global__ __launch_bounds__(64 * WAVES, (D == 64 ? 4 : WAVES <= 6 ? 2 : 1)) void k_attn_bf16(KGeom g, AttnPtrs a, int32_t nQT,
                                                                                int32_t total) {
  using C = TileCfg<D, WAVES>;
  constexpr int BMW = 32 * WAVES;
  extern __shared__ __attribute__((aligned(16))) __bf16 lds_raw[];
  auto lds = reinterpret_cast<__bf16 (*)[2][C::TILE_ELEMS]>(lds_raw);  // [stage][K, V]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // XCD-aware remap of the workgroup id, then longest-head-first order.
  const int w = blockIdx.x;
  const int logical = xcd_logical(w, g.nxcd, kXcdRun);
  if (logical >= total) return;
  const int bh = a.order[logical / nQT];
  const int qt = logical % nQT;
  const int mode = a.modes[bh];

  if (mode == SVG_SKIP) {  // Sparse-vDiT head skipping: the output is zero
    constexpr int OE = OUT_BF16 ? 2 : 4;
    constexpr int CPRO = D * OE / 16;
    const int b = bh / g.H, h = bh % g.H;
    const int64_t obase = (int64_t)b * a.so.b + (int64_t)h * a.so.h;
    char* O = static_cast<char*>(a.o);
    for (int c = tid; c < BMW * CPRO; c += 64 * WAVES) {
      const int r = qt * BMW + c / CPRO;
      if (r < g.L)
        *reinterpret_cast<int4*>(O + (obase + (int64_t)r * a.so.x) * OE + (c % CPRO) * 16) = make_int4(0, 0, 0, 0);
    }
    return;
  }
  if (mode == SVG_TEMPORAL && (a.flags & SVG_FLAG_VIRTUAL_PERMUTE))
    attn_tile<D, OUT_BF16, true, WAVES, STAGES>(g, a, bh, qt, mode, nQT, lds, wave, lane);
  else
    attn_tile<D, OUT_BF16, false, WAVES, STAGES>(g, a, bh, qt, mode, nQT, lds, wave, lane);
}

// Partial (m, l, acc) of one output of one sampled row: acc in the
// accumulator layout order is written back to dims order.  A row with no key
// in the slice (m = -inf) writes only (m, l); the merge skips its acc.
template <int D>
__device__ __forceinline__ void store_partial(const Flash<D>& st, float* acc, float* ml, int hh) {
  const float l_tot = half_sum(st.l_part);
  if (hh == 0) {
    ml[0] = st.m_ref;
    ml[1] = l_tot;
  }
  if (st.m_ref == -INFINITY) return;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = db * 32 + 8 * g4 + 4 * hh;
      *reinterpret_cast<f32x4*>(acc + d0) =
          f32x4{st.o[db][4 * g4], st.o[db][4 * g4 + 1], st.o[db][4 * g4 + 2], st.o[db][4 * g4 + 3]};
    }
}

// ---------------------------------------------------------------------------
// Sampled-row sweeps (profiling and mode search): the attention of the
// sampled rows under one mask, a single online-softmax state swept by the
// same machinery as the attention kernel (8 waves x 32 rows, K/V ring in
// LDS).  Each row's keys are one run [lo, hi) (its working-layout interval of
// the mode) plus the text prefix; the rows of a workgroup are taken in an
// order that keeps their runs close (ascending token for the frame-major
// modes, ascending position for the temporal band), so a workgroup loads only
// the union of their runs, cut into `nsplit` slices of tiles so that the grid
// fills the chip; the merge combines the slices.  VIRT: the temporal band,
// with keys gathered in token-major order through the index map.  Waves skip
// the tiles none of their rows needs.  Workgroup ids are remapped so that the
// chunks of rows sharing one slice of one head run together on one XCD and
// share those K/V tiles in its L2.  The partial state of (row, slice) goes to
// slot ((bh * n_rows + row) * nsplit + slice) * nstates + state.
// One work item of a sweep: rows [chunk * BMW, +BMW) of the sampled rows in
// `rows` order, key slice `split` of their union, head bh, under `mode`.
template <int D, bool VIRT, int WAVES, int STAGES>
__device__ __forceinline__ void prof_item(const KGeom& g, const __bf16* __restrict__ q,
                                          const __bf16* __restrict__ k, const __bf16* __restrict__ v,
                                          const svg_strides& s, const int32_t* __restrict__ rows,
                                          const int32_t* __restrict__ ord_r, int32_t n_rows, int32_t nsplit,
                                          int chunk, int split, int bh, int32_t mode, int32_t state, int32_t nstates,
                                          float* __restrict__ part_acc, float* __restrict__ part_ml,
                                          __bf16 (*lds)[2][TileCfg<D, WAVES>::TILE_ELEMS], int (*wb)[WAVES],
                                          int wave, int lane) {
  constexpr int BMW = 32 * WAVES;
  const int hh = lane >> 5;
  const int b = bh / g.H, h = bh % g.H;
  const int64_t base = (int64_t)b * s.b + (int64_t)h * s.h;
  const int rk = chunk * BMW + wave * 32 + (lane & 31);
  const bool valid = rk < n_rows;
  const int x = sampled_row(g, rows[valid ? rk : n_rows - 1]);
  int lo, hi;
  if (VIRT) {  // the row's band in token-major order: x = T + i*F + j -> T + j*N + i
    const int u = x - g.T;
    const int i = fastdiv(u, g.divF_mul, g.divF_shift), j = u - i * g.F;
    row_interval(g, SVG_TEMPORAL, x < g.T ? x : g.T + j * g.N + i, lo, hi);
  } else {
    row_interval(g, mode, x, lo, hi);
  }
  // the workgroup's union of runs -> tile ranges (text tiles first)
  const int wlo = wave_min_i(valid ? lo : INT_MAX), whi = wave_max_i(valid ? hi : INT_MIN);
  if (lane == 0) {
    wb[0][wave] = wlo;
    wb[1][wave] = whi;
  }
  __syncthreads();
  int ulo = wb[0][0], uhi = wb[1][0];
#pragma unroll
  for (int i = 1; i < WAVES; ++i) {
    ulo = min(ulo, wb[0][i]);
    uhi = max(uhi, wb[1][i]);
  }
  const int bs = ulo / kBN, be = (uhi + kBN - 1) / kBN, te = (g.T + kBN - 1) / kBN;
  int4 u4;
  if (g.T == 0)
    u4 = make_int4(bs, be, 0, 0);
  else if (te >= bs)
    u4 = make_int4(0, max(be, te), 0, 0);
  else
    u4 = make_int4(0, te, bs, be);
  // this workgroup's slice of the concatenated tile sequence
  const int n1 = u4.y - u4.x, nt = n1 + (u4.w - u4.z);
  const int t0 = (int)((int64_t)nt * split / nsplit), t1 = (int)((int64_t)nt * (split + 1) / nsplit);
  int4 rg;
  rg.x = u4.x + min(t0, n1);
  rg.y = u4.x + min(t1, n1);
  rg.z = u4.z + max(t0 - n1, 0);
  rg.w = u4.z + max(t1 - n1, 0);

  bf16x8 qf[D / 16];
  load_q<D>(qf, q + base + (int64_t)x * s.x, hh);
  Flash<D> st;
  run_sweep<D, VIRT, WAVES, STAGES>(st, qf, k + base, v + base, s.x, g, rg, lo, hi, valid, lds, wave, lane);
  if (valid) {
    // temporal rows come in position order; ord_r maps them back
    const int r = VIRT ? min(max(ord_r[rk], 0), n_rows - 1) : rk;  // (a permutation for valid rows)
    const int64_t o = (((int64_t)bh * n_rows + r) * nsplit + split) * nstates + state;
    store_partial<D>(st, part_acc + o * D, part_ml + o * 2, hh);
  }
}

template <int D, bool VIRT, int WAVES, int STAGES>
__global__ __launch_bounds__(64 * WAVES, (WAVES <= 6 ? 2 : 1)) void k_prof_sweep(
    KGeom g, const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    svg_strides s, const int32_t* __restrict__ rows, const int32_t* __restrict__ ord_r, int32_t n_rows,
    int32_t nsplit, int32_t total, int32_t mode, int32_t state, int32_t nstates, float* __restrict__ part_acc,
    float* __restrict__ part_ml) {
  using C = TileCfg<D, WAVES>;
  constexpr int BMW = 32 * WAVES;
  extern __shared__ __attribute__((aligned(16))) __bf16 lds_raw[];
  auto lds = reinterpret_cast<__bf16 (*)[2][C::TILE_ELEMS]>(lds_raw);  // [stage][K, V]
  __shared__ int wb[2][WAVES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int logical = xcd_logical(blockIdx.x, g.nxcd, kXcdRun);
  if (logical >= total) return;
  const int chunks = (n_rows + BMW - 1) / BMW;
  const int chunk = logical % chunks;
  const int split = (logical / chunks) % nsplit, bh = logical / chunks / nsplit;
  prof_item<D, VIRT, WAVES, STAGES>(g, q, k, v, s, rows, ord_r, n_rows, nsplit, chunk, split, bh, mode, state,
                                    nstates, part_acc, part_ml, lds, wb, wave, lane);
}

// All masks of a call in one launch, their work items dealt round-robin
// (item i of mask m at position i * nmask + m): the full-attention items keep
// the matrix cores busy while the short-run masks wait on their loads, and
// the two kinds share each CU instead of running one after the other.  State
// m is mask m; the temporal band goes through the index map (rows in position
// order ord_x, ord_r).
template <int D, int WAVES, int STAGES>
__global__ __launch_bounds__(64 * WAVES, 2) void k_prof_multi(
    KGeom g, const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    svg_strides s, const int32_t* __restrict__ rows, const int32_t* __restrict__ ord_x,
    const int32_t* __restrict__ ord_r, int32_t n_rows, int32_t nsplit, int32_t items, int4 masks, int32_t nmask,
    float* __restrict__ part_acc, float* __restrict__ part_ml) {
  using C = TileCfg<D, WAVES>;
  constexpr int BMW = 32 * WAVES;
  extern __shared__ __attribute__((aligned(16))) __bf16 lds_raw[];
  auto lds = reinterpret_cast<__bf16 (*)[2][C::TILE_ELEMS]>(lds_raw);  // [stage][K, V]
  __shared__ int wb[2][WAVES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int logical = xcd_logical(blockIdx.x, g.nxcd, kXcdRun);
  if (logical >= items * nmask) return;
  const int m = logical % nmask, item = logical / nmask;
  const int mode = m == 0 ? masks.x : m == 1 ? masks.y : m == 2 ? masks.z : masks.w;
  const int chunks = (n_rows + BMW - 1) / BMW;
  const int chunk = item % chunks;
  const int split = (item / chunks) % nsplit, bh = item / chunks / nsplit;
  if (mode == SVG_TEMPORAL)
    prof_item<D, true, WAVES, STAGES>(g, q, k, v, s, ord_x, ord_r, n_rows, nsplit, chunk, split, bh, mode, m, nmask,
                                      part_acc, part_ml, lds, wb, wave, lane);
  else
    prof_item<D, false, WAVES, STAGES>(g, q, k, v, s, rows, nullptr, n_rows, nsplit, chunk, split, bh, mode, m,
                                       nmask, part_acc, part_ml, lds, wb, wave, lane);
}

template <int D, bool OUT_BF16>
static hipError_t launch_attn(const KGeom& g, const AttnPtrs& a, int32_t nQT, int64_t grid, int64_t total,
                              hipStream_t st) {
  constexpr int W = kAttnWaves, S = kAttnStages;
  const size_t lds = (size_t)S * 2 * TileCfg<D>::TILE_ELEMS * sizeof(__bf16);
  auto kern = k_attn_bf16<D, OUT_BF16, W, S>;
  static std::atomic<uint64_t> lds_set{0};
  if (hipError_t e = ensure_dynamic_lds((const void*)kern, lds, lds_set); e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * W), lds, st, g, a, nQT, (int32_t)total);
  return hipGetLastError();
}

hipError_t launch_attention_bf16(const KGeom& g, const AttnPtrs& a, bool out_bf16, hipStream_t st) {
  const int32_t nQT = (g.L + kBM_bf16 - 1) / kBM_bf16;
  const int64_t total = (int64_t)g.B * g.H * nQT;
  const int64_t grid = xcd_grid(total, g.nxcd, kXcdRun);
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  if (g.d == 64)
    return out_bf16 ? launch_attn<64, true>(g, a, nQT, grid, total, st) : launch_attn<64, false>(g, a, nQT, grid, total, st);
  return out_bf16 ? launch_attn<128, true>(g, a, nQT, grid, total, st) : launch_attn<128, false>(g, a, nQT, grid, total, st);
}

template <int D, bool VIRT, int W>
static hipError_t launch_prof(const KGeom& g, const __bf16* q, const __bf16* k, const __bf16* v, svg_strides s,
                              const int32_t* rows, const int32_t* ord_r, int32_t n_rows, int32_t nsplit, int32_t mode,
                              int32_t state, int32_t nstates, float* acc, float* ml, hipStream_t st) {
  constexpr int S = kAttnStages;
  const size_t lds = (size_t)S * 2 * TileCfg<D>::TILE_ELEMS * sizeof(__bf16);
  auto kern = k_prof_sweep<D, VIRT, W, S>;
  static std::atomic<uint64_t> lds_set{0};
  if (hipError_t e = ensure_dynamic_lds((const void*)kern, lds, lds_set); e != hipSuccess) return e;
  const int64_t chunks = (n_rows + 32 * W - 1) / (32 * W);
  const int64_t total = chunks * nsplit * g.B * g.H;
  const int64_t grid = xcd_grid(total, g.nxcd, kXcdRun);
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * W), lds, st, g, q, k, v, s, rows, ord_r, n_rows, nsplit,
                     (int32_t)total, mode, state, nstates, acc, ml);
  return hipGetLastError();
}

// waves per workgroup of the sampled-row sweeps over short runs (4: 128 rows,
// measured faster than 2 and 8 on the HunyuanVideo-shaped layer)
constexpr int kProfWavesBand = 4;

// waves per workgroup of the one-launch sweep of all masks; used at d 64,
// where it measured 17 % faster than one launch per mask on the
// CogVideoX-like layer (at d 128, 2 % slower on the HunyuanVideo-shaped one)
constexpr int kProfWavesMulti = 4;

template <int D>
static hipError_t launch_multi(const KGeom& g, const __bf16* q, const __bf16* k, const __bf16* v, svg_strides s,
                               const int32_t* rows, const int32_t* ord_x, const int32_t* ord_r, int32_t n_rows,
                               int32_t nsplit, const int32_t* modes, int32_t nstates, float* acc, float* ml,
                               hipStream_t st) {
  constexpr int W = kProfWavesMulti, S = kAttnStages;
  if (nstates < 1 || nstates > 4) return hipErrorInvalidValue;
  const size_t lds = (size_t)S * 2 * TileCfg<D>::TILE_ELEMS * sizeof(__bf16);
  auto kern = k_prof_multi<D, W, S>;
  static std::atomic<uint64_t> lds_set{0};
  if (hipError_t e = ensure_dynamic_lds((const void*)kern, lds, lds_set); e != hipSuccess) return e;
  const int64_t chunks = (n_rows + 32 * W - 1) / (32 * W);
  const int64_t items = chunks * nsplit * g.B * g.H;
  const int64_t grid = xcd_grid(items * nstates, g.nxcd, kXcdRun);
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  const int4 masks = make_int4(modes[0], nstates > 1 ? modes[1] : 0, nstates > 2 ? modes[2] : 0,
                               nstates > 3 ? modes[3] : 0);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * W), lds, st, g, q, k, v, s, rows, ord_x, ord_r, n_rows,
                     nsplit, (int32_t)items, masks, nstates, acc, ml);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_sweeps(const KGeom& g, const __bf16* q, const __bf16* k, const __bf16* v, svg_strides s,
                                const int32_t* rows, int32_t n_rows, int32_t ksplit, const int32_t* ord_x,
                                const int32_t* ord_r, const int32_t* modes, int32_t nstates, float* acc, float* ml,
                                hipStream_t st) {
  if constexpr (D == 64) {
    return launch_multi<D>(g, q, k, v, s, rows, ord_x, ord_r, n_rows, ksplit, modes, nstates, acc, ml, st);
  } else {
    for (int32_t i = 0; i < nstates; ++i) {
      hipError_t e;
      // masks with short runs per row take workgroups of kProfWavesBand waves (fewer rows, so the union of
      // their runs stays close to each row's own); full attention the attention kernel's 8
      if (modes[i] == SVG_TEMPORAL)
        e = launch_prof<D, true, kProfWavesBand>(g, q, k, v, s, ord_x, ord_r, n_rows, ksplit, SVG_TEMPORAL, i,
                                                 nstates, acc, ml, st);
      else if (modes[i] == SVG_FULL)
        e = launch_prof<D, false, kAttnWaves>(g, q, k, v, s, rows, nullptr, n_rows, ksplit, modes[i], i, nstates,
                                              acc, ml, st);
      else
        e = launch_prof<D, false, kProfWavesBand>(g, q, k, v, s, rows, nullptr, n_rows, ksplit, modes[i], i,
                                                  nstates, acc, ml, st);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
}

hipError_t launch_sample_sweeps(const KGeom& g, const void* q, const void* k, const void* v, svg_strides s,
                                const int32_t* rows, int32_t n_rows, int32_t ksplit, const int32_t* ord_x,
                                const int32_t* ord_r, const int32_t* modes, int32_t nstates, float* acc, float* ml,
                                hipStream_t st) {
  const __bf16 *bq = static_cast<const __bf16*>(q), *bk = static_cast<const __bf16*>(k),
               *bv = static_cast<const __bf16*>(v);
  if (g.d == 64)
    return launch_sweeps<64>(g, bq, bk, bv, s, rows, n_rows, ksplit, ord_x, ord_r, modes, nstates, acc, ml, st);
  return launch_sweeps<128>(g, bq, bk, bv, s, rows, n_rows, ksplit, ord_x, ord_r, modes, nstates, acc, ml, st);
}

}  // namespace svg
