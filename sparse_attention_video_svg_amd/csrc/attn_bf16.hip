// bf16 block-banded flash attention (svg_sparse_attention) and the bf16
// profiling sweep (svg_profile_heads) for gfx950.
//
// What is computed: per head, O = softmax(Q K^T * scale over the head's
// active keys) V (rebuttal answer to Weakness 1 for the masks; "Sparse
// VideoGen" abstract for the customised kernels and layout transformation;
// Sparse-vDiT review for the per-mode kernels with heads of one mode fused).
//
// How (MI355X-first):
//  * A workgroup is 4 waves x 32 query rows (BM = 128) and walks its key-tile
//    ranges in tiles of BN = 64 keys.  K and V tiles are fetched straight
//    into LDS with global_load_lds_dwordx4 (no VGPR staging), double
//    buffered, one barrier per tile.
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
//  * Workgroup ids are remapped so that each XCD (ids are dealt round-robin to
//    the 8 XCDs) walks runs of consecutive query tiles of one head, which
//    share their K/V band in that XCD's L2; runs are handed out in the
//    longest-head-first order of svg_build_blocks.
#include "svg_device.h"

namespace svg {

constexpr int kBM = kBM_bf16, kBN = kBN_bf16;
constexpr float kRescaleTau = 8.0f;  // log2 headroom before the running max moves
constexpr int kXcdRun = 32;          // consecutive query tiles per XCD turn

template <int D>
struct TileCfg {
  static constexpr int CR = D / 8;                   // 16-byte chunks per row
  static constexpr int RPL = 16 / CR;                // rows per 256-byte LDS line
  static constexpr int CHUNKS = kBN * CR;            // chunks per K (or V) tile
  static constexpr int LOADS = CHUNKS / 256;         // per thread per tensor
  static constexpr int TILE_ELEMS = kBN * D;         // bf16 elements per tile
  // K rows are read 16 keys x one chunk at a time: spread keys over chunks.
  __device__ static __forceinline__ int swz_k(int r) { return (r / RPL) % CR; }
  // V is read 4 keys x 4 chunks at a time (transposing reads): spread the
  // 4 consecutive keys over 4 different 64-byte quarters of the line.
  __device__ static __forceinline__ int swz_v(int r) { return 4 * ((r / RPL) % (CR / 4)); }
};

__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Issue the direct-to-LDS loads of one K tile and one V tile (all 256 threads).
// Chunk p of the tile (row r = p / CR, LDS position pos = p % CR) receives
// global chunk pos ^ swz(r) of key row kt0 + r (clamped to the last row).
template <int D, typename RowMap>
__device__ __forceinline__ void load_kv_tile(const __bf16* __restrict__ K, const __bf16* __restrict__ V,
                                             int64_t sx, int kt0, int L, RowMap phys, __bf16* lds_k,
                                             __bf16* lds_v, int wave, int lane) {
  using C = TileCfg<D>;
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    const int seg = i * 4 + wave;  // 64-chunk segment written by this instruction
    const int p = seg * 64 + lane;
    const int r = p / C::CR, pos = p % C::CR;
    int row = kt0 + r;
    row = row < L ? row : L - 1;
    const int64_t off = (int64_t)phys(row) * sx;
    const __bf16* gk = K + off + ((pos ^ C::swz_k(r)) * 8);
    const __bf16* gv = V + off + ((pos ^ C::swz_v(r)) * 8);
    __builtin_amdgcn_global_load_lds((const void*)gk, (SVG_LDS void*)(lds_k + seg * 64 * 8), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((const void*)gv, (SVG_LDS void*)(lds_v + seg * 64 * 8), 16, 0, 0);
  }
}

// S^T block (32 keys x 32 queries) for key block kb2 of the tile in LDS.
template <int D>
__device__ __forceinline__ f32x16 score_block(const __bf16* lds_k, const bf16x8* qf, int kb2, int lane) {
  using C = TileCfg<D>;
  f32x16 acc = {};
  const int m = kb2 * 32 + (lane & 31);
  const int hh = lane >> 5;
  const int sw = C::swz_k(m);
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const int pos = (2 * ks + hh) ^ sw;
    const bf16x8 kf = *reinterpret_cast<const bf16x8*>(lds_k + m * D + pos * 8);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], acc, 0, 0, 0);
  }
  return acc;
}

// V^T fragment (32 dims x 16 keys) of key step s16 and dim block db, in the
// key order of the score accumulator: element e of lane (dim, h) holds key
// 16*s16 + 8*(e/4) + 4*h + e%4.  Two transposing reads, each serving four
// keys; source lane i of a 16-lane group points at key kbase + i/4, dims
// dbase + 4*(i%4) .. +3.
template <int D>
__device__ __forceinline__ bf16x8 v_fragment(const __bf16* lds_v, int s16, int db, int lane) {
  using C = TileCfg<D>;
  const int grp = lane >> 4, i = lane & 15;
  const int hh = grp >> 1;
  const int dd = db * 32 + (grp & 1) * 16 + 4 * (i & 3);
  const int chunk = dd >> 3, half = (dd >> 2) & 1;
  s16x4 part[2];
#pragma unroll
  for (int e4 = 0; e4 < 2; ++e4) {
    const int key = 16 * s16 + 8 * e4 + 4 * hh + (i >> 2);
    const int pos = chunk ^ C::swz_v(key);
    const SVG_LDS char* addr = (const SVG_LDS char*)lds_v + (key * D + pos * 8) * 2 + half * 8;
    part[e4] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SVG_LDS s16x4*)addr);
  }
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 both = __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, both);
}

// Key index (within the tile) of accumulator register r of block kb2.
__device__ __forceinline__ int acc_key(int kb2, int r, int hh) {
  return kb2 * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
}

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(256, 2) void k_attn_bf16(KGeom g, AttnPtrs a, int32_t nQT, int32_t total) {
  using C = TileCfg<D>;
  __shared__ __attribute__((aligned(16))) __bf16 lds[2][2][C::TILE_ELEMS];  // [buffer][K, V]
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hh = lane >> 5;

  // XCD-aware remap of the workgroup id, then longest-head-first order.
  const int w = blockIdx.x;
  const int xcd = w & 7, slot = w >> 3;
  const int logical = ((slot / kXcdRun) * 8 + xcd) * kXcdRun + (slot % kXcdRun);
  if (logical >= total) return;
  const int bh = a.order[logical / nQT];
  const int qt = logical % nQT;
  const int b = bh / g.H, h = bh % g.H;
  const int mode = a.modes[bh];
  const bool temporal = mode == SVG_TEMPORAL;
  const bool virt = temporal && (a.flags & SVG_FLAG_VIRTUAL_PERMUTE);
  const bool use_p = temporal && !virt;
  const svg_strides sin = use_p ? a.sp : a.s;
  const svg_strides sout = use_p ? a.sop : a.so;
  const int64_t ibase = (int64_t)b * sin.b + (int64_t)h * sin.h;
  const int64_t obase = (int64_t)b * sout.b + (int64_t)h * sout.h;
  const __bf16* Q = static_cast<const __bf16*>(use_p ? a.qp : a.q) + ibase;
  const __bf16* K = static_cast<const __bf16*>(use_p ? a.kp : a.k) + ibase;
  const __bf16* V = static_cast<const __bf16*>(use_p ? a.vp : a.v) + ibase;
  char* O = static_cast<char*>(use_p ? a.op : a.o);
  constexpr int OE = OUT_BF16 ? 2 : 4;  // output element bytes
  const int row0 = qt * kBM;
  const KGeom gg = g;
  auto phys = [gg, virt](int r) { return virt ? perm_inv_row(gg, r) : r; };

  if (mode == SVG_SKIP) {  // Sparse-vDiT head skipping: the output is zero
    constexpr int CPRO = D * OE / 16;
    for (int c = tid; c < kBM * CPRO; c += 256) {
      const int r = row0 + c / CPRO;
      if (r < g.L)
        *reinterpret_cast<int4*>(O + (obase + (int64_t)r * sout.x) * OE + (c % CPRO) * 16) = make_int4(0, 0, 0, 0);
    }
    return;
  }

  const int4 rg = reinterpret_cast<const int4*>(a.ranges)[(int64_t)bh * nQT + qt];
  const int n1 = rg.y - rg.x, nt = n1 + (rg.w - rg.z);
  auto tile_of = [&](int t) { return t < n1 ? rg.x + t : rg.z + (t - n1); };

  if (nt > 0) load_kv_tile<D>(K, V, sin.x, tile_of(0) * kBN, g.L, phys, lds[0][0], lds[0][1], wave, lane);

  // This lane's query row and its Q fragment (B operand of S^T = K Q^T).
  const int xq = row0 + wave * 32 + (lane & 31);
  const bool valid = xq < g.L;
  const int xqc = valid ? xq : g.L - 1;
  bf16x8 qf[D / 16];
  {
    const __bf16* qrow = Q + (int64_t)phys(xqc) * sin.x + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + 16 * ks);
  }
  int lo, hi;
  row_interval(g, mode, xqc, lo, hi);
  // wave-wide run bounds over valid rows: a tile is full for the wave when it
  // lies in every row's run, idle when it lies outside all of them
  const int max_lo = wave_max_i(valid ? lo : INT_MIN);
  const int min_hi = wave_min_i(valid ? hi : INT_MAX);
  const int min_lo = wave_min_i(valid ? lo : INT_MAX);
  const int max_hi = wave_max_i(valid ? hi : INT_MIN);
  const bool wave_rows = wave_max_i(valid ? 1 : 0) != 0;

  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
  float m_ref = -INFINITY, l_part = 0.f;
  const float sl2 = g.scale_log2;

  wait_vm_all();
  __syncthreads();

  for (int t = 0; t < nt; ++t) {
    const int bf = t & 1;
    if (t + 1 < nt)
      load_kv_tile<D>(K, V, sin.x, tile_of(t + 1) * kBN, g.L, phys, lds[bf ^ 1][0], lds[bf ^ 1][1], wave, lane);
    const int kt0 = tile_of(t) * kBN, kt1 = kt0 + kBN;
    const bool idle = kt0 >= g.T && (kt1 <= min_lo || kt0 >= max_hi);
    if (wave_rows && !idle) {
      const bool full = (kt1 <= g.T) || (max(kt0, g.T) >= max_lo && kt1 <= min_hi);
      const __bf16* lk = lds[bf][0];
      const __bf16* lv = lds[bf][1];
      f32x16 s0 = score_block<D>(lk, qf, 0, lane);
      f32x16 s1 = score_block<D>(lk, qf, 1, lane);
      float mx = -INFINITY;
      if (full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s0[r] *= sl2;
          s1[r] *= sl2;
          mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int k0 = kt0 + acc_key(0, r, hh), k1 = kt0 + acc_key(1, r, hh);
          const bool a0 = k0 < g.T || (k0 >= lo && k0 < hi);
          const bool a1 = k1 < g.T || (k1 >= lo && k1 < hi);
          s0[r] = a0 ? s0[r] * sl2 : -INFINITY;
          s1[r] = a1 ? s1[r] * sl2 : -INFINITY;
          mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
        }
      }
      mx = half_max(mx);
      if (__builtin_amdgcn_ballot_w64(mx > m_ref + kRescaleTau) != 0) {
        const float mn = fmaxf(m_ref, mx);
        // rows with nothing accumulated yet have o = l = 0 (and may still have mn = -inf)
        const float alpha = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref - mn);
        l_part *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
        m_ref = mn;
      }
      const float mu = m_ref == -INFINITY ? 0.f : m_ref;
      f32x8 p8[4];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        p8[0][r] = __builtin_amdgcn_exp2f(s0[r] - mu);
        p8[1][r] = __builtin_amdgcn_exp2f(s0[r + 8] - mu);
        p8[2][r] = __builtin_amdgcn_exp2f(s1[r] - mu);
        p8[3][r] = __builtin_amdgcn_exp2f(s1[r + 8] - mu);
      }
#pragma unroll
      for (int s16 = 0; s16 < 4; ++s16) {
#pragma unroll
        for (int r = 0; r < 8; ++r) l_part += p8[s16][r];
        const bf16x8 pb = __builtin_convertvector(p8[s16], bf16x8);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const bf16x8 vf = v_fragment<D>(lv, s16, db, lane);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb, o[db], 0, 0, 0);
        }
      }
    }
    wait_vm_all();
    __syncthreads();
  }

  // Epilogue: lane (query, h) holds dims 32*db + 8*(r/4) + 4*h + r%4.
  const float l_tot = half_sum(l_part);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (valid) {
    char* orow = O + (obase + (int64_t)phys(xq) * sout.x) * OE;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = db * 32 + 8 * g4 + 4 * hh;
        f32x4 v4 = {o[db][4 * g4] * inv, o[db][4 * g4 + 1] * inv, o[db][4 * g4 + 2] * inv, o[db][4 * g4 + 3] * inv};
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

// ---------------------------------------------------------------------------
// Profiling sweep (bf16): every workgroup takes 128 sampled rows of one head
// (4 waves x 32) and one of `ksplit` slices of the key tiles, and keeps three
// online-softmax states per row: full attention, the spatial mask and the
// temporal mask (mod form, frame-major order).  It writes each state's
// (m, l, acc) for the merge kernel.  The scores and the V fragments of a tile
// are shared by the three states.

// Tile-relative active key offsets [a0, b0) U [a1, b1) of one state.
struct Runs {
  int a0, b0, a1, b1;
};
// Clip [a0, b0) U [a1, b1) to the tile; empty runs become [a, a).
__device__ __forceinline__ Runs make_runs(int a0, int b0, int a1, int b1, int n) {
  a0 = min(max(a0, 0), n);
  b0 = min(max(b0, a0), n);
  a1 = min(max(a1, 0), n);
  b1 = min(max(b1, a1), n);
  return Runs{a0, b0, a1, b1};
}
__device__ __forceinline__ bool in_runs(const Runs& r, int e) {
  return (unsigned)(e - r.a0) < (unsigned)(r.b0 - r.a0) || (unsigned)(e - r.a1) < (unsigned)(r.b1 - r.a1);
}

template <int D>
__global__ __launch_bounds__(256, 1) void k_profile_bf16(KGeom g, const __bf16* __restrict__ q,
                                                         const __bf16* __restrict__ k,
                                                         const __bf16* __restrict__ v, svg_strides s,
                                                         const int32_t* __restrict__ rows, int32_t n_rows,
                                                         int32_t ksplit, float* __restrict__ part_acc,
                                                         float* __restrict__ part_ml) {
  using C = TileCfg<D>;
  __shared__ __attribute__((aligned(16))) __bf16 lds[2][2][C::TILE_ELEMS];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hh = lane >> 5;
  const int chunk = blockIdx.x, split = blockIdx.y, bh = blockIdx.z;
  const int b = bh / g.H, h = bh % g.H;
  const int64_t base = (int64_t)b * s.b + (int64_t)h * s.h;
  const __bf16* Q = q + base;
  const __bf16* K = k + base;
  const __bf16* V = v + base;
  auto ident = [](int r) { return r; };

  const int nKT = (g.L + kBN - 1) / kBN;
  const int t_begin = (int)((int64_t)nKT * split / ksplit), t_end = (int)((int64_t)nKT * (split + 1) / ksplit);
  const int nt = t_end - t_begin;
  if (nt > 0) load_kv_tile<D>(K, V, s.x, t_begin * kBN, g.L, ident, lds[0][0], lds[0][1], wave, lane);

  const int ridx = chunk * kProfRows_bf16 + wave * 32 + (lane & 31);
  const bool valid = ridx < n_rows;
  const int x = rows[valid ? ridx : n_rows - 1];
  bf16x8 qf[D / 16];
  {
    const __bf16* qrow = Q + (int64_t)x * s.x + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + 16 * ks);
  }
  // spatial run [slo, shi) of whole frames; temporal positions [jlo, jhi)
  const int u = x - g.T;
  const int fi = fastdiv(u, g.divF_mul, g.divF_shift), fj = u - fi * g.F;
  const int slo = g.T + max(0, fi - g.a1 + 1) * g.F, shi = g.T + min(g.N, fi + g.a1) * g.F;
  const int jlo = max(0, fj - g.a2 + 1), jhi = min(g.F, fj + g.a2);
  const int w_slo = wave_min_i(valid ? slo : INT_MAX), w_shi = wave_max_i(valid ? shi : INT_MIN);

  f32x16 o[3][D / 32];
#pragma unroll
  for (int st = 0; st < 3; ++st)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[st][db] = f32x16{};
  float m_ref[3] = {-INFINITY, -INFINITY, -INFINITY}, l_part[3] = {0.f, 0.f, 0.f};
  const float sl2 = g.scale_log2;

  wait_vm_all();
  __syncthreads();
  for (int t = 0; t < nt; ++t) {
    const int bf = t & 1;
    if (t + 1 < nt)
      load_kv_tile<D>(K, V, s.x, (t_begin + t + 1) * kBN, g.L, ident, lds[bf ^ 1][0], lds[bf ^ 1][1], wave, lane);
    const int kt0 = (t_begin + t) * kBN;
    const __bf16* lk = lds[bf][0];
    const __bf16* lv = lds[bf][1];
    const int nvalid = min(kBN, g.L - kt0);
    const int ntext = max(0, min(kBN, g.T - kt0));
    // active runs of each state, tile-relative
    Runs run[3];
    run[0] = make_runs(0, nvalid, 0, 0, nvalid);
    run[1] = make_runs(0, ntext, slo - kt0, shi - kt0, nvalid);
    const bool tp_simple = kt0 >= g.T && g.F >= kBN;
    if (tp_simple) {  // positions of the tile wrap at most once
      const int uk = kt0 - g.T;
      const int jt0 = uk - fastdiv(uk, g.divF_mul, g.divF_shift) * g.F;
      run[2] = make_runs(jlo - jt0, jhi - jt0, jlo - jt0 + g.F, jhi - jt0 + g.F, nvalid);
    } else {
      run[2] = Runs{0, 0, 0, 0};
    }
    f32x16 sc0 = score_block<D>(lk, qf, 0, lane);
    f32x16 sc1 = score_block<D>(lk, qf, 1, lane);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sc0[r] *= sl2;
      sc1[r] *= sl2;
    }
    // Softmax of one state into bf16 P fragments (masked keys give p = 0, so a
    // state with no active key in the tile contributes nothing).
    auto state_p = [&](int st, bf16x8* pb) {
      f32x16 z0, z1;
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int e0 = acc_key(0, r, hh), e1 = acc_key(1, r, hh);
        bool a0, a1;
        if (st == 2 && !tp_simple) {  // general path: text keys and short frames
          const int k0 = kt0 + e0, k1 = kt0 + e1;
          const int u0 = k0 - g.T, u1 = k1 - g.T;
          const int j0 = u0 - fastdiv(max(u0, 0), g.divF_mul, g.divF_shift) * g.F;
          const int j1 = u1 - fastdiv(max(u1, 0), g.divF_mul, g.divF_shift) * g.F;
          a0 = e0 < nvalid && (k0 < g.T || (j0 >= jlo && j0 < jhi));
          a1 = e1 < nvalid && (k1 < g.T || (j1 >= jlo && j1 < jhi));
        } else {
          a0 = in_runs(run[st], e0);
          a1 = in_runs(run[st], e1);
        }
        z0[r] = a0 ? sc0[r] : -INFINITY;
        z1[r] = a1 ? sc1[r] : -INFINITY;
        mx = fmaxf(mx, fmaxf(z0[r], z1[r]));
      }
      mx = half_max(mx);
      if (__builtin_amdgcn_ballot_w64(mx > m_ref[st] + kRescaleTau) != 0) {
        const float mn = fmaxf(m_ref[st], mx);
        const float alpha = m_ref[st] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref[st] - mn);
        l_part[st] *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) o[st][db] *= alpha;
        m_ref[st] = mn;
      }
      const float mu = m_ref[st] == -INFINITY ? 0.f : m_ref[st];
#pragma unroll
      for (int s16 = 0; s16 < 4; ++s16) {
        f32x8 p8;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const float zz = (s16 >> 1) ? z1[(s16 & 1) * 8 + r] : z0[(s16 & 1) * 8 + r];
          p8[r] = __builtin_amdgcn_exp2f(zz - mu);
          l_part[st] += p8[r];
        }
        pb[s16] = __builtin_convertvector(p8, bf16x8);
      }
    };
    // full and temporal states: every tile
    {
      bf16x8 pf[4], pt[4];
      state_p(0, pf);
      state_p(2, pt);
#pragma unroll
      for (int s16 = 0; s16 < 4; ++s16) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const bf16x8 vf = v_fragment<D>(lv, s16, db, lane);
          o[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[s16], o[0][db], 0, 0, 0);
          o[2][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pt[s16], o[2][db], 0, 0, 0);
        }
      }
    }
    // spatial state: only tiles with text keys or inside the wave's frame run
    if (kt0 < g.T || (kt0 + kBN > w_slo && kt0 < w_shi)) {
      bf16x8 ps[4];
      state_p(1, ps);
#pragma unroll
      for (int s16 = 0; s16 < 4; ++s16) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const bf16x8 vf = v_fragment<D>(lv, s16, db, lane);
          o[1][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, ps[s16], o[1][db], 0, 0, 0);
        }
      }
    }
    wait_vm_all();
    __syncthreads();
  }
  // partial outputs: slot = ((bh * n_rows + ridx) * ksplit + split) * 3 + state
#pragma unroll
  for (int st = 0; st < 3; ++st) {
    const float l_tot = half_sum(l_part[st]);
    if (!valid) continue;
    const int64_t slot = (((int64_t)bh * n_rows + ridx) * ksplit + split) * 3 + st;
    float* acc = part_acc + slot * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = db * 32 + 8 * g4 + 4 * hh;
        *reinterpret_cast<f32x4*>(acc + d0) = f32x4{o[st][db][4 * g4], o[st][db][4 * g4 + 1],
                                                    o[st][db][4 * g4 + 2], o[st][db][4 * g4 + 3]};
      }
    if (hh == 0) {
      part_ml[slot * 2] = m_ref[st];
      part_ml[slot * 2 + 1] = l_tot;
    }
  }
}

hipError_t launch_attention_bf16(const KGeom& g, const AttnPtrs& a, bool out_bf16, hipStream_t st) {
  const int32_t nQT = (g.L + kBM - 1) / kBM;
  const int64_t total = (int64_t)g.B * g.H * nQT;
  const int64_t per_round = 8 * kXcdRun;
  const int64_t grid = (total + per_round - 1) / per_round * per_round;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  if (g.d == 64) {
    if (out_bf16)
      hipLaunchKernelGGL((k_attn_bf16<64, true>), dim3((unsigned)grid), dim3(256), 0, st, g, a, nQT, (int32_t)total);
    else
      hipLaunchKernelGGL((k_attn_bf16<64, false>), dim3((unsigned)grid), dim3(256), 0, st, g, a, nQT, (int32_t)total);
  } else {
    if (out_bf16)
      hipLaunchKernelGGL((k_attn_bf16<128, true>), dim3((unsigned)grid), dim3(256), 0, st, g, a, nQT, (int32_t)total);
    else
      hipLaunchKernelGGL((k_attn_bf16<128, false>), dim3((unsigned)grid), dim3(256), 0, st, g, a, nQT, (int32_t)total);
  }
  return hipGetLastError();
}

hipError_t launch_profile_bf16(const KGeom& g, const void* q, const void* k, const void* v, svg_strides s,
                               const int32_t* rows, int32_t n_rows, int32_t ksplit, float* part_acc,
                               float* part_ml, hipStream_t st) {
  dim3 grid((unsigned)((n_rows + kProfRows_bf16 - 1) / kProfRows_bf16), (unsigned)ksplit, (unsigned)(g.B * g.H));
  const __bf16 *bq = static_cast<const __bf16*>(q), *bk = static_cast<const __bf16*>(k),
               *bv = static_cast<const __bf16*>(v);
  if (g.d == 64)
    hipLaunchKernelGGL(k_profile_bf16<64>, grid, dim3(256), 0, st, g, bq, bk, bv, s, rows, n_rows, ksplit,
                       part_acc, part_ml);
  else
    hipLaunchKernelGGL(k_profile_bf16<128>, grid, dim3(256), 0, st, g, bq, bk, bv, s, rows, n_rows, ksplit,
                       part_acc, part_ml);
  return hipGetLastError();
}

}  // namespace svg
