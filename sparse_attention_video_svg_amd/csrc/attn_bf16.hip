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
//  * Workgroup ids are remapped so that each XCD (ids are dealt round-robin to
//    the 8 XCDs) walks runs of consecutive query tiles of one head, which
//    share their K/V band in that XCD's L2; runs are handed out in the
//    longest-head-first order of svg_build_blocks.
#include <type_traits>

#include "svg_device.h"

namespace svg {

constexpr int kBN = kBN_bf16;
constexpr float kRescaleTau = 8.0f;  // log2 headroom before the running max moves
constexpr int kXcdRun = 32;          // consecutive query tiles per XCD turn


template <int D, int WAVES = 4>
struct TileCfg {
  static constexpr int CR = D / 8;                   // 16-byte chunks per row
  static constexpr int RPL = 16 / CR;                // rows per 256-byte LDS line
  static constexpr int CHUNKS = kBN * CR;            // chunks per K (or V) tile
  static constexpr int SEGS = CHUNKS / 64;                     // 64-chunk segments per tensor
  static constexpr int LOADS = (SEGS + WAVES - 1) / WAVES;     // per thread per tensor (last may be idle)
  static constexpr int TILE_ELEMS = kBN * D;         // bf16 elements per tile
  // K rows are read 16 keys x one chunk at a time: spread keys over chunks.
  __device__ static __forceinline__ int swz_k(int r) { return (r / RPL) % CR; }
  // V is read 4 keys x 4 chunks at a time (transposing reads): spread the
  // 4 consecutive keys over 4 different 64-byte quarters of the line.
  __device__ static __forceinline__ int swz_v(int r) { return 4 * ((r / RPL) % (CR / 4)); }
};

__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// wait until at most N vector-memory loads of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Direct-to-LDS loads of one K tile and one V tile by all 256 threads.
// Chunk p of a tile (row r = p / CR, LDS position pos = p % CR) receives
// global chunk pos ^ swz(r) of key row kt0 + r.  Each lane's byte offsets
// within a tile are fixed, so the hot path is one scalar base per tile plus
// the lane's 32-bit offset (the saddr form of the load).  The last, ragged
// tile clamps rows to L - 1; with VIRT the rows are gathered through the
// token-major index map.
template <int D, bool VIRT, int WAVES = 4>
struct KVLoader {
  using C = TileCfg<D, WAVES>;
  const char* kb;
  const char* vb;
  int64_t sxb;  // token stride in bytes
  uint32_t offk[C::LOADS], offv[C::LOADS];
  int L;

  __device__ __forceinline__ void init(const __bf16* K, const __bf16* V, int64_t sx, int L_, int wave, int lane) {
    kb = reinterpret_cast<const char*>(K);
    vb = reinterpret_cast<const char*>(V);
    sxb = sx * 2;
    L = L_;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int p = min(i * WAVES + wave, C::SEGS - 1) * 64 + lane;
      const int r = p / C::CR, pos = p % C::CR;
      offk[i] = (uint32_t)(r * sxb) + (uint32_t)((pos ^ C::swz_k(r)) * 16);
      offv[i] = (uint32_t)(r * sxb) + (uint32_t)((pos ^ C::swz_v(r)) * 16);
    }
  }

  // one tensor (K: which = 0, V: which = 1) of the tile at key kt0
  template <int WHICH>
  __device__ __forceinline__ void load1(const KGeom& g, int kt0, __bf16* lds_t, int wave, int lane) const {
    const char* base = WHICH == 0 ? kb : vb;
    if (!VIRT && kt0 + kBN <= L) {
      const char* tb = base + kt0 * sxb;
#pragma unroll
      for (int i = 0; i < C::LOADS; ++i) {
        const int seg = i * WAVES + wave;
        if (C::SEGS % WAVES != 0 && seg >= C::SEGS) break;  // wave-uniform
        const uint32_t off = WHICH == 0 ? offk[i] : offv[i];
        __builtin_amdgcn_global_load_lds((const void*)(tb + off), (SVG_LDS void*)(lds_t + seg * 512), 16, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::LOADS; ++i) {
        const int seg = i * WAVES + wave;
        if (C::SEGS % WAVES != 0 && seg >= C::SEGS) break;  // wave-uniform
        const int p = seg * 64 + lane;
        const int r = p / C::CR, pos = p % C::CR;
        int row = kt0 + r;
        row = row < L ? row : L - 1;
        if (VIRT) row = perm_inv_row(g, row);
        const int sw = WHICH == 0 ? C::swz_k(r) : C::swz_v(r);
        __builtin_amdgcn_global_load_lds((const void*)(base + (int64_t)row * sxb + (pos ^ sw) * 16),
                                         (SVG_LDS void*)(lds_t + seg * 512), 16, 0, 0);
      }
    }
  }

  __device__ __forceinline__ void load(const KGeom& g, int kt0, __bf16* lds_k, __bf16* lds_v, int wave, int lane) const {
    load1<0>(g, kt0, lds_k, wave, lane);
    load1<1>(g, kt0, lds_v, wave, lane);
  }
};

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

// Both 32-key blocks of a tile, the two accumulation chains interleaved and
// the K fragments read kAhead steps before their MFMAs, so LDS latency hides
// behind matrix work instead of stalling every pair of MFMAs.
template <int D>
__device__ __forceinline__ void score_tile(const __bf16* lds_k, const bf16x8* qf, int lane, f32x16& s0, f32x16& s1) {
  using C = TileCfg<D>;
  constexpr int KS = D / 16, kAhead = 3;
  const int hh = lane >> 5;
  const int m0 = lane & 31, m1 = 32 + (lane & 31);
  const int sw0 = C::swz_k(m0), sw1 = C::swz_k(m1);
  auto rd = [&](int m, int sw, int ks) {
    return *reinterpret_cast<const bf16x8*>(lds_k + m * D + (((2 * ks + hh) ^ sw) * 8));
  };
  bf16x8 f0[KS], f1[KS];
#pragma unroll
  for (int ks = 0; ks < kAhead; ++ks) {
    f0[ks] = rd(m0, sw0, ks);
    f1[ks] = rd(m1, sw1, ks);
  }
  s0 = f32x16{};
  s1 = f32x16{};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (ks + kAhead < KS) {
      f0[ks + kAhead] = rd(m0, sw0, ks + kAhead);
      f1[ks + kAhead] = rd(m1, sw1, ks + kAhead);
    }
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f0[ks], qf[ks], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f1[ks], qf[ks], s1, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < KS; ++i) {  // keep the issue order: 2 reads, then 2 MFMAs
    if (i == 0) __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAhead, 0);
    if (i + kAhead < KS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  }
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

// Online-softmax state of one output (per lane: one query, the dims of the
// accumulator layout).  m_ref is the running reference max in log2 units; it
// only moves when a lane's tile max exceeds it by more than 2^kRescaleTau, and
// that decision is per lane, so a row's result never depends on which other
// rows share its wave.
template <int D>
struct Flash {
  f32x16 o[D / 32];
  float m_ref, l_part;

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
    m_ref = -INFINITY;
    l_part = 0.f;
  }

  // s0, s1: raw scores of the two 32-key blocks of a tile, masked entries
  // already -inf.  sl2 = scale * log2(e) > 0.  Leaves the tile's weights as
  // bf16 in pbs (key step s16 = 16 keys each) and folds their row sum into
  // l_part; rescales o when the reference max moves.
  __device__ __forceinline__ void softmax(const f32x16& s0, const f32x16& s1, float sl2, bf16x8* pbs) {
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
    mx = half_max(mx) * sl2;
    const bool need = mx > m_ref + kRescaleTau;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      // lanes with nothing accumulated yet (m_ref = -inf) hold o = l = 0
      const float alpha = !need ? 1.f : (m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref - mx));
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
      m_ref = need ? mx : m_ref;
    }
    const float nmu = m_ref == -INFINITY ? 0.f : -m_ref;
    const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int s16 = 0; s16 < 4; ++s16) {
      f32x8 p8;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float sv = (s16 >> 1) ? s1[(s16 & 1) * 8 + r] : s0[(s16 & 1) * 8 + r];
        p8[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv, sl2, nmu));
      }
      const bf16x8 pb = __builtin_convertvector(p8, bf16x8);
      // row sum of the bf16 weights the P.V product actually uses, two per
      // v_dot2_f32_bf16 against (1, 1)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bf16x2 pr = {pb[2 * r], pb[2 * r + 1]};
        l_part = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, l_part, false);
      }
      pbs[s16] = pb;
    }
  }

  // o += P V for the weights of one tile; V^T fragments read from LDS.
  __device__ __forceinline__ void pv(const bf16x8* pbs, const __bf16* lv, int lane) {
#pragma unroll
    for (int s16 = 0; s16 < 4; ++s16) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const bf16x8 vf = v_fragment<D>(lv, s16, db, lane);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pbs[s16], o[db], 0, 0, 0);
      }
    }
  }

  __device__ __forceinline__ void add_tile(const f32x16& s0, const f32x16& s1, const __bf16* lv, int lane,
                                           float sl2) {
    bf16x8 pbs[4];
    softmax(s0, s1, sl2, pbs);
    pv(pbs, lv, lane);
  }
};

// Mask the raw scores of a tile to the lane's active keys [0, T) U [lo, hi).
__device__ __forceinline__ void mask_tile(f32x16& s0, f32x16& s1, int kt0, int hh, int T, int lo, int hi) {
  const unsigned span = (unsigned)(hi - lo);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int k0 = kt0 + acc_key(0, r, hh), k1 = kt0 + acc_key(1, r, hh);
    const bool a0 = (k0 < T) | ((unsigned)(k0 - lo) < span);
    const bool a1 = (k1 < T) | ((unsigned)(k1 - lo) < span);
    s0[r] = a0 ? s0[r] : -INFINITY;
    s1[r] = a1 ? s1[r] : -INFINITY;
  }
}

// Single-output flash sweep of a workgroup over a tile sequence given as two
// ranges [rg.x, rg.y) U [rg.z, rg.w) of key tiles.  Every lane's active keys
// are [0, T) U [lo, hi); `valid` marks lanes with a real query row.  The
// caller has already issued the loads of the first tile into stage 0.  K/V
// tiles go through a ring of STAGES LDS buffers: tile t + STAGES - 1 is in
// flight while tile t is computed, with one barrier per tile.
template <int D, bool VIRT, int WAVES, int STAGES>
__device__ __forceinline__ void sweep(Flash<D>& st, const bf16x8* qf, const KVLoader<D, VIRT, WAVES>& ld,
                                      const KGeom& g, int4 rg, int lo, int hi, bool valid,
                                      __bf16 (*lds)[2][TileCfg<D>::TILE_ELEMS], int wave, int lane) {
  constexpr int PER_TILE = 2 * TileCfg<D, WAVES>::LOADS;  // load instructions per tile per wave
  static_assert(STAGES == 2 || TileCfg<D, WAVES>::SEGS % WAVES == 0,
                "a 3-stage ring counts loads per wave: every wave must issue the same number");
  const int hh = lane >> 5;
  const int T = g.T;
  const float sl2 = g.scale_log2;
  const int n1 = rg.y - rg.x, nt = n1 + (rg.w - rg.z);
  auto tile_of = [&](int t) { return t < n1 ? rg.x + t : rg.z + (t - n1); };
  // wave-wide run bounds over valid rows: a tile is full for the wave when it
  // lies in every row's run, idle when it lies outside all of them
  const int max_lo = wave_max_i(valid ? lo : INT_MIN);
  const int min_hi = wave_min_i(valid ? hi : INT_MAX);
  const int min_lo = wave_min_i(valid ? lo : INT_MAX);
  const int max_hi = wave_max_i(valid ? hi : INT_MIN);
  const bool wave_rows = wave_max_i(valid ? 1 : 0) != 0;
  st.init();
  // prologue: tiles 1 .. STAGES-2 into their stages, then wait for tile 0
#pragma unroll
  for (int p = 1; p <= STAGES - 2; ++p)
    if (p < nt) ld.load(g, tile_of(p) * kBN, lds[p][0], lds[p][1], wave, lane);
  if (STAGES == 3 && nt > 1)
    wait_vm<PER_TILE>();
  else
    wait_vm_all();
  __syncthreads();
  auto step = [&](int t, auto stc) {
    constexpr int sg = decltype(stc)::value;  // t % STAGES
    constexpr int nx = (sg + STAGES - 1) % STAGES;
    if (t + STAGES - 1 < nt) ld.load(g, tile_of(t + STAGES - 1) * kBN, lds[nx][0], lds[nx][1], wave, lane);
    const int kt0 = tile_of(t) * kBN, kt1 = kt0 + kBN;
    const bool idle = kt0 >= T && (kt1 <= min_lo || kt0 >= max_hi);
    if (wave_rows && !idle) {
      const bool full = (kt1 <= T) || (max(kt0, T) >= max_lo && kt1 <= min_hi);
      f32x16 s0, s1;
      score_tile<D>(lds[sg][0], qf, lane, s0, s1);
      if (!full) mask_tile(s0, s1, kt0, hh, T, lo, hi);
      st.add_tile(s0, s1, lds[sg][1], lane, sl2);
    }
    // tile t+1 must have landed; later tiles may still be in flight
    if (STAGES == 3 && t + 2 < nt)
      wait_vm<PER_TILE>();
    else
      wait_vm_all();
    __syncthreads();
  };
  // unrolled by STAGES so that each buffer's LDS offsets are immediates
  for (int t = 0; t < nt; t += STAGES) {
    step(t, std::integral_constant<int, 0>{});
    if (t + 1 < nt) step(t + 1, std::integral_constant<int, 1 % STAGES>{});
    if (STAGES == 3 && t + 2 < nt) step(t + 2, std::integral_constant<int, 2 % STAGES>{});
  }
}


// Sweep of one workgroup's tile ranges into st.
template <int D, bool VIRT, int WAVES, int STAGES>
__device__ __forceinline__ void run_sweep(Flash<D>& st, const bf16x8* qf, const __bf16* K, const __bf16* V, int64_t sx,
                                          const KGeom& g, int4 rg, int lo, int hi, bool valid,
                                          __bf16 (*lds)[2][TileCfg<D>::TILE_ELEMS], int wave, int lane) {
  KVLoader<D, VIRT, WAVES> ld;
  ld.init(K, V, sx, g.L, wave, lane);
  if (rg.y > rg.x)
    ld.load(g, rg.x * kBN, lds[0][0], lds[0][1], wave, lane);
  else if (rg.w > rg.z)
    ld.load(g, rg.z * kBN, lds[0][0], lds[0][1], wave, lane);
  sweep<D, VIRT, WAVES, STAGES>(st, qf, ld, g, rg, lo, hi, valid, lds, wave, lane);
}

template <int D>
__device__ __forceinline__ void load_q(bf16x8* qf, const __bf16* qrow_base, int hh) {
  const __bf16* qrow = qrow_base + 8 * hh;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + 16 * ks);
}

// One query tile (32 * WAVES rows) of one head.  VIRT: a temporal head read
// and written through the token-major index map instead of explicitly
// permuted copies.
template <int D, bool OUT_BF16, bool VIRT, int WAVES, int STAGES>
__device__ __forceinline__ void attn_tile(const KGeom& g, const AttnPtrs& a, int bh, int qt, int mode, int nQT,
                                          __bf16 (*lds)[2][TileCfg<D>::TILE_ELEMS], int wave, int lane) {
  constexpr int BMW = 32 * WAVES;
  const int hh = lane >> 5;
  const int b = bh / g.H, h = bh % g.H;
  const bool use_p = mode == SVG_TEMPORAL && !VIRT;
  const svg_strides sin = use_p ? a.sp : a.s;
  const svg_strides sout = use_p ? a.sop : a.so;
  const int64_t ibase = (int64_t)b * sin.b + (int64_t)h * sin.h;
  const int64_t obase = (int64_t)b * sout.b + (int64_t)h * sout.h;
  const __bf16* Q = static_cast<const __bf16*>(use_p ? a.qp : a.q) + ibase;
  const __bf16* K = static_cast<const __bf16*>(use_p ? a.kp : a.k) + ibase;
  const __bf16* V = static_cast<const __bf16*>(use_p ? a.vp : a.v) + ibase;
  char* O = static_cast<char*>(use_p ? a.op : a.o);
  constexpr int OE = OUT_BF16 ? 2 : 4;  // output element bytes
  auto phys = [&g](int r) { return VIRT ? perm_inv_row(g, r) : r; };

  const int4 rg = reinterpret_cast<const int4*>(a.ranges)[(int64_t)bh * nQT + qt];

  // This lane's query row and its Q fragment (B operand of S^T = K Q^T).
  const int xq = qt * BMW + wave * 32 + (lane & 31);
  const bool valid = xq < g.L;
  const int xqc = valid ? xq : g.L - 1;
  bf16x8 qf[D / 16];
  load_q<D>(qf, Q + (int64_t)phys(xqc) * sin.x, hh);
  int lo, hi;
  row_interval(g, mode, xqc, lo, hi);

  Flash<D> st;
  run_sweep<D, VIRT, WAVES, STAGES>(st, qf, K, V, sin.x, g, rg, lo, hi, valid, lds, wave, lane);

  // Epilogue: lane (query, h) holds dims 32*db + 8*(r/4) + 4*h + r%4.
  const float l_tot = half_sum(st.l_part);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (valid) {
    char* orow = O + (obase + (int64_t)phys(xq) * sout.x) * OE;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = db * 32 + 8 * g4 + 4 * hh;
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

template <int D, bool OUT_BF16, int WAVES, int STAGES>
__global__ __launch_bounds__(64 * WAVES, (WAVES <= 6 ? 2 : 1)) void k_attn_bf16(KGeom g, AttnPtrs a, int32_t nQT,
                                                                                int32_t total) {
  using C = TileCfg<D, WAVES>;
  constexpr int BMW = 32 * WAVES;
  extern __shared__ __attribute__((aligned(16))) __bf16 lds_raw[];
  auto lds = reinterpret_cast<__bf16 (*)[2][C::TILE_ELEMS]>(lds_raw);  // [stage][K, V]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // XCD-aware remap of the workgroup id, then longest-head-first order.
  const int w = blockIdx.x;
  const int xcd = w & 7, slot = w >> 3;
  const int logical = ((slot / kXcdRun) * 8 + xcd) * kXcdRun + (slot % kXcdRun);
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
// accumulator layout order is written back to dims order.
template <int D>
__device__ __forceinline__ void store_partial(const Flash<D>& st, float* acc, float* ml, int hh) {
  const float l_tot = half_sum(st.l_part);
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = db * 32 + 8 * g4 + 4 * hh;
      *reinterpret_cast<f32x4*>(acc + d0) =
          f32x4{st.o[db][4 * g4], st.o[db][4 * g4 + 1], st.o[db][4 * g4 + 2], st.o[db][4 * g4 + 3]};
    }
  if (hh == 0) {
    ml[0] = st.m_ref;
    ml[1] = l_tot;
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
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  const int w = blockIdx.x;
  const int xcd = w & 7, slot = w >> 3;
  const int logical = ((slot / kXcdRun) * 8 + xcd) * kXcdRun + (slot % kXcdRun);
  if (logical >= total) return;
  const int chunks = (n_rows + BMW - 1) / BMW;
  const int chunk = logical % chunks;
  const int split = (logical / chunks) % nsplit, bh = logical / chunks / nsplit;
  const int b = bh / g.H, h = bh % g.H;
  const int64_t base = (int64_t)b * s.b + (int64_t)h * s.h;

  const int rk = chunk * BMW + wave * 32 + (lane & 31);
  const bool valid = rk < n_rows;
  const int x = rows[valid ? rk : n_rows - 1];
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
    const int r = VIRT ? ord_r[rk] : rk;
    const int64_t o = (((int64_t)bh * n_rows + r) * nsplit + split) * nstates + state;
    store_partial<D>(st, part_acc + o * D, part_ml + o * 2, hh);
  }
}

template <int D, bool OUT_BF16>
static hipError_t launch_attn(const KGeom& g, const AttnPtrs& a, int32_t nQT, int64_t grid, int64_t total,
                              hipStream_t st) {
  constexpr int W = kAttnWaves, S = kAttnStages;
  const size_t lds = (size_t)S * 2 * TileCfg<D>::TILE_ELEMS * sizeof(__bf16);
  auto kern = k_attn_bf16<D, OUT_BF16, W, S>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * W), lds, st, g, a, nQT, (int32_t)total);
  return hipGetLastError();
}

hipError_t launch_attention_bf16(const KGeom& g, const AttnPtrs& a, bool out_bf16, hipStream_t st) {
  const int32_t nQT = (g.L + kBM_bf16 - 1) / kBM_bf16;
  const int64_t total = (int64_t)g.B * g.H * nQT;
  const int64_t per_round = 8 * kXcdRun;
  const int64_t grid = (total + per_round - 1) / per_round * per_round;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  if (g.d == 64)
    return out_bf16 ? launch_attn<64, true>(g, a, nQT, grid, total, st) : launch_attn<64, false>(g, a, nQT, grid, total, st);
  return out_bf16 ? launch_attn<128, true>(g, a, nQT, grid, total, st) : launch_attn<128, false>(g, a, nQT, grid, total, st);
}

template <int D, bool VIRT>
static hipError_t launch_prof(const KGeom& g, const __bf16* q, const __bf16* k, const __bf16* v, svg_strides s,
                              const int32_t* rows, const int32_t* ord_r, int32_t n_rows, int32_t nsplit, int32_t mode,
                              int32_t state, int32_t nstates, float* acc, float* ml, hipStream_t st) {
  constexpr int W = kAttnWaves, S = kAttnStages;
  const size_t lds = (size_t)S * 2 * TileCfg<D>::TILE_ELEMS * sizeof(__bf16);
  auto kern = k_prof_sweep<D, VIRT, W, S>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t chunks = (n_rows + 32 * W - 1) / (32 * W);
  const int64_t total = chunks * nsplit * g.B * g.H;
  const int64_t per_round = 8 * kXcdRun;
  const int64_t grid = (total + per_round - 1) / per_round * per_round;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * W), lds, st, g, q, k, v, s, rows, ord_r, n_rows, nsplit,
                     (int32_t)total, mode, state, nstates, acc, ml);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_sweeps(const KGeom& g, const __bf16* q, const __bf16* k, const __bf16* v, svg_strides s,
                                const int32_t* rows, int32_t n_rows, int32_t ksplit, const int32_t* ord_x,
                                const int32_t* ord_r, const int32_t* modes, int32_t nstates, float* acc, float* ml,
                                hipStream_t st) {
  for (int32_t i = 0; i < nstates; ++i) {
    hipError_t e;
    if (modes[i] == SVG_TEMPORAL)
      e = launch_prof<D, true>(g, q, k, v, s, ord_x, ord_r, n_rows, ksplit, SVG_TEMPORAL, i, nstates, acc, ml, st);
    else
      e = launch_prof<D, false>(g, q, k, v, s, rows, nullptr, n_rows, ksplit, modes[i], i, nstates, acc, ml, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
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
