// Building blocks shared by the attention kernels (bf16 and fp8 scores):
// K/V tile configuration and direct-to-LDS loader, the transposed-score and
// P.V MFMA fragments, the online-softmax state, element masks and the
// lock-step sweep of a workgroup over its key tiles.  The design notes are at
// the top of attn_bf16.hip.
#pragma once

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
//
// With VIRT, token-major position x' = T + j*N + i (frame i, position j)
// reads natural row T + i*F + j.  Moving 64 keys on moves i by 64 mod N and
// j by 64 / N (one more when i wraps past N), so the natural row moves by a
// fixed step, plus a fixed correction on a wrap: a tile that directly
// follows the previous one (both all video rows, the new one not ragged)
// takes each lane's row offset and i from the previous tile with adds; other
// tiles (the first of a range, text rows, the ragged end) divide.  At d 64
// the three registers per load do not fit the 128-register kernels, which
// map every row.
template <int D, bool VIRT, int WAVES = 4>
struct KVLoader {
  using C = TileCfg<D, WAVES>;
  static constexpr bool INC = VIRT && D == 128;  // incremental index map
  static constexpr int NM = INC ? C::LOADS : 1;
  const char* kb;
  const char* vb;
  int64_t sxb;  // token stride in bytes
  uint32_t offk[C::LOADS], offv[C::LOADS];  // row + column bytes in the tile (INC: column bytes only)
  int L;
  int64_t vrow[NM];        // INC: byte offset of the lane's row of load i, last tile
  int vfr[NM];             // INC: that row's frame i (meaningful for video rows)
  int vlast;               // INC: first key of the last tile read
  int64_t vstep, vwrap;    // INC: row-offset step per 64 keys, extra on a wrap
  int vm64;                // INC: 64 mod N

  __device__ __forceinline__ void init(const __bf16* K, const __bf16* V, int64_t sx, int L_, int wave, int lane) {
    kb = reinterpret_cast<const char*>(K);
    vb = reinterpret_cast<const char*>(V);
    sxb = sx * 2;
    L = L_;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int p = min(i * WAVES + wave, C::SEGS - 1) * 64 + lane;
      const int r = p / C::CR, pos = p % C::CR;
      const uint32_t rb = INC ? 0u : (uint32_t)(r * sxb);
      offk[i] = rb + (uint32_t)((pos ^ C::swz_k(r)) * 16);
      offv[i] = rb + (uint32_t)((pos ^ C::swz_v(r)) * 16);
    }
  }

  // INC: the constants of the index map (after init).
  __device__ __forceinline__ void init_map(const KGeom& g) {
    const int q64 = (int)fastdiv(64, g.divN_mul, g.divN_shift);
    vm64 = 64 - q64 * g.N;
    vstep = ((int64_t)vm64 * g.F + q64) * sxb;
    vwrap = ((int64_t)1 - (int64_t)g.N * g.F) * sxb;
    vlast = INT_MIN / 2;
  }

  // INC: row offsets of every load of the tile at key kt0 into vrow.
  __device__ __forceinline__ void map_rows(const KGeom& g, int kt0, int wave, int lane) {
    if (kt0 == vlast + kBN && vlast >= g.T && kt0 + kBN <= L) {  // wave-uniform
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        const int fr = vfr[i] + vm64;
        const bool wrap = fr >= g.N;
        vfr[i] = wrap ? fr - g.N : fr;
        vrow[i] += wrap ? vstep + vwrap : vstep;
      }
    } else {
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        const int p = min(i * WAVES + wave, C::SEGS - 1) * 64 + lane;
        int row = kt0 + p / C::CR;
        row = row < L ? row : L - 1;
        int nat = row, fr = 0;
        if (row >= g.T) {
          const int up = row - g.T;
          const int j = (int)fastdiv(up, g.divN_mul, g.divN_shift);
          fr = up - j * g.N;
          nat = g.T + fr * g.F + j;
        }
        vfr[i] = fr;
        vrow[i] = (int64_t)nat * sxb;
      }
    }
    vlast = kt0;
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
    } else if (INC) {  // rows from map_rows
#pragma unroll
      for (int i = 0; i < C::LOADS; ++i) {
        const int seg = i * WAVES + wave;
        if (C::SEGS % WAVES != 0 && seg >= C::SEGS) break;  // wave-uniform
        const uint32_t col = WHICH == 0 ? offk[i] : offv[i];
        __builtin_amdgcn_global_load_lds((const void*)(base + vrow[INC ? i : 0] + col),
                                         (SVG_LDS void*)(lds_t + seg * 512), 16, 0, 0);
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

  __device__ __forceinline__ void load(const KGeom& g, int kt0, __bf16* lds_k, __bf16* lds_v, int wave, int lane) {
    if constexpr (INC) map_rows(g, kt0, wave, lane);
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
// With ACC the products are added to s0, s1 instead of replacing them.
// AHEAD: K fragment steps read ahead (d 64 has four steps and a
// 128-register budget: one).
template <int D, bool ACC = false, int AHEAD = (D == 64 ? 1 : 3)>
__device__ __forceinline__ void score_tile(const __bf16* lds_k, const bf16x8* qf, int lane, f32x16& s0, f32x16& s1) {
  using C = TileCfg<D>;
  constexpr int KS = D / 16, kAhead = AHEAD;
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
  if (!ACC) {
    s0 = f32x16{};
    s1 = f32x16{};
  }
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

// Max of a lane's scores over both 32-key blocks of a tile (its row: the
// lane and its partner lane^32 hold the two halves), in log2 units.
// Two chains of max(max(m, a), b), each step one v_max3_f32: 16 vector
// instructions per tile, where a running max of pairwise maxima compiles to
// 23.  Max is exact in any order.
__device__ __forceinline__ float tile_max(const f32x16& s0, const f32x16& s1, float sl2) {
  float m0 = fmaxf(s0[0], s1[0]), m1 = fmaxf(s0[1], s1[1]);
#pragma unroll
  for (int r = 2; r < 16; r += 2) {
    m0 = fmaxf(fmaxf(m0, s0[r]), s1[r]);
    m1 = fmaxf(fmaxf(m1, s0[r + 1]), s1[r + 1]);
  }
  return half_max(fmaxf(m0, m1)) * sl2;
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

  // Moves the reference max to mx (the tile's max in log2 units) on lanes
  // where it exceeds the reference by more than 2^kRescaleTau, rescaling o
  // and l_part there; a wave-uniform branch, almost never taken after the
  // first tile.
  __device__ __forceinline__ void rescale(float mx) {
    const bool need = mx > m_ref + kRescaleTau;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      // lanes with nothing accumulated yet (m_ref = -inf) hold o = l = 0
      const float alpha = !need ? 1.f : (m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref - mx));
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
      m_ref = need ? mx : m_ref;
    }
  }

  // The weights 2^(s * sl2 - m_ref) of key step s16 (16 keys) as bf16, their
  // row sum folded into l_part.
  __device__ __forceinline__ bf16x8 weights(const f32x16& s0, const f32x16& s1, float sl2, float nmu, int s16) {
    f32x8 p8;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const float sv = (s16 >> 1) ? s1[(s16 & 1) * 8 + r] : s0[(s16 & 1) * 8 + r];
      p8[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv, sl2, nmu));
    }
    const bf16x8 pb = __builtin_convertvector(p8, bf16x8);
    // row sum of the bf16 weights the P.V product actually uses, two per
    // v_dot2_f32_bf16 against (1, 1)
    const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bf16x2 pr = {pb[2 * r], pb[2 * r + 1]};
      l_part = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, l_part, false);
    }
    return pb;
  }

  // s0, s1: raw scores of the two 32-key blocks of a tile, masked entries
  // already -inf.  sl2 = scale * log2(e) > 0.  Leaves the tile's weights as
  // bf16 in pbs (key step s16 = 16 keys each) and folds their row sum into
  // l_part; rescales o when the reference max moves.
  __device__ __forceinline__ void softmax(const f32x16& s0, const f32x16& s1, float sl2, bf16x8* pbs) {
    rescale(tile_max(s0, s1, sl2));
    const float nmu = m_ref == -INFINITY ? 0.f : -m_ref;
#pragma unroll
    for (int s16 = 0; s16 < 4; ++s16) pbs[s16] = weights(s0, s1, sl2, nmu, s16);
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
__device__ __forceinline__ void sweep(Flash<D>& st, const bf16x8* qf, KVLoader<D, VIRT, WAVES>& ld,
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
  if constexpr (KVLoader<D, VIRT, WAVES>::INC) ld.init_map(g);
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

}  // namespace svg
