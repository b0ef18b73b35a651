// FP8-score attention for gfx950: Q and K quantised to FP8 E4M3 (OCP "fn"
// encoding) with power-of-two scales, the scores Q K^T on the FP8 matrix
// cores (v_mfma_scale_f32_32x32x64_f8f6f4, unscaled), softmax and P.V as in
// the bf16 kernel (fp32 softmax, bf16 P and V).
//
// The pages report only that Sparse-vDiT composes with FP8 (Sparse-vDiT
// review, editorial extensions: the appendix adds FP8 on Wan2.1); the
// scheme here is:
//  * Q: one scale per token row; K: one scale per tile of 64 keys of the
//    head's working layout (token-major for TEMPORAL heads), so a tile's
//    scores share one factor.  Each scale is the smallest power of two s with
//    448 * s >= max |x| over its group (1 for an all-zero group); x / s is
//    exact and the only rounding is the conversion to E4M3 (nearest, ties
//    to even).
//  * Scores of a tile are s8 * sq(row) * sk(tile); both factors fold into the
//    one multiplier the softmax already applies (scale * log2 e), so the
//    inner loop is the bf16 one with 4 score MFMAs of K = 64 per tile (d 128)
//    instead of 16 of K = 16, and an 8 KB K tile in LDS instead of 16 KB.
//  * TEMPORAL heads read Q8 and V in natural order through the token-major
//    index map (no permuted copies); K8 is written in token-major order by
//    the quantisation kernel, so its tiles are contiguous.
//  * Workgroups: 8 waves x 32 rows, one per CU, as in the bf16 kernel; with
//    FP8 P.V (every product on the FP8 matrix cores, so the softmax
//    outweighs them) 4 waves taking half of a 256-row query tile, three per
//    CU, out of lock step.
#include "attn_common.h"

namespace svg {

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));

constexpr float kE4M3Max = 448.0f;

// Exponent k of the scale 2^k: the smallest k with 448 * 2^k >= amax.
__device__ __forceinline__ int pow2_scale_exp(float amax) {
  if (!(amax > 0.f)) return 0;
  int e;
  (void)frexpf(amax, &e);  // amax = f * 2^e, f in [0.5, 1)
  int k = e - 9;           // 448 * 2^(e-9) = 0.875 * 2^e
  if (ldexpf(kE4M3Max, k) < amax) ++k;
  return k;
}

// Eight bf16 values scaled by 2^-k and converted to E4M3, packed in 8 bytes.
__device__ __forceinline__ i32x2 to_e4m3(const bf16x8& x, int k) {
  float f[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = ldexpf((float)x[i], -k);
  i32x2 r;
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], hi, true);
  r[0] = lo;
  r[1] = hi;
  return r;
}

// One workgroup per (64-row tile, head): K rows of the tile in the head's
// working layout (per-tile scale), and Q rows of the same natural indices
// (per-row scale).  q8 / k8: [B*H, L, D] bytes; sq: [B*H, L]; sk: [B*H, nKT].
template <int D>
__global__ __launch_bounds__(256) void k_quant_qk(KGeom g, const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                                                  svg_strides s, const int32_t* __restrict__ modes,
                                                  uint8_t* __restrict__ q8, float* __restrict__ sq,
                                                  uint8_t* __restrict__ k8, float* __restrict__ sk, int32_t nKT) {
  constexpr int CPR = D / 8;          // 16-byte chunks of bf16 per row
  constexpr int RPP = 256 / CPR;      // rows per pass
  constexpr int PASSES = 64 / RPP;
  const int t = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int b = bh / g.H, h = bh % g.H;
  const int64_t base = (int64_t)b * s.b + (int64_t)h * s.h;
  const bool temporal = modes[bh] == SVG_TEMPORAL;
  const int c = tid % CPR;
  __shared__ float red[4];

  // K: working-layout rows t*64 .. t*64+63
  bf16x8 kv[PASSES];
  float amax = 0.f;
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int xw = t * 64 + p * RPP + tid / CPR;
    kv[p] = bf16x8{};
    if (xw < g.L) {
      const int xs = temporal ? perm_inv_row(g, xw) : xw;
      kv[p] = *reinterpret_cast<const bf16x8*>(k + base + (int64_t)xs * s.x + c * 8);
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf((float)kv[p][i]));
    }
  }
  amax = wave_max(amax);
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int kk = pow2_scale_exp(amax);
  if (tid == 0) sk[(int64_t)bh * nKT + t] = ldexpf(1.f, kk);
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int xw = t * 64 + p * RPP + tid / CPR;
    if (xw < g.L)
      *reinterpret_cast<i32x2*>(k8 + ((int64_t)bh * g.L + xw) * D + c * 8) = to_e4m3(kv[p], kk);
  }

  // Q: natural rows t*64 .. t*64+63, one scale per row (the CPR lanes of a
  // row are adjacent, so the row max is a butterfly over CPR lanes)
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int x = t * 64 + p * RPP + tid / CPR;
    bf16x8 qv = bf16x8{};
    float m = 0.f;
    if (x < g.L) {
      qv = *reinterpret_cast<const bf16x8*>(q + base + (int64_t)x * s.x + c * 8);
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf((float)qv[i]));
    }
#pragma unroll
    for (int o = 1; o < CPR; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
    const int kq = pow2_scale_exp(m);
    if (x < g.L) {
      *reinterpret_cast<i32x2*>(q8 + ((int64_t)bh * g.L + x) * D + c * 8) = to_e4m3(qv, kq);
      if (c == 0) sq[(int64_t)bh * g.L + x] = ldexpf(1.f, kq);
    }
  }
}

// ---------------------------------------------------------------------------
// V in E4M3 for the FP8 P.V product.  One power-of-two scale per head (E4M3
// is floating point: the scale only sets the range, every value keeps its 3
// mantissa bits), applied once to the output.  Codes are stored per tile of
// 64 keys of the head's working layout, transposed: v8[bh][tile][dim][64],
// the 64 bytes of a dim row in "P-register order": byte p = 32 g + j holds
// key kappa(g, j) = 32 (j / 16) + 8 ((j % 16) / 4) + 4 g + j % 4, the key
// whose weight lane group g of the score accumulator holds in register j.
// grid (BH): amax word of each head cleared (a fill kernel, not a memset).
__global__ void k_v_amax_clear(float* __restrict__ sv, int32_t BH) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < BH) sv[i] = 0.f;
}

// grid (nBlk, BH), 256 threads: max |V| over the head's natural rows, each
// workgroup striding over row blocks of 64 (nBlk <= 32, so at most 32 atomic
// updates per head word), folded in by an atomic max on the bits of a
// non-negative float (their order is the integer order): the result does not
// depend on scheduling.
template <int D>
__global__ __launch_bounds__(256) void k_v_amax(KGeom g, const __bf16* __restrict__ v, svg_strides s,
                                                float* __restrict__ sv, int32_t nKT) {
  constexpr int CPR = D / 8, RPP = 256 / CPR, PASSES = 64 / RPP;
  __shared__ float red[4];
  const int bh = blockIdx.y, tid = threadIdx.x;
  const int b = bh / g.H, h = bh % g.H;
  const int64_t base = (int64_t)b * s.b + (int64_t)h * s.h;
  float amax = 0.f;
  for (int t = blockIdx.x; t < nKT; t += gridDim.x) {
    bf16x8 vv[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int x = min(t * 64 + p * RPP + tid / CPR, g.L - 1);  // a repeated row changes no max
      vv[p] = *reinterpret_cast<const bf16x8*>(v + base + (int64_t)x * s.x + (tid % CPR) * 8);
    }
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf((float)vv[p][i]));
  }
  amax = wave_max(amax);
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  if (tid == 0) {
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    atomicMax(reinterpret_cast<unsigned int*>(sv + bh), __float_as_uint(amax));
  }
}

// grid (nKT, BH), 256 threads: the working-layout tile t of head bh encoded
// with the head's scale (sv[bh] still holds its amax).  The bf16 tile is
// staged in LDS row-major; each thread then builds whole 16-byte chunks of
// the transposed output (16 keys of one dim, read down an LDS column with
// consecutive lanes on consecutive dims), so LDS reads are conflict-free and
// every global write is a 16-byte store.
template <int D>
__global__ __launch_bounds__(256) void k_quant_v(KGeom g, const __bf16* __restrict__ v, svg_strides s,
                                                 const int32_t* __restrict__ modes, const float* __restrict__ sv,
                                                 uint8_t* __restrict__ v8, int32_t nKT) {
  constexpr int CPR = D / 8, RPP = 256 / CPR, PASSES = 64 / RPP;
  __shared__ __attribute__((aligned(16))) __bf16 tile[64 * D];
  const int t = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int b = bh / g.H, h = bh % g.H;
  const int64_t base = (int64_t)b * s.b + (int64_t)h * s.h;
  const bool temporal = modes[bh] == SVG_TEMPORAL;
  const int kv = pow2_scale_exp(sv[bh]);
  const int c = tid % CPR;
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int r = p * RPP + tid / CPR;  // key within the tile
    const int xw = t * 64 + r;
    bf16x8 vv = bf16x8{};  // keys beyond L encode 0
    if (xw < g.L) {
      const int xs = temporal ? perm_inv_row(g, xw) : xw;
      vv = *reinterpret_cast<const bf16x8*>(v + base + (int64_t)xs * s.x + c * 8);
    }
    *reinterpret_cast<bf16x8*>(tile + r * D + c * 8) = vv;
  }
  __syncthreads();
  uint8_t* dst = v8 + ((int64_t)bh * nKT + t) * (D * 64);
  for (int idx = tid; idx < D * 4; idx += 256) {
    const int m = idx % D, q = idx / D;  // dim, 16-byte chunk of its row
    bf16x8 lo, hi;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int p = 16 * q + i;
      const int j = p & 31, grp = p >> 5;
      lo[i] = tile[(32 * (j >> 4) + 8 * ((j & 15) >> 2) + 4 * grp + (j & 3)) * D + m];
      const int p2 = p + 8;
      const int j2 = p2 & 31, grp2 = p2 >> 5;
      hi[i] = tile[(32 * (j2 >> 4) + 8 * ((j2 & 15) >> 2) + 4 * grp2 + (j2 & 3)) * D + m];
    }
    const i32x2 a = to_e4m3(lo, kv), bb = to_e4m3(hi, kv);
    const i32x4 w = {a[0], a[1], bb[0], bb[1]};
    *reinterpret_cast<i32x4*>(dst + m * 64 + q * 16) = w;
  }
}

// grid (BH): the head's amax turned into its scale.
__global__ void k_v_scale(float* __restrict__ sv, int32_t BH) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < BH) sv[i] = ldexpf(1.f, pow2_scale_exp(sv[i]));
}

// K8 tile in LDS: 64 rows of D bytes in 16-byte chunks, XOR-swizzled like the
// bf16 K tile (chunk position ^ (row / rows-per-256-byte-line) % chunks).
template <int D>
struct Fp8Cfg {
  static constexpr int CR = D / 16;      // 16-byte chunks per K8 row
  static constexpr int RPL = 16 / CR;    // rows per 256-byte LDS line
  static constexpr int CHUNKS = kBN * CR;
  static constexpr int SEGS = CHUNKS / 64;
  static constexpr int TILE_BYTES = kBN * D;
  __device__ static __forceinline__ int swz(int r) { return (r / RPL) % CR; }
};

// Loads of one K8 tile (contiguous rows of the working layout) and one bf16
// V tile (gathered through the index map when VIRT) into LDS.
template <int D, bool VIRT, int WAVES>
struct Fp8Loader {
  using C8 = Fp8Cfg<D>;
  using CV = TileCfg<D, WAVES>;
  static constexpr int KLOADS = (C8::SEGS + WAVES - 1) / WAVES;
  const uint8_t* kb;
  const char* vb;
  int64_t sxb;  // V token stride in bytes
  int L;

  __device__ __forceinline__ void init(const uint8_t* K8, const __bf16* V, int64_t sx, int L_) {
    kb = K8;
    vb = reinterpret_cast<const char*>(V);
    sxb = sx * 2;
    L = L_;
  }

  __device__ __forceinline__ void load(const KGeom& g, int kt0, uint8_t* lds_k, __bf16* lds_v, int wave,
                                       int lane) const {
#pragma unroll
    for (int i = 0; i < KLOADS; ++i) {
      const int seg = i * WAVES + wave;
      if (C8::SEGS % WAVES != 0 && seg >= C8::SEGS) break;  // wave-uniform
      const int p = seg * 64 + lane;
      const int r = p / C8::CR, pos = p % C8::CR;
      int row = kt0 + r;
      row = row < L ? row : L - 1;
      __builtin_amdgcn_global_load_lds((const void*)(kb + (int64_t)row * D + (pos ^ C8::swz(r)) * 16),
                                       (SVG_LDS void*)(lds_k + seg * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < CV::LOADS; ++i) {
      const int seg = i * WAVES + wave;
      if (CV::SEGS % WAVES != 0 && seg >= CV::SEGS) break;  // wave-uniform
      const int p = seg * 64 + lane;
      const int r = p / CV::CR, pos = p % CV::CR;
      int row = kt0 + r;
      row = row < L ? row : L - 1;
      if (VIRT) row = perm_inv_row(g, row);
      __builtin_amdgcn_global_load_lds((const void*)(vb + (int64_t)row * sxb + (pos ^ CV::swz_v(r)) * 16),
                                       (SVG_LDS void*)(lds_v + seg * 512), 16, 0, 0);
    }
  }
};

// Scores S^T (64 keys x 32 queries) of a K8 tile: two 32-key chains, D / 64
// MFMAs of K = 64 each.  A operand: lane (key m, half hh) holds the 32 bytes
// of key m at d = 64*ks + 32*hh .. +31; B operand: the query's bytes at the
// same d (the same k order on both sides).
template <int D>
__device__ __forceinline__ void score_tile_fp8(const uint8_t* lk, const i32x8* qf, int lane, f32x16& s0,
                                               f32x16& s1) {
  using C8 = Fp8Cfg<D>;
  constexpr int KS = D / 64;
  const int hh = lane >> 5;
  const int m0 = lane & 31, m1 = 32 + (lane & 31);
  auto rd = [&](int m, int ks) {
    const int sw = C8::swz(m);
    const int c0 = 4 * ks + 2 * hh;
    const i32x4 a = *reinterpret_cast<const i32x4*>(lk + m * D + ((c0 ^ sw) * 16));
    const i32x4 b = *reinterpret_cast<const i32x4*>(lk + m * D + (((c0 + 1) ^ sw) * 16));
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  i32x8 f0[KS], f1[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    f0[ks] = rd(m0, ks);
    f1[ks] = rd(m1, ks);
  }
  s0 = f32x16{};
  s1 = f32x16{};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    s0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f0[ks], qf[ks], s0, 0, 0, 0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f1[ks], qf[ks], s1, 0, 0, 0, 0, 0, 0);
  }
}

// As score_tile_fp8 with the query fragments read from LDS (the lane's 16-byte
// halves at lq + (2 * ks + half) * 1024 + 16 * lane, written by the lane
// itself before the sweep).  The FP8 P.V kernel keeps them there at d 128,
// where at its 168-register cap it otherwise spills one of them, and the
// reload from scratch, counted with the vector-memory loads, made every
// tile's first score MFMA wait for the next tile's K/V loads as well
// (-5 % attention time; at d 64, where nothing spills, +1 %).
template <int D>
inline constexpr bool kFp8PvQInLds = D == 128;
template <int D>
__device__ __forceinline__ void score_tile_fp8_lq(const uint8_t* lk, const uint8_t* lq, int lane, f32x16& s0,
                                                  f32x16& s1) {
  constexpr int KS = D / 64;
  i32x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const i32x4 a = *reinterpret_cast<const i32x4*>(lq + (2 * ks) * 1024 + 16 * lane);
    const i32x4 b = *reinterpret_cast<const i32x4*>(lq + (2 * ks + 1) * 1024 + 16 * lane);
    qf[ks] = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  score_tile_fp8<D>(lk, qf, lane, s0, s1);
}

// Lock-step sweep with fp8 scores (as sweep() in attn_common.h): 2-stage
// ring, one barrier per tile, masks on partial tiles, idle tiles skipped per
// wave.  sl2q = scale * log2(e) * sq(row); sk: this head's K tile scales.
template <int D, bool VIRT, int WAVES>
__device__ __forceinline__ void sweep_fp8(Flash<D>& st, const i32x8* qf, const Fp8Loader<D, VIRT, WAVES>& ld,
                                          const KGeom& g, int4 rg, int lo, int hi, bool valid, float sl2q,
                                          const float* __restrict__ sk, uint8_t* lds_k0, __bf16* lds_v0,
                                          int wave, int lane) {
  constexpr int KB = Fp8Cfg<D>::TILE_BYTES, VE = TileCfg<D>::TILE_ELEMS;
  const int hh = lane >> 5;
  const int T = g.T;
  const int n1 = rg.y - rg.x, nt = n1 + (rg.w - rg.z);
  auto tile_of = [&](int t) { return t < n1 ? rg.x + t : rg.z + (t - n1); };
  const int max_lo = wave_max_i(valid ? lo : INT_MIN);
  const int min_hi = wave_min_i(valid ? hi : INT_MAX);
  const int min_lo = wave_min_i(valid ? lo : INT_MAX);
  const int max_hi = wave_max_i(valid ? hi : INT_MIN);
  const bool wave_rows = wave_max_i(valid ? 1 : 0) != 0;
  st.init();
  if (nt > 0) ld.load(g, tile_of(0) * kBN, lds_k0, lds_v0, wave, lane);
  wait_vm_all();
  __syncthreads();
  auto step = [&](int t, auto stc) {
    constexpr int sg = decltype(stc)::value;
    uint8_t* lk = lds_k0 + sg * KB;
    __bf16* lv = lds_v0 + sg * VE;
    if (t + 1 < nt) ld.load(g, tile_of(t + 1) * kBN, lds_k0 + (sg ^ 1) * KB, lds_v0 + (sg ^ 1) * VE, wave, lane);
    const int kt = tile_of(t), kt0 = kt * kBN, kt1 = kt0 + kBN;
    const bool idle = kt0 >= T && (kt1 <= min_lo || kt0 >= max_hi);
    if (wave_rows && !idle) {
      const bool full = (kt1 <= T) || (max(kt0, T) >= max_lo && kt1 <= min_hi);
      f32x16 s0, s1;
      score_tile_fp8<D>(lk, qf, lane, s0, s1);
      if (!full) mask_tile(s0, s1, kt0, hh, T, lo, hi);
      st.add_tile(s0, s1, lv, lane, sl2q * sk[kt]);
    }
    wait_vm_all();
    __syncthreads();
  };
  for (int t = 0; t < nt; t += 2) {
    step(t, std::integral_constant<int, 0>{});
    if (t + 1 < nt) step(t + 1, std::integral_constant<int, 1>{});
  }
}

// ---------------------------------------------------------------------------
// FP8 P.V.  V8 tiles are 64 keys x D dims transposed: D rows of 64 bytes
// (P-register key order), 4 chunks of 16 bytes per row, stored in LDS
// with chunk position ^ ((row / 4) % 4) so the 16-byte A-operand reads of 16
// consecutive dims hit distinct banks.
template <int D>
struct V8Cfg {
  static constexpr int CHUNKS = D * 4;
  static constexpr int SEGS = CHUNKS / 64;
  static constexpr int TILE_BYTES = D * 64;
  __device__ static __forceinline__ int swz(int m) { return (m >> 2) & 3; }
};

// K8 and V8 tiles of one working-layout tile, both contiguous in global
// memory; the V8 swizzle is applied through the per-lane source offsets.
template <int D, int WAVES>
struct Fp8PvLoader {
  using C8 = Fp8Cfg<D>;
  using CV = V8Cfg<D>;
  static constexpr int KLOADS = (C8::SEGS + WAVES - 1) / WAVES;
  static constexpr int VLOADS = (CV::SEGS + WAVES - 1) / WAVES;
  const uint8_t* kb;
  const uint8_t* vb;  // this head's V8 tiles
  int L;

  __device__ __forceinline__ void load(int kt, uint8_t* lds_k, uint8_t* lds_v, int wave, int lane) const {
    const int kt0 = kt * kBN;
#pragma unroll
    for (int i = 0; i < KLOADS; ++i) {
      const int seg = i * WAVES + wave;
      if (C8::SEGS % WAVES != 0 && seg >= C8::SEGS) break;  // wave-uniform
      const int p = seg * 64 + lane;
      const int r = p / C8::CR, pos = p % C8::CR;
      int row = kt0 + r;
      row = row < L ? row : L - 1;
      __builtin_amdgcn_global_load_lds((const void*)(kb + (int64_t)row * D + (pos ^ C8::swz(r)) * 16),
                                       (SVG_LDS void*)(lds_k + seg * 1024), 16, 0, 0);
    }
    const uint8_t* tv = vb + (int64_t)kt * CV::TILE_BYTES;
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int seg = i * WAVES + wave;
      if (CV::SEGS % WAVES != 0 && seg >= CV::SEGS) break;  // wave-uniform
      const int p = seg * 64 + lane;
      const int m = p >> 2, pos = p & 3;
      __builtin_amdgcn_global_load_lds((const void*)(tv + m * 64 + (pos ^ CV::swz(m)) * 16),
                                       (SVG_LDS void*)(lds_v + seg * 1024), 16, 0, 0);
    }
  }
};

// Online softmax with FP8 weights.  The reference max moves when a tile's
// max exceeds it by more than 2 (log2 units); weights are
// p = 2^(x - m_ref + 6) in E4M3, so they lie in [2^-9, 2^8] (E4M3 keeps
// 3 mantissa bits from 2^-6 up, subnormals to 2^-9, max 448) and a key is
// dropped only when its weight is below 2^-15 of the reference.  The row sum
// is taken from the same E4M3 weights by one extra MFMA against a block of
// ones, so the normalisation matches the weights P.V uses.
template <int D>
struct Flash8 {
  f32x16 o[D / 32];
  float m_ref, l;

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
    m_ref = -INFINITY;
    l = 0.f;
  }

  // s0, s1: raw scores (masked entries -inf), sl2 > 0: their log2 multiplier.
  __device__ __forceinline__ i32x8 softmax(const f32x16& s0, const f32x16& s1, float sl2) {
    const float mx = tile_max(s0, s1, sl2);
    const bool need = mx > m_ref + 2.0f;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      const float alpha = !need ? 1.f : (m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref - mx));
      l *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
      m_ref = need ? mx : m_ref;
    }
    const float bias = (m_ref == -INFINITY ? 0.f : -m_ref) + 6.0f;
    i32x8 p8;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      // register j = 4 w .. 4 w + 3: s0[j] for j < 16, s1[j - 16] after
      const f32x16& sv = w < 4 ? s0 : s1;
      const int r0 = (w & 3) * 4;
      const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[r0], sl2, bias));
      const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[r0 + 1], sl2, bias));
      const float e2 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[r0 + 2], sl2, bias));
      const float e3 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[r0 + 3], sl2, bias));
      int wd = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, 0, false);
      p8[w] = __builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, wd, true);
    }
    return p8;
  }

  // o += V^T P^T for one tile (D / 32 MFMAs of K = 64) and l += the tile's
  // weight sum (one MFMA with A = ones).
  __device__ __forceinline__ void pv(const i32x8& p8, const uint8_t* __restrict__ lv, int lane) {
    using CV = V8Cfg<D>;
    const int hh = lane >> 5;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int m = db * 32 + (lane & 31);
      const int sw = CV::swz(m);
      const i32x4 a = *reinterpret_cast<const i32x4*>(lv + m * 64 + (((2 * hh) ^ sw) * 16));
      const i32x4 b = *reinterpret_cast<const i32x4*>(lv + m * 64 + (((2 * hh + 1) ^ sw) * 16));
      const i32x8 vf = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
      o[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, p8, o[db], 0, 0, 0, 0, 0, 0);
    }
    const int one = 0x38383838;  // E4M3 1.0 in every byte
    const i32x8 ones = {one, one, one, one, one, one, one, one};
    const f32x16 rs = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, p8, f32x16{}, 0, 0, 0, 0, 0, 0);
    l += rs[0];
  }
};

// Sweep with fp8 scores and fp8 P.V (as sweep_fp8).
template <int D, int WAVES>
__device__ __forceinline__ void sweep_fp8pv(Flash8<D>& st, const i32x8* qf, const uint8_t* lq,
                                            const Fp8PvLoader<D, WAVES>& ld,
                                            const KGeom& g, int4 rg, int lo, int hi, bool valid, float sl2q,
                                            const float* __restrict__ sk, uint8_t* lds_k0, uint8_t* lds_v0,
                                            int wave, int lane) {
  constexpr int KB = Fp8Cfg<D>::TILE_BYTES, VB = V8Cfg<D>::TILE_BYTES;
  const int hh = lane >> 5;
  const int T = g.T;
  const int n1 = rg.y - rg.x, nt = n1 + (rg.w - rg.z);
  auto tile_of = [&](int t) { return t < n1 ? rg.x + t : rg.z + (t - n1); };
  const int max_lo = wave_max_i(valid ? lo : INT_MIN);
  const int min_hi = wave_min_i(valid ? hi : INT_MAX);
  const int min_lo = wave_min_i(valid ? lo : INT_MAX);
  const int max_hi = wave_max_i(valid ? hi : INT_MIN);
  const bool wave_rows = wave_max_i(valid ? 1 : 0) != 0;
  st.init();
  if (nt > 0) ld.load(tile_of(0), lds_k0, lds_v0, wave, lane);
  wait_vm_all();
  __syncthreads();
  auto step = [&](int t, auto stc) {
    constexpr int sg = decltype(stc)::value;
    uint8_t* lk = lds_k0 + sg * KB;
    uint8_t* lv = lds_v0 + sg * VB;
    if (t + 1 < nt) ld.load(tile_of(t + 1), lds_k0 + (sg ^ 1) * KB, lds_v0 + (sg ^ 1) * VB, wave, lane);
    const int kt = tile_of(t), kt0 = kt * kBN, kt1 = kt0 + kBN;
    const bool idle = kt0 >= T && (kt1 <= min_lo || kt0 >= max_hi);
    if (wave_rows && !idle) {
      const bool full = (kt1 <= T) || (max(kt0, T) >= max_lo && kt1 <= min_hi);
      f32x16 s0, s1;
      if constexpr (kFp8PvQInLds<D>)
        score_tile_fp8_lq<D>(lk, lq, lane, s0, s1);
      else
        score_tile_fp8<D>(lk, qf, lane, s0, s1);
      if (!full) mask_tile(s0, s1, kt0, hh, T, lo, hi);
      const i32x8 p8 = st.softmax(s0, s1, sl2q * sk[kt]);
      st.pv(p8, lv, lane);
    }
    wait_vm_all();
    __syncthreads();
  };
  for (int t = 0; t < nt; t += 2) {
    step(t, std::integral_constant<int, 0>{});
    if (t + 1 < nt) step(t + 1, std::integral_constant<int, 1>{});
  }
}

struct Fp8Ptrs {
  const uint8_t *q8, *k8, *v8;
  const float *sq, *sk, *svh;  // svh: per-head V scales (FP8 P.V)
  const void* v;
  svg_strides sv;
  void* o;
  svg_strides so;
  const int32_t *modes, *ranges, *order;
  int32_t nKT;
};

template <int D, bool OUT_BF16, bool VIRT, int WAVES>
__device__ __forceinline__ void attn_tile_fp8(const KGeom& g, const Fp8Ptrs& a, int bh, int qt, int rq, int mode, int nQT,
                                              uint8_t* lds_k, __bf16* lds_v, int wave, int lane) {
  constexpr int BMW = 32 * WAVES;
  const int hh = lane >> 5;
  const int b = bh / g.H, h = bh % g.H;
  const int64_t vbase = (int64_t)b * a.sv.b + (int64_t)h * a.sv.h;
  const int64_t obase = (int64_t)b * a.so.b + (int64_t)h * a.so.h;
  constexpr int OE = OUT_BF16 ? 2 : 4;
  auto phys = [&g](int r) { return VIRT ? perm_inv_row(g, r) : r; };

  const int4 rg = reinterpret_cast<const int4*>(a.ranges)[(int64_t)bh * nQT + rq];
  Fp8Loader<D, VIRT, WAVES> ld;
  ld.init(a.k8 + (int64_t)bh * g.L * D, static_cast<const __bf16*>(a.v) + vbase, a.sv.x, g.L);

  const int xq = qt * BMW + wave * 32 + (lane & 31);
  const bool valid = xq < g.L;
  const int xqc = valid ? xq : g.L - 1;
  const int xs = phys(xqc);
  const uint8_t* qrow = a.q8 + ((int64_t)bh * g.L + xs) * D + 32 * hh;
  i32x8 qf[D / 64];
#pragma unroll
  for (int ks = 0; ks < D / 64; ++ks) qf[ks] = *reinterpret_cast<const i32x8*>(qrow + 64 * ks);
  const float sl2q = g.scale_log2 * a.sq[(int64_t)bh * g.L + xs];
  int lo, hi;
  row_interval(g, mode, xqc, lo, hi);

  Flash<D> st;
  sweep_fp8<D, VIRT, WAVES>(st, qf, ld, g, rg, lo, hi, valid, sl2q, a.sk + (int64_t)bh * a.nKT, lds_k, lds_v, wave,
                            lane);

  const float l_tot = half_sum(st.l_part);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (valid) {
    char* orow = static_cast<char*>(a.o) + (obase + (int64_t)phys(xq) * a.so.x) * OE;
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

// One query tile with FP8 P.V (Q8, O through the index map for TEMPORAL heads).
template <int D, bool OUT_BF16, bool VIRT, int WAVES>
__device__ __forceinline__ void attn_tile_fp8pv(const KGeom& g, const Fp8Ptrs& a, int bh, int qt, int rq, int mode, int nQT,
                                                uint8_t* lds_k, uint8_t* lds_v, uint8_t* lds_q, int wave, int lane) {
  constexpr int BMW = 32 * WAVES;
  const int hh = lane >> 5;
  const int b = bh / g.H, h = bh % g.H;
  const int64_t obase = (int64_t)b * a.so.b + (int64_t)h * a.so.h;
  constexpr int OE = OUT_BF16 ? 2 : 4;
  auto phys = [&g](int r) { return VIRT ? perm_inv_row(g, r) : r; };

  const int4 rg = reinterpret_cast<const int4*>(a.ranges)[(int64_t)bh * nQT + rq];
  Fp8PvLoader<D, WAVES> ld;
  ld.kb = a.k8 + (int64_t)bh * g.L * D;
  ld.vb = a.v8 + (int64_t)bh * a.nKT * V8Cfg<D>::TILE_BYTES;
  ld.L = g.L;

  const int xq = qt * BMW + wave * 32 + (lane & 31);
  const bool valid = xq < g.L;
  const int xqc = valid ? xq : g.L - 1;
  const int xs = phys(xqc);
  const uint8_t* qrow = a.q8 + ((int64_t)bh * g.L + xs) * D + 32 * hh;
  // the query fragments, in registers or (d 128) in this wave's own LDS
  // region (16-byte halves, lane-contiguous: conflict-free reads)
  i32x8 qf[D / 64];
  uint8_t* lq = lds_q + wave * (D / 64) * 2048;
#pragma unroll
  for (int ks = 0; ks < D / 64; ++ks) {
    qf[ks] = *reinterpret_cast<const i32x8*>(qrow + 64 * ks);
    if constexpr (kFp8PvQInLds<D>) {
      *reinterpret_cast<i32x4*>(lq + (2 * ks) * 1024 + 16 * lane) = __builtin_shufflevector(qf[ks], qf[ks], 0, 1, 2, 3);
      *reinterpret_cast<i32x4*>(lq + (2 * ks + 1) * 1024 + 16 * lane) =
          __builtin_shufflevector(qf[ks], qf[ks], 4, 5, 6, 7);
    }
  }
  const float sl2q = g.scale_log2 * a.sq[(int64_t)bh * g.L + xs];
  int lo, hi;
  row_interval(g, mode, xqc, lo, hi);

  Flash8<D> st;
  sweep_fp8pv<D, WAVES>(st, qf, lq, ld, g, rg, lo, hi, valid, sl2q, a.sk + (int64_t)bh * a.nKT, lds_k, lds_v,
                        wave, lane);

  // every lane holds its row's whole weight sum (the ones-MFMA sums all keys)
  const float inv = st.l > 0.f ? a.svh[bh] / st.l : 0.f;
  // the output row and column offset are formed anew from the lane id (read
  // in asm so that it is not shared with the one taken before the sweep), so
  // that nothing of them stays live across the key loop
  int lid;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lid));
  const int xo = qt * BMW + wave * 32 + (lid & 31), ho = lid >> 5;
  if (xo < g.L) {
    char* orow = static_cast<char*>(a.o) + (obase + (int64_t)phys(xo) * a.so.x) * OE;
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

// WAVES = 4 (FP8 P.V): a workgroup takes half of a 256-row query tile (with
// that tile's key-tile ranges); three workgroups share a CU and, not being in
// lock step, one's softmax runs under another's MFMAs (all products are FP8
// there, so the softmax outweighs them).  FP8 scores with bf16 P.V keep 8
// waves (measured faster).
template <int D, bool OUT_BF16, int WAVES, bool PV8>
__global__ __launch_bounds__(64 * WAVES, WAVES == 4 ? 3 : 1) void k_attn_fp8(KGeom g, Fp8Ptrs a, int32_t nQT,
                                                                           int32_t total) {
  constexpr int BMW = 32 * WAVES;
  constexpr int SPLIT = kBM_bf16 / BMW;  // workgroups per ranges tile
  extern __shared__ __attribute__((aligned(16))) uint8_t lds8[];
  uint8_t* lds_k = lds8;  // [2][TILE_BYTES], then two V tiles (bf16 or V8)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int w = blockIdx.x;
  const int logical = xcd_logical(w, g.nxcd, kXcdRun);
  if (logical >= total) return;
  const int bh = a.order[logical / (nQT * SPLIT)];
  const int qt = logical % (nQT * SPLIT), rq = qt / SPLIT;
  const int mode = a.modes[bh];
  if (mode == SVG_SKIP) {
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
  if constexpr (PV8) {
    uint8_t* lds_v = lds8 + 2 * Fp8Cfg<D>::TILE_BYTES;
    uint8_t* lds_q = lds_v + 2 * V8Cfg<D>::TILE_BYTES;  // [WAVES][D / 64][2][64 lanes x 16 B]
    if (mode == SVG_TEMPORAL)
      attn_tile_fp8pv<D, OUT_BF16, true, WAVES>(g, a, bh, qt, rq, mode, nQT, lds_k, lds_v, lds_q, wave, lane);
    else
      attn_tile_fp8pv<D, OUT_BF16, false, WAVES>(g, a, bh, qt, rq, mode, nQT, lds_k, lds_v, lds_q, wave, lane);
  } else {
    __bf16* lds_v = reinterpret_cast<__bf16*>(lds8 + 2 * Fp8Cfg<D>::TILE_BYTES);
    if (mode == SVG_TEMPORAL)
      attn_tile_fp8<D, OUT_BF16, true, WAVES>(g, a, bh, qt, rq, mode, nQT, lds_k, lds_v, wave, lane);
    else
      attn_tile_fp8<D, OUT_BF16, false, WAVES>(g, a, bh, qt, rq, mode, nQT, lds_k, lds_v, wave, lane);
  }
}

hipError_t launch_quant_qk(const KGeom& g, const void* q, const void* k, svg_strides s, const int32_t* modes,
                           uint8_t* q8, float* sq, uint8_t* k8, float* sk, hipStream_t st) {
  const int32_t nKT = (g.L + kBN - 1) / kBN;
  dim3 grid((unsigned)nKT, (unsigned)(g.B * g.H));
  const __bf16 *bq = static_cast<const __bf16*>(q), *bk = static_cast<const __bf16*>(k);
  if (g.d == 64)
    hipLaunchKernelGGL(k_quant_qk<64>, grid, dim3(256), 0, st, g, bq, bk, s, modes, q8, sq, k8, sk, nKT);
  else
    hipLaunchKernelGGL(k_quant_qk<128>, grid, dim3(256), 0, st, g, bq, bk, s, modes, q8, sq, k8, sk, nKT);
  return hipGetLastError();
}

hipError_t launch_quant_v(const KGeom& g, const void* v, svg_strides s, const int32_t* modes, uint8_t* v8, float* sv,
                          hipStream_t st) {
  const int32_t nKT = (g.L + kBN - 1) / kBN;
  const int32_t BH = g.B * g.H;
  dim3 grid((unsigned)nKT, (unsigned)BH);
  const __bf16* bv = static_cast<const __bf16*>(v);
  hipLaunchKernelGGL(k_v_amax_clear, dim3((unsigned)((BH + 255) / 256)), dim3(256), 0, st, sv, BH);
  const dim3 agrid((unsigned)(nKT < 32 ? nKT : 32), (unsigned)BH);
  if (g.d == 64) {
    hipLaunchKernelGGL(k_v_amax<64>, agrid, dim3(256), 0, st, g, bv, s, sv, nKT);
    hipLaunchKernelGGL(k_quant_v<64>, grid, dim3(256), 0, st, g, bv, s, modes, sv, v8, nKT);
  } else {
    hipLaunchKernelGGL(k_v_amax<128>, agrid, dim3(256), 0, st, g, bv, s, sv, nKT);
    hipLaunchKernelGGL(k_quant_v<128>, grid, dim3(256), 0, st, g, bv, s, modes, sv, v8, nKT);
  }
  hipLaunchKernelGGL(k_v_scale, dim3((unsigned)((BH + 255) / 256)), dim3(256), 0, st, sv, BH);
  return hipGetLastError();
}

// Waves per workgroup of the FP8 attention kernel, and workgroups per
// 256-row ranges tile.
template <bool PV8>
constexpr int fp8_waves() {
  return PV8 ? 4 : kAttnWaves;
}
template <bool PV8>
constexpr int fp8_split() {
  return kBM_bf16 / (32 * fp8_waves<PV8>());
}

template <int D, bool OUT_BF16, bool PV8>
static hipError_t launch_fp8(const KGeom& g, const Fp8Ptrs& a, int32_t nQT, int64_t grid, int64_t total,
                             hipStream_t st) {
  constexpr int W = fp8_waves<PV8>();
  const size_t vtile = PV8 ? (size_t)V8Cfg<D>::TILE_BYTES : (size_t)TileCfg<D>::TILE_ELEMS * sizeof(__bf16);
  // FP8 P.V: plus each wave's query fragments
  const size_t lds =
      2 * (size_t)Fp8Cfg<D>::TILE_BYTES + 2 * vtile + (PV8 && kFp8PvQInLds<D> ? (size_t)W * (D / 64) * 2048 : 0);
  auto kern = k_attn_fp8<D, OUT_BF16, W, PV8>;
  static std::atomic<uint64_t> lds_set{0};
  if (hipError_t e = ensure_dynamic_lds((const void*)kern, lds, lds_set); e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * W), lds, st, g, a, nQT, (int32_t)total);
  return hipGetLastError();
}

template <bool PV8>
static hipError_t launch_fp8_d(const KGeom& g, const Fp8Ptrs& a, bool out_bf16, hipStream_t st) {
  const int32_t nQT = (g.L + kBM_bf16 - 1) / kBM_bf16;
  const int64_t total = (int64_t)g.B * g.H * nQT * fp8_split<PV8>();
  const int64_t grid = xcd_grid(total, g.nxcd, kXcdRun);
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  if (g.d == 64)
    return out_bf16 ? launch_fp8<64, true, PV8>(g, a, nQT, grid, total, st)
                    : launch_fp8<64, false, PV8>(g, a, nQT, grid, total, st);
  return out_bf16 ? launch_fp8<128, true, PV8>(g, a, nQT, grid, total, st)
                  : launch_fp8<128, false, PV8>(g, a, nQT, grid, total, st);
}

hipError_t launch_attention_fp8(const KGeom& g, const uint8_t* q8, const float* sq, const uint8_t* k8,
                                const float* sk, const void* v, svg_strides sv, void* o, svg_strides so,
                                bool out_bf16, const int32_t* modes, const int32_t* ranges, const int32_t* order,
                                hipStream_t st) {
  Fp8Ptrs a{};
  a.q8 = q8;
  a.sq = sq;
  a.k8 = k8;
  a.sk = sk;
  a.v = v;
  a.sv = sv;
  a.o = o;
  a.so = so;
  a.modes = modes;
  a.ranges = ranges;
  a.order = order;
  a.nKT = (g.L + kBN - 1) / kBN;
  return launch_fp8_d<false>(g, a, out_bf16, st);
}

hipError_t launch_attention_fp8pv(const KGeom& g, const uint8_t* q8, const float* sq, const uint8_t* k8,
                                  const float* sk, const uint8_t* v8, const float* svh, void* o, svg_strides so,
                                  bool out_bf16, const int32_t* modes, const int32_t* ranges, const int32_t* order,
                                  hipStream_t st) {
  Fp8Ptrs a{};
  a.q8 = q8;
  a.sq = sq;
  a.k8 = k8;
  a.sk = sk;
  a.v8 = v8;
  a.svh = svh;
  a.o = o;
  a.so = so;
  a.modes = modes;
  a.ranges = ranges;
  a.order = order;
  a.nKT = (g.L + kBN - 1) / kBN;
  return launch_fp8_d<true>(g, a, out_bf16, st);
}

}  // namespace svg
