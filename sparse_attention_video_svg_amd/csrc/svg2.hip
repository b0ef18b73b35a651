// SVG2: semantic-aware permutation with centroid-based top-p selection
// ("Sparse VideoGen2 ..." explainer, 2. Methodology: A. Q and K tokens
// clustered independently by k-means and reordered so each cluster is
// contiguous; B. attention estimated between cluster centroids, key clusters
// taken in descending estimate until the cumulative score reaches p; C. a
// kernel with dynamic block sizes that loads the scattered keys and computes
// densely on contiguous queries).
//
// Per head, on gfx950:
//  * k-means, one Lloyd iteration = k_km_split (fp32 centroids -> bf16 hi +
//    bf16 lo residual, and 0.5 |mu|^2) -> k_km_assign (scores x . mu on the
//    matrix cores as x . hi + x . lo, centroid tiles streamed through LDS like
//    K tiles, argmax of x . mu - 0.5 |mu|^2, ties to the lower index) ->
//    stable counting sort (k_km_hist: per-block counts and in-block ranks;
//    k_km_scan: per-cluster totals, starts, per-block bases; k_km_scatter)
//    -> k_km_update (mean of each cluster's tokens summed in cluster order:
//    deterministic).  The last iteration's sort is the permutation.
//  * k_svg2_select: per query cluster, fp32 centroid scores against every key
//    cluster, the size-weighted softmax, ranks by comparison, the running sum
//    in rank order, the top-p prefix, and the tile list of the selected key
//    clusters (ranges of at most 64 consecutive keys of the cluster order).
//  * k_gather_rows: K and V copied into cluster order once.
//  * k_svg2_attn: one workgroup per (query cluster, block of 256 of its
//    rows): query rows gathered through the permutation, the tile list swept
//    with the attention kernel's loader, scores, softmax and P.V (the last
//    tile of a key cluster masks its missing keys), rows scattered back.
#include "attn_common.h"

namespace svg {

constexpr int kKmRows = 256;  // tokens per assign / histogram workgroup

__device__ __forceinline__ float block_sum_fixed(float v, float* red) {
  // fixed-tree sum over blockDim.x (a power of two <= 1024) threads
  const int t = threadIdx.x;
  red[t] = v;
  __syncthreads();
  for (int w = blockDim.x / 2; w > 0; w >>= 1) {
    if (t < w) red[t] += red[t + w];
    __syncthreads();
  }
  const float r = red[0];
  __syncthreads();
  return r;
}

// grid (C, BH), D threads: mu[c] = token floor(c * L / C) (fp32).
__global__ void k_km_init(KGeom g, const __bf16* __restrict__ x, svg_strides s, int32_t C, float* __restrict__ mu) {
  const int c = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const int b = bh / g.H, h = bh % g.H;
  const int64_t tok = (int64_t)c * g.L / C;
  mu[((int64_t)bh * C + c) * g.d + t] = (float)x[(int64_t)b * s.b + (int64_t)h * s.h + tok * s.x + t];
}

// grid (C, BH), D threads: hi = bf16(mu), lo = bf16(mu - hi), hn = 0.5 |mu|^2.
__global__ void k_km_split(int32_t C, int32_t D, const float* __restrict__ mu, __bf16* __restrict__ hi,
                           __bf16* __restrict__ lo, float* __restrict__ hn) {
  __shared__ float red[128];
  const int c = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const int64_t o = ((int64_t)bh * C + c) * D + t;
  const float m = mu[o];
  const __bf16 h = (__bf16)m;
  hi[o] = h;
  lo[o] = (__bf16)(m - (float)h);
  const float s = block_sum_fixed(m * m, red);
  if (t == 0) hn[(int64_t)bh * C + c] = 0.5f * s;
}

// grid (ceil(L/256), BH), 8 waves x 32 tokens.  labels[bh*L + x].
template <int D>
__global__ __launch_bounds__(512, 1) void k_km_assign(KGeom g, const __bf16* __restrict__ x, svg_strides s,
                                                      int32_t C, const __bf16* __restrict__ hi,
                                                      const __bf16* __restrict__ lo, const float* __restrict__ hn,
                                                      int32_t* __restrict__ labels) {
  using TC = TileCfg<D, 8>;
  __shared__ __attribute__((aligned(16))) __bf16 lds[2][2][TC::TILE_ELEMS];  // [stage][hi, lo]
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bh = blockIdx.y;
  const int b = bh / g.H, h = bh % g.H;
  const int64_t cb = (int64_t)bh * C;
  KVLoader<D, false, 8> lh, ll;
  lh.init(hi + cb * D, hi + cb * D, D, C, wave, lane);
  ll.init(lo + cb * D, lo + cb * D, D, C, wave, lane);
  const int nct = (C + kBN - 1) / kBN;
  lh.template load1<0>(g, 0, lds[0][0], wave, lane);
  ll.template load1<0>(g, 0, lds[0][1], wave, lane);

  const int tok = blockIdx.x * kKmRows + wave * 32 + (lane & 31);
  const bool valid = tok < g.L;
  bf16x8 qf[D / 16];
  load_q<D>(qf, x + (int64_t)b * s.b + (int64_t)h * s.h + (int64_t)(valid ? tok : g.L - 1) * s.x, hh);
  float best = -INFINITY;
  int bidx = 0x7fffffff;
  wait_vm_all();
  __syncthreads();
  for (int ct = 0; ct < nct; ++ct) {
    const int sg = ct & 1;
    if (ct + 1 < nct) {
      lh.template load1<0>(g, (ct + 1) * kBN, lds[sg ^ 1][0], wave, lane);
      ll.template load1<0>(g, (ct + 1) * kBN, lds[sg ^ 1][1], wave, lane);
    }
    f32x16 a0, a1, b0, b1;
    score_tile<D>(lds[sg][0], qf, lane, a0, a1);
    score_tile<D>(lds[sg][1], qf, lane, b0, b1);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const int c = ct * kBN + acc_key(kb2, r, hh);
        if (c < C) {
          const float v = (kb2 ? a1[r] + b1[r] : a0[r] + b0[r]) - hn[cb + c];
          if (v > best || (v == best && c < bidx)) {
            best = v;
            bidx = c;
          }
        }
      }
    }
    wait_vm_all();
    __syncthreads();
  }
  // the two half-waves hold the same token's other centroids
  const float ob = __shfl_xor(best, 32);
  const int oi = __shfl_xor(bidx, 32);
  if (ob > best || (ob == best && oi < bidx)) bidx = oi;
  if (valid && hh == 0) labels[(int64_t)bh * g.L + tok] = bidx;
}

// grid (nBlk, BH), 256 threads: per-block label counts and each token's rank
// among the earlier tokens of its block with the same label.
__global__ __launch_bounds__(256) void k_km_hist(int32_t L, int32_t C, int32_t nBlk,
                                                 const int32_t* __restrict__ labels, int32_t* __restrict__ hist,
                                                 int32_t* __restrict__ rank) {
  __shared__ int lab[256];
  __shared__ int cnt[1024];
  const int blk = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const int xi = blk * 256 + t;
  for (int c = t; c < C; c += 256) cnt[c] = 0;
  const int l = xi < L ? labels[(int64_t)bh * L + xi] : -1;
  lab[t] = l;
  __syncthreads();
  if (l >= 0) atomicAdd(&cnt[l], 1);
  int r = 0;
  for (int j = 0; j < t; ++j) r += lab[j] == l;
  if (xi < L) rank[(int64_t)bh * L + xi] = r;
  __syncthreads();
  for (int c = t; c < C; c += 256) hist[((int64_t)bh * nBlk + blk) * C + c] = cnt[c];
}

// grid (BH), 1024 threads: cluster totals, starts (start[C] = L) and the
// base position of every (block, cluster) in the cluster order.
__global__ __launch_bounds__(1024) void k_km_scan(int32_t L, int32_t C, int32_t nBlk, const int32_t* __restrict__ hist,
                                                  int32_t* __restrict__ base, int32_t* __restrict__ start) {
  __shared__ int sc[1024];
  const int bh = blockIdx.x, c = threadIdx.x;
  const int64_t hb = (int64_t)bh * nBlk * C;
  int tot = 0;
  if (c < C)
    for (int blk = 0; blk < nBlk; ++blk) tot += hist[hb + (int64_t)blk * C + c];
  sc[c] = c < C ? tot : 0;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {  // inclusive Hillis-Steele scan
    const int v = c >= o ? sc[c - o] : 0;
    __syncthreads();
    sc[c] += v;
    __syncthreads();
  }
  const int st = sc[c] - (c < C ? tot : 0);
  if (c < C) {
    start[(int64_t)bh * (C + 1) + c] = st;
    int run = st;
    for (int blk = 0; blk < nBlk; ++blk) {
      const int64_t o = hb + (int64_t)blk * C + c;
      const int hcount = hist[o];
      base[o] = run;
      run += hcount;
    }
  }
  if (c == 0) start[(int64_t)bh * (C + 1) + C] = L;
}

// grid (nBlk, BH), 256 threads: perm[bh*L + position] = token.
__global__ __launch_bounds__(256) void k_km_scatter(int32_t L, int32_t C, int32_t nBlk,
                                                    const int32_t* __restrict__ labels,
                                                    const int32_t* __restrict__ rank, const int32_t* __restrict__ base,
                                                    int32_t* __restrict__ perm) {
  const int blk = blockIdx.x, bh = blockIdx.y;
  const int xi = blk * 256 + threadIdx.x;
  if (xi >= L) return;
  const int64_t o = (int64_t)bh * L + xi;
  const int pos = base[((int64_t)bh * nBlk + blk) * C + labels[o]] + rank[o];
  perm[(int64_t)bh * L + pos] = xi;
}

// grid (C, BH), D threads: mu = mean of the cluster's tokens, summed in
// cluster order (an empty cluster keeps its centroid).
__global__ void k_km_update(KGeom g, const __bf16* __restrict__ x, svg_strides s, int32_t C,
                            const int32_t* __restrict__ perm, const int32_t* __restrict__ start,
                            float* __restrict__ mu) {
  const int c = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const int b = bh / g.H, h = bh % g.H;
  const __bf16* xb = x + (int64_t)b * s.b + (int64_t)h * s.h + t;
  const int64_t sb = (int64_t)bh * (C + 1);
  const int i0 = start[sb + c], i1 = start[sb + c + 1];
  if (i1 <= i0) return;
  float sum = 0.f;
  for (int i = i0; i < i1; ++i) sum += (float)xb[(int64_t)perm[(int64_t)bh * g.L + i] * s.x];
  mu[((int64_t)bh * C + c) * g.d + t] = sum / (float)(i1 - i0);
}

// grid (Cq, BH), 256 threads.  sel[(bh*Cq + a)*Ck + b]; tiles / ntiles: the
// selected key clusters' keys in cluster order as ranges of <= 64 keys.
__global__ __launch_bounds__(256) void k_svg2_select(KGeom g, int32_t Cq, int32_t Ck, float p,
                                                     const float* __restrict__ mu_q, const float* __restrict__ mu_k,
                                                     const int32_t* __restrict__ start_k, uint8_t* __restrict__ sel,
                                                     int2* __restrict__ tiles, int32_t* __restrict__ ntiles,
                                                     int32_t maxT) {
  __shared__ float P[1024], srt[1024], red[256];
  __shared__ int tsc[1024];
  const int a = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const int D = g.d;
  const float* mq = mu_q + ((int64_t)bh * Cq + a) * D;
  const int64_t sk = (int64_t)bh * (Ck + 1);
  constexpr int PER = 4;  // clusters per thread (Ck <= 1024)
  float z[PER];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int bb = t + 256 * i;
    z[i] = -INFINITY;
    if (bb < Ck && start_k[sk + bb + 1] > start_k[sk + bb]) {
      const float* mk = mu_k + ((int64_t)bh * Ck + bb) * D;
      float dot = 0.f;
      for (int e = 0; e < D; ++e) dot = __builtin_fmaf(mq[e], mk[e], dot);
      z[i] = g.scale * dot;
      m = fmaxf(m, z[i]);
    }
  }
  // block max (fixed tree)
  red[t] = m;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (t < w) red[t] = fmaxf(red[t], red[t + w]);
    __syncthreads();
  }
  m = red[0];
  __syncthreads();
  float e[PER], es = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int bb = t + 256 * i;
    e[i] = 0.f;
    if (bb < Ck && z[i] != -INFINITY) e[i] = (float)(start_k[sk + bb + 1] - start_k[sk + bb]) * expf(z[i] - m);
    es += e[i];
  }
  const float S = block_sum_fixed(es, red);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int bb = t + 256 * i;
    if (bb < Ck) P[bb] = e[i] / S;
  }
  __syncthreads();
  // rank in descending P, ties to the lower index; P in rank order
  int rk[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int bb = t + 256 * i;
    rk[i] = 0;
    if (bb < Ck) {
      const float pb = P[bb];
      int r = 0;
      for (int o = 0; o < Ck; ++o) r += (P[o] > pb) || (P[o] == pb && o < bb);
      rk[i] = r;
      srt[r] = pb;
    }
  }
  __syncthreads();
  // exclusive running sum in rank order, fixed order per element (serial
  // within blocks of 4 ranks, Hillis-Steele across the 256 blocks)
  float loc[PER], run = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int r = 4 * t + i;
    loc[i] = run;
    run += r < Ck ? srt[r] : 0.f;
  }
  red[t] = run;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const float v = t >= o ? red[t - o] : 0.f;
    __syncthreads();
    red[t] += v;
    __syncthreads();
  }
  const float off = red[t] - run;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int r = 4 * t + i;
    if (r < Ck) srt[r] = off + loc[i];  // mass of the clusters ranked before r
  }
  __syncthreads();
  // selection and tile counts, then tile offsets in ascending cluster order
  int nt[PER], tot = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int bb = t + 256 * i;
    nt[i] = 0;
    if (bb < Ck) {
      const int n = start_k[sk + bb + 1] - start_k[sk + bb];
      const bool s = n > 0 && srt[rk[i]] < p;
      sel[((int64_t)bh * Cq + a) * Ck + bb] = s ? 1 : 0;
      nt[i] = s ? (n + kBN - 1) / kBN : 0;
    }
  }
  // tile offsets: cluster bb = t + 256 i; scan over the order (i, t)
#pragma unroll
  for (int i = 0; i < PER; ++i) tsc[t + 256 * i] = nt[i];
  __syncthreads();
  if (t == 0) {
    int acc = 0;
    for (int bb = 0; bb < Ck; ++bb) {
      const int v = tsc[bb];
      tsc[bb] = acc;
      acc += v;
    }
    ntiles[(int64_t)bh * Cq + a] = acc;
  }
  __syncthreads();
  int2* tl = tiles + ((int64_t)bh * Cq + a) * maxT;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int bb = t + 256 * i;
    if (bb < Ck && nt[i] > 0) {
      const int s0 = start_k[sk + bb], s1 = start_k[sk + bb + 1];
      for (int j = 0; j < nt[i]; ++j) tl[tsc[bb] + j] = make_int2(s0 + j * kBN, min(s1, s0 + (j + 1) * kBN));
    }
  }
  (void)tot;
}

// grid (BH): rb_prefix[bh*(Cq+1) + a] = row blocks of 256 before query cluster a.
__global__ void k_svg2_rows(int32_t Cq, const int32_t* __restrict__ start_q, int32_t* __restrict__ rb_prefix) {
  const int bh = blockIdx.x;
  if (threadIdx.x != 0) return;
  int acc = 0;
  for (int a = 0; a < Cq; ++a) {
    rb_prefix[(int64_t)bh * (Cq + 1) + a] = acc;
    const int n = start_q[(int64_t)bh * (Cq + 1) + a + 1] - start_q[(int64_t)bh * (Cq + 1) + a];
    acc += (n + 255) / 256;
  }
  rb_prefix[(int64_t)bh * (Cq + 1) + Cq] = acc;
}

// grid (ceil(L / RPB), BH): dst[bh][i] = src[b, h][perm[bh*L + i]] (rows of D bf16).
template <int D>
__global__ __launch_bounds__(256) void k_gather_rows(KGeom g, const __bf16* __restrict__ src, svg_strides s,
                                                     const int32_t* __restrict__ perm, __bf16* __restrict__ dst) {
  constexpr int CPR = D / 8, RPB = 256 / CPR;
  const int bh = blockIdx.y, t = threadIdx.x;
  const int i = blockIdx.x * RPB + t / CPR, c = t % CPR;
  if (i >= g.L) return;
  const int b = bh / g.H, h = bh % g.H;
  const int xs = perm[(int64_t)bh * g.L + i];
  *reinterpret_cast<int4*>(dst + ((int64_t)bh * g.L + i) * D + c * 8) =
      *reinterpret_cast<const int4*>(src + (int64_t)b * s.b + (int64_t)h * s.h + (int64_t)xs * s.x + c * 8);
}

struct Svg2Ptrs {
  const void *q, *kp, *vp;  // q: caller layout; kp, vp: cluster order [BH][L][D]
  svg_strides s, so;
  void* o;
  const int32_t *perm_q, *start_q, *rb_prefix, *ntiles;
  const int2* tiles;
  int32_t Cq, maxT, max_rb;
};

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(512, 1) void k_svg2_attn(KGeom g, Svg2Ptrs a) {
  constexpr int WAVES = 8;
  using TC = TileCfg<D, WAVES>;
  extern __shared__ __attribute__((aligned(16))) __bf16 lds_raw[];
  auto lds = reinterpret_cast<__bf16 (*)[2][TC::TILE_ELEMS]>(lds_raw);
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bh = blockIdx.x / a.max_rb, j = blockIdx.x % a.max_rb;
  const int32_t* rbp = a.rb_prefix + (int64_t)bh * (a.Cq + 1);
  if (j >= rbp[a.Cq]) return;
  int lo_c = 0, hi_c = a.Cq;  // last cluster with rbp[c] <= j
  while (hi_c - lo_c > 1) {
    const int mid = (lo_c + hi_c) >> 1;
    if (rbp[mid] <= j) lo_c = mid; else hi_c = mid;
  }
  const int cq = lo_c, rb = j - rbp[cq];
  const int32_t* stq = a.start_q + (int64_t)bh * (a.Cq + 1);
  const int p0 = stq[cq] + rb * 256, p1 = stq[cq + 1];
  const int b = bh / g.H, h = bh % g.H;

  KVLoader<D, false, WAVES> ld;
  const __bf16* kp = static_cast<const __bf16*>(a.kp) + (int64_t)bh * g.L * D;
  const __bf16* vp = static_cast<const __bf16*>(a.vp) + (int64_t)bh * g.L * D;
  ld.init(kp, vp, D, g.L, wave, lane);
  const int nt = a.ntiles[(int64_t)bh * a.Cq + cq];
  const int2* tl = a.tiles + ((int64_t)bh * a.Cq + cq) * a.maxT;
  if (nt > 0) ld.load(g, tl[0].x, lds[0][0], lds[0][1], wave, lane);

  const int pos = p0 + wave * 32 + (lane & 31);
  const bool valid = pos < p1;
  const int tok = a.perm_q[(int64_t)bh * g.L + (valid ? pos : p1 - 1)];
  bf16x8 qf[D / 16];
  load_q<D>(qf, static_cast<const __bf16*>(a.q) + (int64_t)b * a.s.b + (int64_t)h * a.s.h + (int64_t)tok * a.s.x, hh);
  const bool wave_rows = wave_max_i(valid ? 1 : 0) != 0;
  Flash<D> st;
  st.init();
  wait_vm_all();
  __syncthreads();
  auto step = [&](int t, auto stc) {
    constexpr int sg = decltype(stc)::value;
    if (t + 1 < nt) ld.load(g, tl[t + 1].x, lds[sg ^ 1][0], lds[sg ^ 1][1], wave, lane);
    if (wave_rows) {
      const int2 rg = tl[t];
      const int cnt = rg.y - rg.x;
      f32x16 s0, s1;
      score_tile<D>(lds[sg][0], qf, lane, s0, s1);
      if (cnt < kBN) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s0[r] = acc_key(0, r, hh) < cnt ? s0[r] : -INFINITY;
          s1[r] = acc_key(1, r, hh) < cnt ? s1[r] : -INFINITY;
        }
      }
      st.add_tile(s0, s1, lds[sg][1], lane, g.scale_log2);
    }
    wait_vm_all();
    __syncthreads();
  };
  for (int t = 0; t < nt; t += 2) {
    step(t, std::integral_constant<int, 0>{});
    if (t + 1 < nt) step(t + 1, std::integral_constant<int, 1>{});
  }
  const float l_tot = half_sum(st.l_part);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (valid) {
    constexpr int OE = OUT_BF16 ? 2 : 4;
    char* orow = static_cast<char*>(a.o) + ((int64_t)b * a.so.b + (int64_t)h * a.so.h + (int64_t)tok * a.so.x) * OE;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = db * 32 + 8 * g4 + 4 * hh;
        f32x4 v4 = {st.o[db][4 * g4] * inv, st.o[db][4 * g4 + 1] * inv, st.o[db][4 * g4 + 2] * inv,
                    st.o[db][4 * g4 + 3] * inv};
        if (OUT_BF16)
          *reinterpret_cast<bf16x4*>(orow + d0 * 2) = __builtin_convertvector(v4, bf16x4);
        else
          *reinterpret_cast<f32x4*>(orow + d0 * 4) = v4;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers

hipError_t launch_kmeans(const KGeom& g, const void* x, svg_strides s, int32_t C, int32_t iters, float* mu,
                         int32_t* labels, int32_t* perm, int32_t* start, const Svg2Scratch& w, hipStream_t st) {
  const unsigned BH = (unsigned)(g.B * g.H);
  const int32_t nBlk = (g.L + kKmRows - 1) / kKmRows;
  const __bf16* bx = static_cast<const __bf16*>(x);
  __bf16* hi = static_cast<__bf16*>(w.hi);
  __bf16* lo = static_cast<__bf16*>(w.lo);
  for (int it = 0; it < iters; ++it) {
    hipLaunchKernelGGL(k_km_split, dim3((unsigned)C, BH), dim3((unsigned)g.d), 0, st, C, g.d, mu, hi, lo, w.hn);
    if (g.d == 64)
      hipLaunchKernelGGL(k_km_assign<64>, dim3((unsigned)nBlk, BH), dim3(512), 0, st, g, bx, s, C, hi, lo, w.hn,
                         labels);
    else
      hipLaunchKernelGGL(k_km_assign<128>, dim3((unsigned)nBlk, BH), dim3(512), 0, st, g, bx, s, C, hi, lo, w.hn,
                         labels);
    hipLaunchKernelGGL(k_km_hist, dim3((unsigned)nBlk, BH), dim3(256), 0, st, g.L, C, nBlk, labels, w.hist, w.rank);
    hipLaunchKernelGGL(k_km_scan, dim3(BH), dim3(1024), 0, st, g.L, C, nBlk, w.hist, w.base, start);
    hipLaunchKernelGGL(k_km_scatter, dim3((unsigned)nBlk, BH), dim3(256), 0, st, g.L, C, nBlk, labels, w.rank, w.base,
                       perm);
    hipLaunchKernelGGL(k_km_update, dim3((unsigned)C, BH), dim3((unsigned)g.d), 0, st, g, bx, s, C, perm, start, mu);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_km_init(const KGeom& g, const void* x, svg_strides s, int32_t C, float* mu, hipStream_t st) {
  hipLaunchKernelGGL(k_km_init, dim3((unsigned)C, (unsigned)(g.B * g.H)), dim3((unsigned)g.d), 0, st, g,
                     static_cast<const __bf16*>(x), s, C, mu);
  return hipGetLastError();
}

hipError_t launch_svg2_select(const KGeom& g, int32_t Cq, int32_t Ck, float p, const float* mu_q, const float* mu_k,
                              const int32_t* start_q, const int32_t* start_k, uint8_t* sel, void* tiles,
                              int32_t* ntiles, int32_t maxT, int32_t* rb_prefix, hipStream_t st) {
  const unsigned BH = (unsigned)(g.B * g.H);
  hipLaunchKernelGGL(k_svg2_select, dim3((unsigned)Cq, BH), dim3(256), 0, st, g, Cq, Ck, p, mu_q, mu_k, start_k, sel,
                     static_cast<int2*>(tiles), ntiles, maxT);
  hipLaunchKernelGGL(k_svg2_rows, dim3(BH), dim3(64), 0, st, Cq, start_q, rb_prefix);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const KGeom& g, const void* src, svg_strides s, const int32_t* perm, void* dst,
                              hipStream_t st) {
  const unsigned BH = (unsigned)(g.B * g.H);
  const int rpb = 256 / (g.d / 8);
  dim3 grid((unsigned)((g.L + rpb - 1) / rpb), BH);
  const __bf16* bs = static_cast<const __bf16*>(src);
  __bf16* bd = static_cast<__bf16*>(dst);
  if (g.d == 64)
    hipLaunchKernelGGL(k_gather_rows<64>, grid, dim3(256), 0, st, g, bs, s, perm, bd);
  else
    hipLaunchKernelGGL(k_gather_rows<128>, grid, dim3(256), 0, st, g, bs, s, perm, bd);
  return hipGetLastError();
}

template <int D, bool OUT_BF16>
static hipError_t launch_svg2_attn_t(const KGeom& g, const Svg2Ptrs& a, hipStream_t st) {
  const size_t lds = (size_t)2 * 2 * TileCfg<D>::TILE_ELEMS * sizeof(__bf16);
  auto kern = k_svg2_attn<D, OUT_BF16>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t grid = (int64_t)g.B * g.H * a.max_rb;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(512), lds, st, g, a);
  return hipGetLastError();
}

hipError_t launch_svg2_attention(const KGeom& g, const void* q, svg_strides s, const void* kp, const void* vp, void* o,
                                 svg_strides so, bool out_bf16, const int32_t* perm_q, const int32_t* start_q,
                                 const int32_t* rb_prefix, const void* tiles, const int32_t* ntiles, int32_t Cq,
                                 int32_t maxT, hipStream_t st) {
  Svg2Ptrs a;
  a.q = q;
  a.kp = kp;
  a.vp = vp;
  a.s = s;
  a.so = so;
  a.o = o;
  a.perm_q = perm_q;
  a.start_q = start_q;
  a.rb_prefix = rb_prefix;
  a.ntiles = ntiles;
  a.tiles = static_cast<const int2*>(tiles);
  a.Cq = Cq;
  a.maxT = maxT;
  a.max_rb = (g.L + 255) / 256 + Cq;
  if (g.d == 64) return out_bf16 ? launch_svg2_attn_t<64, true>(g, a, st) : launch_svg2_attn_t<64, false>(g, a, st);
  return out_bf16 ? launch_svg2_attn_t<128, true>(g, a, st) : launch_svg2_attn_t<128, false>(g, a, st);
}

}  // namespace svg
