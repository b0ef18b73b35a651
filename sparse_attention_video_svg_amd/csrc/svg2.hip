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
//    -> k_km_update (mean of each cluster's tokens, fixed-order partial sums:
//    deterministic).  The last iteration's sort is the permutation.
//  * k_svg2_select: per query cluster, fp32 centroid scores against every key
//    cluster, the size-weighted softmax, ranks by comparison, the running sum
//    in rank order, the top-p prefix, and the segment table of the selected
//    key clusters (first key in the cluster order, offset in the concatenation
//    of the selected clusters' keys).  k_svg2_order: per head, the query
//    clusters in descending work with their row-block prefix sums.
//  * k_gather_rows: K and V copied into cluster order once.
//  * k_svg2_attn: one workgroup per (query cluster, block of 256 of its
//    rows): query rows gathered through the permutation, the selected keys
//    streamed as full 64-key tiles through the segment table (only the last
//    tile masked), scores, softmax and P.V as in the banded kernel, rows
//    scattered back.
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

// grid (ceil(L/256), BH), 8 waves x 32 tokens.  labels[bh*L + x].  The
// scores x . hi and x . lo accumulate into one register pair that starts at
// -|mu|^2 / 2 of its centroids (the half squared norms sit in LDS, read four
// at a time); each lane visits its centroids in increasing index order, so
// a strict > keeps the lowest index among equal scores; two workgroups
// share a CU, so one's loads overlap the other's matrix work.
template <int D>
__global__ __launch_bounds__(512, 4) void k_km_assign(KGeom g, const __bf16* __restrict__ x, svg_strides s,
                                                      int32_t C, const __bf16* __restrict__ hi,
                                                      const __bf16* __restrict__ lo, const float* __restrict__ hn,
                                                      int32_t* __restrict__ labels) {
  using TC = TileCfg<D, 8>;
  __shared__ __attribute__((aligned(16))) __bf16 lds[2][2][TC::TILE_ELEMS];  // [stage][hi, lo]
  __shared__ __attribute__((aligned(16))) float hns[kSvg2MaxClusters];
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
  for (int c = tid; c < C; c += 512) hns[c] = hn[cb + c];

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
    f32x16 a0, a1;
    // accumulator r of block kb2 holds centroid ct*64 + acc_key(kb2, r, hh):
    // four consecutive centroids per group of four registers (entries past
    // C are never selected)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const f32x4 n0 = *reinterpret_cast<const f32x4*>(&hns[ct * kBN + 8 * g4 + 4 * hh]);
      const f32x4 n1 = *reinterpret_cast<const f32x4*>(&hns[ct * kBN + 32 + 8 * g4 + 4 * hh]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a0[4 * g4 + j] = -n0[j];
        a1[4 * g4 + j] = -n1[j];
      }
    }
    // (one step ahead: the kernel is held to 128 registers for two
    // workgroups per CU)
    score_tile<D, true, 1>(lds[sg][0], qf, lane, a0, a1);
    score_tile<D, true, 1>(lds[sg][1], qf, lane, a0, a1);
    const bool full = (ct + 1) * kBN <= C;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = ct * kBN + acc_key(kb2, r, hh);
        const float v = kb2 ? a1[r] : a0[r];
        if ((full || c < C) && v > best) {
          best = v;
          bidx = c;
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
// base position of every (block, cluster) in the cluster order.  Thread
// (part, c) walks part of the histogram blocks of cluster c (P = 1024 / C
// parts of consecutive blocks).
__global__ __launch_bounds__(1024) void k_km_scan(int32_t L, int32_t C, int32_t nBlk, const int32_t* __restrict__ hist,
                                                  int32_t* __restrict__ base, int32_t* __restrict__ start) {
  __shared__ int sc[1024], pt[1024];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int P = 1024 / C;
  const int c = tid % C, part = tid / C;
  const bool act = part < P;
  const int b0 = act ? (int)((int64_t)part * nBlk / P) : 0, b1 = act ? (int)((int64_t)(part + 1) * nBlk / P) : 0;
  const int64_t hb = (int64_t)bh * nBlk * C;
  int tot = 0;
#pragma unroll 8
  for (int blk = b0; blk < b1; ++blk) tot += hist[hb + (int64_t)blk * C + c];
  pt[tid] = tot;  // part totals, [part][c]
  __syncthreads();
  int ctot = 0;
  if (tid < C)
    for (int q = 0; q < P; ++q) ctot += pt[q * C + tid];
  sc[tid] = tid < C ? ctot : 0;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {  // inclusive Hillis-Steele scan
    const int v = tid >= o ? sc[tid - o] : 0;
    __syncthreads();
    sc[tid] += v;
    __syncthreads();
  }
  if (tid < C) start[(int64_t)bh * (C + 1) + tid] = sc[tid] - ctot;
  if (tid == 0) start[(int64_t)bh * (C + 1) + C] = L;
  if (act) {
    int run = (c > 0 ? sc[c - 1] : 0);
    for (int q = 0; q < part; ++q) run += pt[q * C + c];
#pragma unroll 8
    for (int blk = b0; blk < b1; ++blk) {
      const int64_t o = hb + (int64_t)blk * C + c;
      const int hcount = hist[o];
      base[o] = run;
      run += hcount;
    }
  }
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

// grid (C, BH), 256 threads: mu = mean of the cluster's tokens (an empty
// cluster keeps its centroid).  Wave w takes the 64-position chunks w, w+4,
// ... of the cluster: one coalesced load of the chunk's token ids, then row
// gathers 8 at a time (each lane two dims of one row; D = 64: two rows per
// step), into 8 partial sums.  The partials combine in a fixed order: the
// result does not depend on scheduling.
template <int D>
__global__ __launch_bounds__(256) void k_km_update(KGeom g, const __bf16* __restrict__ x, svg_strides s, int32_t C,
                                                   const int32_t* __restrict__ perm,
                                                   const int32_t* __restrict__ start, float* __restrict__ mu) {
  constexpr int HALF = D / 2;      // lanes per token row (two dims each)
  constexpr int TPW = 64 / HALF;   // token rows per wave and step
  constexpr int U = 8;
  __shared__ float2 part[4][64];
  const int c = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int dp = lane % HALF, ts = lane / HALF;
  const int b = bh / g.H, h = bh % g.H;
  const __bf16* xb = x + (int64_t)b * s.b + (int64_t)h * s.h + 2 * dp;
  const int32_t* pp = perm + (int64_t)bh * g.L;
  const int64_t sb = (int64_t)bh * (C + 1);
  const int i0 = start[sb + c], i1 = start[sb + c + 1];
  if (i1 <= i0) return;
  float2 acc[U];
#pragma unroll
  for (int u = 0; u < U; ++u) acc[u] = make_float2(0.f, 0.f);
  for (int chunk = i0 + w * 64; chunk < i1; chunk += 4 * 64) {
    const int n = min(64, i1 - chunk);
    const int ids = pp[chunk + min(lane, n - 1)];
    for (int k = 0; k < n; k += U * TPW) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int e = k + u * TPW + ts;
        const int tk = __shfl(ids, min(e, n - 1));
        const bf16x2 v = *reinterpret_cast<const bf16x2*>(xb + (int64_t)tk * s.x);
        acc[u].x += e < n ? (float)v[0] : 0.f;
        acc[u].y += e < n ? (float)v[1] : 0.f;
      }
    }
  }
  float2 t;
  t.x = ((acc[0].x + acc[1].x) + (acc[2].x + acc[3].x)) + ((acc[4].x + acc[5].x) + (acc[6].x + acc[7].x));
  t.y = ((acc[0].y + acc[1].y) + (acc[2].y + acc[3].y)) + ((acc[4].y + acc[5].y) + (acc[6].y + acc[7].y));
  if (TPW == 2) {  // the two token rows of a wave step; a + b == b + a, so both halves agree
    t.x += __shfl_xor(t.x, 32);
    t.y += __shfl_xor(t.y, 32);
  }
  part[w][lane] = t;
  __syncthreads();
  if (w == 0 && lane < HALF) {
    const float2 r0 = part[0][lane], r1 = part[1][lane], r2 = part[2][lane], r3 = part[3][lane];
    const float n = (float)(i1 - i0);
    float* m = mu + ((int64_t)bh * C + c) * D + 2 * lane;
    m[0] = ((r0.x + r1.x) + (r2.x + r3.x)) / n;
    m[1] = ((r0.y + r1.y) + (r2.y + r3.y)) / n;
  }
}

// grid (Cq, BH), 256 threads.  sel[(bh*Cq + a)*Ck + b]; the selected key
// clusters of a as segments of the cluster order, ascending b:
// segs[(bh*Cq + a)*Ck + i] = (first key position of the i-th selected
// cluster, its offset in the concatenation of the selected clusters' keys);
// nseg / nkeys[bh*Cq + a]: segments and keys in total.
__global__ __launch_bounds__(256) void k_svg2_select(KGeom g, int32_t Cq, int32_t Ck, float p,
                                                     const float* __restrict__ mu_q, const float* __restrict__ mu_k,
                                                     const int32_t* __restrict__ start_k, uint8_t* __restrict__ sel,
                                                     int2* __restrict__ segs, int32_t* __restrict__ nseg,
                                                     int32_t* __restrict__ nkeys) {
  __shared__ float P[1024], srt[1024], red[256], zs[1024];
  __shared__ int tsc[1024], vst[1024];
  const int a = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const int lane = t & 63, wv = t >> 6;
  const int D = g.d;
  const float* mq = mu_q + ((int64_t)bh * Cq + a) * D;
  const int64_t sk = (int64_t)bh * (Ck + 1);
  constexpr int PER = 4;  // clusters per thread (Ck <= 1024)
  // centroid dot products: wave wv takes key clusters wv, wv + 4, ...; the
  // lanes split the dims (lane, lane + 64), a fixed butterfly sums them
  {
    const float q0 = mq[lane], q1 = D > 64 ? mq[lane + 64] : 0.f;
    for (int bb = wv; bb < Ck; bb += 4) {
      const float* mk = mu_k + ((int64_t)bh * Ck + bb) * D;
      float dot = q0 * mk[lane];
      if (D > 64) dot = __builtin_fmaf(q1, mk[lane + 64], dot);
      dot = wave_sum(dot);
      if (lane == 0) zs[bb] = dot;
    }
  }
  __syncthreads();
  float z[PER];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int bb = t + 256 * i;
    z[i] = -INFINITY;
    if (bb < Ck && start_k[sk + bb + 1] > start_k[sk + bb]) {
      z[i] = g.scale * zs[bb];
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
  // selection, then each selected cluster's segment index and key offset in
  // ascending cluster order
  int nsel[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int bb = t + 256 * i;
    nsel[i] = 0;
    if (bb < Ck) {
      const int n = start_k[sk + bb + 1] - start_k[sk + bb];
      const bool s = n > 0 && srt[rk[i]] < p;
      sel[((int64_t)bh * Cq + a) * Ck + bb] = s ? 1 : 0;
      nsel[i] = s ? n : 0;
    }
    tsc[bb] = nsel[i];
  }
  __syncthreads();
  if (t == 0) {
    int ns = 0, nk = 0;
    for (int bb = 0; bb < Ck; ++bb) {
      const int n = tsc[bb];
      tsc[bb] = ns;
      vst[bb] = nk;
      ns += n > 0;
      nk += n;
    }
    nseg[(int64_t)bh * Cq + a] = ns;
    nkeys[(int64_t)bh * Cq + a] = nk;
  }
  __syncthreads();
  int2* sg = segs + ((int64_t)bh * Cq + a) * Ck;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int bb = t + 256 * i;
    if (bb < Ck && nsel[i] > 0) sg[tsc[bb]] = make_int2(start_k[sk + bb], vst[bb]);
  }
}

// grid (BH), 1024 threads: the query clusters of a head in descending work
// (key tiles of their selection; ties to the lower index; clusters without
// rows last): ord[bh*Cq + r] = cluster of rank r, rb_prefix[bh*(Cq+1) + r] =
// row blocks of 256 before rank r (rb_prefix[Cq] = all of the head's).
__global__ __launch_bounds__(1024) void k_svg2_order(int32_t Cq, const int32_t* __restrict__ start_q,
                                                     const int32_t* __restrict__ nkeys, int32_t* __restrict__ ord,
                                                     int32_t* __restrict__ rb_prefix) {
  __shared__ int work[1024], sc[1024];
  const int bh = blockIdx.x, a = threadIdx.x;
  const int64_t sq = (int64_t)bh * (Cq + 1);
  int nrb = 0, wk = -1;
  if (a < Cq) {
    const int n = start_q[sq + a + 1] - start_q[sq + a];
    nrb = (n + 255) / 256;
    wk = n > 0 ? (nkeys[(int64_t)bh * Cq + a] + kBN - 1) / kBN : -1;
  }
  work[a] = wk;
  __syncthreads();
  int r = 0;
  if (a < Cq)
    for (int o = 0; o < Cq; ++o) r += (work[o] > wk) || (work[o] == wk && o < a);
  __syncthreads();
  sc[a] = 0;
  __syncthreads();
  if (a < Cq) {
    ord[(int64_t)bh * Cq + r] = a;
    sc[r] = nrb;
  }
  __syncthreads();
  const int own = sc[a];
  for (int o = 1; o < 1024; o <<= 1) {  // inclusive Hillis-Steele scan over ranks
    const int v = a >= o ? sc[a - o] : 0;
    __syncthreads();
    sc[a] += v;
    __syncthreads();
  }
  if (a < Cq) rb_prefix[sq + a] = sc[a] - own;
  if (a == Cq - 1) rb_prefix[sq + Cq] = sc[a];
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
  const int32_t *perm_q, *start_q, *ord, *rb_prefix, *nseg, *nkeys;
  const int2* segs;
  int32_t Cq, Ck, max_rb, total;
};

// Direct-to-LDS loads of the key tiles of one query cluster: tile t holds
// positions 64t .. 64t+63 of the concatenation of the selected key clusters'
// keys (segments of the cluster-ordered K and V), so only the last tile is
// ragged (its rows clamp to the last key).  The LDS chunk layout and
// swizzles are those of the contiguous loader; each lane's row comes from
// the segment table through a cursor that only moves forward.  The cursor's
// segment (row = base + position) and the position where the next segment
// starts stay in registers, so a tile that crosses no segment boundary
// reads nothing from the table.
template <int D>
struct SegLoader {
  using C = TileCfg<D, 8>;
  const char* kb;
  const char* vb;
  uint32_t colk[C::LOADS], colv[C::LOADS];
  int rr[C::LOADS], cur[C::LOADS], base[C::LOADS], next_y[C::LOADS];

  __device__ __forceinline__ void init(const __bf16* K, const __bf16* V, int wave, int lane) {
    kb = reinterpret_cast<const char*>(K);
    vb = reinterpret_cast<const char*>(V);
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int p = min(i * 8 + wave, C::SEGS - 1) * 64 + lane;
      const int r = p / C::CR, pos = p % C::CR;
      rr[i] = r;
      cur[i] = -1;  // the first load reads the table
      base[i] = 0;
      next_y[i] = INT_MIN;
      colk[i] = (uint32_t)((pos ^ C::swz_k(r)) * 16);
      colv[i] = (uint32_t)((pos ^ C::swz_v(r)) * 16);
    }
  }

  // Every lookup in the LDS segment table comes before the first load is
  // issued: an LDS read behind a direct-to-LDS load in flight would wait for
  // that load to land (the compiler cannot tell the two apart).
  __device__ __forceinline__ void load(int t, const int2* sg, int ns, int nk, __bf16* lds_k, __bf16* lds_v,
                                       int wave) {
    int64_t row[C::LOADS];
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int vpos = min(t * kBN + rr[i], nk - 1);
      if (vpos >= next_y[i]) {  // into a later segment (or the first load)
        int c = max(cur[i], 0);
        while (c + 1 < ns && sg[c + 1].y <= vpos) ++c;
        cur[i] = c;
        const int2 e = sg[c];
        base[i] = e.x - e.y;
        next_y[i] = c + 1 < ns ? sg[c + 1].y : INT_MAX;
      }
      row[i] = (int64_t)(base[i] + vpos) * (D * 2);
    }
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int seg = i * 8 + wave;
      if (C::SEGS % 8 != 0 && seg >= C::SEGS) break;  // wave-uniform
      __builtin_amdgcn_global_load_lds((const void*)(kb + row[i] + colk[i]), (SVG_LDS void*)(lds_k + seg * 512), 16,
                                       0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(vb + row[i] + colv[i]), (SVG_LDS void*)(lds_v + seg * 512), 16,
                                       0, 0);
    }
  }
};

// One workgroup per (head, row block of 256 of a query cluster), the
// clusters of a head in descending work, XCD-aware: consecutive logical ids
// run on one XCD, so the row blocks of a cluster share its key tiles in L2.
template <int D, bool OUT_BF16>
__global__ __launch_bounds__(512, 1) void k_svg2_attn(KGeom g, Svg2Ptrs a) {
  constexpr int WAVES = 8;
  using TC = TileCfg<D, WAVES>;
  extern __shared__ __attribute__((aligned(16))) __bf16 lds_raw[];
  auto lds = reinterpret_cast<__bf16 (*)[2][TC::TILE_ELEMS]>(lds_raw);
  int2* sg = reinterpret_cast<int2*>(lds_raw + 2 * 2 * TC::TILE_ELEMS);  // [Ck] segment table
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int w = blockIdx.x;
  const int logical = xcd_logical(w, g.nxcd, kXcdRun);
  if (logical >= a.total) return;
  const int bh = logical / a.max_rb, j = logical % a.max_rb;
  const int32_t* rbp = a.rb_prefix + (int64_t)bh * (a.Cq + 1);
  if (j >= rbp[a.Cq]) return;
  int lo_r = 0, hi_r = a.Cq;  // last rank with rbp[r] <= j
  while (hi_r - lo_r > 1) {
    const int mid = (lo_r + hi_r) >> 1;
    if (rbp[mid] <= j) lo_r = mid; else hi_r = mid;
  }
  const int cq = a.ord[(int64_t)bh * a.Cq + lo_r], rb = j - rbp[lo_r];
  const int32_t* stq = a.start_q + (int64_t)bh * (a.Cq + 1);
  const int p0 = stq[cq] + rb * 256, p1 = stq[cq + 1];
  const int b = bh / g.H, h = bh % g.H;

  const int64_t ci = (int64_t)bh * a.Cq + cq;
  const int ns = a.nseg[ci], nk = a.nkeys[ci];
  const int2* gsg = a.segs + ci * a.Ck;
  for (int i = tid; i < ns; i += 64 * WAVES) sg[i] = gsg[i];
  __syncthreads();

  SegLoader<D> ld;
  const __bf16* kp = static_cast<const __bf16*>(a.kp) + (int64_t)bh * g.L * D;
  const __bf16* vp = static_cast<const __bf16*>(a.vp) + (int64_t)bh * g.L * D;
  ld.init(kp, vp, wave, lane);
  const int nt = (nk + kBN - 1) / kBN;
  if (nt > 0) ld.load(0, sg, ns, nk, lds[0][0], lds[0][1], wave);

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
    constexpr int sgi = decltype(stc)::value;
    if (t + 1 < nt) ld.load(t + 1, sg, ns, nk, lds[sgi ^ 1][0], lds[sgi ^ 1][1], wave);
    if (wave_rows) {
      const int cnt = nk - t * kBN;
      f32x16 s0, s1;
      score_tile<D>(lds[sgi][0], qf, lane, s0, s1);
      if (cnt < kBN) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s0[r] = acc_key(0, r, hh) < cnt ? s0[r] : -INFINITY;
          s1[r] = acc_key(1, r, hh) < cnt ? s1[r] : -INFINITY;
        }
      }
      st.add_tile(s0, s1, lds[sgi][1], lane, g.scale_log2);
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
    if (g.d == 64)
      hipLaunchKernelGGL(k_km_update<64>, dim3((unsigned)C, BH), dim3(256), 0, st, g, bx, s, C, perm, start, mu);
    else
      hipLaunchKernelGGL(k_km_update<128>, dim3((unsigned)C, BH), dim3(256), 0, st, g, bx, s, C, perm, start, mu);
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
                              const int32_t* start_q, const int32_t* start_k, uint8_t* sel, void* segs,
                              int32_t* nseg, int32_t* nkeys, int32_t* ord, int32_t* rb_prefix, hipStream_t st) {
  const unsigned BH = (unsigned)(g.B * g.H);
  hipLaunchKernelGGL(k_svg2_select, dim3((unsigned)Cq, BH), dim3(256), 0, st, g, Cq, Ck, p, mu_q, mu_k, start_k, sel,
                     static_cast<int2*>(segs), nseg, nkeys);
  hipLaunchKernelGGL(k_svg2_order, dim3(BH), dim3(1024), 0, st, Cq, start_q, nkeys, ord, rb_prefix);
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
static hipError_t launch_svg2_attn_t(const KGeom& g, const Svg2Ptrs& a, int64_t grid, hipStream_t st) {
  const size_t lds = (size_t)2 * 2 * TileCfg<D>::TILE_ELEMS * sizeof(__bf16) + (size_t)kSvg2MaxClusters * sizeof(int2);
  auto kern = k_svg2_attn<D, OUT_BF16>;
  static std::atomic<uint64_t> lds_set{0};
  if (hipError_t e = ensure_dynamic_lds((const void*)kern, lds, lds_set); e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(512), lds, st, g, a);
  return hipGetLastError();
}

hipError_t launch_svg2_attention(const KGeom& g, const void* q, svg_strides s, const void* kp, const void* vp, void* o,
                                 svg_strides so, bool out_bf16, const int32_t* perm_q, const int32_t* start_q,
                                 const int32_t* ord, const int32_t* rb_prefix, const void* segs, const int32_t* nseg,
                                 const int32_t* nkeys, int32_t Cq, int32_t Ck, hipStream_t st) {
  Svg2Ptrs a;
  a.q = q;
  a.kp = kp;
  a.vp = vp;
  a.s = s;
  a.so = so;
  a.o = o;
  a.perm_q = perm_q;
  a.start_q = start_q;
  a.ord = ord;
  a.rb_prefix = rb_prefix;
  a.nseg = nseg;
  a.nkeys = nkeys;
  a.segs = static_cast<const int2*>(segs);
  a.Cq = Cq;
  a.Ck = Ck;
  a.max_rb = (g.L + 255) / 256 + Cq;  // sum over clusters of ceil(n_a / 256) is below this
  const int64_t total = (int64_t)g.B * g.H * a.max_rb;
  const int64_t grid = xcd_grid(total, g.nxcd, kXcdRun);
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  a.total = (int32_t)total;
  if (g.d == 64)
    return out_bf16 ? launch_svg2_attn_t<64, true>(g, a, grid, st) : launch_svg2_attn_t<64, false>(g, a, grid, st);
  return out_bf16 ? launch_svg2_attn_t<128, true>(g, a, grid, st) : launch_svg2_attn_t<128, false>(g, a, grid, st);
}

}  // namespace svg
