// svg_layout_permute: frame-major <-> token-major row transposition.
//
// The abstract of "Sparse VideoGen" introduces a hardware-efficient layout
// transformation; with x = i*F + j (rebuttal, Weakness 1) the token-major
// position of (i, j) is j*N + i, so the temporal slashes become a band.
// The transform is a transpose of an N x F matrix whose elements are whole
// rows of d values.  A workgroup stages an 8 x 8 block of rows in LDS: it
// reads eight runs of eight consecutive source rows and writes eight runs of
// eight consecutive destination rows, so both sides move contiguous
// 8-row segments (1-4 KB) instead of single rows.  Text rows are copied
// through unchanged by extra workgroups.
#include "svg_device.h"

namespace svg {

constexpr int kTI = 8, kTJ = 8;  // frames x positions per workgroup
constexpr int kPermThreads = 256;
typedef int i32x4n __attribute__((ext_vector_type(4)));

// One workgroup moves up to 64 rows of RB bytes (RB = d * element size).
template <int RB>
__global__ __launch_bounds__(kPermThreads) void k_permute(KGeom g, const char* __restrict__ src, svg_strides ss,
                                                 char* __restrict__ dst, svg_strides ds, int elt,
                                                 const int32_t* __restrict__ modes, int inverse,
                                                 int nbi, int nbj, int ntext) {
  constexpr int CPR = RB / 16;  // 16-byte chunks per row
  __shared__ __attribute__((aligned(16))) i32x4n stage[kTI * kTJ * CPR];
  const int bh = blockIdx.y;
  if (modes && modes[bh] != SVG_TEMPORAL) return;
  const int b = bh / g.H, h = bh % g.H;
  const char* sbase = src + ((int64_t)b * ss.b + (int64_t)h * ss.h) * elt;
  char* dbase = dst + ((int64_t)b * ds.b + (int64_t)h * ds.h) * elt;
  const int64_t srow = ss.x * elt, drow = ds.x * elt;
  const int t = threadIdx.x;
  int blk = blockIdx.x;
  if (blk < ntext) {  // text rows: plain copy of up to 64 rows
    const int r0 = blk * 64;
    for (int c = t; c < 64 * CPR; c += kPermThreads) {
      const int r = r0 + c / CPR;
      if (r < g.T) {
        const int4 val = *reinterpret_cast<const int4*>(sbase + r * srow + (c % CPR) * 16);
        *reinterpret_cast<int4*>(dbase + r * drow + (c % CPR) * 16) = val;
      }
    }
    return;
  }
  blk -= ntext;
  // consecutive workgroups take consecutive frame blocks of one position
  // block, so those writing one token-major region (every frame of eight
  // positions) run together (+11 % forward against position blocks first)
  const int i0 = (blk % nbi) * kTI, j0 = (blk / nbi) * kTJ;
  // forward: read runs along j (frame-major rows i*F + j), write runs along i
  // inverse: read runs along i (token-major rows j*N + i), write runs along j
  // (the source is read once: non-temporal loads, +5 % on the forward pass)
  for (int c = t; c < kTI * kTJ * CPR; c += kPermThreads) {
    const int rr = c / CPR, ch = c % CPR;
    int a, bb;  // a: frame offset, bb: position offset
    if (!inverse) {
      a = rr / kTJ;
      bb = rr % kTJ;
    } else {
      bb = rr / kTI;
      a = rr % kTI;
    }
    const int i = i0 + a, j = j0 + bb;
    if (i < g.N && j < g.F) {
      const int64_t row = inverse ? (int64_t)g.T + (int64_t)j * g.N + i : (int64_t)g.T + (int64_t)i * g.F + j;
      stage[(a * kTJ + bb) * CPR + ch] =
          __builtin_nontemporal_load(reinterpret_cast<const i32x4n*>(sbase + row * srow + ch * 16));
    }
  }
  __syncthreads();
  for (int c = t; c < kTI * kTJ * CPR; c += kPermThreads) {
    const int rr = c / CPR, ch = c % CPR;
    int a, bb;
    if (!inverse) {
      bb = rr / kTI;
      a = rr % kTI;
    } else {
      a = rr / kTJ;
      bb = rr % kTJ;
    }
    const int i = i0 + a, j = j0 + bb;
    if (i < g.N && j < g.F) {
      const int64_t row = inverse ? (int64_t)g.T + (int64_t)i * g.F + j : (int64_t)g.T + (int64_t)j * g.N + i;
      *reinterpret_cast<i32x4n*>(dbase + row * drow + ch * 16) = stage[(a * kTJ + bb) * CPR + ch];
    }
  }
}

hipError_t launch_permute(const KGeom& g, int elt, const void* src, svg_strides ss, void* dst,
                          svg_strides ds, const int32_t* modes, int inverse, hipStream_t st) {
  const int nbi = (g.N + kTI - 1) / kTI, nbj = (g.F + kTJ - 1) / kTJ;
  const int ntext = (g.T + 63) / 64;
  dim3 grid((unsigned)(ntext + nbi * nbj), (unsigned)(g.B * g.H));
  const int rb = g.d * elt;
  const char* s = static_cast<const char*>(src);
  char* d = static_cast<char*>(dst);
  switch (rb) {
    case 128:
      hipLaunchKernelGGL(k_permute<128>, grid, dim3(kPermThreads), 0, st, g, s, ss, d, ds, elt, modes, inverse, nbi,
                         nbj, ntext);
      break;
    case 256:
      hipLaunchKernelGGL(k_permute<256>, grid, dim3(kPermThreads), 0, st, g, s, ss, d, ds, elt, modes, inverse, nbi,
                         nbj, ntext);
      break;
    case 512:
      hipLaunchKernelGGL(k_permute<512>, grid, dim3(kPermThreads), 0, st, g, s, ss, d, ds, elt, modes, inverse, nbi,
                         nbj, ntext);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace svg
