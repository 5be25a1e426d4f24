// K1: block-mean pooling of Q (128-row query blocks) and K (64-row key
// blocks) -- the representatives the stage-one predictor scores (SpargeAttn
// abstract, first stage: predict the attention map quickly; iCATS abstract:
// prior work groups query and key tokens independently to estimate scores).
//
// HBM-bound: every element of Q and K is read exactly once with 16-byte
// coalesced loads (a row of D elements is CPR consecutive 16-byte chunks;
// consecutive lanes take consecutive chunks).  Each thread keeps fp32
// partial sums for its VEC columns; the RPP row-partials are combined
// through LDS in a fixed order, so results are deterministic.
#include "sa_device.h"
#include "sa_internal.h"
#include "../../include/sparse_attn.h"

namespace sa {
namespace {

template <typename T>
struct Elem;
template <>
struct Elem<__bf16> {
  static constexpr int VEC = 8;
  __device__ static void add(float* acc, const u32x4& w) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += bf16_lo(w[e]);
      acc[2 * e + 1] += bf16_hi(w[e]);
    }
  }
};
template <>
struct Elem<float> {
  static constexpr int VEC = 4;
  __device__ static void add(float* acc, const u32x4& w) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += __uint_as_float(w[e]);
  }
};

template <typename T, int D>
__global__ __launch_bounds__(256) void pool_kernel(const T* __restrict__ q,
                                                   const T* __restrict__ k,
                                                   float* __restrict__ qbar,
                                                   float* __restrict__ kbar,
                                                   Geometry g) {
  constexpr int VEC = Elem<T>::VEC;
  constexpr int CPR = D / VEC;      // 16-byte chunks per row
  constexpr int RPP = 256 / CPR;    // rows covered per pass
  constexpr int MAXIT = 128 / RPP;  // passes for a full query block
  __shared__ float red[RPP][D];

  const int tid = threadIdx.x;
  const int nq = g.B * g.H * g.nqb;
  int id = blockIdx.x;
  const T* src;
  float* dst;
  int bs, blk, bh;
  if (id < nq) {
    bh = id / g.nqb;
    blk = id - bh * g.nqb;
    src = q;
    dst = qbar + (size_t)id * D;
    bs = 128;
  } else {
    id -= nq;
    bh = id / g.nkb;
    blk = id - bh * g.nkb;
    src = k;
    dst = kbar + (size_t)id * D;
    bs = 64;
  }
  const int b = bh / g.H, h = bh - b * g.H;
  const T* base = src + (int64_t)b * g.sb + (int64_t)h * g.sh;
  const int r0 = blk * bs;
  const int r1 = min(g.N, r0 + bs);
  const int c = tid % CPR, ro = tid / CPR;

  u32x4 buf[MAXIT];
#pragma unroll
  for (int it = 0; it < MAXIT; ++it) {
    const int r = r0 + ro + it * RPP;
    if (r < r1)
      buf[it] = *reinterpret_cast<const u32x4*>(base + (int64_t)r * g.sn + c * VEC);
    else
      buf[it] = u32x4{0u, 0u, 0u, 0u};
  }
  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
#pragma unroll
  for (int it = 0; it < MAXIT; ++it) Elem<T>::add(acc, buf[it]);
#pragma unroll
  for (int e = 0; e < VEC; ++e) red[ro][c * VEC + e] = acc[e];
  __syncthreads();
  const float n = (float)(r1 - r0);
  for (int d = tid; d < D; d += 256) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < RPP; ++r) s += red[r][d];
    dst[d] = s / n;
  }
}

template <typename T, int D>
hipError_t launch_pool_t(const PredictLaunch& a, hipStream_t s) {
  const Geometry& g = a.g;
  const int64_t blocks = (int64_t)g.B * g.H * (g.nqb + g.nkb);
  hipLaunchKernelGGL((pool_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<const T*>(a.q), static_cast<const T*>(a.k), a.qbar,
                     a.kbar, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pool(const PredictLaunch& a, hipStream_t s) {
  if (a.g.dtype == SA_BF16)
    return a.g.D == 128 ? launch_pool_t<__bf16, 128>(a, s) : launch_pool_t<__bf16, 64>(a, s);
  return a.g.D == 128 ? launch_pool_t<float, 128>(a, s) : launch_pool_t<float, 64>(a, s);
}

}  // namespace sa
