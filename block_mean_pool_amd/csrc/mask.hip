// K2: compressed Q.K^T over the block means, predicted block map, and the
// cumulative-mass cut, one workgroup per (batch, head, query block).
//
// Stage one of the SpargeAttn abstract (predict the attention map to skip
// products), built the way the iCATS abstract describes training-free
// sparse attention: score query-key regions, derive a mask with a top-p
// rule, keep only the important candidates; the ENERGY rule weights each
// key block by its estimated total energy (the DynSparse story's
// cumulative-energy target).
//
// Per workgroup (256 threads):
//   1. s_j = sm * <qbar_i, kbar_j> for every admissible key block j, as an
//      fp64 sum of exact fp32 x fp32 products (kbar rows are L2-resident);
//   2. max and sum of the weights exp(s_j - max) [* n_j] (fp64);
//   3. bitonic sort in LDS of the keys (class, s, j): forced blocks first,
//      then s descending, then j ascending -- a strict total order;
//   4. P-hat_j = weight_j / sum in place, blocked fp64 prefix sum over the
//      sorted order, first prefix reaching tau, never below the forced count
//      (the top-k rule keeps a fixed count instead);
//   5. the kept prefix is written in sorted order with its length.
// LDS: val[P2] doubles indexed by j (score, then P-hat) and key[P2] packed
// (class << 16 | j), P2 = max(256, next power of two >= NKB) <= 4096.
#include "sa_device.h"
#include "sa_internal.h"
#include "../../include/sparse_attn.h"

namespace sa {
namespace {

constexpr int kThreads = 256;

// (class, s desc, j asc) order of two packed keys (class << 16 | j); both
// scores are read whatever the classes (every j < P2 has one), so the
// comparison is a chain of selects rather than branches
__device__ __forceinline__ bool sorts_before(int ka, int kb, const double* val) {
  const int ca = ka >> 16, cb = kb >> 16;
  const int ja = ka & 0xffff, jb = kb & 0xffff;
  const double sa_ = val[ja], sb_ = val[jb];
  const bool by_s = sa_ != sb_ ? sa_ > sb_ : ja < jb;
  return ca != cb ? ca < cb : by_s;
}

__device__ __forceinline__ double block_reduce_max(double v, double* scratch) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) scratch[w] = v;
  __syncthreads();
  double r = scratch[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) r = fmax(r, scratch[i]);
  return r;
}

__device__ __forceinline__ double block_reduce_sum(double v, double* scratch) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) scratch[w] = v;
  __syncthreads();
  double r = scratch[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) r += scratch[i];
  return r;
}

template <int D>
__global__ __launch_bounds__(kThreads) void mask_kernel(PredictLaunch a, int P2) {
  extern __shared__ __align__(16) char smem[];
  double* val = reinterpret_cast<double*>(smem);          // [P2]
  int* key = reinterpret_cast<int*>(val + P2);            // [P2]
  double* part = reinterpret_cast<double*>(key + P2);     // [kThreads]
  float* qs = reinterpret_cast<float*>(part + kThreads);  // [D]
  __shared__ double red[kThreads / 64];
  __shared__ int s_counts[2];
  __shared__ int s_kstar;

  const Geometry& g = a.g;
  const int tid = threadIdx.x;
  const int row = blockIdx.x;  // (b*H + h) * nqb + i
  const int bh = row / g.nqb;
  const int i = row - bh * g.nqb;
  const int first_row = i * 128;
  const int last_row = min(g.N, first_row + 128) - 1;
  const float* qb = a.qbar + (size_t)row * D;
  const float* kb = a.kbar + (size_t)bh * g.nkb * D;

  for (int d = tid; d < D; d += kThreads) qs[d] = qb[d];
  if (tid == 0) {
    s_counts[0] = 0;
    s_counts[1] = 0;
    s_kstar = 0x7fffffff;
  }
  __syncthreads();

  // 1. scores and classes (0 forced, 1 admissible, 2 inadmissible, 3 pad).
  // Eight lanes share a key row: lane e reads the row's 16-byte chunks e,
  // e + 8, ..., so one wavefront load covers eight rows in whole cache lines
  // (one row per lane would touch 64 lines per load); the eight fp64 partial
  // sums meet in a butterfly, which leaves the same sum on all eight lanes.
  constexpr int CPL = D / 4 / 8;  // 16-byte chunks per lane
  const int e8 = tid & 7;
  double lmax = -INFINITY;
  int n_adm = 0, n_forced = 0;
  for (int j = tid >> 3; j < P2; j += kThreads / 8) {  // P2 / 32 rounds for every lane
    const bool real = j < g.nkb;
    const int first_key = j * 64;
    const bool adm = real && (!a.causal || first_key <= last_row);
    double acc = 0.0;
    if (adm) {
      const f32x4* kr = reinterpret_cast<const f32x4*>(kb + (size_t)j * D);
#pragma unroll
      for (int u = 0; u < CPL; ++u) {
        const int c = e8 + 8 * u;
        const f32x4 kv = kr[c];
#pragma unroll
        for (int k = 0; k < 4; ++k) acc = fma((double)qs[4 * c + k], (double)kv[k], acc);
      }
    }
    acc += __shfl_xor(acc, 1, 8);
    acc += __shfl_xor(acc, 2, 8);
    acc += __shfl_xor(acc, 4, 8);
    if (e8 == 0) {
      int cls = 3;
      double s = -INFINITY;
      if (adm) {
        s = (double)a.sm * acc;
        const int last_key = min(g.N, first_key + 64) - 1;
        const bool forced = j < a.keep_prefix || (a.causal && last_key >= first_row);
        cls = forced ? 0 : 1;
        lmax = fmax(lmax, s);
        ++n_adm;
        n_forced += forced;
      } else if (real) {
        cls = 2;
      }
      val[j] = s;
      key[j] = (cls << 16) | j;
    }
  }
  if (n_adm) atomicAdd(&s_counts[0], n_adm);
  if (n_forced) atomicAdd(&s_counts[1], n_forced);
  const double smax = block_reduce_max(lmax, red);

  // 2. normaliser of the weights
  double lsum = 0.0;
  for (int j = tid; j < g.nkb; j += kThreads) {
    const int cls = key[j] >> 16;
    if (cls <= 1) {
      double w = exp(val[j] - smax);
      if (a.rule == SA_RULE_ENERGY) w *= (double)(min(g.N, j * 64 + 64) - j * 64);
      lsum += w;
    }
  }
  const double total = block_reduce_sum(lsum, red);
  const int nA = s_counts[0], nF = s_counts[1];

  // 3. bitonic sort of key[] by (class, s desc, j asc); val[] is read-only
  for (int size = 2; size <= P2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = tid; t < (P2 >> 1); t += kThreads) {
        const int lo = 2 * t - (t & (stride - 1));
        const int hi = lo + stride;
        const int klo = key[lo], khi = key[hi];
        const bool asc = (lo & size) == 0;
        // swap when kx sorts before ky: one comparison, no divergent arms
        const int kx = asc ? khi : klo, ky = asc ? klo : khi;
        if (sorts_before(kx, ky, val)) {
          key[lo] = khi;
          key[hi] = klo;
        }
      }
      __syncthreads();
    }
  }

  // 4. P-hat in place (natural order), optional debug copy
  float* bp = a.block_prob ? a.block_prob + (size_t)row * g.nkb : nullptr;
  for (int j = tid; j < g.nkb; j += kThreads) {
    const bool adm = !a.causal || j * 64 <= last_row;
    double p = 0.0;
    if (adm) {
      double w = exp(val[j] - smax);
      if (a.rule == SA_RULE_ENERGY) w *= (double)(min(g.N, j * 64 + 64) - j * 64);
      p = w / total;
    }
    val[j] = p;
    if (bp) bp[j] = (float)p;
  }
  __syncthreads();

  // blocked prefix sum over sorted positions [0, nA)
  const int E = P2 / kThreads;
  const int t0 = tid * E;
  double local = 0.0;
  for (int e = 0; e < E; ++e) {
    const int t = t0 + e;
    if (t < nA) local += val[key[t] & 0xffff];
  }
  part[tid] = local;
  __syncthreads();
  // inclusive Hillis-Steele scan of the per-thread sums
  for (int off = 1; off < kThreads; off <<= 1) {
    const double add = tid >= off ? part[tid - off] : 0.0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  const double tau = (double)a.tau;
  if (tau < 1.0 && a.topk == 0) {
    double run = tid ? part[tid - 1] : 0.0;
    for (int e = 0; e < E; ++e) {
      const int t = t0 + e;
      if (t >= nA) break;
      run += val[key[t] & 0xffff];
      if (run >= tau) {
        atomicMin(&s_kstar, t + 1);
        break;
      }
    }
  }
  __syncthreads();
  int kcount = nA;
  if (a.topk > 0)
    kcount = min(nA, max(nF, a.topk));  // fixed budget, same processing order
  else if (tau < 1.0 && s_kstar != 0x7fffffff)
    kcount = max(nF, s_kstar);

  // 5. compaction: the kept prefix in processing order
  int32_t* out = a.kept_idx + (size_t)row * g.nkb;
  for (int t = tid; t < kcount; t += kThreads) out[t] = key[t] & 0xffff;
  if (tid == 0) a.kept_cnt[row] = kcount;
}

template <int D>
hipError_t launch_mask_t(const PredictLaunch& a, hipStream_t s) {
  const Geometry& g = a.g;
  int P2 = 256;
  while (P2 < g.nkb) P2 <<= 1;
  const size_t lds = (size_t)P2 * (sizeof(double) + sizeof(int)) +
                     kThreads * sizeof(double) + D * sizeof(float);
  const int64_t blocks = (int64_t)g.B * g.H * g.nqb;
  hipLaunchKernelGGL((mask_kernel<D>), dim3((unsigned)blocks), dim3(kThreads), lds, s, a, P2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mask(const PredictLaunch& a, hipStream_t s) {
  return a.g.D == 128 ? launch_mask_t<128>(a, s) : launch_mask_t<64>(a, s);
}

}  // namespace sa
