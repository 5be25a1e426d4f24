// Token reordering for the block-mean predictor: the query tokens and the
// key tokens of each head are clustered, and each side is put in cluster
// order, so that the fixed blocks cut from the reordered sequence hold
// tokens that one mean represents well.
//
// iCATS abstract (arxivdaily.com page): grouping tokens by their query-key
// dot-product interaction estimates block scores better than grouping each
// side by feature similarity, and that objective is a simple quadratic form;
// irregular cluster sizes are handled by merging tails rather than padding.
// PARO abstract (huggingface-mirror search page): reordering tokens turns the
// attention pattern block-wise.
//
// Readings: replacing a query x by c moves its logit with key k by
// sm (x - c) . k, and the mean square of that move over the keys is
// sm^2 (x - c)^T M_K (x - c), M_K = K^T K / N.  So queries cluster under the
// quadratic form of M_K, keys under that of M_Q ("interaction"); "feature"
// uses M = I.  Centroid m starts at token floor((2m+1) N / (2C)); T Lloyd
// passes; ties go to the smaller cluster; a cluster without members keeps its
// centroid; tokens are ordered by (cluster, position), clusters packed back
// to back with no padding.
//
// Kernels, per slot z = 2 (b H + h) + side (side 0 = queries, 1 = keys):
//   moment_kernel    partial X^T X of the other side over a token range
//                    (bf16 MFMA on transposing LDS reads: exact products,
//                    fp32 sums)
//   moment_reduce    sums the partials in a fixed order, divides by N
//   centroid_kernel  the seeds (first pass) or the member means, gathered
//                    through the previous pass's order and summed in a fixed
//                    order
//   metric_kernel    G_m = M c_m as bf16 hi + lo parts, b_m = c_m . G_m
//   assign_kernel    label = argmin_m (b_m - 2 x . G_m), i.e. the quadratic
//                    form without its constant x^T M x; x . G_m by bf16 MFMA
//                    on the hi and lo parts (the tokens are bf16, exact)
//   hist / scan / scatter  stable counting sort of the labels: the order,
//                    each cluster's offset and size
//   export_kernel    the order and labels to the caller's [B,H,N] arrays
//   permute_kernel   row gather (or scatter) by a permutation
// Every reduction runs in a fixed order, so the results are deterministic.
#include "attn_common.h"

namespace sa {
namespace {

__device__ __forceinline__ const __bf16* slot_tokens(const ClusterLaunch& a, int z, bool other) {
  const int bh = z >> 1, side = z & 1;
  const int b = bh / a.g.H, h = bh - b * a.g.H;
  const bool keys = other ? side == 0 : side == 1;
  const __bf16* base = static_cast<const __bf16*>(keys ? a.k : a.q);
  return base + (int64_t)b * a.g.sb + (int64_t)h * a.g.sh;
}

__device__ __forceinline__ int slot_clusters(const ClusterLaunch& a, int z) {
  return (z & 1) ? a.ck : a.cq;
}

__device__ __forceinline__ f32x16 mfma_bf16(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------- moments
constexpr int kMomentTokens = 64;  // tokens per LDS tile

// Partial sum over tokens [c * span, (c + 1) * span) of x x^T for the other
// side's tokens of slot z.  Each 64-token tile is stored row-major in LDS with
// the V-tile chunk permutation of the forward kernel; both MFMA operands
// (8 consecutive tokens of one d column per lane) come from gfx950's
// transposing read ds_read_b64_tr_b16, which permutes the tokens inside one
// MFMA identically for both, so the sum over the 16 tokens is unchanged.
template <int D>
__global__ __launch_bounds__(256) void moment_kernel(ClusterLaunch a, int span) {
  using TL = attn::Tile<__bf16, D>;
  constexpr int RB = TL::RB, CPR = TL::CPR;
  constexpr int NB = D / 32;
  constexpr int TPW = NB * NB / 4;  // 32x32 tiles of M per wavefront
  __shared__ __align__(16) char T[kMomentTokens * RB];
  const int z = blockIdx.y, c = blockIdx.x;
  const __bf16* X = slot_tokens(a, z, true);
  const int t0 = c * span, t1 = min(a.g.N, t0 + span);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // transposing-read bases, as for the V^T operand of the forward kernel
  const int g16 = lane >> 4, s16 = lane & 15;
  const int tr_key = 4 * (g16 >> 1) + (s16 >> 2);
  const int tr_d = 16 * (g16 & 1) + 4 * (s16 & 3);
  uint32_t ro[NB];
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    const int d = 32 * bb + tr_d;
    ro[bb] = (uint32_t)(TL::v_off(tr_key, d >> 3) + (d & 7) * 2);
  }
  auto frag = [&](int kc, int bb) {
    const attn::s16x4 lo =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((attn::lds_s16x4*)(T + ro[bb] + 16 * kc * RB));
    const attn::s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (attn::lds_s16x4*)(T + ro[bb] + (16 * kc + 8) * RB));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return u32x4{l2[0], l2[1], h2[0], h2[1]};
  };

  f32x16 acc[TPW];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[tt][r] = 0.f;

  for (int base = t0; base < t1; base += kMomentTokens) {
    __syncthreads();
#pragma unroll
    for (int e = tid; e < kMomentTokens * CPR; e += 256) {
      const int tok = e / CPR, ch = e - tok * CPR;
      const int row = base + tok;
      const u32x4 v = row < t1 ? *reinterpret_cast<const u32x4*>(X + (int64_t)row * a.g.sn + ch * 8)
                               : u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(T + TL::v_off(tok, ch)) = v;
    }
    __syncthreads();
#pragma unroll
    for (int kc = 0; kc < kMomentTokens / 16; ++kc) {
      if constexpr (TPW == 4) {  // D = 128: row block w against all four column blocks
        const u32x4 fa = frag(kc, w);
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) acc[cb] = mfma_bf16(fa, frag(kc, cb), acc[cb]);
      } else {  // D = 64: one tile (w / 2, w % 2) per wavefront
        acc[0] = mfma_bf16(frag(kc, w >> 1), frag(kc, w & 1), acc[0]);
      }
    }
  }
  float* P = a.mpart + ((size_t)z * a.nchm + c) * D * D;
  const int hh = lane >> 5;
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    const int ti = w * TPW + tt, rb = ti / NB, cb = ti - rb * NB;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 32 * rb + 8 * (r >> 2) + 4 * hh + (r & 3);
      P[i * D + 32 * cb + (lane & 31)] = acc[tt][r];
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void moment_reduce(ClusterLaunch a) {
  const int z = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= D * D) return;
  const float* P = a.mpart + (size_t)z * a.nchm * D * D + e;
  float s = 0.f;
  for (int c = 0; c < a.nchm; ++c) s += P[(size_t)c * D * D];
  a.M[(size_t)z * D * D + e] = s / (float)a.g.N;
}

// -------------------------------------------------------------- centroids
// One workgroup per (cluster, slot).  First pass: the seed token.  Later
// passes: the mean of the members, gathered through the previous pass's
// order.  Thread (g, ch) reads 16-byte chunk ch of members g, g + RG, ...
// (RG row groups in flight), and the RG partial sums of each column are
// added in group order: a fixed order, so the result is deterministic.
constexpr int kGatherRows = 4;  // member rows in flight per thread

template <int D>
__global__ __launch_bounds__(128) void centroid_kernel(ClusterLaunch a, int seed_pass) {
  constexpr int CPR = D / 8;     // 16-byte chunks per row
  constexpr int RG = 128 / CPR;  // rows read at a time
  __shared__ float part[RG][D];
  const int z = blockIdx.y, m = blockIdx.x, tid = threadIdx.x;
  const int C = slot_clusters(a, z);
  if (m >= C) return;
  const __bf16* X = slot_tokens(a, z, false);
  float* c = a.cent + ((size_t)z * a.cmax + m) * D;
  const int64_t sn = a.g.sn;
  if (seed_pass) {
    const int s = (int)(((2LL * m + 1) * a.g.N) / (2LL * C));
    if (tid < D) c[tid] = (float)X[(int64_t)s * sn + tid];
    return;
  }
  const int n = a.cnt[(size_t)z * a.cmax + m];
  if (n == 0) return;  // no member: the centroid stays
  const int32_t* pm = a.perm + (size_t)z * a.g.N + a.seg[(size_t)z * a.cmax + m];
  const int ch = tid % CPR, g = tid / CPR;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  auto add_row = [&](const u32x4& v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += bf16_lo(v[e]);
      acc[2 * e + 1] += bf16_hi(v[e]);
    }
  };
  // kGatherRows member rows per thread in flight (their indices first, then
  // the rows), added in member order: the same sums as one row at a time
  int r = g;
  for (; r + (kGatherRows - 1) * RG < n; r += kGatherRows * RG) {
    int idx[kGatherRows];
#pragma unroll
    for (int u = 0; u < kGatherRows; ++u) idx[u] = pm[r + u * RG];
    u32x4 v[kGatherRows];
#pragma unroll
    for (int u = 0; u < kGatherRows; ++u)
      v[u] = *reinterpret_cast<const u32x4*>(X + (int64_t)idx[u] * sn + ch * 8);
#pragma unroll
    for (int u = 0; u < kGatherRows; ++u) add_row(v[u]);
  }
  for (; r < n; r += RG) add_row(*reinterpret_cast<const u32x4*>(X + (int64_t)pm[r] * sn + ch * 8));
#pragma unroll
  for (int e = 0; e < 8; ++e) part[g][ch * 8 + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
#pragma unroll
    for (int gg = 0; gg < RG; ++gg) s += part[gg][tid];
    c[tid] = s / (float)n;
  }
}

// ----------------------------------------------------------------- metric
constexpr int kMetricClusters = 16;  // clusters per workgroup

// G_m = M c_m for kMetricClusters clusters (M read once per workgroup; M is
// symmetric, so thread i reads column i: coalesced), stored as bf16 hi and
// lo = bf16(G - hi); b_m = c_m . G_m in a fixed order.
template <int D>
__global__ __launch_bounds__(128) void metric_kernel(ClusterLaunch a) {
  __shared__ float cs[kMetricClusters][D];
  __shared__ float gs[kMetricClusters][D];
  const int z = blockIdx.y, m0 = blockIdx.x * kMetricClusters, i = threadIdx.x;
  const int C = slot_clusters(a, z);
  if (m0 >= C) return;
  const int nm = min(kMetricClusters, C - m0);
  const float* cent = a.cent + ((size_t)z * a.cmax + m0) * D;
  for (int e = i; e < nm * D; e += 128) cs[e / D][e % D] = cent[e];
  __syncthreads();
  if (i < D) {
    float g[kMetricClusters];
#pragma unroll
    for (int mm = 0; mm < kMetricClusters; ++mm) g[mm] = 0.f;
    if (a.interaction) {
      const float* Mz = a.M + (size_t)z * D * D;
      for (int j = 0; j < D; ++j) {
        const float mji = Mz[j * D + i];
#pragma unroll
        for (int mm = 0; mm < kMetricClusters; ++mm) g[mm] = fmaf(mji, cs[mm][j], g[mm]);
      }
    } else {
#pragma unroll
      for (int mm = 0; mm < kMetricClusters; ++mm) g[mm] = cs[mm][i];
    }
    for (int mm = 0; mm < nm; ++mm) {
      const __bf16 hi = (__bf16)g[mm];
      const __bf16 lo = (__bf16)(g[mm] - (float)hi);
      const size_t off = ((size_t)z * a.cmax + m0 + mm) * D + i;
      a.ghi[off] = __builtin_bit_cast(uint16_t, hi);
      a.glo[off] = __builtin_bit_cast(uint16_t, lo);
      gs[mm][i] = g[mm];
    }
  }
  __syncthreads();
  if (i < nm) {
    float s = 0.f;
    for (int j = 0; j < D; ++j) s = fmaf(cs[i][j], gs[i][j], s);
    a.bvec[(size_t)z * a.cmax + m0 + i] = s;
  }
}

// ----------------------------------------------------------------- assign
// kAssignTokens tokens per workgroup: kAssignGroups MFMA columns of 32 tokens per
// wavefront, which share every A fragment.
// Cluster tiles of 32 rows of G (hi and lo) go through LDS in two buffers:
// the global loads of tile t + 1 are issued before the MFMAs of tile t and
// land in the other buffer after them, one barrier per tile.  The product
// D[m][x] = G_m . x comes out with lane -> token column, so each lane scans
// 16 clusters per tile in increasing order and the two lane halves merge at
// the end (ties to the smaller index).
constexpr int kAssignGroups = 4;
constexpr int kAssignTokens = 4 * 32 * kAssignGroups;

template <int D>
__global__ __launch_bounds__(256, 2) void assign_kernel(ClusterLaunch a) {
  constexpr int NG = kAssignGroups;
  constexpr int NKK = D / 16;
  constexpr int RS = D * 2 + 16;           // LDS row stride in bytes (padded)
  constexpr int TILE = 2 * 32 * RS;        // hi rows, then lo rows
  constexpr int CPT = 2 * 32 * (D / 8);    // 16-byte chunks per tile
  constexpr int LPT = CPT / 256;           // chunks per thread
  __shared__ __align__(16) char tiles[2][TILE];
  __shared__ float bt[2][32];
  const int z = blockIdx.y;
  const int C = slot_clusters(a, z);
  const __bf16* X = slot_tokens(a, z, false);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int tok0 = blockIdx.x * kAssignTokens + w * 32 * NG;
  const uint16_t* ghi = a.ghi + (size_t)z * a.cmax * D;
  const uint16_t* glo = a.glo + (size_t)z * a.cmax * D;
  const float* bz = a.bvec + (size_t)z * a.cmax;

  // chunk e of a tile: part (hi / lo), row r, 16-byte column ch
  u32x4 stage[LPT];
  float bstage = 0.f;
  auto fetch = [&](int m0) {
#pragma unroll
    for (int n = 0; n < LPT; ++n) {
      const int e = tid + 256 * n;
      const int part = e / (32 * (D / 8)), rem = e - part * (32 * (D / 8));
      const int r = rem / (D / 8), ch = rem - r * (D / 8);
      const int m = m0 + r;
      stage[n] = m < C ? *reinterpret_cast<const u32x4*>((part ? glo : ghi) + (size_t)m * D +
                                                         ch * 8)
                       : u32x4{0u, 0u, 0u, 0u};
    }
    if (tid < 32) bstage = m0 + tid < C ? bz[m0 + tid] : 0.f;
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int n = 0; n < LPT; ++n) {
      const int e = tid + 256 * n;
      const int part = e / (32 * (D / 8)), rem = e - part * (32 * (D / 8));
      const int r = rem / (D / 8), ch = rem - r * (D / 8);
      *reinterpret_cast<u32x4*>(&tiles[buf][part * 32 * RS + r * RS + ch * 16]) = stage[n];
    }
    if (tid < 32) bt[buf][tid] = bstage;
  };

  u32x4 xf[NG][NKK];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const int row = tok0 + 32 * gi + l32;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      xf[gi][kk] = row < a.g.N ? *reinterpret_cast<const u32x4*>(X + (int64_t)row * a.g.sn +
                                                                 16 * kk + 8 * hh)
                               : u32x4{0u, 0u, 0u, 0u};
  }
  float best[NG];
  int bidx[NG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    best[gi] = INFINITY;
    bidx[gi] = 0;
  }

  fetch(0);
  store(0);
  __syncthreads();
  const int ntiles = (C + 31) / 32;
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1, m0 = 32 * t;
    const bool more = t + 1 < ntiles;
    if (more) fetch(m0 + 32);
    const char* A = tiles[buf];
    f32x16 acc[NG];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[gi][r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const u32x4 ah = *reinterpret_cast<const u32x4*>(A + l32 * RS + (16 * kk + 8 * hh) * 2);
      const u32x4 al =
          *reinterpret_cast<const u32x4*>(A + 32 * RS + l32 * RS + (16 * kk + 8 * hh) * 2);
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        acc[gi] = mfma_bf16(ah, xf[gi][kk], acc[gi]);
        acc[gi] = mfma_bf16(al, xf[gi][kk], acc[gi]);
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 8 * (r >> 2) + 4 * hh + (r & 3);
      if (m0 + i < C) {
        const float bi = bt[buf][i];
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
          const float dist = fmaf(-2.f, acc[gi][r], bi);
          if (dist < best[gi]) {
            best[gi] = dist;
            bidx[gi] = m0 + i;
          }
        }
      }
    }
    // the other buffer was last read in iteration t - 1, before the barrier
    // that ended it
    if (more) store(buf ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const float pd = __shfl_xor(best[gi], 32, 64);
    const int pi = __shfl_xor(bidx[gi], 32, 64);
    if (pd < best[gi] || (pd == best[gi] && pi < bidx[gi])) bidx[gi] = pi;
    const int row = tok0 + 32 * gi + l32;
    if (hh == 0 && row < a.g.N) a.labels[(size_t)z * a.g.N + row] = bidx[gi];
  }
}

// ------------------------------------------------------------ counting sort
constexpr int kSortTokens = 256;  // tokens per chunk

__global__ __launch_bounds__(256) void hist_kernel(ClusterLaunch a) {
  extern __shared__ int32_t hs[];
  const int z = blockIdx.y, ch = blockIdx.x, tid = threadIdx.x;
  const int C = slot_clusters(a, z);
  for (int e = tid; e < C; e += 256) hs[e] = 0;
  __syncthreads();
  const int x = ch * kSortTokens + tid;
  if (x < a.g.N) atomicAdd(&hs[a.labels[(size_t)z * a.g.N + x]], 1);
  __syncthreads();
  int32_t* row = a.hist + ((size_t)z * a.nch + ch) * a.cmax;
  for (int e = tid; e < C; e += 256) row[e] = hs[e];
}

// Per slot: cluster sizes, their exclusive prefix (cluster offsets), and the
// chunk counts turned in place into each (chunk, cluster) start position.
__global__ __launch_bounds__(1024) void scan_kernel(ClusterLaunch a) {
  __shared__ int32_t tot[kMaxClusters];
  const int z = blockIdx.x, tid = threadIdx.x;
  const int C = slot_clusters(a, z);
  int32_t* H = a.hist + (size_t)z * a.nch * a.cmax;
  for (int m = tid; m < C; m += 1024) {
    int s = 0;
#pragma unroll 16
    for (int c = 0; c < a.nch; ++c) s += H[(size_t)c * a.cmax + m];
    tot[m] = s;
    a.cnt[(size_t)z * a.cmax + m] = s;
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int m = 0; m < C; ++m) {
      const int t = tot[m];
      tot[m] = run;
      run += t;
    }
  }
  __syncthreads();
  // counts -> bases, 16 chunks at a time: all loads of a batch are issued
  // before its stores
  constexpr int BATCH = 16;
  for (int m = tid; m < C; m += 1024) {
    int run = tot[m];
    a.seg[(size_t)z * a.cmax + m] = run;
    for (int c0 = 0; c0 < a.nch; c0 += BATCH) {
      int v[BATCH];
#pragma unroll
      for (int u = 0; u < BATCH; ++u)
        v[u] = c0 + u < a.nch ? H[(size_t)(c0 + u) * a.cmax + m] : 0;
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        if (c0 + u < a.nch) H[(size_t)(c0 + u) * a.cmax + m] = run;
        run += v[u];
      }
    }
  }
}

// Each token's position: its (chunk, cluster) start plus the number of
// earlier tokens of the chunk in the same cluster (stable).
__global__ __launch_bounds__(256) void scatter_kernel(ClusterLaunch a) {
  __shared__ int32_t lab[kSortTokens];
  const int z = blockIdx.y, ch = blockIdx.x, tid = threadIdx.x;
  const int x = ch * kSortTokens + tid;
  const int L = x < a.g.N ? a.labels[(size_t)z * a.g.N + x] : -1;
  lab[tid] = L;
  __syncthreads();
  if (x < a.g.N) {
    int rank = 0;
    for (int t = 0; t < tid; ++t) rank += lab[t] == L ? 1 : 0;
    const int pos = a.hist[((size_t)z * a.nch + ch) * a.cmax + L] + rank;
    a.perm[(size_t)z * a.g.N + pos] = x;
  }
}

__global__ __launch_bounds__(256) void export_kernel(ClusterLaunch a) {
  const int z = blockIdx.y, bh = z >> 1, side = z & 1;
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= a.g.N) return;
  const size_t src = (size_t)z * a.g.N + r, dst = (size_t)bh * a.g.N + r;
  (side ? a.perm_k : a.perm_q)[dst] = a.perm[src];
  int32_t* lab = side ? a.labels_k : a.labels_q;
  if (lab) lab[dst] = a.labels[src];
}

// ---------------------------------------------------------------- permute
// One 16-byte chunk per thread.  perm entries outside [0, N) are skipped.
__global__ __launch_bounds__(256) void permute_kernel(PermuteLaunch a) {
  const int cpr = a.row_bytes / 16, rpw = 256 / cpr;
  const int bh = blockIdx.y, tid = threadIdx.x;
  const int r = blockIdx.x * rpw + tid / cpr, ch = tid - (tid / cpr) * cpr;
  if (tid / cpr >= rpw || r >= a.g.N) return;
  const int p = a.perm[(size_t)bh * a.g.N + r];
  if ((unsigned)p >= (unsigned)a.g.N) return;
  const int src_row = a.inverse ? r : p, dst_row = a.inverse ? p : r;
  const int b = bh / a.g.H, h = bh - b * a.g.H;
  const int64_t off = ((int64_t)b * a.g.sb + (int64_t)h * a.g.sh) * a.esz;
  const int64_t rs = a.g.sn * a.esz;
  *reinterpret_cast<u32x4*>(static_cast<char*>(a.y) + off + dst_row * rs + ch * 16) =
      *reinterpret_cast<const u32x4*>(static_cast<const char*>(a.x) + off + src_row * rs + ch * 16);
}

template <int D>
hipError_t launch_cluster_t(const ClusterLaunch& a, hipStream_t s) {
  const int z2 = 2 * a.g.B * a.g.H;
  if (a.interaction) {
    hipLaunchKernelGGL((moment_kernel<D>), dim3(a.nchm, z2), dim3(256), 0, s, a, a.mspan);
    hipLaunchKernelGGL((moment_reduce<D>), dim3((D * D + 255) / 256, z2), dim3(256), 0, s, a);
  }
  const dim3 gc(a.cmax, z2), gm((a.cmax + kMetricClusters - 1) / kMetricClusters, z2);
  const dim3 ga((a.g.N + kAssignTokens - 1) / kAssignTokens, z2), gs(a.nch, z2);
  for (int t = 0; t < a.iters; ++t) {
    hipLaunchKernelGGL((centroid_kernel<D>), gc, dim3(128), 0, s, a, t == 0 ? 1 : 0);
    hipLaunchKernelGGL((metric_kernel<D>), gm, dim3(128), 0, s, a);
    hipLaunchKernelGGL((assign_kernel<D>), ga, dim3(256), 0, s, a);
    hipLaunchKernelGGL(hist_kernel, gs, dim3(256), a.cmax * sizeof(int32_t), s, a);
    hipLaunchKernelGGL(scan_kernel, dim3(z2), dim3(1024), 0, s, a);
    hipLaunchKernelGGL(scatter_kernel, gs, dim3(256), 0, s, a);
  }
  hipLaunchKernelGGL(export_kernel, dim3((a.g.N + 255) / 256, z2), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_cluster(const ClusterLaunch& a, hipStream_t s) {
  return a.g.D == 128 ? launch_cluster_t<128>(a, s) : launch_cluster_t<64>(a, s);
}

hipError_t launch_permute(const PermuteLaunch& a, hipStream_t s) {
  const int rpw = 256 / (a.row_bytes / 16);
  hipLaunchKernelGGL(permute_kernel, dim3((a.g.N + rpw - 1) / rpw, a.g.B * a.g.H), dim3(256), 0,
                     s, a);
  return hipGetLastError();
}

}  // namespace sa
