// Internal interface between the C-ABI host layer (api.hip) and the kernel
// launchers.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

struct Geometry {
  int B, H, N, D;
  int nqb, nkb;              // ceil(N/128), ceil(N/64)
  int64_t sb, sh, sn;        // element strides of Q/K/V/O
  int dtype;                 // SA_F32 | SA_BF16
};

struct PredictLaunch {
  Geometry g;
  const void* q;
  const void* k;
  float* qbar;               // [B,H,NQB,D]
  float* kbar;               // [B,H,NKB,D]
  int32_t* kept_idx;
  int32_t* kept_cnt;
  float* block_prob;         // optional
  int causal, rule, keep_prefix;
  float sm;
  float tau;
  int topk;                  // > 0: keep this many blocks (top-k rule)
};

struct ForwardLaunch {
  Geometry g;
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;                // optional
  uint32_t* skip_bits;       // optional
  const int32_t* kept_idx;
  const int32_t* kept_cnt;
  int causal;
  int o_fp32;                // O stored as fp32 (else bf16)
  float sm;
  float lambda;
  int recall_on;             // skip rule: 0 lambda, 1 recall
  float recall;              // target recall rho (recall rule)
  int group_rows;            // rows per skip group G: 16, 32, 64 or 128
  int qmax;                  // quantised variant: Q/K code range [-qmax, qmax]
  int v_pow2;                // quantised variant: power-of-two V scales
  // quantised variant: workspace buffers
  int8_t* qc;                // [B,H,N,D]
  int8_t* kc;                // [B,H,N,D]
  uint8_t* vt;               // [B,H,NKB,D,64]
  float* sq;                 // [B,H,NQB]
  float* sk;                 // [B,H,NKB]
  float* sv;                 // [B,H,NKB]
};

constexpr int kMaxClusters = 4096;  // clusters per side of one head

// Token clustering (all heads, both sides).  Slot z = 2 (b H + h) + side,
// side 0 = queries, 1 = keys; per-slot arrays are strided by cmax or N.
struct ClusterLaunch {
  Geometry g;
  const void* q;             // bf16
  const void* k;
  int cq, ck, cmax;          // clusters of the query / key side, max of both
  int iters;
  int interaction;           // 1: quadratic form of the other side's moment
  int nch;                   // sort chunks: ceil(N / 256)
  int nchm, mspan;           // moment partials and tokens per partial
  float* M;                  // [2BH][D][D]
  float* mpart;              // [2BH][nchm][D][D]
  float* cent;               // [2BH][cmax][D]
  uint16_t* ghi;             // [2BH][cmax][D] bf16 bits
  uint16_t* glo;
  float* bvec;               // [2BH][cmax]
  int32_t* labels;           // [2BH][N]
  int32_t* perm;             // [2BH][N]
  int32_t* hist;             // [2BH][nch][cmax]
  int32_t* seg;              // [2BH][cmax]
  int32_t* cnt;              // [2BH][cmax]
  int32_t* perm_q;           // outputs [B,H,N]
  int32_t* perm_k;
  int32_t* labels_q;         // optional
  int32_t* labels_k;
};

struct PermuteLaunch {
  Geometry g;
  const void* x;
  void* y;
  const int32_t* perm;       // [B,H,N]
  int inverse;               // 0: y[r] = x[perm[r]]; 1: y[perm[r]] = x[r]
  int esz;                   // element bytes (2 or 4)
  int row_bytes;             // D * esz
};

hipError_t launch_pool(const PredictLaunch& a, hipStream_t s);
hipError_t launch_mask(const PredictLaunch& a, hipStream_t s);
hipError_t launch_attn(const ForwardLaunch& a, hipStream_t s);
hipError_t launch_attn_pipe(const ForwardLaunch& a, hipStream_t s);
hipError_t launch_quant(const ForwardLaunch& a, hipStream_t s);
hipError_t launch_attn_q(const ForwardLaunch& a, hipStream_t s);
hipError_t launch_cluster(const ClusterLaunch& a, hipStream_t s);
hipError_t launch_permute(const PermuteLaunch& a, hipStream_t s);

}  // namespace sa
