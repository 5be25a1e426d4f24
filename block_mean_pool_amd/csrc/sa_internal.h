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
  // quantised variant: workspace buffers
  int8_t* qc;                // [B,H,N,D]
  int8_t* kc;                // [B,H,N,D]
  uint8_t* vt;               // [B,H,NKB,D,64]
  float* sq;                 // [B,H,NQB]
  float* sk;                 // [B,H,NKB]
  float* sv;                 // [B,H,NKB]
};

hipError_t launch_pool(const PredictLaunch& a, hipStream_t s);
hipError_t launch_mask(const PredictLaunch& a, hipStream_t s);
hipError_t launch_attn(const ForwardLaunch& a, hipStream_t s);
hipError_t launch_attn_pipe(const ForwardLaunch& a, hipStream_t s);
hipError_t launch_quant(const ForwardLaunch& a, hipStream_t s);
hipError_t launch_attn_q(const ForwardLaunch& a, hipStream_t s);

}  // namespace sa
