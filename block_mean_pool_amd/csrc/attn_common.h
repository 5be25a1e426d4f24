// Shared pieces of the forward kernels: argument block, LDS tile layout
// (row-major K/V tiles with XOR-permuted 16-byte chunks) and small wave
// helpers.
#pragma once

#include "sa_device.h"
#include "sa_internal.h"
#include "../../include/sparse_attn.h"

namespace sa {
namespace attn {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// two fp32 -> packed bf16x2 (round to nearest even), one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// max / sum of x over this lane and lane ^ 32 (the other half of the wave):
// after v_permlane32_swap each lane holds both values, in some order.
__device__ __forceinline__ float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The query block a workgroup runs.
// * Default: consecutive ids stay on one XCD and one head (xcd_remap), so
//   each XCD works through whole heads and the head's K and V are shared in
//   its L2.  Under causality a head's query blocks run last-first: block i
//   has 2 i + 2 admissible key blocks, so the heaviest start first and the
//   light ones fill the end of the grid.
// * window (non-causal calls whose K and V would stream from HBM, eight
//   heads in flight exceeding the 256 MiB Infinity Cache): xcd_window_remap
//   with windows of 512 query blocks, what the chip holds at once (2
//   workgroups on each of 256 CUs).  The whole chip works on one or two
//   heads at a time, whose K and V then stay in the Infinity Cache, and each
//   XCD runs 64 consecutive query blocks, which share its L2.
constexpr int kWindowPerXcd = 64;
struct QueryBlock {
  int row;  // (b H + h) nqb + i: index into the mask arrays
  int bh;
  int i;
};
__device__ __forceinline__ QueryBlock query_block(int nwg, int nqb, bool causal,
                                                bool window = false) {
  const int wg = window ? xcd_window_remap(blockIdx.x, nwg, kWindowPerXcd) : xcd_remap(blockIdx.x, nwg);
  const int bh = wg / nqb;
  const int j = wg - bh * nqb;
  const int i = causal ? nqb - 1 - j : j;
  return QueryBlock{bh * nqb + i, bh, i};
}

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  uint32_t* skip_bits;
  const int32_t* kept_idx;
  const int32_t* kept_cnt;
  int H, N, nqb, nkb, nwg, skip_words;
  int64_t sb, sh, sn;
  float c2;     // sm * log2(e)
  float lam2;   // lambda * log2(e)
  int lam_off;  // lambda == -inf: never skip
  int o_fp32;   // O stored as fp32
  int recall_on;  // recall skip rule instead of lambda
  float omr;      // 1 - recall
};

template <typename T, int D>
struct Tile {
  static constexpr int E = sizeof(T);
  static constexpr int RB = D * E;        // LDS row bytes (one key)
  static constexpr int CPR = RB / 16;     // 16-byte chunks per row
  static constexpr int TBYTES = 64 * RB;  // one K or V tile
  static constexpr int STAGE = 2 * TBYTES;
  static constexpr int NLD = CPR / 4;     // 16 B loads per thread per tile
  static constexpr int NKK = D / 16;      // 16-wide k chunks of S
  static constexpr int NDT = D / 32;      // 32-row d tiles of O^T
  // chunk permutation of row r: K rows are read 16 consecutive rows at a
  // time (one chunk each), V rows 4 at a time (64 bytes each)
  __device__ static int swz_k(int r) { return CPR >= 16 ? (r & 15) : ((r >> 1) & 7); }
  __device__ static int swz_v(int r) {
    if constexpr (E != 2) return 0;
    return CPR >= 16 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
  }
  __device__ static int k_off(int r, int c) { return r * RB + ((c ^ swz_k(r)) << 4); }
  __device__ static int v_off(int r, int c) { return r * RB + ((c ^ swz_v(r)) << 4); }
};


inline AttnArgs make_args(const ForwardLaunch& f) {
  const Geometry& g = f.g;
  AttnArgs a;
  a.q = f.q;
  a.k = f.k;
  a.v = f.v;
  a.o = f.o;
  a.lse = f.lse;
  a.skip_bits = f.skip_bits;
  a.kept_idx = f.kept_idx;
  a.kept_cnt = f.kept_cnt;
  a.H = g.H;
  a.N = g.N;
  a.nqb = g.nqb;
  a.nkb = g.nkb;
  a.nwg = g.B * g.H * g.nqb;
  a.skip_words = (g.nkb + 31) / 32;
  a.sb = g.sb;
  a.sh = g.sh;
  a.sn = g.sn;
  a.c2 = f.sm * kLog2e;
  a.lam_off = f.lambda == -INFINITY;
  a.lam2 = a.lam_off ? 0.f : f.lambda * kLog2e;
  a.o_fp32 = f.o_fp32;
  a.recall_on = f.recall_on;
  a.omr = 1.0f - f.recall;
  if (a.recall_on) a.lam_off = 1;
  return a;
}

}  // namespace attn
}  // namespace sa
