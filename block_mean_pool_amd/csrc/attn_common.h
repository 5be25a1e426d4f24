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

// Skip groups of G rows: 16 (half a wavefront), 32 (one wavefront), 64 (a
// wavefront pair) or 128 (the whole query block).  `need_lane` holds for a
// lane whose row needs the tile's P.V product; lanes l and l ^ 32 hold the
// same row.  wave_need: some row of the wavefront needs it.  For G = 16,
// half_split tells the halves apart: 0 when both halves decide alike
// (both need it, or neither), else 1 (only rows 0-15 need it) or 2 (only
// rows 16-31).
__device__ __forceinline__ bool wave_need(bool need_lane) { return __any(need_lane); }
__device__ __forceinline__ uint32_t half_split(bool need_lane) {
  const uint64_t bal = __builtin_amdgcn_ballot_w64(need_lane);
  const uint64_t lo = 0x0000ffff0000ffffull;
  const bool a = (bal & lo) != 0, b = (bal & ~lo) != 0;
  return a == b ? 0u : (a ? 1u : 2u);
}
// G >= 64: the group needs the product if one of its wavefronts does
// (votes[w] = 1 when wavefront w needs it, published before a barrier).
__device__ __forceinline__ bool group_need(const uint32_t* votes, int w, int G) {
  const int per = G >> 5, g0 = w & ~(per - 1);  // per = 2 or 4
  uint32_t any = 0;
  for (int i = 0; i < per; ++i) any |= votes[g0 + i];
  return any != 0u;
}
// Whether this lane's row (l32 = lane % 32) is kept by a half split.
__device__ __forceinline__ bool split_keeps(uint32_t split, int l32) {
  return (split >> (l32 >> 4)) & 1u;
}

// Edge-tile masking of a lane's 32 scores of a 64-key tile (first key key0):
// score r of key half kt is key key0 + 32 kt + 8 (r / 4) + 4 hh + r % 4, set
// to -inf past N, for rows past N, and (causal) after the lane's row.  The
// per-score offsets are compile-time constants against one scalar and one
// per-lane value, so no per-score lane offsets stay live.  A row past N gets
// a lane offset beyond every limit (N <= 2^18) instead of a separate test:
// `qvalid && ...` became exec-masked code that wrote the masked scores to
// new registers, and the unmasked path then copied all 32 scores to match.
template <bool CAUSAL, typename F>
__device__ __forceinline__ void mask_scores(F (&s)[2], int key0, int N, int hh, int qrow,
                                            bool qvalid) {
  const int lim = N - key0;  // offsets >= lim are keys past N
  const int hh4 = qvalid ? 4 * hh : (1 << 30);
  const int dq = hh4 - (qrow - key0);  // causal: offset hh4 + c visible iff dq <= -c
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int c = 32 * kt + 8 * (r >> 2) + (r & 3);
      const bool ok = hh4 < lim - c && (!CAUSAL || dq <= -c);
      s[kt][r] = ok ? s[kt][r] : -INFINITY;
    }
}

// Skip-bit output of one wavefront: skip_bits is [rows of the mask,
// 128 / G, words]; group slot g, list entry t -> bit t % 32 of word t / 32.
// G = 16: a wavefront writes slots 2 w and 2 w + 1 (TWO kernels handle that
// case; a TWO kernel with another G writes one slot); G = 32: slot w;
// G >= 64: the group's first wavefront writes slot w / (G / 32), the others
// nothing.  The words are wavefront-uniform (scalar registers).
template <bool TWO>
struct SkipOut {
  uint32_t* out;  // the wavefront's first slot; null: nothing to write
  int second;     // words from the first slot to the second (G = 16), else 0
  uint32_t w0, w1;
  __device__ void init(uint32_t* bits, int row, int w, int G, int words) {
    out = nullptr;
    second = G == 16 ? words : 0;
    w0 = w1 = 0;
    if (!bits) return;
    uint32_t* base = bits + (size_t)row * (128 / G) * words;
    if (G == 16) out = base + (size_t)(2 * w) * words;
    else if (G == 32) out = base + (size_t)w * words;
    else if ((w & ((G >> 5) - 1)) == 0) out = base + (size_t)(w >> (G == 64 ? 1 : 2)) * words;
  }
  // the final decision on list entry t (of cnt): `need` for the group, or
  // (TWO) a half split (half_split) when the halves differ
  __device__ void put(int t, int cnt, bool need, uint32_t split, int lane) {
    if (!out) return;
    bool s0 = !need, s1 = !need;  // skipped: rows 0-15, rows 16-31
    if (TWO && split) {
      s0 = split == 2u;
      s1 = split == 1u;
    }
    w0 |= (s0 ? 1u : 0u) << (t & 31);
    if (TWO) w1 |= (s1 ? 1u : 0u) << (t & 31);
    if ((t & 31) == 31 || t + 1 == cnt) {
      if (lane == 0) {
        out[t >> 5] = w0;
        if (TWO && second) out[second + (t >> 5)] = w1;
      }
      w0 = w1 = 0;
    }
  }
};

// Skip-group handling compiled into a forward kernel: one wavefront per
// group (G = 32), half wavefronts (G = 16), or several wavefronts (G = 64,
// 128; the count is a launch argument).
enum GroupMode { kGroupWave = 0, kGroupHalf = 1, kGroupMulti = 2 };
inline int group_mode(int G) { return G == 16 ? kGroupHalf : (G > 32 ? kGroupMulti : kGroupWave); }

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
  int G;          // rows per skip group: 16, 32, 64 or 128
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
  a.G = f.group_rows;
  return a;
}

}  // namespace attn
}  // namespace sa
