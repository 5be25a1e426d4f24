// K3 for bf16 inputs: block-sparse flash attention with the per-wavefront
// softmax-aware skip, software-pipelined so that the matrix cores and the
// vector ALU of each wavefront work at the same time.
//
// Same method, tile shapes, operand layouts and results as the generic
// kernel in attn.hip (see there for the reading of the SpargeAttn abstract's
// stage two); what differs is the schedule:
//
//   iteration t (tile = t-th kept key block, in list order):
//     scalar part of the softmax of tile t: masking (edge tiles only),
//           row max, lambda ballot, running max (the recall rule decides
//           after the region, once tile t's energy is summed).  The VOTE
//           variant runs it at the end of iteration t - 1 instead, as soon
//           as tile t's Q.K^T is complete, and votes on tile t's V transfer;
//     one region, in four chunks of 16 keys: the 4 MFMAs of P.V for tile
//           t-1 (not issued when tile t-1 was skipped), 4 MFMAs of Q.K^T
//           for tile t+1, and 8 exp2/FMA/add plus bf16 packing of tile t's
//           softmax; after the first chunk, the DMA of K of tile t+2 and V
//           of tile t (unless no wavefront multiplies tile t), global -> LDS
//           directly (buffer_load ... lds, no staging registers), into the
//           stages whose previous contents iteration t-1 finished reading;
//     wait until this wave's DMA has landed, barrier.
//
// LDS: two stages of K and of V (64 KiB, two workgroups per CU), each stage
// its own array so the compiler sees that DMA into one does not alias reads
// of another; the loop is unrolled twice so every stage choice, and every
// LDS read offset, is a compile-time constant plus a per-lane base.  DMA is
// issued every iteration (rows past N read as zero).
// The exponent offset is the exact running max m: P = exp2(c S - m) <= 1,
// so the key holding a row's maximum has P = 1, exact in bf16 (a lazily
// raised offset would leave that dominant weight with up to 2^-8 relative
// rounding, which alone can move O by 1e-2).  l is rescaled at once when m
// grows; acc one step later, before the P.V of the tile that set the new m
// (in score order m grows on about 2 % of a wavefront's tiles).
#include <algorithm>
#include <type_traits>

#include "attn_common.h"

namespace sa {
namespace {

using namespace attn;

typedef __attribute__((address_space(3))) void lds_void;

struct Soft {
  float m;        // running max (log2 units), the exponent offset
  float l;        // this lane's share of sum exp2(c S - m)
  float resc_a;   // acc factor applied at the start of the next step
  float resc_b;   // acc factor of the latest scalar part, one step later
  float drop;     // recall rule: energy the row has dropped, same offset as l
};

template <int I>
using Int = std::integral_constant<int, I>;

// Two workgroups per CU at d = 128 (256 VGPRs per lane); three at d = 64,
// where the compiler fits the kernel in 168 VGPRs by spilling a few (six
// dwords reloaded once per step): 5-8 % faster than two on the video and
// causal workloads at d = 64, identical output.
template <int D, bool CAUSAL, bool VOTE, int GM>
__global__ __launch_bounds__(256, D == 64 ? 3 : 2) void attn_pipe_kernel(AttnArgs a) {
  static_assert(!(CAUSAL && VOTE), "the V vote is a non-causal schedule");
  // skip groups: SPLIT = halves of a wavefront (G = 16); MULTI = several
  // wavefronts (G = 64, 128), whose decision in the plain schedule is final
  // only after the barrier that follows the wavefronts' votes (DEFER)
  constexpr bool SPLIT = GM == kGroupHalf, MULTI = GM == kGroupMulti;
  constexpr bool DEFER = MULTI && !VOTE;
  using TL = Tile<__bf16, D>;
  constexpr int RB = TL::RB, TB = TL::TBYTES;
  constexpr int NI = TB / 4096;  // DMA wave-instructions per tile per wave
  constexpr int NKK = D / 16, NDT = D / 32;
  constexpr int ROWS_PER_4K = 4096 / RB;
  static_assert(NKK % 4 == 0, "the region splits the d chunks in quarters");
  __shared__ __align__(16) char k0[TB];
  __shared__ __align__(16) char k1[TB];
  __shared__ __align__(16) char v0[TB];
  __shared__ __align__(16) char v1[TB];
  // per tile parity and wavefront: 1 if the wavefront needs the tile's P.V.
  // VOTE kernels publish the lambda decision one step early, and a tile no
  // wavefront needs gets no V; groups of G > 32 rows decide by OR-ing their
  // wavefronts' votes (published before a barrier)
  __shared__ __align__(16) uint32_t vote[2][4];
  auto kst = [&](auto s) -> char* {
    if constexpr (decltype(s)::value % 2 == 0) return k0;
    else return k1;
  };
  auto vst = [&](auto s) -> char* {
    if constexpr (decltype(s)::value % 2 == 0) return v0;
    else return v1;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const QueryBlock qblk = query_block(a.nwg, a.nqb, CAUSAL, VOTE);
  const int wg = qblk.row;  // the query block's row in the mask arrays
  const int bh = qblk.bh;
  const int i = qblk.i;
  const int b = bh / a.H, h = bh - b * a.H;
  const int64_t head_off = ((int64_t)b * a.sb + (int64_t)h * a.sh) * 2;
  const int64_t row_bytes = a.sn * 2;
  const uint32_t rbg = (uint32_t)row_bytes;
  const char* qbase = static_cast<const char*>(a.q) + head_off;

  const int wrow0 = i * 128 + 32 * w;
  const int qrow = wrow0 + l32;
  const bool qvalid = qrow < a.N;
  const bool wave_partial = wrow0 + 32 > a.N;

  u32x4 qf[NKK];  // d = 16 kk + 8 hh + [0, 8) of row qrow
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk)
    qf[kk] = qvalid ? *reinterpret_cast<const u32x4*>(qbase + (int64_t)qrow * row_bytes +
                                                      (16 * kk + 8 * hh) * 2)
                    : u32x4{0u, 0u, 0u, 0u};

  int cnt = a.kept_cnt[wg];
  cnt = cnt < 0 ? 0 : (cnt > a.nkb ? a.nkb : cnt);
  const int32_t* lst = a.kept_idx + (size_t)wg * a.nkb;
  auto key_of = [&](int j) { return (unsigned)j < (unsigned)a.nkb ? j * 64 : a.N; };
  // list window: lane e of `win` holds entry wbase + e, `nxt` the next 64
  int wbase = 0;
  int win = lane < cnt ? lst[lane] : 0;
  int nxt = 64 + lane < cnt ? lst[64 + lane] : 0;
  auto entry_key = [&](int e) {  // key of entry e < wbase + 64, or N past the list
    return e < cnt ? key_of(__builtin_amdgcn_readlane(win, e - wbase)) : a.N;
  };
  SkipOut<SPLIT> skip_out;
  skip_out.init(a.skip_bits, wg, w, a.G, a.skip_words);

  // buffer resources for K and V of this head (rows >= N read as zero)
  const uint32_t span = (uint32_t)((int64_t)(a.N - 1) * row_bytes + D * 2);
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(static_cast<const char*>(a.k) + head_off), (short)0, (int)span, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(static_cast<const char*>(a.v) + head_off), (short)0, (int)span, 0x00020000);

  // DMA: wave-instruction n of wave w fills LDS bytes [(4 n + w) KiB, +1 KiB)
  // of a tile, lane e the 16 bytes at e * 16: LDS row r, position p holds the
  // global chunk p ^ swizzle(r) of key row r.  Instruction n covers rows
  // n * 4096 / RB further on, which leaves both swizzles unchanged, so one
  // per-lane offset per tensor serves every n.
  uint32_t dk0, dv0;
  {
    const int pos = w * 1024 + lane * 16;
    const int r = pos / RB, pch = (pos % RB) >> 4;
    dk0 = (uint32_t)r * rbg + (uint32_t)((pch ^ TL::swz_k(r)) << 4);
    dv0 = (uint32_t)r * rbg + (uint32_t)((pch ^ TL::swz_v(r)) << 4);
  }
  // LDS read bases: K row l32 (+ 32 kt), chunk 2 kk + hh; V^T transpose
  // reads from key 16 c + 8 half + tr_key, d = 32 dt + tr_d
  uint32_t kro[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) kro[kk] = (uint32_t)TL::k_off(l32, 2 * kk + hh);
  const int g16 = lane >> 4, s16 = lane & 15;
  const int tr_key = 4 * (g16 >> 1) + (s16 >> 2);
  const int tr_d = 16 * (g16 & 1) + 4 * (s16 & 3);
  uint32_t vro[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    const int d = 32 * dt + tr_d;
    vro[dt] = (uint32_t)(TL::v_off(tr_key, d >> 3) + (d & 7) * 2);
  }

  auto dma = [&](const __amdgpu_buffer_rsrc_t& rs, uint32_t lane_off, char* dst, int key0) {
    const uint32_t base = (uint32_t)key0 * rbg + lane_off;
#pragma unroll
    for (int n = 0; n < NI; ++n)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + (4 * n + w) * 1024), 16,
                                               base + n * ROWS_PER_4K * rbg, 0, 0, 0);
  };
  auto qk_mfma = [&](const char* kb, int kt, int kk, f32x16 acc_s) {
    const u32x4 kv = *reinterpret_cast<const u32x4*>(kb + kro[kk] + 32 * kt * RB);
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kv),
                                                   __builtin_bit_cast(bf16x8, qf[kk]), acc_s, 0, 0,
                                                   0);
  };
  auto pv_mfma = [&](const char* vb, int c, int dt, const u32x4& pb, f32x16 acc_o) {
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(vb + vro[dt] + 16 * c * RB));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(vb + vro[dt] + (16 * c + 8) * RB));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    const u32x4 va{l2[0], l2[1], h2[0], h2[1]};
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va),
                                                   __builtin_bit_cast(bf16x8, pb), acc_o, 0, 0, 0);
  };

  f32x16 acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
  f32x16 sA[2], sB[2];
  u32x4 pf[4];  // P of the previous tile, bf16, as the P.V B operand
#pragma unroll
  for (int c = 0; c < 4; ++c) pf[c] = u32x4{0u, 0u, 0u, 0u};
  Soft ss{-INFINITY, 0.f, 1.f, 1.f, 0.f};
  bool pv_prev = false;
  float pend_E = 0.f;     // DEFER, recall rule: the row's energy in the tile awaiting its vote
  uint32_t sp_new = 0;    // SPLIT: the half split of the latest scalar part
  // VOTE kernels (chosen by the host for non-causal calls whose K and V
  // would stream from HBM; they also take the windowed workgroup order)
  // vote on each tile's V transfer: the lambda decision is known once
  // the tile's Q.K^T is complete, so the scalar part runs at the end of the
  // previous step and the vote is in LDS by the barrier before the tile's
  // step; a tile no wavefront multiplies is not fetched (a third of them at
  // tau = 0.9 on the video workloads).  The recall rule decides after the
  // tile's energy is summed, so it always fetches V.  The other kernels run
  // the scalar part at the start of the step.
  const bool vote_on = VOTE && !a.lam_off && !a.recall_on;

  // softmax, scalar part of the tile whose scores are s (first key key0):
  // masking, row max, lambda ballot, running max; the acc factor for a
  // raised m goes to resc_b and reaches acc at the start of the step whose
  // region multiplies this tile's P.V
  auto scalar_part = [&](f32x16(&s)[2], int key0, int u) -> bool {
    const bool need_mask = (key0 + 64 > a.N) || wave_partial || (CAUSAL && key0 + 63 > wrow0);
    // a select per score, not a branch: this file is built with SimplifyCFG's
    // sinking and hoisting off, which would leave `if (!ok)` as one branch per
    // score (a third more code; 4 % slower on the video workload)
    if (need_mask) mask_scores<CAUSAL>(s, key0, a.N, hh, qrow, qvalid);
    float mloc = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, s[kt][r]);
    mloc = xhalf_max(mloc) * a.c2;
    const float mnew = fmaxf(ss.m, mloc);
    bool do_pv = true;
    sp_new = 0u;
    if (!a.lam_off) {
      const bool nl = (mloc != -INFINITY) && (mloc - mnew >= a.lam2);
      do_pv = wave_need(nl);
      if constexpr (SPLIT) sp_new = half_split(nl);
    }
    if (__any(mnew != ss.m)) {
      // 0 when m was -inf (nothing accumulated yet), 1 where m did not move
      const float f = (mnew == ss.m) ? 1.f : __builtin_amdgcn_exp2f(ss.m - mnew);
      ss.l *= f;
      ss.drop *= f;
      ss.resc_b *= f;
      ss.m = mnew;
    }
    if (vote_on && lane == 0) vote[u & 1][w] = do_pv ? 1u : 0u;
    return do_pv;
  };

  // the final decision on entry tt (SPLIT: with its half split): the recall
  // rule's dropped energy, the zero P of a skipping half wavefront, the skip
  // bits, and whether the next step multiplies the tile's P.V
  auto finish = [&](int tt, bool nd, uint32_t split, float E) {
    if constexpr (SPLIT) {
      const bool keep = split ? split_keeps(split, l32) : nd;
      if (a.recall_on && !keep) ss.drop += E;
      if (split) {  // the skipping half's rows multiply a zero P (acc + 0 = acc)
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int e = 0; e < 4; ++e) pf[c][e] = keep ? pf[c][e] : 0u;
      }
    } else {
      if (a.recall_on && !nd) ss.drop += E;
    }
    skip_out.put(tt, cnt, nd, split, lane);
    pv_prev = nd;
  };

  int kq0 = entry_key(0), kq1 = entry_key(1);  // keys of entries t, t + 1

  // prologue: K of entries 0 and 1, S of entry 0
  dma(krs, dk0, kst(Int<0>{}), kq0);
  dma(krs, dk0, kst(Int<1>{}), kq1);
  __syncthreads();
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) sA[kt][r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) sA[kt] = qk_mfma(kst(Int<0>{}), kt, kk, sA[kt]);
  }
  bool dpv_next = true;  // the lambda decision of the next tile (VOTE kernels)
  uint32_t dsp_next = 0u;
  if (VOTE && cnt > 0) {
    dpv_next = scalar_part(sA, kq0, 0);
    dsp_next = sp_new;
  }
  __syncthreads();  // stage 0 of K is refilled in iteration 0; entry 0's vote

  // one pipeline step for entry t with phase PH = t % 2
  auto step = [&](auto ph, int t, f32x16(&sc)[2], f32x16(&sn)[2]) {
    constexpr int PH = decltype(ph)::value;
    char* k_next = kst(Int<PH + 1>{});  // K of entry t + 1
    char* k_free = kst(Int<PH>{});      // K of entry t (read) -> entry t + 2
    char* v_prev = vst(Int<PH + 1>{});  // V of entry t - 1
    char* v_free = vst(Int<PH>{});      // V of entry t - 2 (read) -> entry t

    if (t + 2 - wbase >= 64) {  // slide the list window
      win = nxt;
      wbase += 64;
      nxt = wbase + 64 + lane < cnt ? lst[wbase + 64 + lane] : 0;
    }
    const int key_far = entry_key(t + 2);
    const int key_cur = kq0;
    bool need_v = true;
    if (vote_on) {
      const u32x4 vv = *reinterpret_cast<const u32x4*>(vote[t & 1]);
      need_v = __builtin_amdgcn_readfirstlane((vv[0] | vv[1] | vv[2] | vv[3]) != 0u);
    }
    // the DMA of this step goes out after the region's first chunk: the first
    // MFMAs start without waiting behind it, and it still has the rest of
    // the region to land
    auto issue_dma = [&]() {
      dma(krs, dk0, k_free, key_far);
      if (need_v) dma(vrs, dv0, v_free, key_cur);
    };

    if constexpr (DEFER) {
      if (t > 0) finish(t - 1, group_need(vote[(t - 1) & 1], w, a.G), 0u, pend_E);
    }
    bool do_pv = dpv_next;  // the lambda decision of tile t
    uint32_t split = dsp_next;
    if constexpr (!VOTE) {
      do_pv = scalar_part(sc, key_cur, t);
      split = sp_new;
    } else if constexpr (MULTI) {
      if (vote_on) do_pv = group_need(vote[t & 1], w, a.G);
    }
    if (__any(ss.resc_a != 1.f)) {  // m grew at t - 1
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] *= ss.resc_a;
    }
    ss.resc_a = ss.resc_b;
    ss.resc_b = 1.f;

    const float negm = (ss.m == -INFINITY) ? 0.f : -ss.m;
    const float c2 = a.c2;

    // region: [P.V of t-1] + Q.K^T of t+1 + exp/sum/pack of t.  Chunk c:
    // P.V MFMAs of key chunk c of tile t-1, Q.K^T MFMAs for the c-th quarter
    // of the d chunks kk (both key halves), softmax of this lane's 8 scores
    // 8 half + [0, 8) of key half kt = c / 2 of tile t.
    u32x4 pn[4];
    float psum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) sn[kt][r] = 0.f;
    auto chunk_qk = [&](int c) {
#pragma unroll
      for (int kk = c * (NKK / 4); kk < (c + 1) * (NKK / 4); ++kk) {
        sn[0] = qk_mfma(k_next, 0, kk, sn[0]);
        sn[1] = qk_mfma(k_next, 1, kk, sn[1]);
      }
    };
    auto chunk_pv = [&](int c) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) acc[dt] = pv_mfma(v_prev, c, dt, pf[c], acc[dt]);
    };
    auto chunk_soft = [&](int c) {
      const int kt = c >> 1, half = c & 1;
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        pv[e] = __builtin_amdgcn_exp2f(fmaf(sc[kt][8 * half + e], c2, negm));
      psum += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
#pragma unroll
      for (int e = 0; e < 4; ++e) pn[c][e] = pack2(pv[2 * e], pv[2 * e + 1]);
    };
    if (pv_prev) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        chunk_pv(c);
        chunk_qk(c);
        chunk_soft(c);
        if (c == 0) issue_dma();
      }
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        chunk_qk(c);
        chunk_soft(c);
        if (c == 0) issue_dma();
      }
    }
    ss.l += psum;
#pragma unroll
    for (int c = 0; c < 4; ++c) pf[c] = pn[c];
    float E = 0.f;
    if (a.recall_on) {  // drop the tile if the rows' dropped share stays <= 1 - recall
      E = xhalf_sum(psum);
      const bool nl = !(ss.drop + E <= a.omr * xhalf_sum(ss.l));
      do_pv = wave_need(nl);
      if constexpr (SPLIT) split = half_split(nl);
    }
    if constexpr (DEFER) {
      if (lane == 0) vote[t & 1][w] = do_pv ? 1u : 0u;
      pend_E = E;
    } else {
      finish(t, do_pv, split, E);
    }
    kq0 = kq1;
    kq1 = key_far;
    if (VOTE && t + 1 < cnt) {
      dpv_next = scalar_part(sn, kq0, t + 1);
      dsp_next = sp_new;
    }
    // the DMA issued above is what iteration t + 1 reads; the vote on its V
    __syncthreads();
  };

  int t = 0;
  for (; t + 2 <= cnt; t += 2) {
    step(Int<0>{}, t, sA, sB);
    step(Int<1>{}, t + 1, sB, sA);
  }
  if (t < cnt) step(Int<0>{}, t, sA, sB);

  if (cnt > 0) {
    if constexpr (DEFER) finish(cnt - 1, group_need(vote[(cnt - 1) & 1], w, a.G), 0u, pend_E);
    if (__any(ss.resc_a != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] *= ss.resc_a;
    }
    if (pv_prev) {  // P.V of the last entry, V in stage (cnt - 1) % 2
      const char* vlast = ((cnt - 1) & 1) ? v1 : v0;
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) acc[dt] = pv_mfma(vlast, c, dt, pf[c], acc[dt]);
    }
  }

  // epilogue: O = acc / l; lse = (m + log2 l) ln 2
  const float l = xhalf_sum(ss.l);
  if (qvalid) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int oe = a.o_fp32 ? 4 : 2;
    char* orow = static_cast<char*>(a.o) +
                 ((int64_t)b * a.sb + (int64_t)h * a.sh + (int64_t)qrow * a.sn) * oe;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * dt + 8 * g4 + 4 * hh;
        const float o0 = acc[dt][4 * g4] * inv, o1 = acc[dt][4 * g4 + 1] * inv;
        const float o2 = acc[dt][4 * g4 + 2] * inv, o3 = acc[dt][4 * g4 + 3] * inv;
        if (a.o_fp32)
          *reinterpret_cast<f32x4*>(orow + d * 4) = f32x4{o0, o1, o2, o3};
        else
          *reinterpret_cast<u32x2*>(orow + d * 2) = u32x2{pack2(o0, o1), pack2(o2, o3)};
      }
    if (a.lse && hh == 0)
      a.lse[(int64_t)bh * a.N + qrow] = l > 0.f ? (ss.m + __log2f(l)) * kLn2 : -INFINITY;
  }
}

// The VOTE variant (windowed workgroup order + V vote) pays where K and V
// would stream from HBM: when the K and V of eight heads, one per XCD in the
// default order, exceed the 256 MiB Infinity Cache.  Rotated medians at
// N = 119056 (488 MB), bit-identical output: the V vote alone -4.8 %, with
// the windowed order -11.8 % (lambda = -5) and -15.3 % (lambda = -inf).  At
// N = 32760 (134 MB, cache-resident either way) the variant measured
// between -2 % and +1.6 % on different boxes, so the plain kernel stays.
// The recall rule with groups of several wavefronts decides after each
// tile's region, too late for the VOTE schedule's early vote: such calls
// run the plain schedule.
bool vote_pays(const ForwardLaunch& f) {
  const int64_t heads = std::min<int64_t>(8, (int64_t)f.g.B * f.g.H);
  if (f.recall_on && f.group_rows > 32) return false;
  return !f.causal && heads * 2 * f.g.N * (int64_t)f.g.D * 2 > (int64_t)256 << 20;
}

template <int D, int GM>
hipError_t launch_pipe_t(const ForwardLaunch& f, hipStream_t s) {
  const AttnArgs a = make_args(f);
  if (f.causal)
    hipLaunchKernelGGL((attn_pipe_kernel<D, true, false, GM>), dim3(a.nwg), dim3(256), 0, s, a);
  else if (vote_pays(f))
    hipLaunchKernelGGL((attn_pipe_kernel<D, false, true, GM>), dim3(a.nwg), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((attn_pipe_kernel<D, false, false, GM>), dim3(a.nwg), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_pipe_d(const ForwardLaunch& f, hipStream_t s) {
  switch (group_mode(f.group_rows)) {
    case kGroupHalf: return launch_pipe_t<D, kGroupHalf>(f, s);
    case kGroupMulti: return launch_pipe_t<D, kGroupMulti>(f, s);
    default: return launch_pipe_t<D, kGroupWave>(f, s);
  }
}

}  // namespace

hipError_t launch_attn_pipe(const ForwardLaunch& f, hipStream_t s) {
  return f.g.D == 128 ? launch_pipe_d<128>(f, s) : launch_pipe_d<64>(f, s);
}

}  // namespace sa
