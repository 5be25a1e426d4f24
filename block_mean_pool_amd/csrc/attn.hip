// K3: block-sparse flash attention over the kept-block lists, with the
// softmax-aware skip of P.V products evaluated per wavefront.
//
// Stage two of the SpargeAttn abstract: an online softmax-aware filter that
// costs nothing extra and skips more matrix products.  Reading: for each
// kept tile, a group of G query rows (by default a wavefront's 32) skips its
// P.V product when max over its rows of (tile max - new running max) <
// lambda; m and l are updated either way.  G = 16 zeroes the P of the half
// wavefront that skips; G = 64 and 128 OR the wavefronts' decisions through
// LDS.  Tiles are processed in list order (the predictor's
// sorted order), which fixes which tiles the filter can skip.
//
// Workgroup = one (batch, head, 128-row query block), 4 wavefronts x 32 rows.
// Per kept key block j (64 keys), per wavefront:
//   S^T = K_j Q^T   v_mfma_f32_32x32x16_bf16 (fp32 inputs: 32x32x2f32),
//                   computed transposed so that a lane owns one query row
//                   and 32 of the 64 keys: the row max and row sum are
//                   in-lane reductions plus one v_permlane32_swap;
//   online softmax in the exp2 domain (scale * log2 e folded into one FMA);
//   lambda test: one wave-wide ballot, a uniform branch around P.V;
//   O^T += V_j^T P^T  with P taken straight from the S^T accumulator
//                   layout as the B operand (the key order inside one MFMA
//                   is permuted identically on both operands).
//
// LDS layout: K and V tiles are both stored row-major (a row = one key,
// D elements), with the 16-byte chunks of each row permuted by an XOR of
// the row index, so that the staging stores are contiguous 16-byte writes
// and every operand read spreads over all LDS banks.  The V^T operand of
// P.V is read with ds_read_b64_tr_b16: within 16 lanes, source lane
// 4 j + q names 4 d-values of key K0 + j and lane i receives key K0 + j's
// value at d = D0 + i, i.e. a 4-key column segment of V^T per lane.
// K/V tiles are double buffered: tile t+1 is loaded into registers while
// tile t is computed and written to the other buffer afterwards, one barrier
// per tile.  K and V are read through buffer resources that end at row N-1,
// so ragged or empty tiles read zeros without branches.  Workgroup ids are
// remapped so that consecutive query blocks of one head run on one XCD.
#include "attn_common.h"

namespace sa {
namespace {

using namespace attn;

// Global -> registers -> LDS for one K/V tile.  K and V of the head are read
// through buffer resources whose size ends at row N - 1, so rows >= N (the
// ragged last block, or an empty tile whose offset starts at row N) read as
// zero without a branch.
template <typename T, int D>
struct Stager {
  using TL = Tile<T, D>;
  u32x4 kr[TL::NLD];
  u32x4 vr[TL::NLD];
  __amdgpu_buffer_rsrc_t krs, vrs;
  uint32_t row_bytes;

  __device__ void init(const char* kbase, const char* vbase, uint32_t rb, uint32_t span) {
    krs = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kbase), (short)0, (int)span, 0x00020000);
    vrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vbase), (short)0, (int)span, 0x00020000);
    row_bytes = rb;
  }

  // tile_off = first key of the tile * row_bytes; chunk id = tid + 256 s
  __device__ void load(uint32_t tile_off, int tid) {
#pragma unroll
    for (int s = 0; s < TL::NLD; ++s) {
      const int id = tid + s * 256;
      const uint32_t off = tile_off + (uint32_t)(id / TL::CPR) * row_bytes + (id % TL::CPR) * 16;
      kr[s] = __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0);
      vr[s] = __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, 0);
    }
  }

  __device__ void store(char* stage, int tid) {
#pragma unroll
    for (int s = 0; s < TL::NLD; ++s) {
      const int id = tid + s * 256;
      const int r = id / TL::CPR, c = id % TL::CPR;
      *reinterpret_cast<u32x4*>(stage + TL::k_off(r, c)) = kr[s];
      *reinterpret_cast<u32x4*>(stage + TL::TBYTES + TL::v_off(r, c)) = vr[s];
    }
  }
};

// S^T sub-tile kt (32 keys) = K Q^T.  Q fragment kk holds d = 16 kk + 8 hh
// + [0, 8) of this lane's query row (fp32: fragments 2 kk and 2 kk + 1).
template <typename T, int D>
__device__ __forceinline__ f32x16 qk_sub(const char* ks, const u32x4* qf, int kt, int l32, int hh) {
  using TL = Tile<T, D>;
  f32x16 s;
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = 0.f;
  const int row = 32 * kt + l32;
  if constexpr (TL::E == 2) {
#pragma unroll
    for (int kk = 0; kk < TL::NKK; ++kk) {
      const u32x4 kv = *reinterpret_cast<const u32x4*>(ks + TL::k_off(row, 2 * kk + hh));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kv),
                                                  __builtin_bit_cast(bf16x8, qf[kk]), s, 0, 0, 0);
    }
  } else {
    // 8 fp32 values = 2 chunks; eight k=2 MFMAs, k-slot (lane / 32) <-> element
#pragma unroll
    for (int kk = 0; kk < TL::NKK; ++kk) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const f32x4 kv =
            *reinterpret_cast<const f32x4*>(ks + TL::k_off(row, 4 * kk + 2 * hh + half));
        const u32x4 q = qf[2 * kk + half];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          s = __builtin_amdgcn_mfma_f32_32x32x2f32(kv[e], __uint_as_float(q[e]), s, 0, 0, 0);
      }
    }
  }
  return s;
}

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256, (sizeof(T) == 4 && D == 128) ? 1 : 2) void attn_kernel(AttnArgs a) {
  using TL = Tile<T, D>;
  constexpr int NQF = TL::E == 2 ? TL::NKK : 2 * TL::NKK;  // 16-byte Q fragments
  __shared__ __align__(16) char smem[2 * TL::STAGE];
  __shared__ uint32_t vote[4];  // G >= 64: 1 if wavefront w needs the tile's P.V

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const QueryBlock qblk = query_block(a.nwg, a.nqb, CAUSAL);
  const int wg = qblk.row;  // the query block's row in the mask arrays
  const int bh = qblk.bh;
  const int i = qblk.i;
  const int b = bh / a.H, h = bh - b * a.H;
  const int64_t head_off = ((int64_t)b * a.sb + (int64_t)h * a.sh) * TL::E;
  const int64_t row_bytes = a.sn * TL::E;
  const char* qbase = static_cast<const char*>(a.q) + head_off;
  const char* kbase = static_cast<const char*>(a.k) + head_off;
  const char* vbase = static_cast<const char*>(a.v) + head_off;

  const int row0 = i * 128;
  const int wrow0 = row0 + 32 * w;
  const int qrow = wrow0 + l32;
  const bool qvalid = qrow < a.N;
  const bool wave_partial = wrow0 + 32 > a.N;

  // Q fragments: row qrow, d = 16 kk + 8 hh + [0, 8) (fp32: two 16 B halves)
  u32x4 qf[NQF];
#pragma unroll
  for (int f = 0; f < NQF; ++f) {
    const int byte =
        TL::E == 2 ? (16 * f + 8 * hh) * 2 : (16 * (f >> 1) + 8 * hh + 4 * (f & 1)) * 4;
    qf[f] = qvalid ? *reinterpret_cast<const u32x4*>(qbase + (int64_t)qrow * row_bytes + byte)
                   : u32x4{0u, 0u, 0u, 0u};
  }

  int cnt = a.kept_cnt[wg];
  cnt = cnt < 0 ? 0 : (cnt > a.nkb ? a.nkb : cnt);
  const int32_t* lst = a.kept_idx + (size_t)wg * a.nkb;
  // an entry outside [0, NKB) is an empty tile: its keys start at N
  auto key_start = [&](int j) { return (unsigned)j < (unsigned)a.nkb ? j * 64 : a.N; };
  // list entries travel 64 at a time in one VGPR (lane e holds entry
  // base + e) and are picked with readlane; the next chunk is prefetched
  int lvec = lane < cnt ? lst[lane] : 0;
  int nvec = 64 + lane < cnt ? lst[64 + lane] : 0;
  SkipOut<true> skip_out;
  skip_out.init(a.skip_bits, wg, w, a.G, a.skip_words);

  f32x16 acc[TL::NDT];
#pragma unroll
  for (int dt = 0; dt < TL::NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
  float m = -INFINITY;  // running max, log2 units
  float l = 0.f;        // this lane's share of the running sum
  float drop = 0.f;     // recall rule: energy this row has dropped (row total)

  // V^T transpose reads: this lane's source key (within a 16-key chunk, +8
  // for the second read) and d offset (within a 32-wide d tile)
  const int g16 = lane >> 4, s16 = lane & 15;
  const int tr_key = 4 * (g16 >> 1) + (s16 >> 2);
  const int tr_d = 16 * (g16 & 1) + 4 * (s16 & 3);

  Stager<T, D> st;
  st.init(kbase, vbase, (uint32_t)row_bytes,
          (uint32_t)((int64_t)(a.N - 1) * row_bytes + D * TL::E));
  if (cnt > 0) {
    st.load((uint32_t)key_start(__builtin_amdgcn_readlane(lvec, 0)) * (uint32_t)row_bytes, tid);
    st.store(smem, tid);
  }
  __syncthreads();

  for (int t = 0; t < cnt; ++t) {
    const int key0 = key_start(__builtin_amdgcn_readlane(lvec, t & 63));
    const char* stage = smem + (t & 1) * TL::STAGE;
    if (t + 1 < cnt) {
      const int jn = ((t + 1) & 63) ? __builtin_amdgcn_readlane(lvec, (t + 1) & 63)
                                    : __builtin_amdgcn_readlane(nvec, 0);
      st.load((uint32_t)key_start(jn) * (uint32_t)row_bytes, tid);
    }

    f32x16 s[2];
    s[0] = qk_sub<T, D>(stage, qf, 0, l32, hh);
    s[1] = qk_sub<T, D>(stage, qf, 1, l32, hh);

    // masking: keys past N, rows past N, future keys under causality
    const bool need_mask = (key0 + 64 > a.N) || wave_partial || (CAUSAL && key0 + 63 > wrow0);
    if (need_mask) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * kt + 8 * (r >> 2) + 4 * hh + (r & 3);
          const bool ok = qvalid && key < a.N && (!CAUSAL || key <= qrow);
          if (!ok) s[kt][r] = -INFINITY;
        }
    }

    float mloc = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, s[kt][r]);
    mloc = xhalf_max(mloc);
    const float mloc2 = mloc * a.c2;
    const float mnew = fmaxf(m, mloc2);
    bool need = true;     // some row of the group needs the tile's P.V
    uint32_t split = 0u;  // G = 16: the halves of the wavefront decide apart
    if (!a.lam_off) {
      const bool nl = (mloc2 != -INFINITY) && (mloc2 - mnew >= a.lam2);
      need = wave_need(nl);
      if (a.G == 16) split = half_split(nl);
    }
    const float alpha = (mnew == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m - mnew);
    const float negm = (mnew == -INFINITY) ? 0.f : -mnew;
    float psum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[kt][r], a.c2, negm));
        s[kt][r] = p;
        psum += p;
      }
    l = alpha * l + psum;
    m = mnew;
    float E = 0.f;
    if (a.recall_on) {  // drop the tile if the rows' dropped share stays <= 1 - recall
      drop *= alpha;
      E = xhalf_sum(psum);
      const bool nl = !(drop + E <= a.omr * xhalf_sum(l));
      need = wave_need(nl);
      split = a.G == 16 ? half_split(nl) : 0u;
    }
    if (a.G > 32) {  // the group's decision, voted through LDS
      if (lane == 0) vote[w] = need ? 1u : 0u;
      __syncthreads();
      need = group_need(vote, w, a.G);
    }
    const bool keep = split ? split_keeps(split, l32) : need;
    if (a.recall_on && !keep) drop += E;
    if (split) {  // G = 16, one half skips: its P is zero
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kt][r] = keep ? s[kt][r] : 0.f;
    }
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < TL::NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
    }

    if (need) {
      // O^T += V^T P^T.  Chunk c of 16 keys uses p values [8 (c & 1), +8) of
      // sub-tile c >> 1: lane half hh holds keys 16 c + 8 (e / 4) + 4 hh +
      // e % 4 for e in [0, 8).
      const char* vst = stage + TL::TBYTES;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int kt = c >> 1, half = c & 1;
        if constexpr (TL::E == 2) {
          u32x4 pb;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            pb[e] = pack2(s[kt][8 * half + 2 * e], s[kt][8 * half + 2 * e + 1]);
#pragma unroll
          for (int dt = 0; dt < TL::NDT; ++dt) {
            // source: key 16 c + tr_key (+ 8), d = 32 dt + tr_d .. + 3
            const int d = 32 * dt + tr_d;
            const int k0 = 16 * c + tr_key;
            const int cd = d >> 3, hb = (d & 7) * 2;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4*)(vst + TL::v_off(k0, cd) + hb));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4*)(vst + TL::v_off(k0 + 8, cd) + hb));
            const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
            const u32x4 va{l2[0], l2[1], h2[0], h2[1]};
            acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, va), __builtin_bit_cast(bf16x8, pb), acc[dt], 0, 0, 0);
          }
        } else {
          // fp32: V^T element (d = 32 dt + l32, key) is one 4-byte read of
          // row `key`; eight k=2 MFMAs per chunk
#pragma unroll
          for (int dt = 0; dt < TL::NDT; ++dt) {
            const int d = 32 * dt + l32;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int key = 16 * c + 8 * (e >> 2) + 4 * hh + (e & 3);
              const float vv =
                  *reinterpret_cast<const float*>(vst + TL::v_off(key, d >> 2) + (d & 3) * 4);
              acc[dt] =
                  __builtin_amdgcn_mfma_f32_32x32x2f32(vv, s[kt][8 * half + e], acc[dt], 0, 0, 0);
            }
          }
        }
      }
    }

    skip_out.put(t, cnt, need, split, lane);

    if (t + 1 < cnt) st.store(smem + ((t + 1) & 1) * TL::STAGE, tid);
    if (((t + 1) & 63) == 0) {
      lvec = nvec;
      nvec = t + 65 + lane < cnt ? lst[t + 65 + lane] : 0;
    }
    __syncthreads();
  }

  // epilogue: O = acc / l; lse = (m + log2 l) ln 2
  l = xhalf_sum(l);
  if (qvalid) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int oe = a.o_fp32 ? 4 : 2;  // bytes per O element
    char* orow = static_cast<char*>(a.o) +
                 ((int64_t)b * a.sb + (int64_t)h * a.sh + (int64_t)qrow * a.sn) * oe;
#pragma unroll
    for (int dt = 0; dt < TL::NDT; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * dt + 8 * g4 + 4 * hh;
        const float o0 = acc[dt][4 * g4] * inv, o1 = acc[dt][4 * g4 + 1] * inv;
        const float o2 = acc[dt][4 * g4 + 2] * inv, o3 = acc[dt][4 * g4 + 3] * inv;
        if (a.o_fp32) {
          *reinterpret_cast<f32x4*>(orow + d * 4) = f32x4{o0, o1, o2, o3};
        } else {
          *reinterpret_cast<u32x2*>(orow + d * 2) = u32x2{pack2(o0, o1), pack2(o2, o3)};
        }
      }
    if (a.lse && hh == 0) {
      const int64_t li = (int64_t)bh * a.N + qrow;
      a.lse[li] = l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
    }
  }
}

template <typename T, int D>
hipError_t launch_t(const ForwardLaunch& f, hipStream_t s) {
  const AttnArgs a = make_args(f);
  if (f.causal)
    hipLaunchKernelGGL((attn_kernel<T, D, true>), dim3(a.nwg), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((attn_kernel<T, D, false>), dim3(a.nwg), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn(const ForwardLaunch& f, hipStream_t s) {
  if (f.g.dtype == SA_BF16) return launch_attn_pipe(f, s);
  return f.g.D == 128 ? launch_t<float, 128>(f, s) : launch_t<float, 64>(f, s);
}

}  // namespace sa
