// K3: block-sparse flash attention over the kept-block lists, with the
// softmax-aware skip of P.V products evaluated per wavefront.
//
// Stage two of the SpargeAttn abstract: an online softmax-aware filter that
// costs nothing extra and skips more matrix products.  Reading: for each
// kept tile, a wavefront (32 query rows) skips its P.V product when
// max over its rows of (tile max - new running max) < lambda; m and l are
// updated either way.  Tiles are processed in list order (the predictor's
// sorted order), which fixes which tiles the filter can skip.
//
// Workgroup = one (batch, head, 128-row query block), 4 wavefronts x 32 rows.
// Per kept key block j (64 keys):
//   S^T = K_j Q^T   on v_mfma_f32_32x32x16_bf16 (fp32 inputs: 32x32x2f32),
//                   computed transposed so that a lane owns one query row
//                   and 32 of the 64 keys: the row max and row sum are
//                   in-lane reductions plus one exchange with lane ^ 32;
//   online softmax in the exp2 domain (scale * log2 e folded into one FMA);
//   lambda test: one wave-wide ballot, a uniform branch around P.V;
//   O^T += V_j^T P^T  with P taken straight from the S^T accumulator
//                   layout as the B operand (the key order inside one MFMA
//                   is permuted identically on both operands).
// K_j is staged row-major and V_j transposed (d-major) in LDS, double
// buffered: tile t+1 is loaded into registers while tile t is computed and
// written to the other buffer afterwards, one barrier per tile.  Row
// paddings of 16 B (K) and 8/16 B (V^T) make the MFMA operand reads
// bank-conflict free.  Workgroup ids are remapped so that consecutive query
// blocks of one head run on one XCD and share its L2.
#include "sa_device.h"
#include "sa_internal.h"
#include "../../include/sparse_attn.h"

namespace sa {
namespace {

template <typename T>
struct Mfma;

template <>
struct Mfma<__bf16> {
  // 8 consecutive bf16 of one row / column: one 16-byte fragment
  struct Frag {
    u32x4 v;
  };
  __device__ static Frag load(const void* p) { return Frag{*reinterpret_cast<const u32x4*>(p)}; }
  __device__ static Frag zero() { return Frag{u32x4{0u, 0u, 0u, 0u}}; }
  __device__ static f32x16 mma(const Frag& a, const Frag& b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a.v),
                                                   __builtin_bit_cast(bf16x8, b.v), c, 0, 0, 0);
  }
};

template <>
struct Mfma<float> {
  // 8 consecutive fp32: eight k=2 MFMAs, k-slot (lane / 32) <-> element e
  struct Frag {
    f32x4 lo, hi;
  };
  __device__ static Frag load(const void* p) {
    const f32x4* q = reinterpret_cast<const f32x4*>(p);
    return Frag{q[0], q[1]};
  }
  __device__ static Frag zero() { return Frag{f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}}; }
  __device__ static f32x16 mma(const Frag& a, const Frag& b, f32x16 c) {
#pragma unroll
    for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[e], b.lo[e], c, 0, 0, 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[e], b.hi[e], c, 0, 0, 0);
    return c;
  }
};

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
};

template <typename T, int D>
struct Tile {
  static constexpr int E = sizeof(T);
  static constexpr int VEC = 16 / E;                     // elements per 16 B
  static constexpr int CPR = D * E / 16;                 // 16 B chunks per row
  static constexpr int KS = D * E + 16;                  // K row stride (bytes)
  static constexpr int VS = 64 * E + (E == 2 ? 8 : 16);  // V^T row stride (bytes)
  static constexpr int KBYTES = 64 * KS;
  static constexpr int VBYTES = D * VS;
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int KLD = CPR / 4;                    // K 16 B loads per thread
  static constexpr int VTASK = (16 * CPR + 255) / 256;   // 4-key x 16 B tasks per thread
  static constexpr int NKK = D / 16;                     // 16-wide k chunks of S
  static constexpr int NDT = D / 32;                     // 32-row d tiles of O^T
};

// Global -> registers for one K/V tile (rows >= N read as zero).
template <typename T, int D>
struct Stager {
  using TL = Tile<T, D>;
  u32x4 kr[TL::KLD];
  u32x4 vr[TL::VTASK][4];

  __device__ void load(const char* kbase, const char* vbase, int64_t row_bytes, int key0,
                       int N, int tid) {
#pragma unroll
    for (int s = 0; s < TL::KLD; ++s) {
      const int id = tid + s * 256;
      const int r = id / TL::CPR, c = id % TL::CPR;
      const int key = key0 + r;
      kr[s] = key < N ? *reinterpret_cast<const u32x4*>(kbase + (int64_t)key * row_bytes + c * 16)
                      : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int s = 0; s < TL::VTASK; ++s) {
      const int task = tid + s * 256;
      if (task < 16 * TL::CPR) {
        const int quad = task / TL::CPR, c = task % TL::CPR;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int key = key0 + 4 * quad + u;
          vr[s][u] = key < N ? *reinterpret_cast<const u32x4*>(vbase + (int64_t)key * row_bytes + c * 16)
                             : u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  }

  __device__ void store(char* stage, int tid) {
    char* ks = stage;
    char* vs = stage + TL::KBYTES;
#pragma unroll
    for (int s = 0; s < TL::KLD; ++s) {
      const int id = tid + s * 256;
      const int r = id / TL::CPR, c = id % TL::CPR;
      *reinterpret_cast<u32x4*>(ks + r * TL::KS + c * 16) = kr[s];
    }
#pragma unroll
    for (int s = 0; s < TL::VTASK; ++s) {
      const int task = tid + s * 256;
      if (task < 16 * TL::CPR) {
        const int quad = task / TL::CPR, c = task % TL::CPR;
        if constexpr (TL::E == 2) {
          // 4 keys x 8 bf16 -> for each of the 8 d: 4 keys = 8 bytes of V^T
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int w = e >> 1;
            const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
            u32x2 out;
            out[0] = __builtin_amdgcn_perm(vr[s][1][w], vr[s][0][w], sel);
            out[1] = __builtin_amdgcn_perm(vr[s][3][w], vr[s][2][w], sel);
            *reinterpret_cast<u32x2*>(vs + (c * 8 + e) * TL::VS + quad * 8) = out;
          }
        } else {
          // 4 keys x 4 fp32 -> for each of the 4 d: 4 keys = 16 bytes of V^T
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            u32x4 out{vr[s][0][e], vr[s][1][e], vr[s][2][e], vr[s][3][e]};
            *reinterpret_cast<u32x4*>(vs + (c * 4 + e) * TL::VS + quad * 16) = out;
          }
        }
      }
    }
  }
};

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256, (sizeof(T) == 4 && D == 128) ? 1 : 2) void attn_kernel(AttnArgs a) {
  using TL = Tile<T, D>;
  using M = Mfma<T>;
  __shared__ __align__(16) char smem[2 * TL::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int wg = xcd_remap(blockIdx.x, a.nwg);
  const int bh = wg / a.nqb;
  const int i = wg - bh * a.nqb;
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

  // Q fragment: row qrow, d = 16 kk + 8 hh + [0, 8)
  typename M::Frag qf[TL::NKK];
#pragma unroll
  for (int kk = 0; kk < TL::NKK; ++kk)
    qf[kk] = qvalid ? M::load(qbase + (int64_t)qrow * row_bytes + (16 * kk + 8 * hh) * TL::E)
                    : M::zero();

  int cnt = a.kept_cnt[wg];
  cnt = cnt < 0 ? 0 : (cnt > a.nkb ? a.nkb : cnt);
  const int32_t* lst = a.kept_idx + (size_t)wg * a.nkb;
  // an entry outside [0, NKB) is an empty tile: its keys start at N
  auto key_start = [&](int j) { return (unsigned)j < (unsigned)a.nkb ? j * 64 : a.N; };
  uint32_t* skip_out =
      a.skip_bits ? a.skip_bits + ((size_t)wg * 4 + w) * a.skip_words : nullptr;

  f32x16 acc[TL::NDT];
#pragma unroll
  for (int dt = 0; dt < TL::NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
  float m = -INFINITY;  // running max, log2 units
  float l = 0.f;        // this lane's share of the running sum
  uint32_t skip_word = 0;

  Stager<T, D> st;
  if (cnt > 0) {
    st.load(kbase, vbase, row_bytes, key_start(lst[0]), a.N, tid);
    st.store(smem, tid);
  }
  __syncthreads();

  for (int t = 0; t < cnt; ++t) {
    const int key0 = key_start(lst[t]);
    const char* stage = smem + (t & 1) * TL::STAGE;
    if (t + 1 < cnt) st.load(kbase, vbase, row_bytes, key_start(lst[t + 1]), a.N, tid);

    // S^T = K Q^T: two 32-key sub-tiles
    f32x16 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kt][r] = 0.f;
      const char* krow = stage + (32 * kt + l32) * TL::KS + 8 * hh * TL::E;
#pragma unroll
      for (int kk = 0; kk < TL::NKK; ++kk)
        s[kt] = M::mma(M::load(krow + 16 * kk * TL::E), qf[kk], s[kt]);
    }

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
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    const float mloc2 = mloc * a.c2;
    const float mnew = fmaxf(m, mloc2);
    bool do_pv = true;
    if (!a.lam_off) {
      const bool raises = (mloc2 != -INFINITY) && (mloc2 - mnew >= a.lam2);
      do_pv = __any(raises);
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
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < TL::NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
    }

    if (do_pv) {
      // O^T += V^T P^T; chunk c of 16 keys uses p values [8 (c & 1), +8) of
      // sub-tile c >> 1: lane half hh holds keys 32 kt + 16 (c & 1) +
      // 8 (e / 4) + 4 hh + e % 4 for e in [0, 8).
      const char* vst = stage + TL::KBYTES;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int kt = c >> 1, half = c & 1;
        const int kbase_c = 32 * kt + 16 * half + 4 * hh;
        if constexpr (TL::E == 2) {
          u32x4 pb;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            pb[e] = pack_bf16x2(s[kt][8 * half + 2 * e], s[kt][8 * half + 2 * e + 1]);
#pragma unroll
          for (int dt = 0; dt < TL::NDT; ++dt) {
            const char* vr = vst + (32 * dt + l32) * TL::VS + kbase_c * 2;
            const u32x2 v0 = *reinterpret_cast<const u32x2*>(vr);
            const u32x2 v1 = *reinterpret_cast<const u32x2*>(vr + 16);
            const u32x4 va{v0[0], v0[1], v1[0], v1[1]};
            acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, va), __builtin_bit_cast(bf16x8, pb), acc[dt], 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int dt = 0; dt < TL::NDT; ++dt) {
            const char* vr = vst + (32 * dt + l32) * TL::VS + kbase_c * 4;
            const f32x4 v0 = *reinterpret_cast<const f32x4*>(vr);
            const f32x4 v1 = *reinterpret_cast<const f32x4*>(vr + 32);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              acc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(v0[e], s[kt][8 * half + e], acc[dt], 0, 0, 0);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              acc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(v1[e], s[kt][8 * half + 4 + e], acc[dt], 0, 0, 0);
          }
        }
      }
    }

    if (skip_out) {
      skip_word |= (do_pv ? 0u : 1u) << (t & 31);
      if ((t & 31) == 31 || t + 1 == cnt) {
        if (lane == 0) skip_out[t >> 5] = skip_word;
        skip_word = 0;
      }
    }

    if (t + 1 < cnt) st.store(smem + ((t + 1) & 1) * TL::STAGE, tid);
    __syncthreads();
  }

  // epilogue: O = acc / l; lse = (m + log2 l) ln 2
  l += __shfl_xor(l, 32, 64);
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
          u32x2 pk{pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
          *reinterpret_cast<u32x2*>(orow + d * 2) = pk;
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
  if (f.causal)
    hipLaunchKernelGGL((attn_kernel<T, D, true>), dim3(a.nwg), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((attn_kernel<T, D, false>), dim3(a.nwg), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn(const ForwardLaunch& f, hipStream_t s) {
  if (f.g.dtype == SA_BF16)
    return f.g.D == 128 ? launch_t<__bf16, 128>(f, s) : launch_t<__bf16, 64>(f, s);
  return f.g.D == 128 ? launch_t<float, 128>(f, s) : launch_t<float, 64>(f, s);
}

}  // namespace sa
