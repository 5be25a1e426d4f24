// Quantised stage two: INT8 Q.K^T and FP8 (OCP e4m3) P.V.
//
// The SpargeAttn abstract calls the method sparse *and quantized*; the
// DynSparse story notes the filter combines with quantization.  The pages fix
// no format, so this follows the stated reading:
//   Q, K: one scale per (b, h, block) = block absmax / 127 (1 if zero),
//         code = rint(x / scale) clamped to [-127, 127] (fp32 division);
//   V:    one scale per key block = absmax / 448, code = e4m3(x / scale);
//   P:    e4m3(2^8 p), the product rescaled by scale_v * 2^-8; the running
//         sum l uses the unquantised p.
//
// quant_kernel: one workgroup per Q block, K block or V block; the block is
// read once into registers, its absmax reduced, and its codes written.  V
// codes are written per key block transposed ([D][64] bytes) through LDS, so
// the attention kernel stages V^T with plain 16-byte copies.
// attn_q_kernel: the same tiling, online softmax and per-wavefront lambda
// test as the bf16 kernel, with v_mfma_i32_32x32x32_i8 for S^T = K Q^T and
// v_mfma_f32_32x32x16_fp8_fp8 for O^T += V^T P^T.
#include "sa_device.h"
#include "sa_internal.h"
#include "../../include/sparse_attn.h"

namespace sa {
namespace {

constexpr int D = 128;

__device__ __forceinline__ float block_max(float v, float* scratch) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) scratch[w] = v;
  __syncthreads();
  return fmaxf(fmaxf(scratch[0], scratch[1]), fmaxf(scratch[2], scratch[3]));
}

// Q: 128-row blocks, K and V: 64-row blocks.  D = 128 bf16 = 16 chunks of
// 16 B per row; thread -> chunk tid % 16, rows tid / 16 + 16 * it.
__global__ __launch_bounds__(256) void quant_kernel(ForwardLaunch f) {
  __shared__ float scratch[4];
  __shared__ __align__(16) uint8_t vt_tile[D * 64];
  const Geometry& g = f.g;
  const int tid = threadIdx.x;
  const int c = tid & 15, ro = tid >> 4;
  const int nq = g.B * g.H * g.nqb;
  const int nk = g.B * g.H * g.nkb;
  int id = blockIdx.x;
  int kind, bh, blk, bs;
  if (id < nq) {
    kind = 0;
    bh = id / g.nqb;
    blk = id - bh * g.nqb;
    bs = 128;
  } else if (id < nq + nk) {
    id -= nq;
    kind = 1;
    bh = id / g.nkb;
    blk = id - bh * g.nkb;
    bs = 64;
  } else {
    id -= nq + nk;
    kind = 2;
    bh = id / g.nkb;
    blk = id - bh * g.nkb;
    bs = 64;
  }
  const int b = bh / g.H, h = bh - b * g.H;
  const __bf16* src = static_cast<const __bf16*>(kind == 0 ? f.q : kind == 1 ? f.k : f.v) +
                      (int64_t)b * g.sb + (int64_t)h * g.sh;
  const int r0 = blk * bs, r1 = min(g.N, r0 + bs);

  u32x4 buf[8];
  float amax = 0.f;
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int r = r0 + ro + 16 * it;
    buf[it] = u32x4{0u, 0u, 0u, 0u};
    if (r < r1) buf[it] = *reinterpret_cast<const u32x4*>(src + (int64_t)r * g.sn + c * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(buf[it][e])), fabsf(bf16_hi(buf[it][e]))));
  }
  amax = block_max(amax, scratch);

  if (kind < 2) {
    const float scale = amax > 0.f ? __fdiv_rn(amax, 127.0f) : 1.0f;
    int8_t* dst = (kind == 0 ? f.qc : f.kc) + (size_t)bh * g.N * D;
    if (tid == 0) (kind == 0 ? f.sq : f.sk)[bh * (kind == 0 ? g.nqb : g.nkb) + blk] = scale;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int r = r0 + ro + 16 * it;
      if (r < r1) {
        uint32_t packed[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t w = buf[it][e >> 1];
          const float x = (e & 1) ? bf16_hi(w) : bf16_lo(w);
          float qv = rintf(__fdiv_rn(x, scale));
          qv = fminf(fmaxf(qv, -127.f), 127.f);
          packed[e >> 2] |= ((uint32_t)(int)qv & 0xffu) << (8 * (e & 3));
        }
        *reinterpret_cast<u32x2*>(dst + (int64_t)r * D + c * 8) = u32x2{packed[0], packed[1]};
      }
    }
  } else {
    const float scale = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
    if (tid == 0) f.sv[bh * g.nkb + blk] = scale;
    // rows ro + 16 it (it < 4) of this key block; transposed into LDS
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int rr = ro + 16 * it;  // key within block
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const uint32_t w = buf[it][e >> 1];
        const float x0 = __fdiv_rn(bf16_lo(w), scale);
        const float x1 = __fdiv_rn(bf16_hi(w), scale);
        const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
        vt_tile[(c * 8 + e) * 64 + rr] = (uint8_t)(pk & 0xff);
        vt_tile[(c * 8 + e + 1) * 64 + rr] = (uint8_t)((pk >> 8) & 0xff);
      }
    }
    __syncthreads();
    uint8_t* dst = f.vt + ((size_t)bh * g.nkb + blk) * D * 64;
    // 8 KB tile = 512 chunks of 16 B, two per thread
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int ch = tid + 256 * s;
      *reinterpret_cast<u32x4*>(dst + ch * 16) = *reinterpret_cast<const u32x4*>(vt_tile + ch * 16);
    }
  }
}

struct AttnQArgs {
  const int8_t* qc;
  const int8_t* kc;
  const uint8_t* vt;
  const float* sq;
  const float* sk;
  const float* sv;
  void* o;
  float* lse;
  uint32_t* skip_bits;
  const int32_t* kept_idx;
  const int32_t* kept_cnt;
  int H, N, nqb, nkb, nwg, skip_words;
  int64_t sb, sh, sn;  // strides of O (elements)
  float c2, lam2;
  int lam_off;
  int o_fp32;
};

constexpr int KS = D + 16;  // int8 K row stride (bytes)
constexpr int VS = 64 + 4;  // e4m3 V^T row stride (bytes)
constexpr int KBYTES = 64 * KS;
constexpr int VBYTES = D * VS;
constexpr int STAGE = KBYTES + VBYTES;

struct StagerQ {
  u32x4 kr[2];  // 64 rows x 8 chunks = 512 chunks
  u32x4 vr[2];  // 128 d rows x 4 chunks = 512 chunks
  __device__ void load(const int8_t* kc, const uint8_t* vt_blocks, int j, int N, int tid) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int id = tid + 256 * s;
      const int r = id >> 3, c = id & 7;
      const int key = j * 64 + r;
      kr[s] = key < N ? *reinterpret_cast<const u32x4*>(kc + (int64_t)key * D + c * 16)
                      : u32x4{0u, 0u, 0u, 0u};
      vr[s] = *reinterpret_cast<const u32x4*>(vt_blocks + (size_t)j * D * 64 + id * 16);
    }
  }
  __device__ void store(char* stage, int tid) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int id = tid + 256 * s;
      const int r = id >> 3, c = id & 7;
      *reinterpret_cast<u32x4*>(stage + r * KS + c * 16) = kr[s];
      const int d = id >> 2, cv = id & 3;
      uint32_t* vp = reinterpret_cast<uint32_t*>(stage + KBYTES + d * VS + cv * 16);
      vp[0] = vr[s][0];
      vp[1] = vr[s][1];
      vp[2] = vr[s][2];
      vp[3] = vr[s][3];
    }
  }
};

template <bool CAUSAL>
__global__ __launch_bounds__(256, 2) void attn_q_kernel(AttnQArgs a) {
  __shared__ __align__(16) char smem[2 * STAGE];
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int wg = xcd_remap(blockIdx.x, a.nwg);
  const int bh = wg / a.nqb;
  const int i = wg - bh * a.nqb;
  const int b = bh / a.H, h = bh - b * a.H;
  const int row0 = i * 128;
  const int wrow0 = row0 + 32 * w;
  const int qrow = wrow0 + l32;
  const bool qvalid = qrow < a.N;
  const bool wave_partial = wrow0 + 32 > a.N;
  const int8_t* qc = a.qc + (size_t)bh * a.N * D;
  const int8_t* kc = a.kc + (size_t)bh * a.N * D;
  const uint8_t* vt = a.vt + (size_t)bh * a.nkb * D * 64;

  u32x4 qf[4];  // d = 32 kk + 16 hh + [0, 16)
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    qf[kk] = qvalid ? *reinterpret_cast<const u32x4*>(qc + (int64_t)qrow * D + 32 * kk + 16 * hh)
                    : u32x4{0u, 0u, 0u, 0u};
  const float cq = a.c2 * a.sq[wg];

  int cnt = a.kept_cnt[wg];
  cnt = cnt < 0 ? 0 : (cnt > a.nkb ? a.nkb : cnt);
  const int32_t* lst = a.kept_idx + (size_t)wg * a.nkb;
  uint32_t* skip_out =
      a.skip_bits ? a.skip_bits + ((size_t)wg * 4 + w) * a.skip_words : nullptr;

  f32x16 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
  float m = -INFINITY, l = 0.f;
  uint32_t skip_word = 0;

  StagerQ st;
  auto valid_block = [&](int j) { return (unsigned)j < (unsigned)a.nkb ? j : -1; };
  if (cnt > 0) {
    const int j0 = valid_block(lst[0]);
    if (j0 >= 0) {
      st.load(kc, vt, j0, a.N, tid);
      st.store(smem, tid);
    }
  }
  __syncthreads();

  for (int t = 0; t < cnt; ++t) {
    const int j = valid_block(lst[t]);
    const char* stage = smem + (t & 1) * STAGE;
    if (t + 1 < cnt) {
      const int jn = valid_block(lst[t + 1]);
      if (jn >= 0) st.load(kc, vt, jn, a.N, tid);
    }
    const int key0 = j >= 0 ? j * 64 : a.N;  // an invalid entry is an empty tile
    const float csc = j >= 0 ? cq * a.sk[(size_t)bh * a.nkb + j] : 0.f;
    const float vsc = j >= 0 ? a.sv[(size_t)bh * a.nkb + j] * (1.0f / 256.0f) : 0.f;

    f32x16 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      i32x16 si;
#pragma unroll
      for (int r = 0; r < 16; ++r) si[r] = 0;
      const char* krow = stage + (32 * kt + l32) * KS + 16 * hh;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const u32x4 kv = *reinterpret_cast<const u32x4*>(krow + 32 * kk);
        si = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, kv),
                                                   __builtin_bit_cast(i32x4, qf[kk]), si, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kt][r] = (float)si[r];
    }

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
    // logits in log2 units: s * (sm log2e sq sk); max taken on scaled values
    float mloc = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[kt][r] *= csc;
        mloc = fmaxf(mloc, s[kt][r]);
      }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    const float mnew = fmaxf(m, mloc);
    bool do_pv = true;
    if (!a.lam_off) do_pv = __any((mloc != -INFINITY) && (mloc - mnew >= a.lam2));
    const float alpha = (mnew == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m - mnew);
    const float negm = (mnew == -INFINITY) ? 0.f : -mnew;
    float psum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(s[kt][r] + negm);
        s[kt][r] = p;
        psum += p;
      }
    l = alpha * l + psum;
    m = mnew;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
    }

    if (do_pv) {
      // P codes: chunk c holds p[kt][8 half + e], e in [0, 8), as e4m3(256 p)
      uint64_t pc[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int kt = c >> 1, half = c & 1;
        float pp[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pp[e] = s[kt][8 * half + e];
        int lo = __builtin_amdgcn_cvt_pk_fp8_f32(pp[0] * 256.f, pp[1] * 256.f, 0, false);
        lo = __builtin_amdgcn_cvt_pk_fp8_f32(pp[2] * 256.f, pp[3] * 256.f, lo, true);
        int hi = __builtin_amdgcn_cvt_pk_fp8_f32(pp[4] * 256.f, pp[5] * 256.f, 0, false);
        hi = __builtin_amdgcn_cvt_pk_fp8_f32(pp[6] * 256.f, pp[7] * 256.f, hi, true);
        pc[c] = (uint64_t)(uint32_t)lo | ((uint64_t)(uint32_t)hi << 32);
      }
      const char* vst = stage + KBYTES;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        f32x16 tmp;
#pragma unroll
        for (int r = 0; r < 16; ++r) tmp[r] = 0.f;
        const char* vr = vst + (32 * dt + l32) * VS + 4 * hh;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int kb = 16 * c;  // = 32 kt + 16 half
          const uint32_t v0 = *reinterpret_cast<const uint32_t*>(vr + kb);
          const uint32_t v1 = *reinterpret_cast<const uint32_t*>(vr + kb + 8);
          const uint64_t va = (uint64_t)v0 | ((uint64_t)v1 << 32);
          tmp = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8((long)va, (long)pc[c], tmp, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] = fmaf(vsc, tmp[r], acc[dt][r]);
      }
    }

    if (skip_out) {
      skip_word |= (do_pv ? 0u : 1u) << (t & 31);
      if ((t & 31) == 31 || t + 1 == cnt) {
        if (lane == 0) skip_out[t >> 5] = skip_word;
        skip_word = 0;
      }
    }
    if (t + 1 < cnt) st.store(smem + ((t + 1) & 1) * STAGE, tid);
    __syncthreads();
  }

  l += __shfl_xor(l, 32, 64);
  if (qvalid) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int oe = a.o_fp32 ? 4 : 2;
    char* orow = static_cast<char*>(a.o) +
                 ((int64_t)b * a.sb + (int64_t)h * a.sh + (int64_t)qrow * a.sn) * oe;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
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
    if (a.lse && hh == 0)
      a.lse[(int64_t)bh * a.N + qrow] = l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_quant(const ForwardLaunch& f, hipStream_t s) {
  const Geometry& g = f.g;
  const int64_t blocks = (int64_t)g.B * g.H * (g.nqb + 2 * g.nkb);
  hipLaunchKernelGGL(quant_kernel, dim3((unsigned)blocks), dim3(256), 0, s, f);
  return hipGetLastError();
}

hipError_t launch_attn_q(const ForwardLaunch& f, hipStream_t s) {
  const Geometry& g = f.g;
  AttnQArgs a;
  a.qc = f.qc;
  a.kc = f.kc;
  a.vt = f.vt;
  a.sq = f.sq;
  a.sk = f.sk;
  a.sv = f.sv;
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
    hipLaunchKernelGGL((attn_q_kernel<true>), dim3(a.nwg), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((attn_q_kernel<false>), dim3(a.nwg), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace sa
