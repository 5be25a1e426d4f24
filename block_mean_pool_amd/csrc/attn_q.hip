// Quantised stage two: INT8 Q.K^T and FP8 (OCP e4m3) P.V.
//
// The SpargeAttn abstract calls the method sparse *and quantized*; the
// DynSparse story notes the filter combines with quantization.  The pages fix
// no format, so this follows the stated reading:
//   Q, K: one scale per (b, h, block) = block absmax / qmax (1 if zero),
//         code = rint(x / scale) clamped to [-qmax, qmax] (fp32 division);
//         qmax = 127 (INT8), or 7 for 4-bit codes (the PARO abstract on the
//         search page reports INT4 attention after token reordering; gfx950
//         has no INT4 MFMA, so 4-bit codes run on the INT8 one);
//   V:    one scale per key block = absmax / 448, code = e4m3(x / scale);
//         or (the power-of-two variant) 2^e with e the smallest integer such
//         that absmax <= 448 * 2^e, the E8M0 block scale of the OCP
//         microscaling formats, which the scaled MFMA applies in hardware;
//   P:    e4m3(2^8 p), the product rescaled by scale_v * 2^-8; the running
//         sum l uses the unquantised p.
//
// quant_kernel: one workgroup per Q block, K block or V block; the block is
// read once into registers, its absmax reduced, and its codes written.  V
// codes are written per key block transposed ([D][64] bytes) through LDS, so
// the attention kernel stages V^T with plain 16-byte copies.  Both kernels
// take the head dimension D (64 or 128) as a template parameter.
// attn_q_kernel: the same tiling, online softmax and per-wavefront lambda
// test as the bf16 kernel, with v_mfma_i32_32x32x32_i8 for S^T = K Q^T and
// v_mfma_f32_32x32x64_f8f6f4 (e4m3 x e4m3) for O^T += V^T P^T.
#include <type_traits>

#include "attn_common.h"

namespace sa {
namespace {

__device__ __forceinline__ float block_max(float v, float* scratch) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) scratch[w] = v;
  __syncthreads();
  return fmaxf(fmaxf(scratch[0], scratch[1]), fmaxf(scratch[2], scratch[3]));
}

// Q: 128-row blocks, K and V: 64-row blocks.  A row of D bf16 is CPR = D / 8
// chunks of 16 B; thread -> chunk tid % CPR, rows tid / CPR + RPI * it.
template <int D>
__global__ __launch_bounds__(256) void quant_kernel(ForwardLaunch f) {
  constexpr int CPR = D / 8;       // 16-byte chunks per row
  constexpr int RPI = 256 / CPR;   // rows per pass of the workgroup
  constexpr int NIT = 128 / RPI;   // passes over a query block
  __shared__ float scratch[4];
  __shared__ __align__(16) uint8_t vt_tile[D * 64];
  const Geometry& g = f.g;
  const int tid = threadIdx.x;
  const int c = tid % CPR, ro = tid / CPR;
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

  u32x4 buf[NIT];
  float amax = 0.f;
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int r = r0 + ro + RPI * it;
    buf[it] = u32x4{0u, 0u, 0u, 0u};
    if (r < r1) buf[it] = *reinterpret_cast<const u32x4*>(src + (int64_t)r * g.sn + c * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(buf[it][e])), fabsf(bf16_hi(buf[it][e]))));
  }
  amax = block_max(amax, scratch);

  if (kind < 2) {
    const float qm = (float)f.qmax;
    const float scale = amax > 0.f ? __fdiv_rn(amax, qm) : 1.0f;
    int8_t* dst = (kind == 0 ? f.qc : f.kc) + (size_t)bh * g.N * D;
    if (tid == 0) (kind == 0 ? f.sq : f.sk)[bh * (kind == 0 ? g.nqb : g.nkb) + blk] = scale;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int r = r0 + ro + RPI * it;
      if (r < r1) {
        uint32_t packed[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t w = buf[it][e >> 1];
          const float x = (e & 1) ? bf16_hi(w) : bf16_lo(w);
          float qv = rintf(__fdiv_rn(x, scale));
          qv = fminf(fmaxf(qv, -qm), qm);
          packed[e >> 2] |= ((uint32_t)(int)qv & 0xffu) << (8 * (e & 3));
        }
        *reinterpret_cast<u32x2*>(dst + (int64_t)r * D + c * 8) = u32x2{packed[0], packed[1]};
      }
    }
  } else {
    float scale = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
    if (f.v_pow2) {
      // amax = fr 2^E with fr in [0.5, 1); 448 = 0.875 * 2^9: the smallest
      // 2^e with amax <= 448 * 2^e is 2^(E - 9) if fr <= 0.875, else 2^(E - 8)
      int E = 0;
      const float fr = frexpf(amax, &E);
      scale = amax > 0.f ? ldexpf(1.0f, fr <= 0.875f ? E - 9 : E - 8) : 1.0f;
    }
    if (tid == 0) f.sv[bh * g.nkb + blk] = scale;
    // rows ro + RPI it (it < 64 / RPI) of this key block; transposed into
    // LDS, key k = 32 t + 8 g + 4 h + e at position 32 h + 16 t + 4 g + e: the
    // order of a 32x32 MFMA accumulator lane's keys, so that a lane's 32 P
    // codes and the 32 V codes it multiplies are both contiguous
#pragma unroll
    for (int it = 0; it < 64 / RPI; ++it) {
      const int rr = ro + RPI * it;  // key within block
      const int pos = 32 * ((rr >> 2) & 1) + 16 * (rr >> 5) + 4 * ((rr >> 3) & 3) + (rr & 3);
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const uint32_t w = buf[it][e >> 1];
        const float x0 = __fdiv_rn(bf16_lo(w), scale);
        const float x1 = __fdiv_rn(bf16_hi(w), scale);
        const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
        vt_tile[(c * 8 + e) * 64 + pos] = (uint8_t)(pk & 0xff);
        vt_tile[(c * 8 + e + 1) * 64 + pos] = (uint8_t)((pk >> 8) & 0xff);
      }
    }
    __syncthreads();
    uint8_t* dst = f.vt + ((size_t)bh * g.nkb + blk) * D * 64;
    // a D x 64-byte tile = D * 4 chunks of 16 B, D / 64 per thread
#pragma unroll
    for (int s = 0; s < D / 64; ++s) {
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
  int recall_on;  // recall skip rule instead of lambda
  float omr;      // 1 - recall
  int G;          // rows per skip group: 16, 32, 64 or 128
};

typedef __attribute__((address_space(3))) void lds_void_q;
typedef int i32x8 __attribute__((ext_vector_type(8)));

// Stage two in INT8 / FP8, software-pipelined like the bf16 kernel
// (attn_pipe.hip): K codes (64 rows x 128 B) and V^T codes (128 rows x 64 B)
// are DMA'd global -> LDS in two stages each, 16-byte chunks XOR-permuted
// per row so that the operand reads are free of bank conflicts; iteration t
// holds, in one region, the FP8 P.V MFMAs of tile t-1, the INT8 Q.K^T MFMAs
// of tile t+1 and the softmax of tile t.  Unlike the bf16 kernel the
// exponent offset is the exact running max m (P codes are e4m3(2^8 P) with
// P <= 1, as the reading fixes), so acc is rescaled whenever m grows.  The
// factor 2^8 is folded into the exponent and into l: O = acc / l and lse are
// unchanged.  P.V uses v_mfma_f32_32x32x64_f8f6f4 (all 64 keys of a tile in
// one MFMA per 32 d-rows); each tile's product is added as acc += s_v * tmp.
//
// PM (precision mode): 0 = absmax / 448 V scales; 1 and 2 = power-of-two V
// scales, applied by the scaled MFMA, which then accumulates into acc
// directly; these modes normalise O by the sum of the quantised weights (the
// mode's reading), summed by one more scaled MFMA per tile with an all-ones
// operand instead of 31 adds per lane.  Mode 2 (the recall rule) still sums
// the unquantised weights on the VALU for the rule's energies.
// Two workgroups per CU at d = 128, three at d = 64 (168 VGPRs; the
// power-of-two mode spills a few registers there and still runs 12 % faster
// than at two, the absmax mode as fast).
template <int D, bool CAUSAL, int GM, int PM>
__global__ __launch_bounds__(256, D == 64 ? 3 : 2) void attn_q_kernel(AttnQArgs a) {
  constexpr bool VP2 = PM != 0, ROWSUM_VALU = PM != 1;
  // 32-wide d chunks: the K extent of one INT8 Q.K^T MFMA, and the d rows of
  // one FP8 P.V MFMA; a region of four chunks issues the MFMAs of one d chunk
  // every CSTEP chunks (every chunk at D = 128, every other one at D = 64)
  constexpr int NKK = D / 32, CSTEP = 4 / NKK;
  constexpr int NI = 64 * D / 4096;  // DMA instructions per tile and wavefront
  // skip groups: SPLIT = halves of a wavefront (G = 16); DEFER = several
  // wavefronts (G = 64, 128), final after the barrier that follows the votes
  constexpr bool SPLIT = GM == attn::kGroupHalf, DEFER = GM == attn::kGroupMulti;
  constexpr int TK = 64 * D;  // K codes of a tile, D * 64 bytes
  constexpr int TV = D * 64;  // V^T codes of a tile, D * 64 bytes
  __shared__ __align__(16) char k0[TK];
  __shared__ __align__(16) char k1[TK];
  __shared__ __align__(16) char v0[TV];
  __shared__ __align__(16) char v1[TV];
  // per tile parity and wavefront: 1 if the wavefront needs the tile's P.V;
  // groups of G > 32 rows OR their wavefronts' votes, published before the
  // barrier that ends the step
  __shared__ __align__(16) uint32_t vote[2][4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const attn::QueryBlock qblk = attn::query_block(a.nwg, a.nqb, CAUSAL);
  const int wg = qblk.row;  // the query block's row in the mask arrays
  const int bh = qblk.bh;
  const int i = qblk.i;
  const int b = bh / a.H, h = bh - b * a.H;
  const int wrow0 = i * 128 + 32 * w;
  const int qrow = wrow0 + l32;
  const bool qvalid = qrow < a.N;
  const bool wave_partial = wrow0 + 32 > a.N;
  const int8_t* qc = a.qc + (size_t)bh * a.N * D;

  u32x4 qf[NKK];  // Q codes, d = 32 kk + 16 hh + [0, 16) of row qrow
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk)
    qf[kk] = qvalid ? *reinterpret_cast<const u32x4*>(qc + (int64_t)qrow * D + 32 * kk + 16 * hh)
                    : u32x4{0u, 0u, 0u, 0u};
  const float cq = a.c2 * a.sq[wg];
  const float* skp = a.sk + (size_t)bh * a.nkb;
  const float* svp = a.sv + (size_t)bh * a.nkb;

  int cnt = a.kept_cnt[wg];
  cnt = cnt < 0 ? 0 : (cnt > a.nkb ? a.nkb : cnt);
  const int32_t* lst = a.kept_idx + (size_t)wg * a.nkb;
  int wbase = 0;
  int win = lane < cnt ? lst[lane] : 0;
  int nxt = 64 + lane < cnt ? lst[64 + lane] : 0;
  // block of entry e (< wbase + 64), or nkb (an empty tile) past the list
  auto entry_blk = [&](int e) {
    if (e >= cnt) return a.nkb;
    const int j = __builtin_amdgcn_readlane(win, e - wbase);
    return (unsigned)j < (unsigned)a.nkb ? j : a.nkb;
  };
  attn::SkipOut<SPLIT> skip_out;
  skip_out.init(a.skip_bits, wg, w, a.G, a.skip_words);

  // K codes of the head: rows >= N read as zero; V^T codes: block nkb (an
  // empty tile) reads as zero
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(a.kc + (size_t)bh * a.N * D), (short)0, (int)(a.N * D), 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.vt + (size_t)bh * a.nkb * TV), (short)0, (int)(a.nkb * TV),
      0x00020000);

  // DMA: wave-instruction n (< NI) of wave w fills bytes [(4 n + w) KiB,
  // +1 KiB) of a tile, lane e 16 bytes at e * 16.  K: LDS row r (D bytes),
  // position p holds global chunk p ^ swk(r), swk(r) = (r >> 1) & 7 at
  // D = 128 and (r >> 2) & 3 at D = 64, so that the 16 rows a K operand read
  // touches at one chunk index fall on distinct banks; V^T: LDS row d (64 B),
  // position p holds chunk p ^ swv(d), swv(d) = (d >> 2) & 3.  Instruction n
  // is 32 K rows / 64 V rows further on, which leaves both permutations
  // unchanged.
  auto swk = [](int r) { return D == 128 ? (r >> 1) & 7 : (r >> 2) & 3; };
  auto swv = [](int d) { return (d >> 2) & 3; };
  uint32_t dk0, dv0;
  {
    const int pos = w * 1024 + lane * 16;
    const int r = pos >> (D == 128 ? 7 : 6), pk = (pos & (D - 1)) >> 4;
    dk0 = (uint32_t)(r * D + ((pk ^ swk(r)) << 4));
    const int d = pos >> 6, pv = (pos & 63) >> 4;
    dv0 = (uint32_t)(d * 64 + ((pv ^ swv(d)) << 4));
  }
  // LDS read bases: K row l32 (+32 kt), chunk 2 kk + hh; V^T row l32
  // (+32 dt), chunks 2 hh and 2 hh + 1
  uint32_t kro[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk)
    kro[kk] = (uint32_t)(l32 * D + (((2 * kk + hh) ^ swk(l32)) << 4));
  const uint32_t vro0 = (uint32_t)(l32 * 64 + (((2 * hh) ^ swv(l32)) << 4));
  const uint32_t vro1 = (uint32_t)(l32 * 64 + (((2 * hh + 1) ^ swv(l32)) << 4));

  // K(blk) into kdst, V(vblk) into vdst (a block index of nkb is an empty
  // tile and reads as zero)
  auto dma = [&](char* kdst, int blk, char* vdst, int vblk) {
    const uint32_t kb = (uint32_t)blk * 64u * D + dk0;
    const uint32_t vb = (uint32_t)vblk * TV + dv0;
#pragma unroll
    for (int n = 0; n < NI; ++n) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void_q*)(kdst + (4 * n + w) * 1024), 16,
                                               kb + n * 4096, 0, 0, 0);
      if (vdst)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void_q*)(vdst + (4 * n + w) * 1024),
                                                 16, vb + n * 4096, 0, 0, 0);
    }
  };
  auto qk_mfma = [&](const char* kbuf, int kt, int kk, i32x16 acc_s) {
    const u32x4 kv = *reinterpret_cast<const u32x4*>(kbuf + kro[kk] + 32 * kt * D);
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, kv),
                                                 __builtin_bit_cast(i32x4, qf[kk]), acc_s, 0, 0, 0);
  };
  // VP2 (power-of-two V scales): the MFMA applies the V scale (E8M0 = the
  // fp32 exponent field of 2^e) and accumulates into acc directly
  auto pv_mfma_acc = [&](const char* vbuf, int dt, const i32x8& pb, f32x16 acc_o,
                         int vexp) {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(vbuf + vro0 + 32 * dt * 64);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(vbuf + vro1 + 32 * dt * 64);
    const i32x8 va{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                   (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pb, acc_o, 0, 0, 0, vexp, 0, 127);
  };
  auto pv_mfma = [&](const char* vbuf, int dt, const i32x8& pb) {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(vbuf + vro0 + 32 * dt * 64);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(vbuf + vro1 + 32 * dt * 64);
    const i32x8 va{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                   (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    f32x16 z;
#pragma unroll
    for (int r = 0; r < 16; ++r) z[r] = 0.f;
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pb, z, 0, 0, 0, 0, 0, 0);
  };

  f32x16 acc[NKK];
#pragma unroll
  for (int dt = 0; dt < NKK; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
  i32x16 sA[2], sB[2];
  i32x8 pf;  // e4m3(2^8 P) of the previous tile, byte j = key 32 kt + ... (S^T order)
#pragma unroll
  for (int e = 0; e < 8; ++e) pf[e] = 0;
  float m = -INFINITY, l = 0.f, rescale = 1.f, vsc_prev = 0.f;
  int vexp_prev = 0;  // VP2: E8M0 of the previous tile's V scale
  f32x16 lacc;        // VP2: running sum of the quantised weights (every row alike)
#pragma unroll
  for (int r = 0; r < 16; ++r) lacc[r] = 0.f;
  i32x8 ones;  // e4m3 1.0 in every byte: the all-ones operand of the row sums
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = 0x38383838;
  float drop = 0.f;  // recall rule: energy the row has dropped, same scale as l
  bool pv_prev = false;
  float pend_E = 0.f;  // recall rule, G > 32: the row's energy in the tile awaiting its vote
  // the final decision on entry tt (for G = 16 with a half split): dropped
  // energy (recall rule), zero P codes of a skipping half wavefront, skip
  // bits, and whether the next step multiplies the tile's P.V
  auto finish = [&](int tt, bool nd, uint32_t split, float E) {
    if constexpr (SPLIT) {
      const bool keep = split ? attn::split_keeps(split, l32) : nd;
      if (a.recall_on && !keep) drop += E;
      if (split) {
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[e] = keep ? pf[e] : 0;
      }
    } else {
      if (a.recall_on && !nd) drop += E;
    }
    skip_out.put(tt, cnt, nd, split, lane);
    pv_prev = nd;
  };

  int jq0 = entry_blk(0), jq1 = entry_blk(1);  // blocks of entries t, t + 1

  // prologue: K of entries 0 and 1, S of entry 0
  dma(k0, jq0, nullptr, 0);
  dma(k1, jq1, nullptr, 0);
  __syncthreads();
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) sA[kt][r] = 0;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) sA[kt] = qk_mfma(k0, kt, kk, sA[kt]);
  }
  __syncthreads();

  auto step = [&](auto ph, int t, i32x16(&sc)[2], i32x16(&sn)[2]) {
    constexpr int PH = decltype(ph)::value;
    char* k_next = PH ? k0 : k1;  // K of entry t + 1
    char* k_free = PH ? k1 : k0;  // K of entry t (read) -> entry t + 2
    char* v_prev = PH ? v0 : v1;  // V of entry t - 1
    char* v_free = PH ? v1 : v0;  // V of entry t - 2 (read) -> entry t

    if (t + 2 - wbase >= 64) {
      win = nxt;
      wbase += 64;
      nxt = wbase + 64 + lane < cnt ? lst[wbase + 64 + lane] : 0;
    }
    const int j_far = entry_blk(t + 2);
    // K(t+2) into the stage of K(t); V(t) into the stage of V(t-2)
    dma(k_free, j_far, v_free, jq0);
    if constexpr (DEFER) {
      if (t > 0) finish(t - 1, attn::group_need(vote[(t - 1) & 1], w, a.G), 0u, pend_E);
    }
    const int j_cur = jq0;
    const int key_cur = j_cur < a.nkb ? j_cur * 64 : a.N;
    const float csc = j_cur < a.nkb ? cq * skp[j_cur] : 0.f;
    const float vsc = j_cur < a.nkb ? svp[j_cur] : 0.f;
    const int vexp = (int)(__float_as_uint(vsc) >> 23);  // VP2: 2^e -> e + 127

    if (__any(rescale != 1.f)) {  // m grew at t - 1
#pragma unroll
      for (int dt = 0; dt < NKK; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] *= rescale;
      rescale = 1.f;
    }

    // integer scores Q~.K~ of tile t (exact in fp32: |Q~.K~| < 2^22); masked -inf
    f32x16 x[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) x[kt][r] = (float)sc[kt][r];
    const bool need_mask =
        (key_cur + 64 > a.N) || wave_partial || (CAUSAL && key_cur + 63 > wrow0);
    // a select per score, not a branch: this file is built with SimplifyCFG's
    // sinking and hoisting off, which would leave `if (!ok)` as one branch per
    // score (a third more code)
    if (need_mask) attn::mask_scores<CAUSAL>(x, key_cur, a.N, hh, qrow, qvalid);
    float xmax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) xmax = fmaxf(xmax, x[kt][r]);
    xmax = attn::xhalf_max(xmax);
    // logits in log2 units: csc * x, csc = sm log2(e) sq sk > 0
    const float mloc = xmax * csc;
    const float mnew = fmaxf(m, mloc);
    bool do_pv = true;
    uint32_t split = 0u;  // G = 16: the halves of the wavefront decide apart
    if (!a.lam_off) {
      const bool nl = (mloc != -INFINITY) && (mloc - mnew >= a.lam2);
      do_pv = attn::wave_need(nl);
      if constexpr (SPLIT) split = attn::half_split(nl);
    }
    if (mnew != m) {
      const float f = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - mnew);
      l *= f;
      drop *= f;
      rescale = f;
      m = mnew;
      if constexpr (VP2) {
#pragma unroll
        for (int r = 0; r < 16; ++r) lacc[r] *= f;
      }
    }
    // 2^8 P = exp2(csc * x + cb), cb = 8 - m
    const float cb = (m == -INFINITY) ? 0.f : 8.f - m;

    i32x8 pn;
    float psum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) sn[kt][r] = 0;
    // chunk c: softmax of this lane's scores 8c .. 8c+7; and, for c a
    // multiple of CSTEP (u = c / CSTEP), P.V of tile t-1 for d rows
    // 32u..32u+31 and Q.K^T of tile t+1 for kk = u (both key halves)
    auto chunk_pv = [&](int u) {  // d rows 32 u .. 32 u + 31
      if constexpr (VP2) {
        acc[u] = pv_mfma_acc(v_prev, u, pf, acc[u], vexp_prev);
      } else {
        const f32x16 tmp = pv_mfma(v_prev, u, pf);
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[u][r] = fmaf(vsc_prev, tmp[r], acc[u][r]);
      }
    };
    auto chunk_qk = [&](int u) {  // d chunk kk = u
      sn[0] = qk_mfma(k_next, 0, u, sn[0]);
      sn[1] = qk_mfma(k_next, 1, u, sn[1]);
    };
    auto chunk_soft = [&](int c) {
      const int kt = c >> 1, r0 = 8 * (c & 1);
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(x[kt][r0 + e], csc, cb));
      if constexpr (ROWSUM_VALU)
        psum += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      // the first conversion of each word writes its low half; the second
      // overwrites the high half, so the word's old contents do not matter
      int lo, hi;  // defined by empty asm: no instruction, no zeroing move
      asm("" : "=v"(lo) : "v"(p[0]));
      asm("" : "=v"(hi) : "v"(p[4]));
      lo = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], lo, false);
      lo = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], lo, true);
      hi = __builtin_amdgcn_cvt_pk_fp8_f32(p[4], p[5], hi, false);
      hi = __builtin_amdgcn_cvt_pk_fp8_f32(p[6], p[7], hi, true);
      pn[2 * c] = lo;
      pn[2 * c + 1] = hi;
    };
    if (pv_prev) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (c % CSTEP == 0) {
          chunk_pv(c / CSTEP);
          chunk_qk(c / CSTEP);
        }
        chunk_soft(c);
      }
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (c % CSTEP == 0) chunk_qk(c / CSTEP);
        chunk_soft(c);
      }
    }
    l += psum;
    pf = pn;
    // VP2: the row sums of this tile's quantised weights (before a half
    // split zeroes any codes of pf: the skipped mass stays in the sum)
    if constexpr (VP2)
      lacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, pn, lacc, 0, 0, 0, 127, 0, 127);
    vsc_prev = vsc;
    vexp_prev = vexp;
    float E = 0.f;
    if (a.recall_on) {  // drop the tile if the rows' dropped share stays <= 1 - recall
      E = attn::xhalf_sum(psum);
      const bool nl = !(drop + E <= a.omr * attn::xhalf_sum(l));
      do_pv = attn::wave_need(nl);
      if constexpr (SPLIT) split = attn::half_split(nl);
    }
    if constexpr (DEFER) {
      if (lane == 0) vote[t & 1][w] = do_pv ? 1u : 0u;
      pend_E = E;
    } else {
      finish(t, do_pv, split, E);
    }
    jq0 = jq1;
    jq1 = j_far;
    __syncthreads();
  };

  int t = 0;
  for (; t + 2 <= cnt; t += 2) {
    step(std::integral_constant<int, 0>{}, t, sA, sB);
    step(std::integral_constant<int, 1>{}, t + 1, sB, sA);
  }
  if (t < cnt) step(std::integral_constant<int, 0>{}, t, sA, sB);

  if (cnt > 0) {
    if constexpr (DEFER)
      finish(cnt - 1, attn::group_need(vote[(cnt - 1) & 1], w, a.G), 0u, pend_E);
    if (__any(rescale != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < NKK; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] *= rescale;
    }
    if (pv_prev) {  // P.V of the last entry, V in stage (cnt - 1) % 2
      const char* vlast = ((cnt - 1) & 1) ? v1 : v0;
#pragma unroll
      for (int dt = 0; dt < NKK; ++dt) {
        if constexpr (VP2) {
          acc[dt] = pv_mfma_acc(vlast, dt, pf, acc[dt], vexp_prev);
        } else {
          const f32x16 tmp = pv_mfma(vlast, dt, pf);
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[dt][r] = fmaf(vsc_prev, tmp[r], acc[dt][r]);
        }
      }
    }
  }

  // epilogue: O = acc / l (both carry the factor 2^8); lse = (m + log2 l - 8) ln 2;
  // VP2 normalises by the quantised weights' sum (each lane holds its row's)
  l = VP2 ? lacc[0] : attn::xhalf_sum(l);
  if (qvalid) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int oe = a.o_fp32 ? 4 : 2;
    char* orow = static_cast<char*>(a.o) +
                 ((int64_t)b * a.sb + (int64_t)h * a.sh + (int64_t)qrow * a.sn) * oe;
#pragma unroll
    for (int dt = 0; dt < NKK; ++dt)
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
      a.lse[(int64_t)bh * a.N + qrow] = l > 0.f ? (m + __log2f(l) - 8.f) * kLn2 : -INFINITY;
  }
}

template <int D, int GM, int PM>
void launch_q(const AttnQArgs& a, bool causal, hipStream_t s) {
  if (causal)
    hipLaunchKernelGGL((attn_q_kernel<D, true, GM, PM>), dim3(a.nwg), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((attn_q_kernel<D, false, GM, PM>), dim3(a.nwg), dim3(256), 0, s, a);
}

// precision mode: 0 absmax / 448 V scales; power-of-two V scales with the
// lambda rule (1) or the recall rule (2)
template <int D, int GM>
void launch_q(const AttnQArgs& a, bool causal, bool v_pow2, hipStream_t s) {
  if (!v_pow2) launch_q<D, GM, 0>(a, causal, s);
  else if (a.recall_on) launch_q<D, GM, 2>(a, causal, s);
  else launch_q<D, GM, 1>(a, causal, s);
}

template <int D>
void launch_q_d(const AttnQArgs& a, int group_rows, bool causal, bool v_pow2, hipStream_t s) {
  switch (attn::group_mode(group_rows)) {
    case attn::kGroupHalf: launch_q<D, attn::kGroupHalf>(a, causal, v_pow2, s); break;
    case attn::kGroupMulti: launch_q<D, attn::kGroupMulti>(a, causal, v_pow2, s); break;
    default: launch_q<D, attn::kGroupWave>(a, causal, v_pow2, s); break;
  }
}

}  // namespace

hipError_t launch_quant(const ForwardLaunch& f, hipStream_t s) {
  const Geometry& g = f.g;
  const int64_t blocks = (int64_t)g.B * g.H * (g.nqb + 2 * g.nkb);
  if (g.D == 128)
    hipLaunchKernelGGL(quant_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, s, f);
  else
    hipLaunchKernelGGL(quant_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, s, f);
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
  a.recall_on = f.recall_on;
  a.omr = 1.0f - f.recall;
  if (a.recall_on) a.lam_off = 1;
  a.G = f.group_rows;
  if (g.D == 128)
    launch_q_d<128>(a, f.group_rows, f.causal, f.v_pow2, s);
  else
    launch_q_d<64>(a, f.group_rows, f.causal, f.v_pow2, s);
  return hipGetLastError();
}

}  // namespace sa
