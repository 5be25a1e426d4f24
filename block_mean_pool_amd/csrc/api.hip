// Host side of the C ABI declared in include/sparse_attn.h: argument
// validation, workspace layout, launch of the gfx950 kernels on the caller's
// stream, and error reporting.  Nothing is enqueued unless every check
// passes; no exception crosses the ABI.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "sa_internal.h"
#include "../../include/sparse_attn.h"

// Scratch of sparse_attn_predict_noalloc: the predict workspace (the block
// means) for callers that cannot allocate device memory.  Each GPU the
// library runs on holds one copy for the life of the process.  Host code
// never passes this name to a kernel or a copy: on the host it is only a
// stand-in for the symbol, and each device's address comes from
// hipGetSymbolAddress (noalloc_scratch below).
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {

thread_local char g_err[512];

sa_status fail(sa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

sa_status ok() {
  g_err[0] = 0;
  return SA_OK;
}

constexpr size_t kAlign = 256;
constexpr int kDefaultGroupRows = 32;  // one wavefront's rows
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Validates the parameter block and fills the geometry.  `empty` is set for
// problems with B, H or N equal to zero.
sa_status check_params(const sa_params* p, sa::Geometry* g, bool* empty) {
  if (!p) return fail(SA_ERR_INVALID_ARG, "params is NULL");
  if (p->B < 0 || p->H < 0 || p->N < 0 || p->D <= 0)
    return fail(SA_ERR_INVALID_ARG, "negative shape (B=%d H=%d N=%d D=%d)", p->B, p->H, p->N, p->D);
  if (p->D != 64 && p->D != 128) return fail(SA_ERR_UNSUPPORTED, "D=%d (supported: 64, 128)", p->D);
  if (p->block_q != 128 || p->block_k != 64)
    return fail(SA_ERR_UNSUPPORTED, "block sizes %dx%d (supported: 128x64)", p->block_q, p->block_k);
  if (p->dtype != SA_F32 && p->dtype != SA_BF16) return fail(SA_ERR_INVALID_ARG, "dtype=%d", p->dtype);
  if (p->prec != SA_PREC_NATIVE && p->prec != SA_PREC_I8_FP8 && p->prec != SA_PREC_I4_FP8 &&
      p->prec != SA_PREC_I8_MXFP8)
    return fail(SA_ERR_INVALID_ARG, "prec=%d", p->prec);
  if (p->prec != SA_PREC_NATIVE && p->dtype != SA_BF16)
    return fail(SA_ERR_UNSUPPORTED, "INT8/INT4/FP8 variants need bf16 inputs");
  if (p->rule != SA_RULE_TOPCDF && p->rule != SA_RULE_ENERGY && p->rule != SA_RULE_TOPK)
    return fail(SA_ERR_INVALID_ARG, "rule=%d", p->rule);
  if (p->rule == SA_RULE_TOPK && p->topk_blocks < 1)
    return fail(SA_ERR_INVALID_ARG, "topk_blocks=%d (must be >= 1)", p->topk_blocks);
  if (p->causal != 0 && p->causal != 1) return fail(SA_ERR_INVALID_ARG, "causal=%d", p->causal);
  if (!(p->tau > 0.f) || std::isnan(p->tau))
    return fail(SA_ERR_INVALID_ARG, "tau=%g (must be in (0, 1]; >= 1 keeps all)", (double)p->tau);
  if (std::isnan(p->lambda)) return fail(SA_ERR_INVALID_ARG, "lambda is NaN");
  if (p->skip_rule != SA_SKIP_LAMBDA && p->skip_rule != SA_SKIP_RECALL)
    return fail(SA_ERR_INVALID_ARG, "skip_rule=%d", p->skip_rule);
  if (p->skip_rule == SA_SKIP_RECALL && !(p->recall > 0.f && p->recall <= 1.f))
    return fail(SA_ERR_INVALID_ARG, "recall=%g (must be in (0, 1])", (double)p->recall);
  if (!(p->sm_scale >= 0.f) || std::isinf(p->sm_scale))
    return fail(SA_ERR_INVALID_ARG, "sm_scale=%g", (double)p->sm_scale);
  if (p->keep_prefix_kblocks < 0) return fail(SA_ERR_INVALID_ARG, "keep_prefix_kblocks < 0");
  if (p->lambda_group_rows != 0 && p->lambda_group_rows != 16 && p->lambda_group_rows != 32 &&
      p->lambda_group_rows != 64 && p->lambda_group_rows != 128)
    return fail(SA_ERR_UNSUPPORTED, "lambda_group_rows=%d (supported: 16, 32, 64, 128)",
                p->lambda_group_rows);
  if (p->N > 262144) return fail(SA_ERR_UNSUPPORTED, "N=%d > 262144", p->N);
  if (p->o_fp32 != 0 && p->o_fp32 != 1) return fail(SA_ERR_INVALID_ARG, "o_fp32=%d", p->o_fp32);
  const int64_t esz = p->dtype == SA_BF16 ? 2 : 4;
  g->B = p->B;
  g->H = p->H;
  g->N = p->N;
  g->D = p->D;
  g->nqb = (p->N + 127) / 128;
  g->nkb = (p->N + 63) / 64;
  g->dtype = p->dtype;
  g->sn = p->stride_n ? p->stride_n : p->D;
  g->sh = p->stride_h ? p->stride_h : (int64_t)p->N * g->sn;
  g->sb = p->stride_b ? p->stride_b : (int64_t)p->H * g->sh;
  if (g->sn < p->D || g->sh < 0 || g->sb < 0)
    return fail(SA_ERR_INVALID_ARG, "strides (b=%lld h=%lld n=%lld) do not fit D=%d",
                (long long)g->sb, (long long)g->sh, (long long)g->sn, p->D);
  if ((g->sn * esz) % 16 || (g->sh * esz) % 16 || (g->sb * esz) % 16)
    return fail(SA_ERR_INVALID_ARG, "strides must keep rows 16-byte aligned");
  if ((int64_t)(p->N + 64) * g->sn * esz >= (1LL << 31))
    return fail(SA_ERR_UNSUPPORTED, "one head spans >= 2 GiB (N=%d, stride_n=%lld)", p->N,
                (long long)g->sn);
  *empty = p->B == 0 || p->H == 0 || p->N == 0;
  const int64_t wgs = (int64_t)p->B * p->H * (g->nqb + g->nkb);
  if (wgs > 0x7fffffffLL) return fail(SA_ERR_UNSUPPORTED, "problem too large for one grid");
  return SA_OK;
}

struct PredictLayout {
  size_t qbar, kbar, total;
};
PredictLayout predict_layout(const sa::Geometry& g) {
  PredictLayout L;
  L.qbar = 0;
  L.kbar = round_up((size_t)g.B * g.H * g.nqb * g.D * sizeof(float));
  L.total = L.kbar + round_up((size_t)g.B * g.H * g.nkb * g.D * sizeof(float));
  return L;
}

struct ForwardLayout {
  size_t qc, kc, vt, sq, sk, sv, total;
};
ForwardLayout forward_layout(const sa::Geometry& g, int prec) {
  ForwardLayout L{};
  if (prec == SA_PREC_NATIVE) return L;
  const size_t bh = (size_t)g.B * g.H;
  L.qc = 0;
  L.kc = L.qc + round_up(bh * g.N * g.D);
  L.vt = L.kc + round_up(bh * g.N * g.D);
  L.sq = L.vt + round_up(bh * g.nkb * g.D * 64);
  L.sk = L.sq + round_up(bh * g.nqb * sizeof(float));
  L.sv = L.sk + round_up(bh * g.nkb * sizeof(float));
  L.total = L.sv + round_up(bh * g.nkb * sizeof(float));
  return L;
}

float softmax_scale(const sa_params* p) {
  return p->sm_scale > 0.f ? p->sm_scale : 1.0f / sqrtf((float)p->D);
}

}  // namespace

extern "C" {

sa_status sparse_attn_mask_shape(const sa_params* p, int64_t* nqb, int64_t* nkb) {
  sa::Geometry g;
  bool empty;
  sa_status st = check_params(p, &g, &empty);
  if (st) return st;
  if (nqb) *nqb = g.nqb;
  if (nkb) *nkb = g.nkb;
  return ok();
}

sa_status sparse_attn_workspace_size(const sa_params* p, size_t* predict_ws, size_t* forward_ws) {
  sa::Geometry g;
  bool empty;
  sa_status st = check_params(p, &g, &empty);
  if (st) return st;
  if (predict_ws) *predict_ws = empty ? 0 : predict_layout(g).total;
  if (forward_ws) *forward_ws = empty ? 0 : forward_layout(g, p->prec).total;
  return ok();
}

}  // extern "C"

namespace {

// The mask rules of sparse_attn_check_mask, on host copies of the mask.
sa_status check_mask_host(const sa::Geometry& g, const sa_params* p, const int32_t* idx,
                          const int32_t* cnt, int64_t* bad_row) {
  std::vector<uint8_t> seen(g.nkb);
  const int64_t rows = (int64_t)g.B * g.H * g.nqb;
  for (int64_t row = 0; row < rows; ++row) {
    const int i = (int)(row % g.nqb);
    const int first_row = i * 128, last_row = std::min(g.N, first_row + 128) - 1;
    // admissible key blocks: all, or (causal) those whose first key <= last_row
    const int n_adm = p->causal ? last_row / 64 + 1 : g.nkb;
    auto forced = [&](int j) {
      const int last_key = std::min(g.N, j * 64 + 64) - 1;
      return j < p->keep_prefix_kblocks || (p->causal && last_key >= first_row);
    };
    int n_forced = 0;
    for (int j = 0; j < n_adm; ++j) n_forced += forced(j);
    if (bad_row) *bad_row = row;
    const int c = cnt[row];
    if (c < std::max(1, n_forced) || c > n_adm)
      return fail(SA_ERR_INVALID_ARG, "mask row %lld: kept_cnt %d outside [%d, %d]",
                  (long long)row, c, std::max(1, n_forced), n_adm);
    std::fill(seen.begin(), seen.end(), 0);
    const int32_t* lst = idx + row * g.nkb;
    for (int t = 0; t < c; ++t) {
      const int j = lst[t];
      if (j < 0 || j >= n_adm)
        return fail(SA_ERR_INVALID_ARG, "mask row %lld entry %d: key block %d not admissible",
                    (long long)row, t, j);
      if (seen[j]) return fail(SA_ERR_INVALID_ARG, "mask row %lld: key block %d repeated",
                               (long long)row, j);
      seen[j] = 1;
      if (forced(j) != (t < n_forced))
        return fail(SA_ERR_INVALID_ARG, "mask row %lld entry %d: the %d forced blocks do not "
                    "come first", (long long)row, t, n_forced);
    }
  }
  if (bad_row) *bad_row = -1;
  return SA_OK;
}

// Opt-in validation of the mask forward receives: with the environment
// variable SA_CHECK_MASK set to 1, forward copies the mask to the host (a
// synchronisation on the stream) and checks it before any launch.
bool check_mask_requested() {
  const char* e = std::getenv("SA_CHECK_MASK");
  return e && e[0] == '1';
}

// predict / forward with a dry-run mode that validates everything and
// enqueues nothing (so a composite call can check all of its parts first).
// pool_only: stage one's block means alone (no mask arguments).
sa_status predict_impl(const sa_params* p, const void* q, const void* k, const sa_mask* out,
                       void* ws, size_t ws_bytes, void* stream, bool dry,
                       bool pool_only = false) {
  sa::Geometry g;
  bool empty;
  sa_status st = check_params(p, &g, &empty);
  if (st) return st;
  if (empty) return ok();
  if (!q || !k) return fail(SA_ERR_INVALID_ARG, "q or k is NULL");
  if (!aligned16(q) || !aligned16(k)) return fail(SA_ERR_INVALID_ARG, "q/k not 16-byte aligned");
  if (!pool_only && (!out || !out->kept_idx || !out->kept_cnt))
    return fail(SA_ERR_INVALID_ARG, "mask output (kept_idx, kept_cnt) is NULL");
  const PredictLayout L = predict_layout(g);
  if (!ws || ws_bytes < L.total)
    return fail(SA_ERR_WORKSPACE, "predict workspace %zu < %zu bytes", ws_bytes, L.total);
  if (!aligned16(ws)) return fail(SA_ERR_INVALID_ARG, "workspace not 16-byte aligned");
  sa::PredictLaunch a;
  a.g = g;
  a.q = q;
  a.k = k;
  a.qbar = reinterpret_cast<float*>(static_cast<char*>(ws) + L.qbar);
  a.kbar = reinterpret_cast<float*>(static_cast<char*>(ws) + L.kbar);
  a.kept_idx = pool_only ? nullptr : out->kept_idx;
  a.kept_cnt = pool_only ? nullptr : out->kept_cnt;
  a.block_prob = pool_only ? nullptr : out->block_prob;
  a.causal = p->causal;
  a.rule = p->rule;
  a.keep_prefix = p->keep_prefix_kblocks;
  a.sm = softmax_scale(p);
  a.tau = p->tau;
  a.topk = p->rule == SA_RULE_TOPK ? p->topk_blocks : 0;
  if (dry) return ok();
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = sa::launch_pool(a, s);
  if (e != hipSuccess) return fail(SA_ERR_HIP, "pool launch: %s", hipGetErrorString(e));
  if (pool_only) return ok();
  e = sa::launch_mask(a, s);
  if (e != hipSuccess) return fail(SA_ERR_HIP, "mask launch: %s", hipGetErrorString(e));
  return ok();
}

sa_status forward_impl(const sa_params* p, const void* q, const void* k, const void* v,
                       const sa_mask* mask, void* o, float* lse, uint32_t* skip_bits, void* ws,
                       size_t ws_bytes, void* stream, bool dry) {
  sa::Geometry g;
  bool empty;
  sa_status st = check_params(p, &g, &empty);
  if (st) return st;
  if (empty) return ok();
  if (!q || !k || !v || !o) return fail(SA_ERR_INVALID_ARG, "q, k, v or o is NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(SA_ERR_INVALID_ARG, "q/k/v/o not 16-byte aligned");
  if (!mask || !mask->kept_idx || !mask->kept_cnt)
    return fail(SA_ERR_INVALID_ARG, "mask (kept_idx, kept_cnt) is NULL");
  const ForwardLayout L = forward_layout(g, p->prec);
  if (L.total && (!ws || ws_bytes < L.total))
    return fail(SA_ERR_WORKSPACE, "forward workspace %zu < %zu bytes", ws_bytes, L.total);
  if (L.total && !aligned16(ws)) return fail(SA_ERR_INVALID_ARG, "workspace not 16-byte aligned");
  sa::ForwardLaunch a{};
  a.g = g;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.skip_bits = skip_bits;
  a.kept_idx = mask->kept_idx;
  a.kept_cnt = mask->kept_cnt;
  a.causal = p->causal;
  a.sm = softmax_scale(p);
  a.lambda = p->lambda;
  a.recall_on = p->skip_rule == SA_SKIP_RECALL;
  a.recall = p->recall;
  a.group_rows = p->lambda_group_rows ? p->lambda_group_rows : kDefaultGroupRows;
  a.o_fp32 = p->o_fp32 || p->dtype == SA_F32;
  if (dry) return ok();
  if (check_mask_requested()) {
    const size_t rows = (size_t)g.B * g.H * g.nqb;
    std::vector<int32_t> hidx(rows * g.nkb), hcnt(rows);
    hipStream_t cs = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(hcnt.data(), mask->kept_cnt, rows * sizeof(int32_t),
                                  hipMemcpyDeviceToHost, cs);
    if (e == hipSuccess)
      e = hipMemcpyAsync(hidx.data(), mask->kept_idx, hidx.size() * sizeof(int32_t),
                         hipMemcpyDeviceToHost, cs);
    if (e == hipSuccess) e = hipStreamSynchronize(cs);
    if (e != hipSuccess) return fail(SA_ERR_HIP, "mask check copy: %s", hipGetErrorString(e));
    st = check_mask_host(g, p, hidx.data(), hcnt.data(), nullptr);
    if (st) return st;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (p->prec != SA_PREC_NATIVE) {
    a.qmax = p->prec == SA_PREC_I4_FP8 ? 7 : 127;
    a.v_pow2 = p->prec == SA_PREC_I8_MXFP8;
    char* w = static_cast<char*>(ws);
    a.qc = reinterpret_cast<int8_t*>(w + L.qc);
    a.kc = reinterpret_cast<int8_t*>(w + L.kc);
    a.vt = reinterpret_cast<uint8_t*>(w + L.vt);
    a.sq = reinterpret_cast<float*>(w + L.sq);
    a.sk = reinterpret_cast<float*>(w + L.sk);
    a.sv = reinterpret_cast<float*>(w + L.sv);
    e = sa::launch_quant(a, s);
    if (e != hipSuccess) return fail(SA_ERR_HIP, "quantise launch: %s", hipGetErrorString(e));
    e = sa::launch_attn_q(a, s);
    if (e != hipSuccess) return fail(SA_ERR_HIP, "attention (int8/fp8) launch: %s", hipGetErrorString(e));
  } else {
    e = sa::launch_attn(a, s);
    if (e != hipSuccess) return fail(SA_ERR_HIP, "attention launch: %s", hipGetErrorString(e));
  }
  return ok();
}

}  // namespace

extern "C" {

sa_status sparse_attn_predict(const sa_params* p, const void* q, const void* k, const sa_mask* out,
                              void* ws, size_t ws_bytes, void* stream) {
  return predict_impl(p, q, k, out, ws, ws_bytes, stream, false);
}

sa_status sparse_attn_pool(const sa_params* p, const void* q, const void* k, void* ws,
                           size_t ws_bytes, void* stream) {
  return predict_impl(p, q, k, nullptr, ws, ws_bytes, stream, false, true);
}

sa_status sparse_attn_forward(const sa_params* p, const void* q, const void* k, const void* v,
                              const sa_mask* mask, void* o, float* lse, uint32_t* skip_bits,
                              void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(p, q, k, v, mask, o, lse, skip_bits, ws, ws_bytes, stream, false);
}

sa_status sparse_attn_step(const sa_params* p, sa_schedule* sched, const void* q, const void* k,
                           const void* v, const sa_mask* mask, void* o, float* lse,
                           uint32_t* skip_bits, void* predict_ws, size_t predict_ws_bytes,
                           void* forward_ws, size_t forward_ws_bytes, void* stream) {
  if (!p) return fail(SA_ERR_INVALID_ARG, "params is NULL");
  if (!sched) return fail(SA_ERR_INVALID_ARG, "schedule is NULL");
  if (sched->refresh_every < 1 || sched->dense_steps < 0 || sched->step < 0)
    return fail(SA_ERR_INVALID_ARG, "schedule refresh_every=%d dense_steps=%d step=%d",
                sched->refresh_every, sched->dense_steps, sched->step);
  if (sched->tau_by_step && sched->n_tau < 1)
    return fail(SA_ERR_INVALID_ARG, "schedule n_tau=%d with a tau table", sched->n_tau);
  // the call's parameters: a dense step keeps every admissible block and
  // skips nothing; a sparse step predicts on its first call and every
  // refresh_every-th call after, and otherwise reuses the caller's mask
  sa_params run = *p;
  bool refresh;
  if (sched->step < sched->dense_steps) {
    // every admissible block: tau = 1 under a cumulative-mass rule; a top-k
    // budget would still cut, so a dense call reads it as top-cdf
    run.tau = 1.0f;
    if (run.rule == SA_RULE_TOPK) run.rule = SA_RULE_TOPCDF;
    run.topk_blocks = 0;
    run.skip_rule = SA_SKIP_LAMBDA;
    run.lambda = -INFINITY;
    refresh = true;
  } else {
    refresh = (sched->step - sched->dense_steps) % sched->refresh_every == 0;
    if (sched->tau_by_step) {
      const int e = sched->step < sched->n_tau ? sched->step : sched->n_tau - 1;
      run.tau = sched->tau_by_step[e];  // validated with the rest of run below
    }
  }
  sa_status st = SA_OK;
  if (refresh) st = predict_impl(&run, q, k, mask, predict_ws, predict_ws_bytes, stream, true);
  if (st) return st;
  st = forward_impl(&run, q, k, v, mask, o, lse, skip_bits, forward_ws, forward_ws_bytes, stream,
                    true);
  if (st) return st;
  if (refresh) st = predict_impl(&run, q, k, mask, predict_ws, predict_ws_bytes, stream, false);
  if (st) return st;
  st = forward_impl(&run, q, k, v, mask, o, lse, skip_bits, forward_ws, forward_ws_bytes, stream,
                    false);
  if (st) return st;
  sched->refreshed = refresh ? 1 : 0;
  sched->step += 1;
  return ok();
}

}  // extern "C"

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};  // per device: the address of `scratch` there

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
sa_status noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SA_ERR_UNSUPPORTED, "device %d (the no-alloc scratch serves devices 0..%d)", dev,
                kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(SA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return SA_OK;
}

}  // namespace

extern "C" {

sa_status sparse_attn_predict_noalloc(const sa_params* p, const void* q, const void* k,
                                      const sa_mask* out, void* stream) {
  sa::Geometry g;
  bool empty;
  sa_status st = check_params(p, &g, &empty);
  if (st) return st;
  if (empty) return ok();
  const size_t need = predict_layout(g).total;
  if (need > kNoAllocScratchBytes)
    return fail(SA_ERR_WORKSPACE,
                "sparse_attn_predict_noalloc needs %zu bytes of scratch, more than the %zu of "
                "its static scratch; call sparse_attn_predict with a workspace",
                need, kNoAllocScratchBytes);
  void* ws = nullptr;
  st = noalloc_scratch(&ws);
  if (st) return st;
  return predict_impl(p, q, k, out, ws, kNoAllocScratchBytes, stream, false);
}

}  // extern "C"

namespace {

struct ClusterLayout {
  size_t M, mpart, cent, ghi, glo, bvec, labels, perm, hist, seg, cnt, total;
  int nch, nchm, mspan, cmax;
};

ClusterLayout cluster_layout(const sa::Geometry& g, const sa_cluster_params* cp) {
  ClusterLayout L{};
  const size_t z2 = 2 * (size_t)g.B * g.H;
  const bool inter = cp->metric == SA_METRIC_INTERACTION;
  L.cmax = cp->clusters_q > cp->clusters_k ? cp->clusters_q : cp->clusters_k;
  L.nch = (g.N + 255) / 256;
  L.nchm = 0;
  L.mspan = 0;
  if (inter) {
    const int want = (g.N + 2047) / 2048;
    L.nchm = want < 1 ? 1 : (want > 16 ? 16 : want);
    const int per = (g.N + L.nchm - 1) / L.nchm;
    L.mspan = (per + 63) / 64 * 64;
  }
  const size_t D = g.D, C = L.cmax, N = g.N;
  size_t o = 0;
  L.M = o;
  o += inter ? round_up(z2 * D * D * 4) : 0;
  L.mpart = o;
  o += inter ? round_up(z2 * L.nchm * D * D * 4) : 0;
  L.cent = o;
  o += round_up(z2 * C * D * 4);
  L.ghi = o;
  o += round_up(z2 * C * D * 2);
  L.glo = o;
  o += round_up(z2 * C * D * 2);
  L.bvec = o;
  o += round_up(z2 * C * 4);
  L.labels = o;
  o += round_up(z2 * N * 4);
  L.perm = o;
  o += round_up(z2 * N * 4);
  L.hist = o;
  o += round_up(z2 * L.nch * C * 4);
  L.seg = o;
  o += round_up(z2 * C * 4);
  L.cnt = o;
  o += round_up(z2 * C * 4);
  L.total = o;
  return L;
}

sa_status check_cluster(const sa_params* p, const sa_cluster_params* cp, sa::Geometry* g,
                        bool* empty) {
  sa_status st = check_params(p, g, empty);
  if (st) return st;
  if (!cp) return fail(SA_ERR_INVALID_ARG, "cluster params is NULL");
  if (p->dtype != SA_BF16) return fail(SA_ERR_UNSUPPORTED, "token clustering needs bf16 Q and K");
  if (p->causal)
    return fail(SA_ERR_INVALID_ARG, "token reordering is defined for non-causal attention only");
  if (cp->metric != SA_METRIC_FEATURE && cp->metric != SA_METRIC_INTERACTION)
    return fail(SA_ERR_INVALID_ARG, "metric=%d", cp->metric);
  if (cp->iters < 1 || cp->iters > 64)
    return fail(SA_ERR_INVALID_ARG, "iters=%d (must be in [1, 64])", cp->iters);
  const int cap = p->N < sa::kMaxClusters ? p->N : sa::kMaxClusters;
  if (!*empty && (cp->clusters_q < 1 || cp->clusters_q > cap || cp->clusters_k < 1 ||
                  cp->clusters_k > cap))
    return fail(SA_ERR_INVALID_ARG, "clusters_q=%d clusters_k=%d (must be in [1, min(N, %d)])",
                cp->clusters_q, cp->clusters_k, sa::kMaxClusters);
  if (2LL * p->B * p->H > 65535)
    return fail(SA_ERR_UNSUPPORTED, "B*H=%lld > 32767 for token clustering",
                (long long)p->B * p->H);
  return SA_OK;
}

}  // namespace

extern "C" {

sa_status sparse_attn_cluster_workspace_size(const sa_params* p, const sa_cluster_params* cp,
                                             size_t* ws) {
  sa::Geometry g;
  bool empty;
  sa_status st = check_cluster(p, cp, &g, &empty);
  if (st) return st;
  if (ws) *ws = empty ? 0 : cluster_layout(g, cp).total;
  return ok();
}

sa_status sparse_attn_cluster(const sa_params* p, const sa_cluster_params* cp, const void* q,
                              const void* k, const sa_reorder* out, void* ws, size_t ws_bytes,
                              void* stream) {
  sa::Geometry g;
  bool empty;
  sa_status st = check_cluster(p, cp, &g, &empty);
  if (st) return st;
  if (empty) return ok();
  if (!q || !k) return fail(SA_ERR_INVALID_ARG, "q or k is NULL");
  if (!aligned16(q) || !aligned16(k)) return fail(SA_ERR_INVALID_ARG, "q/k not 16-byte aligned");
  if (!out || !out->perm_q || !out->perm_k)
    return fail(SA_ERR_INVALID_ARG, "reorder output (perm_q, perm_k) is NULL");
  const ClusterLayout L = cluster_layout(g, cp);
  if (!ws || ws_bytes < L.total)
    return fail(SA_ERR_WORKSPACE, "cluster workspace %zu < %zu bytes", ws_bytes, L.total);
  if (!aligned16(ws)) return fail(SA_ERR_INVALID_ARG, "workspace not 16-byte aligned");
  char* w = static_cast<char*>(ws);
  sa::ClusterLaunch a{};
  a.g = g;
  a.q = q;
  a.k = k;
  a.cq = cp->clusters_q;
  a.ck = cp->clusters_k;
  a.cmax = L.cmax;
  a.iters = cp->iters;
  a.interaction = cp->metric == SA_METRIC_INTERACTION;
  a.nch = L.nch;
  a.nchm = L.nchm;
  a.mspan = L.mspan;
  a.M = reinterpret_cast<float*>(w + L.M);
  a.mpart = reinterpret_cast<float*>(w + L.mpart);
  a.cent = reinterpret_cast<float*>(w + L.cent);
  a.ghi = reinterpret_cast<uint16_t*>(w + L.ghi);
  a.glo = reinterpret_cast<uint16_t*>(w + L.glo);
  a.bvec = reinterpret_cast<float*>(w + L.bvec);
  a.labels = reinterpret_cast<int32_t*>(w + L.labels);
  a.perm = reinterpret_cast<int32_t*>(w + L.perm);
  a.hist = reinterpret_cast<int32_t*>(w + L.hist);
  a.seg = reinterpret_cast<int32_t*>(w + L.seg);
  a.cnt = reinterpret_cast<int32_t*>(w + L.cnt);
  a.perm_q = out->perm_q;
  a.perm_k = out->perm_k;
  a.labels_q = out->labels_q;
  a.labels_k = out->labels_k;
  hipError_t e = sa::launch_cluster(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SA_ERR_HIP, "cluster launch: %s", hipGetErrorString(e));
  return ok();
}

sa_status sparse_attn_permute(const sa_params* p, const void* x, const int32_t* perm,
                              int32_t inverse, int32_t elem_bytes, void* y, void* stream) {
  sa::Geometry g;
  bool empty;
  sa_status st = check_params(p, &g, &empty);
  if (st) return st;
  if (inverse != 0 && inverse != 1) return fail(SA_ERR_INVALID_ARG, "inverse=%d", inverse);
  if (elem_bytes != 2 && elem_bytes != 4)
    return fail(SA_ERR_INVALID_ARG, "elem_bytes=%d (2 or 4)", elem_bytes);
  if (empty) return ok();
  if (!x || !y || !perm) return fail(SA_ERR_INVALID_ARG, "x, y or perm is NULL");
  if (x == y) return fail(SA_ERR_INVALID_ARG, "x and y must be different buffers");
  if (!aligned16(x) || !aligned16(y)) return fail(SA_ERR_INVALID_ARG, "x/y not 16-byte aligned");
  if ((g.sn * elem_bytes) % 16 || (g.sh * elem_bytes) % 16 || (g.sb * elem_bytes) % 16)
    return fail(SA_ERR_INVALID_ARG, "strides must keep rows 16-byte aligned");
  sa::PermuteLaunch a{};
  a.g = g;
  a.x = x;
  a.y = y;
  a.perm = perm;
  a.inverse = inverse;
  a.esz = elem_bytes;
  a.row_bytes = g.D * elem_bytes;
  hipError_t e = sa::launch_permute(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SA_ERR_HIP, "permute launch: %s", hipGetErrorString(e));
  return ok();
}

sa_status sparse_attn_check_mask(const sa_params* p, const int32_t* kept_idx,
                                 const int32_t* kept_cnt, int64_t* bad_row) {
  if (bad_row) *bad_row = -1;
  sa::Geometry g;
  bool empty;
  sa_status st = check_params(p, &g, &empty);
  if (st) return st;
  if (empty) return ok();
  if (!kept_idx || !kept_cnt) return fail(SA_ERR_INVALID_ARG, "kept_idx or kept_cnt is NULL");
  st = check_mask_host(g, p, kept_idx, kept_cnt, bad_row);
  return st ? st : ok();
}

sa_status sparse_attn_info(int32_t* default_group_rows, int32_t* version) {
  if (default_group_rows) *default_group_rows = kDefaultGroupRows;
  if (version) *version = SPARSE_ATTN_VERSION;
  return ok();
}

const char* sparse_attn_status_str(int32_t status) {
  switch (status) {
    case SA_OK: return "SA_OK";
    case SA_ERR_INVALID_ARG: return "SA_ERR_INVALID_ARG";
    case SA_ERR_UNSUPPORTED: return "SA_ERR_UNSUPPORTED";
    case SA_ERR_WORKSPACE: return "SA_ERR_WORKSPACE";
    case SA_ERR_HIP: return "SA_ERR_HIP";
    default: return "SA_ERR_UNKNOWN";
  }
}

const char* sparse_attn_last_error(void) { return g_err; }

}  // extern "C"
