"""Python binding of libsparse_attn.so (the C ABI in include/sparse_attn.h).

Argument marshalling only: every step of block-sparse attention runs in the
library's HIP kernels.  PyTorch supplies device memory and the current
stream; tensors are passed by ``data_ptr()``, after a check that each is a
device tensor of the expected element type whose storage covers the shape
the parameters describe (raw integer pointers pass unchecked).  Importing
this module fails loudly when the library has not been built (``python
block_mean_pool_amd/build.py``) -- there is no CPU fallback.

Entry points have the C names:

    sparse_attn_mask_shape(params) -> (nqb, nkb)
    sparse_attn_workspace_size(params) -> (predict_bytes, forward_bytes)
    sparse_attn_predict(params, q, k, mask, ws, stream=None)
    sparse_attn_pool(params, q, k, ws, stream=None)
    sparse_attn_predict_noalloc(params, q, k, mask, stream=None)
    sparse_attn_forward(params, q, k, v, mask, o, lse=None, skip_bits=None,
                        ws=None, stream=None)
    sparse_attn_step(params, schedule, q, k, v, mask, o, lse=None,
                     skip_bits=None, predict_ws=None, forward_ws=None, stream=None)
    sparse_attn_cluster_workspace_size(params, cluster_params) -> bytes
    sparse_attn_cluster(params, cluster_params, q, k, reorder, ws, stream=None)
    sparse_attn_permute(params, x, perm, inverse, y, stream=None)
    sparse_attn_check_mask(params, kept_idx_host, kept_cnt_host) -> -1
    sparse_attn_info() -> (default_group_rows, version)
    sparse_attn_status_str(code) -> str
    sparse_attn_last_error() -> str
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
# SA_LIBRARY names another build of the same library (the host-sanitizer
# build the CPU tests run the boundary checks against); by default the
# in-tree build
LIB_PATH = os.environ.get("SA_LIBRARY") or os.path.join(HERE, "libsparse_attn.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "sparse_attn.h")

SA_OK, SA_ERR_INVALID_ARG, SA_ERR_UNSUPPORTED, SA_ERR_WORKSPACE, SA_ERR_HIP = range(5)
SA_F32, SA_BF16 = 0, 1
SA_PREC_NATIVE, SA_PREC_I8_FP8, SA_PREC_I4_FP8, SA_PREC_I8_MXFP8 = 0, 1, 2, 3
SA_RULE_TOPCDF, SA_RULE_ENERGY, SA_RULE_TOPK = 0, 1, 2
SA_SKIP_LAMBDA, SA_SKIP_RECALL = 0, 1
SA_METRIC_FEATURE, SA_METRIC_INTERACTION = 0, 1


class SaParams(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32),
        ("D", ctypes.c_int32), ("block_q", ctypes.c_int32), ("block_k", ctypes.c_int32),
        ("causal", ctypes.c_int32), ("dtype", ctypes.c_int32), ("prec", ctypes.c_int32),
        ("rule", ctypes.c_int32), ("tau", ctypes.c_float), ("lam", ctypes.c_float),
        ("sm_scale", ctypes.c_float), ("keep_prefix_kblocks", ctypes.c_int32),
        ("lambda_group_rows", ctypes.c_int32), ("o_fp32", ctypes.c_int32),
        ("stride_b", ctypes.c_int64),
        ("stride_h", ctypes.c_int64), ("stride_n", ctypes.c_int64),
        ("skip_rule", ctypes.c_int32), ("recall", ctypes.c_float),
        ("topk_blocks", ctypes.c_int32),
    ]


class SaMask(ctypes.Structure):
    _fields_ = [("kept_idx", ctypes.c_void_p), ("kept_cnt", ctypes.c_void_p),
                ("block_prob", ctypes.c_void_p)]


class SaSchedule(ctypes.Structure):
    _fields_ = [("refresh_every", ctypes.c_int32), ("dense_steps", ctypes.c_int32),
                ("step", ctypes.c_int32), ("refreshed", ctypes.c_int32),
                ("tau_by_step", ctypes.POINTER(ctypes.c_float)), ("n_tau", ctypes.c_int32)]


class SaClusterParams(ctypes.Structure):
    _fields_ = [("clusters_q", ctypes.c_int32), ("clusters_k", ctypes.c_int32),
                ("iters", ctypes.c_int32), ("metric", ctypes.c_int32)]


class SaReorder(ctypes.Structure):
    _fields_ = [("perm_q", ctypes.c_void_p), ("perm_k", ctypes.c_void_p),
                ("labels_q", ctypes.c_void_p), ("labels_k", ctypes.c_void_p)]


class SparseAttnError(RuntimeError):
    def __init__(self, code: int, where: str, msg: str):
        super().__init__(f"{where}: {status_name(code)}: {msg}")
        self.code = code


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python block_mean_pool_amd/build.py); there is no fallback path")
    # torch ships its own HIP runtime under the same soname
    # (libamdhip64.so.7) as the ROCm one this library is linked against.
    # Importing torch first makes the library's dependency resolve to the
    # runtime torch already loaded, so the process holds one HIP runtime
    # (two would each open the device, and the second finds none).
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    vp = ctypes.c_void_p
    sig = {
        "sparse_attn_mask_shape": [P(SaParams), P(ctypes.c_int64), P(ctypes.c_int64)],
        "sparse_attn_workspace_size": [P(SaParams), P(ctypes.c_size_t), P(ctypes.c_size_t)],
        "sparse_attn_predict": [P(SaParams), vp, vp, P(SaMask), vp, ctypes.c_size_t, vp],
        "sparse_attn_pool": [P(SaParams), vp, vp, vp, ctypes.c_size_t, vp],
        "sparse_attn_predict_noalloc": [P(SaParams), vp, vp, P(SaMask), vp],
        "sparse_attn_check_mask": [P(SaParams), vp, vp, P(ctypes.c_int64)],
        "sparse_attn_forward": [P(SaParams), vp, vp, vp, P(SaMask), vp, vp, vp, vp,
                                ctypes.c_size_t, vp],
        "sparse_attn_info": [P(ctypes.c_int32), P(ctypes.c_int32)],
        "sparse_attn_step": [P(SaParams), P(SaSchedule), vp, vp, vp, P(SaMask), vp, vp, vp, vp,
                             ctypes.c_size_t, vp, ctypes.c_size_t, vp],
        "sparse_attn_cluster_workspace_size": [P(SaParams), P(SaClusterParams),
                                               P(ctypes.c_size_t)],
        "sparse_attn_cluster": [P(SaParams), P(SaClusterParams), vp, vp, P(SaReorder), vp,
                                ctypes.c_size_t, vp],
        "sparse_attn_permute": [P(SaParams), vp, vp, ctypes.c_int32, ctypes.c_int32, vp, vp],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.sparse_attn_status_str.argtypes = [ctypes.c_int32]
    lib.sparse_attn_status_str.restype = ctypes.c_char_p
    lib.sparse_attn_last_error.argtypes = []
    lib.sparse_attn_last_error.restype = ctypes.c_char_p
    return lib


lib = _load()


def status_name(code: int) -> str:
    return lib.sparse_attn_status_str(int(code)).decode()


def sparse_attn_status_str(code: int) -> str:
    return status_name(code)


def sparse_attn_last_error() -> str:
    return lib.sparse_attn_last_error().decode()


def _check(code: int, where: str):
    if code != SA_OK:
        raise SparseAttnError(code, where, sparse_attn_last_error())


def make_params(B, H, N, D, *, dtype="bf16", causal=False, tau=0.95, lam=-math.inf,
                sm_scale=0.0, rule="topcdf", prec="native", keep_prefix_kblocks=0,
                block_q=128, block_k=64, lambda_group_rows=0, o_fp32=False,
                strides=(0, 0, 0), skip_rule="lambda", recall=1.0,
                topk_blocks=0) -> SaParams:
    """A parameter block; ``strides`` are element strides (b, h, n), 0 =
    packed [B, H, N, D]; ``o_fp32`` writes O as float32; ``skip_rule`` is
    "lambda" (threshold ``lam``) or "recall" (target share ``recall``)."""
    return SaParams(
        B, H, N, D, block_q, block_k, int(bool(causal)),
        {"f32": SA_F32, "bf16": SA_BF16}[dtype] if isinstance(dtype, str) else int(dtype),
        {"native": SA_PREC_NATIVE, "i8fp8": SA_PREC_I8_FP8, "i4fp8": SA_PREC_I4_FP8,
         "i8mxfp8": SA_PREC_I8_MXFP8}[prec] if isinstance(prec, str) else int(prec),
        {"topcdf": SA_RULE_TOPCDF, "energy": SA_RULE_ENERGY, "topk": SA_RULE_TOPK}[rule]
        if isinstance(rule, str) else int(rule),
        float(tau), float(lam), float(sm_scale), int(keep_prefix_kblocks),
        int(lambda_group_rows), int(bool(o_fp32)), int(strides[0]), int(strides[1]),
        int(strides[2]),
        {"lambda": SA_SKIP_LAMBDA, "recall": SA_SKIP_RECALL}[skip_rule]
        if isinstance(skip_rule, str) else int(skip_rule),
        float(recall), int(topk_blocks))


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


# Checks on the tensors handed to the library, made before any call: a host
# tensor, a wrong element type or a buffer too short for the described shape
# would otherwise reach the kernels.  Raw integer pointers are passed through
# unchecked (the caller vouches for them).
def _dtype_name(t) -> str:
    return str(t.dtype).replace("torch.", "")


def _need(t, name, dtypes=None, elems=None):
    if t is None or isinstance(t, int):
        return
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name} must be a device tensor (got {getattr(t, 'device', type(t))})")
    if dtypes is not None and _dtype_name(t) not in dtypes:
        raise TypeError(f"{name} has dtype {_dtype_name(t)}, expected {' or '.join(dtypes)}")
    if elems is not None:
        avail = t.untyped_storage().nbytes() // t.element_size() - t.storage_offset()
        if avail < elems:
            raise ValueError(f"{name} holds {avail} elements from its data pointer, "
                             f"{elems} needed")


def _extent(p: SaParams) -> int:
    """Elements spanned by a [B, H, N, D] tensor with the strides of ``p``."""
    if p.B <= 0 or p.H <= 0 or p.N <= 0:
        return 0
    sn = p.stride_n or p.D
    sh = p.stride_h or p.N * sn
    sb = p.stride_b or p.H * sh
    return (p.B - 1) * sb + (p.H - 1) * sh + (p.N - 1) * sn + p.D


def _io_dtype(p: SaParams):
    return ("bfloat16",) if p.dtype == SA_BF16 else ("float32",)


def _check_qkv(p: SaParams, **tensors):
    n = _extent(p)
    for name, t in tensors.items():
        _need(t, name, _io_dtype(p), n)


def _check_outputs(p: SaParams, o, lse, skip_bits):
    _need(o, "o", ("float32",) if p.o_fp32 else _io_dtype(p), _extent(p))
    bhn = max(p.B, 0) * max(p.H, 0) * max(p.N, 0)
    _need(lse, "lse", ("float32",), bhn)
    nqb, nkb = (p.N + 127) // 128, (p.N + 63) // 64
    groups = 128 // (p.lambda_group_rows or 32) if p.lambda_group_rows in (0, 16, 32, 64, 128) \
        else 4  # an unsupported G is rejected by the library
    _need(skip_bits, "skip_bits", ("int32", "uint32"),
          max(p.B, 0) * max(p.H, 0) * nqb * groups * ((nkb + 31) // 32))


def sparse_attn_mask_shape(p: SaParams):
    nq, nk = ctypes.c_int64(), ctypes.c_int64()
    _check(lib.sparse_attn_mask_shape(ctypes.byref(p), ctypes.byref(nq), ctypes.byref(nk)),
           "sparse_attn_mask_shape")
    return nq.value, nk.value


def sparse_attn_workspace_size(p: SaParams):
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib.sparse_attn_workspace_size(ctypes.byref(p), ctypes.byref(a), ctypes.byref(b)),
           "sparse_attn_workspace_size")
    return a.value, b.value


def sparse_attn_check_mask(p: SaParams, kept_idx, kept_cnt):
    """Checks a mask held in host memory (numpy int32 arrays [B,H,NQB,NKB]
    and [B,H,NQB]).  Returns -1 when it is valid; raises SparseAttnError
    naming the first offending row otherwise."""
    import numpy as np
    idx = np.ascontiguousarray(kept_idx, dtype=np.int32)
    cnt = np.ascontiguousarray(kept_cnt, dtype=np.int32)
    nqb, nkb = sparse_attn_mask_shape(p)
    rows = max(p.B, 0) * max(p.H, 0) * nqb
    if idx.size != rows * nkb or cnt.size != rows:
        raise ValueError(f"mask arrays hold {idx.size} / {cnt.size} entries, expected "
                         f"{rows * nkb} / {rows}")
    bad = ctypes.c_int64(-1)
    _check(lib.sparse_attn_check_mask(ctypes.byref(p), idx.ctypes.data, cnt.ctypes.data,
                                      ctypes.byref(bad)), "sparse_attn_check_mask")
    return bad.value


def sparse_attn_info():
    g, v = ctypes.c_int32(), ctypes.c_int32()
    _check(lib.sparse_attn_info(ctypes.byref(g), ctypes.byref(v)), "sparse_attn_info")
    return g.value, v.value


def make_mask(kept_idx, kept_cnt, block_prob=None) -> SaMask:
    _need(kept_idx, "kept_idx", ("int32",))
    _need(kept_cnt, "kept_cnt", ("int32",))
    _need(block_prob, "block_prob", ("float32",))
    return SaMask(_ptr(kept_idx), _ptr(kept_cnt), _ptr(block_prob))


def sparse_attn_predict(p: SaParams, q, k, mask: SaMask, ws, stream=None, ws_bytes=None):
    """Stage one.  ``q``, ``k``: device tensors; ``mask``: SaMask over device
    int32 buffers; ``ws``: device buffer of sparse_attn_workspace_size()[0]
    bytes."""
    _check_qkv(p, q=q, k=k)
    _need(ws, "ws", ("uint8", "int8"))
    nb = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check(lib.sparse_attn_predict(ctypes.byref(p), _ptr(q), _ptr(k), ctypes.byref(mask),
                                   _ptr(ws), nb, _stream(stream)), "sparse_attn_predict")


def sparse_attn_predict_noalloc(p: SaParams, q, k, mask: SaMask, stream=None):
    """Stage one with the library's static scratch instead of a caller
    workspace (for callers that cannot allocate; problems whose predict
    workspace exceeds 64 MiB are rejected)."""
    _check_qkv(p, q=q, k=k)
    _check(lib.sparse_attn_predict_noalloc(ctypes.byref(p), _ptr(q), _ptr(k),
                                           ctypes.byref(mask), _stream(stream)),
           "sparse_attn_predict_noalloc")


def sparse_attn_pool(p: SaParams, q, k, ws, stream=None, ws_bytes=None):
    """Stage one's block means alone, written to ``ws`` (a predict
    workspace) in its layout: qbar float [B,H,NQB,D] at offset 0, kbar float
    [B,H,NKB,D] at the next 256-byte boundary."""
    _check_qkv(p, q=q, k=k)
    _need(ws, "ws", ("uint8", "int8"))
    nb = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check(lib.sparse_attn_pool(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(ws), nb,
                                _stream(stream)), "sparse_attn_pool")


def sparse_attn_forward(p: SaParams, q, k, v, mask: SaMask, o, lse=None, skip_bits=None,
                        ws=None, stream=None, ws_bytes=None):
    """Stage two.  Writes ``o`` (and ``lse`` / ``skip_bits`` when given)."""
    _check_qkv(p, q=q, k=k, v=v)
    _check_outputs(p, o, lse, skip_bits)
    _need(ws, "ws", ("uint8", "int8"))
    nb = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check(lib.sparse_attn_forward(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v),
                                   ctypes.byref(mask), _ptr(o), _ptr(lse), _ptr(skip_bits),
                                   _ptr(ws), nb, _stream(stream)), "sparse_attn_forward")


def make_schedule(refresh_every=1, dense_steps=0, tau_by_step=None) -> SaSchedule:
    """A mask-reuse schedule for sparse_attn_step, at step 0.  ``tau_by_step``
    (a sequence of floats) gives the tau of each call's prediction; the
    schedule keeps the host array alive."""
    sched = SaSchedule(int(refresh_every), int(dense_steps), 0, 0, None, 0)
    if tau_by_step is not None:
        arr = (ctypes.c_float * len(tau_by_step))(*[float(t) for t in tau_by_step])
        sched._tau_array = arr
        sched.tau_by_step = ctypes.cast(arr, ctypes.POINTER(ctypes.c_float))
        sched.n_tau = len(tau_by_step)
    return sched


def sparse_attn_step(p: SaParams, sched: SaSchedule, q, k, v, mask: SaMask, o, lse=None,
                     skip_bits=None, predict_ws=None, forward_ws=None, stream=None,
                     predict_ws_bytes=None, forward_ws_bytes=None):
    """One call of a sequence: stage one when ``sched`` says so, then stage
    two.  Updates ``sched`` (step, refreshed)."""
    _check_qkv(p, q=q, k=k, v=v)
    _check_outputs(p, o, lse, skip_bits)
    _need(predict_ws, "predict_ws", ("uint8", "int8"))
    _need(forward_ws, "forward_ws", ("uint8", "int8"))
    pb = _nbytes(predict_ws) if predict_ws_bytes is None else predict_ws_bytes
    fb = _nbytes(forward_ws) if forward_ws_bytes is None else forward_ws_bytes
    _check(lib.sparse_attn_step(ctypes.byref(p), ctypes.byref(sched), _ptr(q), _ptr(k), _ptr(v),
                                ctypes.byref(mask), _ptr(o), _ptr(lse), _ptr(skip_bits),
                                _ptr(predict_ws), pb, _ptr(forward_ws), fb, _stream(stream)),
           "sparse_attn_step")


def make_cluster_params(clusters_q, clusters_k, iters=4, metric="interaction") -> SaClusterParams:
    """Token clustering parameters; ``metric`` is "interaction" or "feature"."""
    m = {"feature": SA_METRIC_FEATURE, "interaction": SA_METRIC_INTERACTION}[metric] \
        if isinstance(metric, str) else int(metric)
    return SaClusterParams(int(clusters_q), int(clusters_k), int(iters), m)


def make_reorder(perm_q, perm_k, labels_q=None, labels_k=None) -> SaReorder:
    for name, t in (("perm_q", perm_q), ("perm_k", perm_k), ("labels_q", labels_q),
                    ("labels_k", labels_k)):
        _need(t, name, ("int32",))
    return SaReorder(_ptr(perm_q), _ptr(perm_k), _ptr(labels_q), _ptr(labels_k))


def sparse_attn_cluster_workspace_size(p: SaParams, cp: SaClusterParams) -> int:
    n = ctypes.c_size_t()
    _check(lib.sparse_attn_cluster_workspace_size(ctypes.byref(p), ctypes.byref(cp),
                                                  ctypes.byref(n)),
           "sparse_attn_cluster_workspace_size")
    return n.value


def sparse_attn_cluster(p: SaParams, cp: SaClusterParams, q, k, out: SaReorder, ws,
                        stream=None, ws_bytes=None):
    """Clusters query and key tokens; writes the orders (and labels) of
    ``out`` (SaReorder over device int32 [B, H, N] buffers)."""
    _check_qkv(p, q=q, k=k)
    _need(ws, "ws", ("uint8", "int8"))
    nb = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check(lib.sparse_attn_cluster(ctypes.byref(p), ctypes.byref(cp), _ptr(q), _ptr(k),
                                   ctypes.byref(out), _ptr(ws), nb, _stream(stream)),
           "sparse_attn_cluster")


def sparse_attn_permute(p: SaParams, x, perm, inverse, y, stream=None, elem_bytes=None):
    """Row gather (inverse=0: y[r] = x[perm[r]]) or scatter (inverse=1:
    y[perm[r]] = x[r]) of [B, H, N, D] tensors; ``elem_bytes`` defaults to
    x's element size."""
    eb = x.element_size() if elem_bytes is None else int(elem_bytes)
    n = _extent(p)
    for name, t in (("x", x), ("y", y)):
        _need(t, name, None, None)
        if t is not None and not isinstance(t, int):
            if t.element_size() != eb:
                raise TypeError(f"{name} has {t.element_size()}-byte elements, {eb} expected")
            _need(t, name, None, n)
    _need(perm, "perm", ("int32",), max(p.B, 0) * max(p.H, 0) * max(p.N, 0))
    _check(lib.sparse_attn_permute(ctypes.byref(p), _ptr(x), _ptr(perm), int(inverse), eb,
                                   _ptr(y), _stream(stream)), "sparse_attn_permute")


__all__ = [
    "SaParams", "SaMask", "SparseAttnError", "make_params", "make_mask",
    "sparse_attn_mask_shape", "sparse_attn_workspace_size", "sparse_attn_predict",
    "sparse_attn_forward", "sparse_attn_pool", "sparse_attn_predict_noalloc",
    "sparse_attn_check_mask", "sparse_attn_info", "sparse_attn_status_str",
    "SaClusterParams", "SaReorder", "make_cluster_params", "make_reorder",
    "sparse_attn_cluster_workspace_size", "sparse_attn_cluster", "sparse_attn_permute",
    "SaSchedule", "make_schedule", "sparse_attn_step",
    "sparse_attn_last_error", "lib", "LIB_PATH", "HEADER",
]
