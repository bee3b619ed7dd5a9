"""ctypes binding of libmoe.so (C ABI in include/moe.h).

Argument marshalling only: every function passes device pointers, sizes and
the current HIP stream to the entry point of the same name and raises
``MoeError`` on a nonzero status.  PyTorch supplies device memory and the
stream; all computation happens in the library.  Importing this module loads
the library and fails loudly when it has not been built.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libmoe.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built: run `python -m mixture_experts_layer_layout_amd.build`")

_lib = ctypes.CDLL(LIB_PATH)

c_int32 = ctypes.c_int32
c_void_p = ctypes.c_void_p

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE = 0, -1, -2, -3
MOE_ERR_HIP, MOE_ERR_TIMEOUT, MOE_ERR_INVALID_ROUTE = -4, -5, -6
MOE_F32, MOE_BF16, MOE_MXFP8 = 0, 1, 2
MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID = 0, 1
MOE_FLAG_DIRECT_PULL = 0x1
MOE_FLAG_PERSISTENT_SPLIT = 0x2
MOE_FLAG_PERSISTENT_WGRAD_APART = 0x4
MOE_FLAG_PERSISTENT_SINGLE = 0x8
MOE_FLAG_BIAS_SELECT_ONLY = 0x10
MOE_FLAG_SPIN_LIMIT_TINY = 0x100
MOE_FLAG_TEST_DROP_READY = 0x200
MOE_FLAG_TEST_SHUFFLE_CLAIMS = 0x400
MOE_FLAG_PERSISTENT_GEMM_APART = 0x800
MOE_FLAG_MXFP8_WGRAD = 0x1000

_DT = {"f32": MOE_F32, "bf16": MOE_BF16, "mxfp8": MOE_MXFP8}
_SC = {"softmax": MOE_SCORE_SOFTMAX, "sigmoid": MOE_SCORE_SIGMOID}


class MoeDesc(ctypes.Structure):
    _fields_ = [("T", c_int32), ("d", c_int32), ("E", c_int32), ("k", c_int32),
                ("I", c_int32), ("act_dtype", c_int32), ("expert_dtype", c_int32),
                ("score", c_int32), ("renorm", c_int32), ("fused", c_int32),
                ("stage_rows", c_int32), ("n_workgroups", c_int32),
                ("flags", ctypes.c_uint32), ("n_group", c_int32), ("topk_group", c_int32),
                ("routed_scale", ctypes.c_float), ("macro_tokens", c_int32),
                ("n_producer_cus", c_int32)]


class MoeWeights(ctypes.Structure):
    _fields_ = [("w1", c_void_p), ("w3", c_void_p), ("w2", c_void_p),
                ("w1_scale", c_void_p), ("w3_scale", c_void_p), ("w2_scale", c_void_p)]


class MoeSaved(ctypes.Structure):
    _fields_ = [("logits", c_void_p), ("topk_idx", c_void_p), ("gate", c_void_p),
                ("counts", c_void_p), ("offsets", c_void_p), ("perm", c_void_p),
                ("inv", c_void_p), ("a", c_void_p), ("b", c_void_p), ("h", c_void_p),
                ("status", c_void_p)]


_P = ctypes.POINTER
_lib.moe_workspace_size.argtypes = [_P(MoeDesc), _P(ctypes.c_size_t)]
_lib.moe_route.argtypes = [_P(MoeDesc), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]
_lib.moe_layout.argtypes = [_P(MoeDesc), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                            c_void_p, c_void_p, ctypes.c_size_t, c_void_p]
_lib.moe_gather.argtypes = [_P(MoeDesc), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]
_lib.moe_quantize_mxfp8.argtypes = [c_void_p, ctypes.c_int64, ctypes.c_int64, c_void_p,
                                    c_void_p, c_void_p]
_lib.moe_quantize_mxfp8_t.argtypes = [c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                      c_void_p, c_void_p, c_void_p]
_lib.moe_combine.argtypes = [_P(MoeDesc), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]
_lib.moe_forward.argtypes = [_P(MoeDesc), c_void_p, c_void_p, c_void_p, _P(MoeWeights),
                             c_void_p, _P(MoeSaved), c_void_p, ctypes.c_size_t, c_void_p]
_lib.moe_forward_noalloc.argtypes = [_P(MoeDesc), c_void_p, c_void_p, c_void_p, _P(MoeWeights),
                                     c_void_p, _P(MoeSaved), c_void_p]
_lib.moe_backward.argtypes = [_P(MoeDesc), c_void_p, c_void_p, _P(MoeWeights), _P(MoeSaved),
                              c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                              ctypes.c_size_t, c_void_p]
_lib.moe_router_backward.argtypes = [_P(MoeDesc), c_void_p, c_void_p, c_void_p, _P(MoeSaved),
                                     c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                     ctypes.c_size_t, c_void_p]
_lib.moe_status_string.argtypes = [ctypes.c_int]
_lib.moe_status_string.restype = ctypes.c_char_p
for _f in ("moe_workspace_size", "moe_route", "moe_layout", "moe_gather", "moe_quantize_mxfp8",
           "moe_quantize_mxfp8_t", "moe_combine", "moe_forward", "moe_forward_noalloc", "moe_backward",
           "moe_router_backward"):
    getattr(_lib, _f).restype = ctypes.c_int

EXPORTS = ("moe_workspace_size", "moe_route", "moe_layout", "moe_gather",
           "moe_quantize_mxfp8", "moe_quantize_mxfp8_t", "moe_combine", "moe_forward", "moe_forward_noalloc",
           "moe_backward", "moe_router_backward", "moe_status_string")
MOE_NOALLOC_SCRATCH_BYTES = 256 << 20


class MoeError(RuntimeError):
    def __init__(self, code, where):
        self.code = code
        super().__init__(f"{where}: {moe_status_string(code)} ({code})")


def moe_status_string(code: int) -> str:
    return _lib.moe_status_string(int(code)).decode()


def _check(rc, where):
    if rc != MOE_OK:
        raise MoeError(rc, where)


def _p(t):
    return None if t is None else c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return c_void_p(stream.cuda_stream)


def make_desc(T, d, E, k, I, act="bf16", experts="bf16", score="sigmoid", renorm=True,
              fused=True, stage_rows=0, n_workgroups=0, flags=0, n_group=0, topk_group=0,
              routed_scale=0.0, macro_tokens=0, n_producer_cus=0) -> MoeDesc:
    return MoeDesc(T, d, E, k, I, _DT[act], _DT[experts], _SC[score], int(bool(renorm)),
                   int(bool(fused)), stage_rows, n_workgroups, flags, n_group, topk_group,
                   routed_scale, macro_tokens, n_producer_cus)


def moe_workspace_size(desc: MoeDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib.moe_workspace_size(ctypes.byref(desc), ctypes.byref(n)), "moe_workspace_size")
    return n.value


def moe_route(desc, logits, bias, topk_idx, gate, stream=None):
    _check(_lib.moe_route(ctypes.byref(desc), _p(logits), _p(bias), _p(topk_idx), _p(gate),
                          _stream(stream)), "moe_route")


def moe_layout(desc, topk_idx, counts, offsets, perm, inv, status, workspace, stream=None):
    _check(_lib.moe_layout(ctypes.byref(desc), _p(topk_idx), _p(counts), _p(offsets), _p(perm),
                           _p(inv), _p(status), _p(workspace),
                           0 if workspace is None else workspace.numel(), _stream(stream)),
           "moe_layout")


def moe_gather(desc, x, perm, xp, xp_scale=None, stream=None, inv=None):
    _check(_lib.moe_gather(ctypes.byref(desc), _p(x), _p(perm), _p(inv), _p(xp), _p(xp_scale),
                           _stream(stream)), "moe_gather")


def moe_quantize_mxfp8(src, codes, scales, stream=None):
    rows, K = src.shape[0], src.shape[-1]
    rows = src.numel() // K
    _check(_lib.moe_quantize_mxfp8(_p(src), rows, K, _p(codes), _p(scales), _stream(stream)),
           "moe_quantize_mxfp8")


def moe_quantize_mxfp8_t(src, codes, scales, stream=None):
    """src [batch, rows, cols] (or [rows, cols]) -> codes [batch, cols, rows],
    scales [batch, cols, rows/32]."""
    batch = 1 if src.dim() == 2 else src.shape[0]
    rows, cols = src.shape[-2], src.shape[-1]
    _check(_lib.moe_quantize_mxfp8_t(_p(src), batch, rows, cols, _p(codes), _p(scales), _stream(stream)),
           "moe_quantize_mxfp8_t")


def moe_combine(desc, yp, gate, inv, y, stream=None):
    _check(_lib.moe_combine(ctypes.byref(desc), _p(yp), _p(gate), _p(inv), _p(y), _stream(stream)),
           "moe_combine")


def make_weights(w1, w3, w2, w1_scale=None, w3_scale=None, w2_scale=None) -> MoeWeights:
    return MoeWeights(_p(w1), _p(w3), _p(w2), _p(w1_scale), _p(w3_scale), _p(w2_scale))


def make_saved(**bufs) -> MoeSaved:
    s = MoeSaved()
    for name, t in bufs.items():
        setattr(s, name, None if t is None else t.data_ptr())
    return s


def moe_forward(desc, x, wr, bias, weights: MoeWeights, y, saved: MoeSaved | None, workspace,
                stream=None):
    _check(_lib.moe_forward(ctypes.byref(desc), _p(x), _p(wr), _p(bias), ctypes.byref(weights),
                            _p(y), None if saved is None else ctypes.byref(saved), _p(workspace),
                            0 if workspace is None else workspace.numel(), _stream(stream)),
           "moe_forward")


def moe_forward_noalloc(desc, x, wr, bias, weights: MoeWeights, y, saved: MoeSaved | None, stream=None):
    _check(_lib.moe_forward_noalloc(ctypes.byref(desc), _p(x), _p(wr), _p(bias), ctypes.byref(weights),
                                    _p(y), None if saved is None else ctypes.byref(saved), _stream(stream)),
           "moe_forward_noalloc")


def moe_backward(desc, dy, x, weights: MoeWeights, saved: MoeSaved, dx, dw1, dw3, dw2, dgate,
                 workspace, stream=None):
    _check(_lib.moe_backward(ctypes.byref(desc), _p(dy), _p(x), ctypes.byref(weights),
                             ctypes.byref(saved), _p(dx), _p(dw1), _p(dw3), _p(dw2), _p(dgate),
                             _p(workspace), 0 if workspace is None else workspace.numel(),
                             _stream(stream)), "moe_backward")


def moe_router_backward(desc, x, wr, bias, saved: MoeSaved, dgate, dlogits, dwr, dbias, dx,
                        workspace, stream=None):
    _check(_lib.moe_router_backward(ctypes.byref(desc), _p(x), _p(wr), _p(bias), ctypes.byref(saved),
                                    _p(dgate), _p(dlogits), _p(dwr), _p(dbias), _p(dx), _p(workspace),
                                    0 if workspace is None else workspace.numel(), _stream(stream)),
           "moe_router_backward")
