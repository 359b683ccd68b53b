"""Fused chunked top-K KL distillation loss on AMD MI355X (gfx950).

Thin binding over the C ABI in ``include/fckl.h`` (``libfckl.so``, built in-tree by
``python -m chunked_top_kl_chunk_amd.build``).  This module only marshals
arguments: torch supplies device memory and the stream, and every step of the
loss runs in the library's HIP kernels.  There is no CPU or eager fallback; if
the library is missing every call raises.

    import chunked_top_kl_chunk_amd as fckl
    loss_tok, lse, loss_mean = fckl.forward(h, W, topk_idx, topk_logit, T=1.0)
    dH, dW = fckl.backward(h, W, topk_idx, topk_logit, lse, T=1.0)
    # or both in one call (the loss is the last operation of the step):
    loss_tok, lse, loss_mean, dH, dW = fckl.forward_backward(h, W, topk_idx, topk_logit, T=1.0)

Optional per-token ``weights`` (float32 [N], 0 masks a token) make the mean
sum_i w_i loss_i / sum_i w_i.  ``FusedChunkedKLLoss`` (``chunked_top_kl_chunk_amd.loss``)
wraps the two passes as a torch autograd module.

Shapes: h [N,H] bf16, W [V,H] bf16, topk_idx [N,K] int32, topk_logit [N,K] bf16 or
float32, all contiguous on one HIP device.  Outputs are float32.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfckl.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_INDEX, ERR_HIP = range(6)
DTYPE_BF16, DTYPE_F32 = 0, 1
FLAG_VALIDATE, FLAG_DW_ACCUMULATE, FLAG_TOPK_FULL_FIRST_PASS = 1, 2, 4

# Every symbol include/fckl.h declares.
EXPORTS = ("fckl_plan", "fckl_workspace_size", "fckl_forward", "fckl_backward", "fckl_forward_ex",
           "fckl_backward_ex", "fckl_forward_noalloc", "fckl_single_plan", "fckl_forward_backward", "fckl_topk_workspace_size", "fckl_topk",
           "fckl_topk_async", "fckl_full_plan", "fckl_full_forward_backward", "fckl_scale", "fckl_status_string",
           "fckl_version")


KERNELS = ("prepare", "fwd_logits", "combine", "mean", "bwd_logits", "dh", "dh_reduce", "dw", "transpose",
           "softmax_grad", "weights", "full_teacher", "full_student", "full_combine", "full_grad")


class Profile(ctypes.Structure):
    """Mirror of struct fckl_profile (per-kernel hipEvent brackets)."""
    _fields_ = [("kernel_mask", ctypes.c_uint32), ("capacity", ctypes.c_int32), ("count", ctypes.c_int32),
                ("events", ctypes.POINTER(ctypes.c_void_p)), ("kernel_ids", ctypes.POINTER(ctypes.c_int32)),
                ("work", ctypes.POINTER(ctypes.c_int32)), ("vocab_rows", ctypes.POINTER(ctypes.c_int32))]


class Desc(ctypes.Structure):
    """Mirror of struct fckl_desc."""
    _fields_ = [("N", ctypes.c_int64), ("H", ctypes.c_int32), ("V", ctypes.c_int32), ("K", ctypes.c_int32),
                ("T", ctypes.c_float), ("chunk", ctypes.c_int32), ("logit_dtype", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("profile", ctypes.POINTER(Profile)), ("vocab_slab", ctypes.c_int32)]


class FCKLError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, status_string(status), status))


_lib: Optional[ctypes.CDLL] = None


def load() -> ctypes.CDLL:
    """Load libfckl.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libfckl.so not found at %s; build it with `python -m chunked_top_kl_chunk_amd.build`"
                          % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, vp, sz = ctypes.POINTER, ctypes.c_void_p, ctypes.c_size_t
    lib.fckl_plan.argtypes = [P(Desc), sz, P(ctypes.c_int32), P(sz)]
    lib.fckl_single_plan.argtypes = [P(Desc), sz, P(ctypes.c_int32), P(sz)]
    lib.fckl_workspace_size.argtypes = [P(Desc), ctypes.c_int32, P(sz)]
    lib.fckl_forward.argtypes = [P(Desc), vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.fckl_backward.argtypes = [P(Desc), vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, sz, vp]
    lib.fckl_forward_ex.argtypes = [P(Desc), vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.fckl_forward_noalloc.argtypes = [P(Desc), vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.fckl_backward_ex.argtypes = [P(Desc), vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp, sz, vp]
    lib.fckl_forward_backward.argtypes = [P(Desc), vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp, vp, vp,
                                          sz, vp]
    lib.fckl_status_string.argtypes = [ctypes.c_int]
    lib.fckl_status_string.restype = ctypes.c_char_p
    lib.fckl_version.argtypes = []
    lib.fckl_version.restype = ctypes.c_int32
    lib.fckl_topk_workspace_size.argtypes = [P(Desc), ctypes.c_int32, P(sz)]
    lib.fckl_topk.argtypes = [P(Desc), vp, vp, vp, vp, vp, sz, vp]
    lib.fckl_topk_async.argtypes = [P(Desc), vp, vp, vp, vp, vp, sz, vp, vp]
    lib.fckl_full_plan.argtypes = [P(Desc), ctypes.c_int32, sz, P(ctypes.c_int32), P(sz)]
    lib.fckl_full_forward_backward.argtypes = [P(Desc), ctypes.c_int32, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp,
                                               vp, vp, vp, vp, sz, vp]
    lib.fckl_scale.argtypes = [vp, ctypes.c_int64, vp, vp]
    for f in ("fckl_plan", "fckl_single_plan", "fckl_workspace_size", "fckl_forward", "fckl_backward",
              "fckl_forward_ex", "fckl_forward_noalloc", "fckl_backward_ex", "fckl_forward_backward", "fckl_topk_workspace_size", "fckl_topk",
              "fckl_topk_async", "fckl_full_plan", "fckl_full_forward_backward", "fckl_scale"):
        getattr(lib, f).restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().fckl_status_string(int(status)).decode()


def version() -> int:
    return int(load().fckl_version())


def make_desc(N: int, H: int, V: int, K: int, T: float = 1.0, chunk: int = 0, logit_dtype: int = DTYPE_BF16,
              flags: int = 0, profile: Optional[Profile] = None, vocab_slab: int = 0) -> Desc:
    """vocab_slab: vocabulary rows per slab of the two-pass backward (a multiple of 256;
    0 = the library's choice)."""
    d = Desc(int(N), int(H), int(V), int(K), float(T), int(chunk), int(logit_dtype), int(flags))
    if profile is not None:
        d.profile = ctypes.pointer(profile)
    d.vocab_slab = int(vocab_slab)
    return d


def _call(name: str, *args) -> None:
    st = getattr(load(), name)(*args)
    if st != OK:
        raise FCKLError(st, name)


def device_budget(device=None) -> int:
    """Default workspace budget for the chunk scheduler: a quarter of the device memory
    that is free right now (torch.cuda.mem_get_info), so that the loss leaves most of
    the card to the rest of the step.  On an idle MI355X that admits the scheduler's
    largest chunk; on a nearly full one it shrinks the chunk instead of failing."""
    import torch
    free, _ = torch.cuda.mem_get_info(device)
    return max(int(free) // 4, 1)


def plan(desc: Desc, budget_bytes: Optional[int] = None, device=None) -> Tuple[int, int]:
    """(tokens per chunk, workspace bytes) chosen by the library's chunk scheduler for
    fckl_forward / fckl_backward.  budget_bytes None: device_budget(device); 0: the
    library's own default (12 GiB)."""
    load()      # a missing library fails first, before any device query
    if budget_bytes is None:
        budget_bytes = device_budget(device)
    c, ws = ctypes.c_int32(0), ctypes.c_size_t(0)
    _call("fckl_plan", ctypes.byref(desc), ctypes.c_size_t(budget_bytes), ctypes.byref(c), ctypes.byref(ws))
    return int(c.value), int(ws.value)


def single_plan(desc: Desc, budget_bytes: Optional[int] = None, device=None) -> Tuple[int, int]:
    """The same for fckl_forward_backward, whose workspace also holds the kept
    exponentials of the chunk (fckl_single_plan).  With desc.chunk > 0 that chunk is
    kept and its workspace size returned."""
    load()      # a missing library fails first, before any device query
    if budget_bytes is None:
        budget_bytes = device_budget(device)
    c, ws = ctypes.c_int32(0), ctypes.c_size_t(0)
    _call("fckl_single_plan", ctypes.byref(desc), ctypes.c_size_t(budget_bytes), ctypes.byref(c), ctypes.byref(ws))
    return int(c.value), int(ws.value)


def workspace_size(desc: Desc, chunk: int) -> int:
    ws = ctypes.c_size_t(0)
    _call("fckl_workspace_size", ctypes.byref(desc), ctypes.c_int32(chunk), ctypes.byref(ws))
    return int(ws.value)


# ---------------------------------------------------------------- torch-facing calls

def _check_inputs(h, W, topk_idx, topk_logit):
    import torch
    for name, t in (("h", h), ("W", W), ("topk_idx", topk_idx), ("topk_logit", topk_logit)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError("%s must be a device tensor" % name)
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
    if h.dtype != torch.bfloat16 or W.dtype != torch.bfloat16:
        raise ValueError("h and W must be bfloat16")
    if topk_idx.dtype != torch.int32:
        raise ValueError("topk_idx must be int32")
    if topk_logit.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("topk_logit must be bfloat16 or float32")
    if h.dim() != 2 or W.dim() != 2 or topk_idx.dim() != 2 or topk_logit.shape != topk_idx.shape:
        raise ValueError("expected h[N,H], W[V,H], topk_idx[N,K], topk_logit[N,K]")
    if W.shape[1] != h.shape[1] or topk_idx.shape[0] != h.shape[0]:
        raise ValueError("shape mismatch: h%s W%s topk_idx%s" % (tuple(h.shape), tuple(W.shape),
                                                                tuple(topk_idx.shape)))
    devs = {t.device for t in (h, W, topk_idx, topk_logit)}
    if len(devs) != 1:
        raise ValueError("all tensors must be on one device")


def desc_for(h, W, topk_idx, topk_logit, T: float, chunk: int = 0, flags: int = 0,
             profile: Optional[Profile] = None, vocab_slab: int = 0) -> Desc:
    import torch
    ld = DTYPE_F32 if topk_logit.dtype == torch.float32 else DTYPE_BF16
    return make_desc(h.shape[0], h.shape[1], W.shape[0], topk_idx.shape[1], T, chunk, ld, flags, profile,
                     vocab_slab)


def _stream_handle(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _out(t, shape, device, name):
    import torch
    if t is None:
        return torch.empty(shape, dtype=torch.float32, device=device)
    if t.dtype != torch.float32 or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or t.device != device:
        raise ValueError("%s must be a contiguous float32 tensor of shape %s on %s" % (name, shape, device))
    return t


def _workspace(desc: Desc, ws, device, single: bool = False):
    import torch
    if single:
        desc.chunk, need = single_plan(desc, None, device)
    elif desc.chunk == 0:
        desc.chunk, need = plan(desc, None, device)
    else:
        need = workspace_size(desc, desc.chunk)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=device)
    if ws.numel() * ws.element_size() < need or not ws.is_contiguous():
        raise ValueError("workspace of %d bytes needed" % need)
    return ws


def _weights(weights, N, device):
    """None, or a contiguous float32 [N] tensor on `device` (its pointer is passed as is)."""
    import torch
    if weights is None:
        return None
    if (not isinstance(weights, torch.Tensor) or weights.dtype != torch.float32 or tuple(weights.shape) != (N,)
            or not weights.is_contiguous() or weights.device != device):
        raise ValueError("weights must be a contiguous float32 tensor of shape (%d,) on %s" % (N, device))
    return weights


def _ptr(t):
    return None if t is None else t.data_ptr()


def forward(h, W, topk_idx, topk_logit, T: float = 1.0, chunk: int = 0, ws=None, validate: bool = False,
            loss_tok=None, lse=None, loss_mean=None, stream=None, profile: Optional[Profile] = None,
            weights=None, vocab_slab: int = 0):
    """Per-token loss, saved lse (log-sum-exp of z/T) and the mean loss (weighted when
    `weights` is given), via fckl_forward / fckl_forward_ex.  vocab_slab only sizes the
    workspace (the backward's slabs), so that one workspace serves both passes."""
    _check_inputs(h, W, topk_idx, topk_logit)
    dev = h.device
    desc = desc_for(h, W, topk_idx, topk_logit, T, chunk, FLAG_VALIDATE if validate else 0, profile, vocab_slab)
    ws = _workspace(desc, ws, dev)
    N = h.shape[0]
    weights = _weights(weights, N, dev)
    loss_tok = _out(loss_tok, (N,), dev, "loss_tok")
    lse = _out(lse, (N,), dev, "lse")
    loss_mean = _out(loss_mean, (1,), dev, "loss_mean")
    common = (h.data_ptr(), W.data_ptr(), topk_idx.data_ptr(), topk_logit.data_ptr())
    tail = (loss_tok.data_ptr(), lse.data_ptr(), loss_mean.data_ptr(), ws.data_ptr(),
            ctypes.c_size_t(ws.numel() * ws.element_size()), _stream_handle(stream))
    if weights is None:
        _call("fckl_forward", ctypes.byref(desc), *common, *tail)
    else:
        _call("fckl_forward_ex", ctypes.byref(desc), *common, weights.data_ptr(), *tail)
    return loss_tok, lse, loss_mean


def forward_noalloc(h, W, topk_idx, topk_logit, loss_tok, lse, loss_mean=None, T: float = 1.0, chunk: int = 0,
                    weights=None, validate: bool = False, stream=None):
    """The forward pass without a workspace (fckl_forward_noalloc): the chunk's buffers are
    the library's own device array.  The outputs must be given (nothing is allocated
    here either).  Returns (loss_tok, lse, loss_mean)."""
    _check_inputs(h, W, topk_idx, topk_logit)
    dev, N = h.device, h.shape[0]
    desc = desc_for(h, W, topk_idx, topk_logit, T, chunk, FLAG_VALIDATE if validate else 0)
    weights = _weights(weights, N, dev)
    loss_tok = _out(loss_tok, (N,), dev, "loss_tok")
    lse = _out(lse, (N,), dev, "lse")
    if loss_mean is not None:
        loss_mean = _out(loss_mean, (1,), dev, "loss_mean")
    _call("fckl_forward_noalloc", ctypes.byref(desc), h.data_ptr(), W.data_ptr(), topk_idx.data_ptr(),
          topk_logit.data_ptr(), _ptr(weights), loss_tok.data_ptr(), lse.data_ptr(), _ptr(loss_mean),
          _stream_handle(stream))
    return loss_tok, lse, loss_mean


def backward(h, W, topk_idx, topk_logit, lse, T: float = 1.0, grad_scale: float = 1.0, chunk: int = 0, ws=None,
             dH=None, dW=None, accumulate: bool = False, validate: bool = False, stream=None,
             profile: Optional[Profile] = None, weights=None, grad_scale_dev=None, vocab_slab: int = 0):
    """dH [N,H] and dW [V,H] (float32) of grad_scale * (weighted) mean loss, via
    fckl_backward / fckl_backward_ex.  grad_scale_dev (float32 [1] on the device) further
    multiplies grad_scale without a host read-back.  vocab_slab: vocabulary rows per
    slab (a multiple of 256, 0 = the library's choice)."""
    import torch
    _check_inputs(h, W, topk_idx, topk_logit)
    if lse.dtype != torch.float32 or tuple(lse.shape) != (h.shape[0],) or lse.device != h.device:
        raise ValueError("lse must be float32 [N] on the inputs' device")
    dev = h.device
    flags = (FLAG_VALIDATE if validate else 0) | (FLAG_DW_ACCUMULATE if accumulate else 0)
    desc = desc_for(h, W, topk_idx, topk_logit, T, chunk, flags, profile, vocab_slab)
    ws = _workspace(desc, ws, dev)
    weights = _weights(weights, h.shape[0], dev)
    if grad_scale_dev is not None and (grad_scale_dev.dtype != torch.float32 or grad_scale_dev.numel() != 1
                                       or grad_scale_dev.device != dev):
        raise ValueError("grad_scale_dev must be a float32 scalar tensor on the inputs' device")
    dH = _out(dH, tuple(h.shape), dev, "dH")
    dW = _out(dW, tuple(W.shape), dev, "dW")
    common = (h.data_ptr(), W.data_ptr(), topk_idx.data_ptr(), topk_logit.data_ptr())
    tail = (dH.data_ptr(), dW.data_ptr(), ws.data_ptr(), ctypes.c_size_t(ws.numel() * ws.element_size()),
            _stream_handle(stream))
    if weights is None and grad_scale_dev is None:
        _call("fckl_backward", ctypes.byref(desc), *common, lse.data_ptr(), ctypes.c_float(grad_scale), *tail)
    else:
        _call("fckl_backward_ex", ctypes.byref(desc), *common, _ptr(weights), lse.data_ptr(),
              ctypes.c_float(grad_scale), _ptr(grad_scale_dev), *tail)
    return dH, dW


def forward_backward(h, W, topk_idx, topk_logit, T: float = 1.0, grad_scale: float = 1.0, weights=None,
                     chunk: int = 0, ws=None, loss_tok=None, lse=None, loss_mean=None, dH=None, dW=None,
                     accumulate: bool = False, validate: bool = False, stream=None,
                     profile: Optional[Profile] = None, vocab_slab: int = 0):
    """Loss and gradients in one call (fckl_forward_backward): the logits of each chunk
    are formed once.  vocab_slab as for backward.  Returns (loss_tok, lse, loss_mean, dH, dW)."""
    _check_inputs(h, W, topk_idx, topk_logit)
    dev = h.device
    flags = (FLAG_VALIDATE if validate else 0) | (FLAG_DW_ACCUMULATE if accumulate else 0)
    desc = desc_for(h, W, topk_idx, topk_logit, T, chunk, flags, profile, vocab_slab)
    ws = _workspace(desc, ws, dev, single=True)
    N = h.shape[0]
    weights = _weights(weights, N, dev)
    loss_tok = _out(loss_tok, (N,), dev, "loss_tok")
    lse = _out(lse, (N,), dev, "lse")
    loss_mean = _out(loss_mean, (1,), dev, "loss_mean")
    dH = _out(dH, tuple(h.shape), dev, "dH")
    dW = _out(dW, tuple(W.shape), dev, "dW")
    _call("fckl_forward_backward", ctypes.byref(desc), h.data_ptr(), W.data_ptr(), topk_idx.data_ptr(),
          topk_logit.data_ptr(), _ptr(weights), ctypes.c_float(grad_scale), loss_tok.data_ptr(), lse.data_ptr(),
          loss_mean.data_ptr(), dH.data_ptr(), dW.data_ptr(), ws.data_ptr(),
          ctypes.c_size_t(ws.numel() * ws.element_size()), _stream_handle(stream))
    return loss_tok, lse, loss_mean, dH, dW


def topk_workspace_size(desc: Desc, chunk: int = 0) -> int:
    ws = ctypes.c_size_t(0)
    _call("fckl_topk_workspace_size", ctypes.byref(desc), ctypes.c_int32(chunk), ctypes.byref(ws))
    return int(ws.value)


def topk(h, W, K: int, chunk: int = 0, logits_f32: bool = False, ws=None, topk_idx=None, topk_logit=None,
         stream=None, full_first_pass: bool = False, status=None):
    """Teacher-side extraction (fckl_topk): per token the K largest z = h W^T, descending,
    equal values by the smaller index.  Returns (topk_idx int32 [N,K], topk_logit [N,K]
    bf16, or float32 with logits_f32).  full_first_pass: FCKL_FLAG_TOPK_FULL_FIRST_PASS.
    status: a one-element int32 device tensor selects fckl_topk_async (no host
    synchronisation; the call's status is written there on the stream)."""
    import torch
    for name, t in (("h", h), ("W", W)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous() or t.dtype != torch.bfloat16:
            raise ValueError("%s must be a contiguous bfloat16 device tensor" % name)
    if h.dim() != 2 or W.dim() != 2 or W.shape[1] != h.shape[1] or h.device != W.device:
        raise ValueError("expected h[N,H] and W[V,H] on one device")
    N, dev = h.shape[0], h.device
    desc = make_desc(N, h.shape[1], W.shape[0], K, 1.0, chunk, DTYPE_F32 if logits_f32 else DTYPE_BF16,
                     FLAG_TOPK_FULL_FIRST_PASS if full_first_pass else 0)
    need = topk_workspace_size(desc, chunk)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    if ws.numel() * ws.element_size() < need or not ws.is_contiguous():
        raise ValueError("workspace of %d bytes needed" % need)
    if topk_idx is None:
        topk_idx = torch.empty((N, K), dtype=torch.int32, device=dev)
    ldt = torch.float32 if logits_f32 else torch.bfloat16
    if topk_logit is None:
        topk_logit = torch.empty((N, K), dtype=ldt, device=dev)
    for name, t, dt in (("topk_idx", topk_idx, torch.int32), ("topk_logit", topk_logit, ldt)):
        if t.dtype != dt or tuple(t.shape) != (N, K) or not t.is_contiguous() or t.device != dev:
            raise ValueError("%s must be a contiguous %s tensor of shape (%d, %d)" % (name, dt, N, K))
    if status is not None:
        if (not isinstance(status, torch.Tensor) or status.dtype != torch.int32 or status.numel() != 1
                or status.device != dev):
            raise ValueError("status must be a one-element int32 tensor on the device of h")
        _call("fckl_topk_async", ctypes.byref(desc), h.data_ptr(), W.data_ptr(), topk_idx.data_ptr(),
              topk_logit.data_ptr(), ws.data_ptr(), ctypes.c_size_t(ws.numel() * ws.element_size()),
              status.data_ptr(), _stream_handle(stream))
    else:
        _call("fckl_topk", ctypes.byref(desc), h.data_ptr(), W.data_ptr(), topk_idx.data_ptr(),
              topk_logit.data_ptr(), ws.data_ptr(), ctypes.c_size_t(ws.numel() * ws.element_size()),
              _stream_handle(stream))
    return topk_idx, topk_logit


def full_plan(desc: Desc, H_teacher: int, budget_bytes: int = 0) -> Tuple[int, int]:
    """(tokens per chunk, workspace bytes) of the full-teacher variant (fckl_full_plan)."""
    c, ws = ctypes.c_int32(0), ctypes.c_size_t(0)
    _call("fckl_full_plan", ctypes.byref(desc), ctypes.c_int32(H_teacher), ctypes.c_size_t(budget_bytes),
          ctypes.byref(c), ctypes.byref(ws))
    return int(c.value), int(ws.value)


def full_forward_backward(h, W, h_t, W_t, T: float = 1.0, grad_scale: float = 1.0, weights=None, chunk: int = 0,
                          budget_bytes: int = 0, ws=None, loss_tok=None, lse=None, loss_mean=None, dH=None, dW=None,
                          accumulate: bool = False, stream=None, profile: Optional[Profile] = None,
                          vocab_slab: int = 0):
    """Online distillation against the teacher's full distribution
    (fckl_full_forward_backward): the student (h, W) and the teacher (h_t, W_t) share the
    vocabulary.  vocab_slab as for backward.  Returns (loss_tok, lse, loss_mean, dH, dW)."""
    import torch
    for name, t in (("h", h), ("W", W), ("h_t", h_t), ("W_t", W_t)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous() or t.dtype != torch.bfloat16:
            raise ValueError("%s must be a contiguous bfloat16 device tensor" % name)
        if t.dim() != 2 or t.device != h.device:
            raise ValueError("%s must be 2-D on the device of h" % name)
    N, H = h.shape
    V, Ht = W.shape[0], h_t.shape[1]
    if W.shape[1] != H or h_t.shape[0] != N or tuple(W_t.shape) != (V, Ht):
        raise ValueError("expected h[N,H], W[V,H], h_t[N,Ht], W_t[V,Ht]")
    dev = h.device
    flags = FLAG_DW_ACCUMULATE if accumulate else 0
    desc = make_desc(N, H, V, 1, T, chunk, DTYPE_BF16, flags, profile, vocab_slab)
    desc.chunk, need = full_plan(desc, Ht, budget_bytes if budget_bytes else device_budget(dev))
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    if ws.numel() * ws.element_size() < need or not ws.is_contiguous():
        raise ValueError("workspace of %d bytes needed" % need)
    weights = _weights(weights, N, dev)
    loss_tok = _out(loss_tok, (N,), dev, "loss_tok")
    lse = _out(lse, (N,), dev, "lse")
    loss_mean = _out(loss_mean, (1,), dev, "loss_mean")
    dH = _out(dH, (N, H), dev, "dH")
    dW = _out(dW, (V, H), dev, "dW")
    _call("fckl_full_forward_backward", ctypes.byref(desc), ctypes.c_int32(Ht), h.data_ptr(), W.data_ptr(),
          h_t.data_ptr(), W_t.data_ptr(), _ptr(weights), ctypes.c_float(grad_scale), loss_tok.data_ptr(),
          lse.data_ptr(), loss_mean.data_ptr(), dH.data_ptr(), dW.data_ptr(), ws.data_ptr(),
          ctypes.c_size_t(ws.numel() * ws.element_size()), _stream_handle(stream))
    return loss_tok, lse, loss_mean, dH, dW


def scale_(x, scale, stream=None):
    """x *= scale[0] in place on the device (fckl_scale); x contiguous float32, scale a
    float32 device tensor of one element.  Returns x."""
    import torch
    for name, t in (("x", x), ("scale", scale)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous() or t.dtype != torch.float32:
            raise ValueError("%s must be a contiguous float32 device tensor" % name)
    if scale.numel() != 1 or scale.device != x.device:
        raise ValueError("scale must hold one element on the device of x")
    _call("fckl_scale", x.data_ptr(), ctypes.c_int64(x.numel()), scale.data_ptr(), _stream_handle(stream))
    return x


__all__ = ["Desc", "Profile", "KERNELS", "FCKLError", "load", "plan", "single_plan", "device_budget",
           "workspace_size", "forward", "forward_noalloc", "backward",
           "forward_backward", "topk", "topk_workspace_size", "full_plan", "full_forward_backward", "scale_", "make_desc", "desc_for", "status_string", "version", "EXPORTS", "LIB_PATH"]
