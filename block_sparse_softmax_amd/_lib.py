"""ctypes binding over the C ABI in include/bss_attn.h.

Argument marshalling only: every step of the attention runs in the HIP
library.  torch supplies device memory (tensors, the workspace) and the
current stream.  If the shared library is missing or cannot be loaded, every
entry point raises; there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import numpy as np

# BSS_ATTN_CHECKED=1 loads the checked build (forward kernels with range checks; see attn_checks)
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                        "libbss_attn_checked.so" if os.environ.get("BSS_ATTN_CHECKED") == "1" else "libbss_attn.so")

ATTN_OK, ATTN_E_INVAL, ATTN_E_UNSUPPORTED, ATTN_E_WORKSPACE, ATTN_E_HIP, ATTN_E_NOMEM = 0, -1, -2, -3, -4, -5
KINDS = {"full": 0, "chunk": 1, "window": 2, "block": 3}
STATUS_NAMES = {0: "ATTN_OK", -1: "ATTN_E_INVAL", -2: "ATTN_E_UNSUPPORTED", -3: "ATTN_E_WORKSPACE",
                -4: "ATTN_E_HIP", -5: "ATTN_E_NOMEM"}

# every symbol the header declares
EXPORTS = ("attn_masked_fwd", "attn_masked_fwd_noalloc", "attn_workspace_bytes", "attn_workspace_release", "attn_plan_create", "attn_plan_tiles",
           "attn_plan_pairs", "attn_plan_schedule", "attn_plan_kernel", "attn_plan_workspace_bytes", "attn_plan_upload",
           "attn_masked_fwd_plan", "attn_masked_fwd_group", "attn_rr_workspace_bytes", "attn_rr_search",
           "attn_reorder_tokens", "attn_masked_fwd_lse", "attn_bwd_workspace_bytes", "attn_bwd_lists",
           "attn_bwd_upload",
           "attn_masked_bwd", "attn_decode_workspace_bytes", "attn_decode_fwd", "attn_checks",
           "attn_plan_destroy", "attn_last_error", "attn_version")


class AttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class AttnTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p),
                ("B", ctypes.c_int64), ("L", ctypes.c_int64), ("H", ctypes.c_int64), ("D", ctypes.c_int64),
                ("stride_b", ctypes.c_int64), ("stride_l", ctypes.c_int64), ("stride_h", ctypes.c_int64)]


class RrParams(ctypes.Structure):
    _fields_ = [("stride", ctypes.c_int64), ("block", ctypes.c_int64), ("tau", ctypes.c_float),
                ("protect_last", ctypes.c_int32)]


class MaskDesc(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("chunk", ctypes.c_int64), ("left", ctypes.c_int64), ("right", ctypes.c_int64),
                ("head_left", ctypes.POINTER(ctypes.c_int64)),
                ("block", ctypes.c_int64), ("block_mask", ctypes.POINTER(ctypes.c_uint8)),
                ("block_mask_heads", ctypes.c_int32), ("prefix", ctypes.c_int64)]


class DecodeDesc(ctypes.Structure):
    _fields_ = [("window", ctypes.c_int64), ("prefix", ctypes.c_int64)]


class Launch(ctypes.Structure):
    _fields_ = [("stream", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("softmax_scale", ctypes.c_float),
                ("start_event", ctypes.c_void_p), ("stop_event", ctypes.c_void_p)]


_lib = None
_lib_lock = threading.Lock()


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it is not built."""
    global _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(f"HIP library not built: {path} is missing (run __graft_entry__.build())")
        lib = ctypes.CDLL(path)
        P = ctypes.POINTER
        i64, i32, sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        vp = ctypes.c_void_p
        plan_p = vp
        sig = {
            "attn_masked_fwd": [P(AttnTensor), P(AttnTensor), P(AttnTensor), P(MaskDesc), vp, P(AttnTensor), P(Launch)],
            "attn_workspace_bytes": [P(MaskDesc), i64, i64, i64, P(sz)],
            "attn_workspace_release": [vp],
            "attn_masked_fwd_noalloc": [P(AttnTensor), P(AttnTensor), P(AttnTensor), P(MaskDesc), vp, P(AttnTensor),
                                        P(Launch)],
            "attn_plan_create": [P(MaskDesc), i64, i64, i64, P(plan_p)],
            "attn_plan_tiles": [plan_p, P(i32), P(i32), P(i64), P(i64), P(P(i32)), P(P(i32)), P(P(ctypes.c_uint8))],
            "attn_plan_pairs": [plan_p, P(i64), P(i64)],
            "attn_plan_schedule": [plan_p, P(i64), P(P(i32))],
            "attn_plan_kernel": [plan_p, P(i32)],
            "attn_plan_workspace_bytes": [plan_p, P(sz)],
            "attn_plan_upload": [plan_p, vp, sz, vp],
            "attn_masked_fwd_plan": [plan_p, P(AttnTensor), P(AttnTensor), P(AttnTensor), vp, P(AttnTensor), P(Launch)],
            "attn_masked_fwd_group": [i32, P(vp), P(AttnTensor), P(AttnTensor), P(AttnTensor), P(vp), P(AttnTensor),
                                      P(vp), P(sz), P(Launch)],
            "attn_rr_workspace_bytes": [P(AttnTensor), P(RrParams), P(sz)],
            "attn_rr_search": [P(AttnTensor), P(AttnTensor), P(RrParams), vp, vp, P(Launch)],
            "attn_reorder_tokens": [P(AttnTensor), i32, P(AttnTensor), i32, i64, i64, P(Launch)],
            "attn_masked_fwd_lse": [plan_p, P(AttnTensor), P(AttnTensor), P(AttnTensor), vp, P(AttnTensor), vp,
                                    P(Launch)],
            "attn_bwd_workspace_bytes": [plan_p, i64, i64, P(sz)],
            "attn_bwd_upload": [plan_p, i64, vp, sz, vp],
            "attn_bwd_lists": [plan_p, i64, P(i64), P(P(i32)), P(i64), P(P(i32)), P(i64), P(P(i32))],
            "attn_masked_bwd": [plan_p, P(AttnTensor), P(AttnTensor), P(AttnTensor), P(AttnTensor), P(AttnTensor),
                                vp, vp, P(AttnTensor), P(AttnTensor), P(AttnTensor), vp, P(Launch)],
            "attn_decode_workspace_bytes": [P(AttnTensor), P(AttnTensor), i64, P(DecodeDesc), P(sz)],
            "attn_decode_fwd": [P(AttnTensor), P(AttnTensor), P(AttnTensor), vp, i64, P(DecodeDesc), vp,
                                P(AttnTensor), P(Launch)],
            "attn_checks": [P(i32), P(ctypes.c_uint32), i32],
        }
        for name, args in sig.items():
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        lib.attn_plan_destroy.argtypes = [plan_p]
        lib.attn_plan_destroy.restype = None
        lib.attn_last_error.restype = ctypes.c_char_p
        lib.attn_version.restype = ctypes.c_char_p
        _lib = lib
        return lib


def checks(clear: bool = True):
    """(enabled, bits) of the loaded library's range checks (attn_checks); synchronize first."""
    lib = load_library()
    en, bits = ctypes.c_int32(), ctypes.c_uint32()
    _check(lib.attn_checks(ctypes.byref(en), ctypes.byref(bits), 1 if clear else 0))
    return bool(en.value), int(bits.value)


def _check(status: int):
    if status != ATTN_OK:
        msg = load_library().attn_last_error().decode()
        raise AttnError(status, msg)


def mask_key(mask: dict) -> tuple:
    """Hashable content key of a mask dict (arrays by value)."""
    items = []
    for k in sorted(mask):
        v = mask[k]
        if isinstance(v, np.ndarray):
            v = (v.shape, str(v.dtype), hash(v.tobytes()))
        elif isinstance(v, (list, tuple)):
            v = tuple(int(x) for x in v)
        items.append((k, v))
    return tuple(items)


def build_desc(mask: dict, H: int):
    """MaskDesc plus the numpy arrays it points into (keep them alive)."""
    d = MaskDesc()
    keep = []
    kind = mask["kind"]
    if kind not in KINDS:
        raise ValueError(f"unknown mask kind {kind!r}")
    d.kind = KINDS[kind]
    d.causal = 1 if mask.get("causal", False) else 0
    d.chunk = int(mask.get("chunk", 0))
    d.left = int(mask.get("left", 0))
    d.right = int(mask.get("right", 0))
    hl = mask.get("head_left")
    if hl is not None:
        arr = np.ascontiguousarray(np.asarray(hl, dtype=np.int64))
        if arr.shape != (H,):
            raise ValueError("head_left must have one entry per head")
        keep.append(arr)
        d.head_left = arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    d.block = int(mask.get("block", 0))
    bm = mask.get("block_mask")
    if bm is not None:
        arr = np.ascontiguousarray(np.asarray(bm, dtype=np.uint8))
        if arr.ndim == 2:
            arr = arr[None]
        keep.append(arr)
        d.block_mask = arr.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))
        d.block_mask_heads = arr.shape[0]
    d.prefix = int(mask.get("prefix", 0) or 0)
    return d, keep


class Plan:
    """A compiled mask for (L, H, D): tile lists, schedule, pair counts, device image."""

    def __init__(self, mask: dict, L: int, H: int, D: int):
        lib = load_library()
        self.mask, self.L, self.H, self.D = mask, L, H, D
        desc, keep = build_desc(mask, H)
        h = ctypes.c_void_p()
        _check(lib.attn_plan_create(ctypes.byref(desc), L, H, D, ctypes.byref(h)))
        self._h = h
        del keep

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.attn_plan_destroy(h)
            self._h = None

    @property
    def handle(self):
        return self._h

    def tiles(self):
        lib = load_library()
        bm, bn = ctypes.c_int32(), ctypes.c_int32()
        nr, nnz = ctypes.c_int64(), ctypes.c_int64()
        rp, kv = ctypes.POINTER(ctypes.c_int32)(), ctypes.POINTER(ctypes.c_int32)()
        fl = ctypes.POINTER(ctypes.c_uint8)()
        _check(lib.attn_plan_tiles(self._h, ctypes.byref(bm), ctypes.byref(bn), ctypes.byref(nr),
                                   ctypes.byref(nnz), ctypes.byref(rp), ctypes.byref(kv), ctypes.byref(fl)))
        n_rows, n = nr.value, nnz.value
        row_ptr = np.ctypeslib.as_array(rp, shape=(n_rows + 1,)).copy()
        kv_tile = np.ctypeslib.as_array(kv, shape=(n,)).copy() if n else np.zeros(0, np.int32)
        flags = np.ctypeslib.as_array(fl, shape=(n,)).copy() if n else np.zeros(0, np.uint8)
        return bm.value, bn.value, row_ptr, kv_tile, flags

    def pairs(self):
        lib = load_library()
        per = np.zeros(self.H, dtype=np.int64)
        tot = ctypes.c_int64()
        _check(lib.attn_plan_pairs(self._h, per.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), ctypes.byref(tot)))
        return per, tot.value

    def schedule(self):
        lib = load_library()
        n = ctypes.c_int64()
        it = ctypes.POINTER(ctypes.c_int32)()
        _check(lib.attn_plan_schedule(self._h, ctypes.byref(n), ctypes.byref(it)))
        return np.ctypeslib.as_array(it, shape=(n.value, 8)).copy() if n.value else np.zeros((0, 8), np.int32)

    def kernel(self) -> str:
        """Forward kernel of the plan's launches: "swizzled" (d 64, 80), "single" or "pingpong"."""
        lib = load_library()
        k = ctypes.c_int32()
        _check(lib.attn_plan_kernel(self._h, ctypes.byref(k)))
        return {0: "swizzled", 1: "single", 2: "pingpong"}[k.value]

    def bwd_lists(self, kv_heads: int):
        """Transposed lists of the backward: (n_blocks, col_ptr, entries, items (n, 8))."""
        lib = load_library()
        nb, ne, ni = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        cp, en, it = (ctypes.POINTER(ctypes.c_int32)() for _ in range(3))
        _check(lib.attn_bwd_lists(self._h, kv_heads, ctypes.byref(nb), ctypes.byref(cp), ctypes.byref(ne),
                                  ctypes.byref(en), ctypes.byref(ni), ctypes.byref(it)))
        col_ptr = np.ctypeslib.as_array(cp, shape=(kv_heads * nb.value + 1,)).copy()
        entries = np.ctypeslib.as_array(en, shape=(ne.value,)).copy() if ne.value else np.zeros(0, np.int32)
        items = np.ctypeslib.as_array(it, shape=(ni.value, 8)).copy() if ni.value else np.zeros((0, 8), np.int32)
        return nb.value, col_ptr, entries, items

    def workspace_bytes(self) -> int:
        lib = load_library()
        b = ctypes.c_size_t()
        _check(lib.attn_plan_workspace_bytes(self._h, ctypes.byref(b)))
        return b.value

    def upload(self, workspace, stream=None):
        """Copy the device image into `workspace` (a uint8 CUDA tensor)."""
        lib = load_library()
        _check(lib.attn_plan_upload(self._h, ctypes.c_void_p(workspace.data_ptr()),
                                    workspace.numel() * workspace.element_size(), _stream_ptr(stream, workspace)))


# ---------------------------------------------------------------------------
# torch-facing helpers
# ---------------------------------------------------------------------------

def _stream_ptr(stream, like):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(like.device)
    return ctypes.c_void_p(stream.cuda_stream)


def tensor_view(t, layout: str = "blhd") -> AttnTensor:
    """AttnTensor over a bf16 CUDA tensor stored as [B, L, H, D] ('blhd') or [B, H, L, D] ('bhld')."""
    import torch
    if t.dtype != torch.bfloat16:
        raise TypeError("attention tensors must be bfloat16")
    if not t.is_cuda:
        raise TypeError("attention tensors must be on the GPU")
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("expected a 4-d tensor with a contiguous last dimension")
    a = AttnTensor()
    a.data = t.data_ptr()
    if layout == "blhd":
        a.B, a.L, a.H, a.D = t.shape
        a.stride_b, a.stride_l, a.stride_h = t.stride(0), t.stride(1), t.stride(2)
    elif layout == "bhld":
        a.B, a.H, a.L, a.D = t.shape
        a.stride_b, a.stride_h, a.stride_l = t.stride(0), t.stride(1), t.stride(2)
    else:
        raise ValueError(layout)
    return a


def _release(workspace):
    """Tell the library that a workspace it has seen is about to be freed (its upload record goes).
    Quiet at interpreter exit, when the module's globals may already be gone."""
    try:
        if workspace is not None and _lib is not None:
            _lib.attn_workspace_release(ctypes.c_void_p(workspace.data_ptr()))
    except (TypeError, AttributeError):
        pass


class PreparedMask:
    """A plan plus a device workspace holding its uploaded image.  The workspace belongs to the stream
    it was created for (its partial states are per launch, so launches on other streams need their
    own PreparedMask)."""

    def __init__(self, mask: dict, L: int, H: int, D: int, device, stream=None):
        import torch
        self.plan = Plan(mask, L, H, D)
        stream = torch.cuda.current_stream(device) if stream is None else stream
        with torch.cuda.stream(stream):
            self.workspace = torch.empty(max(256, self.plan.workspace_bytes()), dtype=torch.uint8, device=device)
        self.plan.upload(self.workspace, stream)

    def __del__(self):
        _release(getattr(self, "workspace", None))

    def bind(self, q, k, v, o, sink=None, layout="blhd", stream=None, softmax_scale: float = 0.0):
        """Marshal the arguments once; the returned callable launches with a single C call.

        The tensors must stay alive (and keep their storage) while the callable is used.
        """
        lib = load_library()
        qv, kv, vv, ov = (tensor_view(x, layout) for x in (q, k, v, o))
        ln = Launch()
        ln.stream = _stream_ptr(stream, q).value
        ln.workspace = self.workspace.data_ptr()
        ln.workspace_bytes = self.workspace.numel()
        ln.softmax_scale = softmax_scale
        sp = _sink_ptr(sink, self.plan.H)
        args = (self.plan.handle, ctypes.byref(qv), ctypes.byref(kv), ctypes.byref(vv), sp,
                ctypes.byref(ov), ctypes.byref(ln))
        keep = (qv, kv, vv, ov, ln, q, k, v, o, sink)
        fn = lib.attn_masked_fwd_plan

        def run(start_event=None, stop_event=None):
            """Launch; optional torch.cuda.Events (already created, e.g. recorded once) are set at
            the kernel's start and end by the launch itself."""
            ln.start_event = None if start_event is None else start_event.cuda_event
            ln.stop_event = None if stop_event is None else stop_event.cuda_event
            _check(fn(*args))
            return keep[8]
        return run

    def launch(self, q, k, v, o, sink=None, layout="blhd", stream=None, softmax_scale: float = 0.0):
        lib = load_library()
        qv, kv, vv, ov = (tensor_view(x, layout) for x in (q, k, v, o))
        ln = Launch()
        ln.stream = _stream_ptr(stream, q).value
        ln.workspace = self.workspace.data_ptr()
        ln.workspace_bytes = self.workspace.numel()
        ln.softmax_scale = softmax_scale
        sp = _sink_ptr(sink, self.plan.H)
        _check(lib.attn_masked_fwd_plan(self.plan.handle, ctypes.byref(qv), ctypes.byref(kv), ctypes.byref(vv),
                                        sp, ctypes.byref(ov), ctypes.byref(ln)))
        return o


def _sink_ptr(sink, H):
    if sink is None:
        return None
    import torch
    if sink.dtype != torch.float32 or not sink.is_cuda or sink.numel() != H or not sink.is_contiguous():
        raise TypeError("sink must be a contiguous float32 CUDA tensor with one entry per head")
    return ctypes.c_void_p(sink.data_ptr())


def _f32_ptr(t, n, name):
    import torch
    if t.dtype != torch.float32 or not t.is_cuda or t.numel() != n or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous float32 CUDA tensor of {n} elements")
    return ctypes.c_void_p(t.data_ptr())


class PreparedBackward:
    """A plan plus a workspace prepared by attn_bwd_upload for batch B and kv_heads K/V heads: it serves
    the forward that also writes the row log-sum-exp (attn_masked_fwd_lse) and the backward
    (attn_masked_bwd)."""

    def __init__(self, mask: dict, L: int, H: int, D: int, B: int, kv_heads: int, device, stream=None):
        import torch
        lib = load_library()
        self.plan = Plan(mask, L, H, D)
        self.B, self.kv_heads = B, kv_heads
        nbytes = ctypes.c_size_t()
        _check(lib.attn_bwd_workspace_bytes(self.plan.handle, B, kv_heads, ctypes.byref(nbytes)))
        stream = torch.cuda.current_stream(device) if stream is None else stream
        with torch.cuda.stream(stream):
            self.workspace = torch.empty(max(256, nbytes.value), dtype=torch.uint8, device=device)
        _check(lib.attn_bwd_upload(self.plan.handle, kv_heads, ctypes.c_void_p(self.workspace.data_ptr()),
                                   self.workspace.numel(), ctypes.c_void_p(stream.cuda_stream)))

    def __del__(self):
        _release(getattr(self, "workspace", None))

    def _launch(self, like, stream, softmax_scale):
        ln = Launch()
        ln.stream = _stream_ptr(stream, like).value
        ln.workspace = self.workspace.data_ptr()
        ln.workspace_bytes = self.workspace.numel()
        ln.softmax_scale = softmax_scale
        return ln

    def bind_forward(self, q, k, v, o, lse, sink=None, layout="blhd", stream=None, softmax_scale: float = 0.0):
        """Marshal attn_masked_fwd_lse once; the returned callable launches it (lse: float32 [B, H, L])."""
        lib = load_library()
        qv, kv, vv, ov = (tensor_view(x, layout) for x in (q, k, v, o))
        lp = _f32_ptr(lse, qv.B * qv.H * qv.L, "lse")
        sp = _sink_ptr(sink, self.plan.H)
        ln = self._launch(q, stream, softmax_scale)
        args = (self.plan.handle, ctypes.byref(qv), ctypes.byref(kv), ctypes.byref(vv), sp, ctypes.byref(ov), lp,
                ctypes.byref(ln))
        keep = (qv, kv, vv, ov, ln, q, k, v, o, lse, sink)
        fn = lib.attn_masked_fwd_lse

        def run(start_event=None, stop_event=None):
            ln.start_event = None if start_event is None else start_event.cuda_event
            ln.stop_event = None if stop_event is None else stop_event.cuda_event
            _check(fn(*args))
            return keep[8], keep[9]
        return run

    def bind_backward(self, q, k, v, o, dout, lse, dq, dk, dv, sink=None, dsink=None, layout="blhd", stream=None,
                      softmax_scale: float = 0.0):
        """Marshal attn_masked_bwd once; the returned callable launches it and returns (dq, dk, dv, dsink)."""
        lib = load_library()
        views = [tensor_view(x, layout) for x in (q, k, v, o, dout, dq, dk, dv)]
        qv = views[0]
        lp = _f32_ptr(lse, qv.B * qv.H * qv.L, "lse")
        sp = _sink_ptr(sink, self.plan.H)
        dsp = None if dsink is None else _f32_ptr(dsink, self.plan.H, "dsink")
        ln = self._launch(q, stream, softmax_scale)
        args = (self.plan.handle, *(ctypes.byref(x) for x in views[:5]), lp, sp,
                *(ctypes.byref(x) for x in views[5:]), dsp, ctypes.byref(ln))
        keep = (views, ln, q, k, v, o, dout, lse, sink, (dq, dk, dv, dsink))
        fn = lib.attn_masked_bwd

        def run(start_event=None, stop_event=None):
            ln.start_event = None if start_event is None else start_event.cuda_event
            ln.stop_event = None if stop_event is None else stop_event.cuda_event
            _check(fn(*args))
            return keep[9]
        return run


_prepared_bwd = {}


def prepare_backward(mask: dict, L: int, H: int, D: int, B: int, kv_heads: int, device,
                     stream=None) -> PreparedBackward:
    """The PreparedBackward of (mask, L, H, D, B, kv_heads) for `stream` (default: the current stream),
    cached (its workspace holds per-launch statistics and partial sums, so each stream has its own)."""
    import torch
    stream = torch.cuda.current_stream(device) if stream is None else stream
    key = (mask_key(mask), L, H, D, B, kv_heads, str(device), stream.cuda_stream)
    with _prepared_lock:
        pb = _prepared_bwd.get(key)
        if pb is None:
            pb = PreparedBackward(mask, L, H, D, B, kv_heads, device, stream)
            _prepared_bwd[key] = pb
        return pb


def _shape(q, layout):
    if layout == "blhd":
        B, L, H, D = q.shape
    else:
        B, H, L, D = q.shape
    return B, L, H, D


def masked_fwd_lse(q, k, v, mask: dict, sink=None, layout: str = "blhd", stream=None, softmax_scale: float = 0.0):
    """(O, lse) of masked softmax attention: lse float32 [B, H, L] is each row's log-sum-exp (natural log,
    sink included), which masked_bwd needs."""
    import torch
    B, L, H, D = _shape(q, layout)
    kvh = k.shape[2] if layout == "blhd" else k.shape[1]
    stream = torch.cuda.current_stream(q.device) if stream is None else stream
    pb = prepare_backward(mask, L, H, D, B, kvh, q.device, stream)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, L), dtype=torch.float32, device=q.device)
    return pb.bind_forward(q, k, v, out, lse, sink=sink, layout=layout, stream=stream,
                           softmax_scale=softmax_scale)()


def masked_bwd(q, k, v, o, dout, lse, mask: dict, sink=None, layout: str = "blhd", stream=None,
               softmax_scale: float = 0.0):
    """Gradients (dq, dk, dv, dsink) of masked softmax attention (see attn_masked_bwd in
    include/bss_attn.h); dsink is None without a sink."""
    import torch
    B, L, H, D = _shape(q, layout)
    kvh = k.shape[2] if layout == "blhd" else k.shape[1]
    stream = torch.cuda.current_stream(q.device) if stream is None else stream
    pb = prepare_backward(mask, L, H, D, B, kvh, q.device, stream)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dsink = None if sink is None else torch.empty(H, dtype=torch.float32, device=q.device)
    return pb.bind_backward(q, k, v, o, dout, lse, dq, dk, dv, sink=sink, dsink=dsink, layout=layout,
                            stream=stream, softmax_scale=softmax_scale)()


def bind_group(prepared, qs, ks, vs, outs, sinks=None, layout="blhd", stream=None, softmax_scale: float = 0.0):
    """Marshal a grouped launch (attn_masked_fwd_group) of PreparedMasks once; the returned callable
    launches all of them as one kernel.  Lists are per launch; outputs must be distinct tensors."""
    lib = load_library()
    n = len(prepared)
    if not (len(qs) == len(ks) == len(vs) == len(outs) == n):
        raise ValueError("one q, k, v and output per prepared mask")
    sinks = [None] * n if sinks is None else list(sinks)
    ta = AttnTensor * n
    qv, kv, vv, ov = (ta(*(tensor_view(x, layout) for x in xs)) for xs in (qs, ks, vs, outs))
    for j, sk in enumerate(sinks):
        if sk is not None:
            import torch
            if sk.dtype != torch.float32 or not sk.is_cuda or sk.numel() != prepared[j].plan.H:
                raise TypeError("sink must be a float32 CUDA tensor with one entry per head")
    plans = (ctypes.c_void_p * n)(*(pm.plan.handle.value for pm in prepared))
    sk = (ctypes.c_void_p * n)(*(None if x is None else x.data_ptr() for x in sinks))
    ws = (ctypes.c_void_p * n)(*(pm.workspace.data_ptr() for pm in prepared))
    wb = (ctypes.c_size_t * n)(*(pm.workspace.numel() for pm in prepared))
    ln = Launch()
    ln.stream = _stream_ptr(stream, qs[0]).value
    ln.softmax_scale = softmax_scale
    keep = (qv, kv, vv, ov, plans, sk, ws, wb, ln, prepared, qs, ks, vs, outs, sinks)
    fn = lib.attn_masked_fwd_group

    def run(start_event=None, stop_event=None):
        ln.start_event = None if start_event is None else start_event.cuda_event
        ln.stop_event = None if stop_event is None else stop_event.cuda_event
        _check(fn(n, plans, qv, kv, vv, sk, ov, ws, wb, ctypes.byref(ln)))
        return keep[13]
    return run


class RrSearch:
    """RRAttention's block-pattern search (attn_rr_search) for one q/k shape and parameter set, with
    its workspace and outputs allocated once."""

    def __init__(self, q, stride: int, block: int, tau: float, protect_last: bool = True, layout: str = "blhd"):
        import torch
        lib = load_library()
        self.layout = layout
        self.prm = RrParams(stride, block, tau, 1 if protect_last else 0)
        qv = tensor_view(q, layout)
        nbytes = ctypes.c_size_t()
        _check(lib.attn_rr_workspace_bytes(ctypes.byref(qv), ctypes.byref(self.prm), ctypes.byref(nbytes)))
        self.workspace = torch.empty(max(256, nbytes.value), dtype=torch.uint8, device=q.device)
        nb = -(-qv.L // block)
        self.block_mask = torch.empty((qv.B, qv.H, nb, nb), dtype=torch.uint8, device=q.device)
        self.block_score = torch.empty((qv.B, qv.H, nb, nb), dtype=torch.float32, device=q.device)

    def __call__(self, q, k, stream=None, start_event=None, stop_event=None):
        """Queue the search; returns (block_mask uint8 [B, H, Nb, Nb], block_score float32 [B, H, Nb, Nb])."""
        lib = load_library()
        qv, kv = tensor_view(q, self.layout), tensor_view(k, self.layout)
        ln = Launch()
        ln.stream = _stream_ptr(stream, q).value
        ln.workspace = self.workspace.data_ptr()
        ln.workspace_bytes = self.workspace.numel()
        ln.start_event = None if start_event is None else start_event.cuda_event
        ln.stop_event = None if stop_event is None else stop_event.cuda_event
        _check(lib.attn_rr_search(ctypes.byref(qv), ctypes.byref(kv), ctypes.byref(self.prm),
                                  ctypes.c_void_p(self.block_mask.data_ptr()),
                                  ctypes.c_void_p(self.block_score.data_ptr()), ctypes.byref(ln)))
        return self.block_mask, self.block_score


def rr_search(q, k, stride: int, block: int, tau: float, protect_last: bool = True, layout: str = "blhd"):
    """RRAttention's block-pattern search of bf16 CUDA tensors q, k (see include/bss_attn.h):
    returns (block_mask uint8 [B, H, Nb, Nb], block_score float32 [B, H, Nb, Nb]) on the device."""
    return RrSearch(q, stride, block, tau, protect_last, layout)(q, k)


def _token_view(t) -> AttnTensor:
    """AttnTensor [B, 1, H, D] over a bf16 CUDA tensor [B, H, D] (one token per sequence)."""
    import torch
    if t.dtype != torch.bfloat16 or not t.is_cuda or t.dim() != 3 or t.stride(2) != 1:
        raise TypeError("decode queries and outputs must be bf16 CUDA tensors [B, H, D] with contiguous D")
    a = AttnTensor()
    a.data = t.data_ptr()
    a.B, a.L, a.H, a.D = t.shape[0], 1, t.shape[1], t.shape[2]
    a.stride_b, a.stride_h = t.stride(0), t.stride(1)
    a.stride_l = max(t.shape[2], t.stride(1) * t.shape[1])   # unused for one token; any valid value
    return a


class PreparedDecode:
    """attn_decode_fwd for one shape (q [B, H, D], caches [B, Lmax, Hkv, D] in `layout`), window, prefix
    and max_len, with its workspace allocated once."""

    def __init__(self, q, k_cache, max_len: int, window: int = 0, prefix: int = 0, layout: str = "blhd"):
        import torch
        lib = load_library()
        self.layout, self.max_len = layout, int(max_len)
        self.desc = DecodeDesc(int(window), int(prefix))
        qv, kv = _token_view(q), tensor_view(k_cache, layout)
        nbytes = ctypes.c_size_t()
        _check(lib.attn_decode_workspace_bytes(ctypes.byref(qv), ctypes.byref(kv), self.max_len,
                                               ctypes.byref(self.desc), ctypes.byref(nbytes)))
        self.workspace_bytes = nbytes.value
        self.workspace = torch.empty(max(256, nbytes.value), dtype=torch.uint8, device=q.device)

    def bind(self, q, k_cache, v_cache, seq_lens, o, sink=None, stream=None, softmax_scale: float = 0.0):
        """Marshal once; the returned callable launches (optional events mark the kernels)."""
        import torch
        lib = load_library()
        qv, ov = _token_view(q), _token_view(o)
        kv, vv = tensor_view(k_cache, self.layout), tensor_view(v_cache, self.layout)
        if seq_lens.dtype != torch.int32 or not seq_lens.is_cuda or seq_lens.numel() != qv.B \
                or not seq_lens.is_contiguous():
            raise TypeError("seq_lens must be a contiguous int32 CUDA tensor with one entry per sequence")
        sp = _sink_ptr(sink, qv.H)
        ln = Launch()
        ln.stream = _stream_ptr(stream, q).value
        ln.workspace = self.workspace.data_ptr()
        ln.workspace_bytes = self.workspace.numel()
        ln.softmax_scale = softmax_scale
        args = (ctypes.byref(qv), ctypes.byref(kv), ctypes.byref(vv), ctypes.c_void_p(seq_lens.data_ptr()),
                self.max_len, ctypes.byref(self.desc), sp, ctypes.byref(ov), ctypes.byref(ln))
        keep = (qv, kv, vv, ov, ln, q, k_cache, v_cache, seq_lens, o, sink)
        fn = lib.attn_decode_fwd

        def run(start_event=None, stop_event=None):
            ln.start_event = None if start_event is None else start_event.cuda_event
            ln.stop_event = None if stop_event is None else stop_event.cuda_event
            _check(fn(*args))
            return keep[9]
        return run


def decode_fwd(q, k_cache, v_cache, seq_lens, max_len: int, window: int = 0, prefix: int = 0, sink=None, out=None,
               layout: str = "blhd", stream=None, softmax_scale: float = 0.0):
    """One decode step (attn_decode_fwd): q bf16 [B, H, D] (the newest token of each sequence), caches bf16
    [B, Lmax, Hkv, D] ('blhd') or [B, Hkv, Lmax, D] ('bhld'), seq_lens int32 [B] on the device; returns
    bf16 [B, H, D]."""
    import torch
    if out is None:
        out = torch.empty_like(q)
    pd = PreparedDecode(q, k_cache, max_len, window, prefix, layout)
    pd.bind(q, k_cache, v_cache, seq_lens, out, sink=sink, stream=stream, softmax_scale=softmax_scale)()
    torch.cuda.current_stream(q.device).synchronize()   # the workspace lives until the kernels have run
    return out


ORDERS = {"raster": 0, "block_row": 1, "block_col": 2}


def reorder_tokens(x, src: str, dst: str, grid_h: int, grid_w: int, out=None, layout: str = "blhd", stream=None,
                   start_event=None, stop_event=None):
    """Re-permute the tokens of bf16 CUDA tensor x from serialisation order `src` to `dst`
    (attn_reorder_tokens; orders 'raster', 'block_row', 'block_col')."""
    import torch
    lib = load_library()
    if out is None:
        out = torch.empty_like(x)
    iv, ov = tensor_view(x, layout), tensor_view(out, layout)
    ln = Launch()
    ln.stream = _stream_ptr(stream, x).value
    ln.start_event = None if start_event is None else start_event.cuda_event
    ln.stop_event = None if stop_event is None else stop_event.cuda_event
    _check(lib.attn_reorder_tokens(ctypes.byref(iv), ORDERS[src], ctypes.byref(ov), ORDERS[dst], grid_h, grid_w,
                                   ctypes.byref(ln)))
    return out


_prepared = {}
_prepared_lock = threading.Lock()


def prepare(mask: dict, L: int, H: int, D: int, device, stream=None) -> PreparedMask:
    """The PreparedMask of (mask, L, H, D) for `stream` (default: the device's current stream), cached."""
    import torch
    stream = torch.cuda.current_stream(device) if stream is None else stream
    key = (mask_key(mask), L, H, D, str(device), stream.cuda_stream)
    with _prepared_lock:
        pm = _prepared.get(key)
        if pm is None:
            pm = PreparedMask(mask, L, H, D, device, stream)
            _prepared[key] = pm
        return pm


def masked_fwd(q, k, v, mask: dict, sink=None, out=None, layout: str = "blhd", stream=None,
               softmax_scale: float = 0.0):
    """O = masked softmax attention of bf16 CUDA tensors q, k, v (see include/bss_attn.h).

    layout 'blhd' = [B, L, H, D] (the default) or 'bhld' = [B, H, L, D].
    The compiled plan and its uploaded workspace are cached per (mask, L, H, D, device, stream).
    """
    import torch
    if layout == "blhd":
        B, L, H, D = q.shape
    else:
        B, H, L, D = q.shape
    stream = torch.cuda.current_stream(q.device) if stream is None else stream
    pm = prepare(mask, L, H, D, q.device, stream)
    if out is None:
        out = torch.empty_like(q)
    return pm.launch(q, k, v, out, sink=sink, layout=layout, stream=stream, softmax_scale=softmax_scale)


# Workspaces of the one-shot entry point, one per (device, stream), kept for the life of the process:
# the library records the plan image each holds, so repeated calls with one mask copy nothing.
_oneshot_ws = {}
_oneshot_lock = threading.Lock()


def _oneshot_workspace(device, stream, nbytes: int):
    import torch
    key = (str(device), stream.cuda_stream)
    with _oneshot_lock:
        ws = _oneshot_ws.get(key)
        if ws is None or ws.numel() < nbytes:
            _release(ws)                  # the old buffer goes back to the allocator (stream-ordered)
            with torch.cuda.stream(stream):
                ws = torch.empty(max(256, nbytes), dtype=torch.uint8, device=device)
            _oneshot_ws[key] = ws
        return ws


def masked_fwd_oneshot(q, k, v, mask: dict, sink=None, out=None, layout: str = "blhd", stream=None,
                       softmax_scale: float = 0.0):
    """The one-shot C entry point attn_masked_fwd (plan from the library's cache; the image is copied
    into the stream's workspace only when it does not hold it already).  Asynchronous."""
    import torch
    lib = load_library()
    qv, kv, vv = (tensor_view(x, layout) for x in (q, k, v))
    if out is None:
        out = torch.empty_like(q)
    ov = tensor_view(out, layout)
    desc, keep = build_desc(mask, qv.H)
    nbytes = ctypes.c_size_t()
    _check(lib.attn_workspace_bytes(ctypes.byref(desc), qv.L, qv.H, qv.D, ctypes.byref(nbytes)))
    stream = torch.cuda.current_stream(q.device) if stream is None else stream
    ws = _oneshot_workspace(q.device, stream, nbytes.value)
    ln = Launch()
    ln.stream = stream.cuda_stream
    ln.workspace = ws.data_ptr()
    ln.workspace_bytes = ws.numel()
    ln.softmax_scale = softmax_scale
    _check(lib.attn_masked_fwd(ctypes.byref(qv), ctypes.byref(kv), ctypes.byref(vv), ctypes.byref(desc),
                               _sink_ptr(sink, qv.H), ctypes.byref(ov), ctypes.byref(ln)))
    del keep
    return out
