"""ctypes binding of ``libjfa.so`` (the C ABI in include/jfa.h).

Argument marshalling only: every step of the attention path runs in the library's HIP kernels.
PyTorch provides device memory and the current stream. If the library is missing or cannot be
loaded, importing the binding raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
# torch must be loaded before libjfa.so: the library's libamdhip64 dependency then resolves to the HIP
# runtime torch already carries, so one runtime owns the device, the streams and the pointers that
# torch hands to the library. Loading the library first would bring in a second runtime.
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libjfa.so")

JFA_OK = 0
STATUS_NAMES = {0: "JFA_OK", 1: "JFA_ERR_NULL_ARG", 2: "JFA_ERR_BAD_OFFSETS", 3: "JFA_ERR_BAD_SHAPE",
                4: "JFA_ERR_UNSUPPORTED", 5: "JFA_ERR_MISALIGNED", 6: "JFA_ERR_WORKSPACE", 7: "JFA_ERR_HIP",
                8: "JFA_ERR_HOST_ONLY"}
MASKS = {"none": 0, "causal": 1}
ACTS = {"softmax": 0, "silu": 1, "gelu_tanh": 2}
BIASES = {"none": 0, "scalar": 1, "bucket": 2}
DTYPES = {"bf16": 0, "f32": 1}
PLAN_HOST_ONLY = 0x1
PLAN_NO_SPLIT = 0x2
PLAN_SHARED_Q = 0x4
PLAN_MXFP8 = 0x8
KERNELS = {"forward": 0, "combine": 1, "dkdv": 3, "dq": 4, "reduce": 5, "dbias": 6, "mx_quantize": 7, "bwd_fused": 8}
SYMBOLS = ["jfa_plan", "jfa_workspace_bytes", "jfa_forward", "jfa_backward", "jfa_backward_noalloc",
           "jfa_plan_schedule", "jfa_plan_info", "jfa_timing_enable", "jfa_timing_read", "jfa_plan_destroy",
           "jfa_status_string", "jfa_last_error"]
NOALLOC_SCRATCH_BYTES = 64 << 20  # JFA_NOALLOC_SCRATCH_BYTES


class JfaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("q_offsets_host", ctypes.POINTER(ctypes.c_int32)), ("kv_offsets_host", ctypes.POINTER(ctypes.c_int32)),
                ("mask", ctypes.c_int32), ("act", ctypes.c_int32), ("bias", ctypes.c_int32), ("scale", ctypes.c_float),
                ("out_dtype", ctypes.c_int32), ("grad_dtype", ctypes.c_int32), ("num_slots", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("window", ctypes.c_int32), ("block", ctypes.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m jagged_sequence_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i32, st = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int
    lib.jfa_plan.argtypes = [ctypes.POINTER(Problem), vp, ctypes.POINTER(vp)]
    lib.jfa_workspace_bytes.argtypes = [vp, ctypes.POINTER(sz), ctypes.POINTER(sz)]
    lib.jfa_forward.argtypes = [vp] * 9 + [vp, sz, vp]
    lib.jfa_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.jfa_backward_noalloc.argtypes = [vp] * 15
    lib.jfa_plan_schedule.argtypes = [vp, i32, ctypes.POINTER(ctypes.c_int32), sz, ctypes.POINTER(sz)]
    lib.jfa_plan_info.argtypes = [vp, ctypes.POINTER(ctypes.c_int32), sz]
    lib.jfa_timing_enable.argtypes = [vp, i32]
    lib.jfa_timing_read.argtypes = [vp, i32, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_int32)]
    lib.jfa_plan_destroy.argtypes = [vp]
    lib.jfa_plan_destroy.restype = None
    lib.jfa_status_string.argtypes = [st]
    lib.jfa_status_string.restype = ctypes.c_char_p
    lib.jfa_last_error.argtypes = []
    lib.jfa_last_error.restype = ctypes.c_char_p
    for name in ["jfa_plan", "jfa_workspace_bytes", "jfa_forward", "jfa_backward", "jfa_backward_noalloc",
                 "jfa_plan_schedule", "jfa_plan_info", "jfa_timing_enable", "jfa_timing_read"]:
        getattr(lib, name).restype = st
    return lib


LIB = _load()


def _check(status: int):
    if status != JFA_OK:
        raise JfaError(status, LIB.jfa_last_error().decode())


def _check_tensors(specs):
    """Raise ValueError unless every ``(name, tensor, shape, dtype)`` names a contiguous tensor of that
    shape and dtype, all on one GPU.

    The library sees bare pointers: a tensor of the wrong size, type or layout would make the kernels
    read or write past it, so every tensor is checked here, before the call. Shapes, dtypes and layouts
    are checked for all tensors first and devices last, so the structural checks also run on CPU
    tensors."""
    for name, t, shape, dtype in specs:
        if t is None:
            raise ValueError(f"{name} is required")
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name} must be a torch tensor")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if t.dtype != dtype:
            raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    dev = specs[0][1].device
    for name, t, _, _ in specs:
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a GPU tensor (it is on {t.device})")
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, {specs[0][0]} on {dev}")
    return dev


def _ptr(t) -> Optional[int]:
    """Device pointer of a torch tensor (or None)."""
    if t is None:
        return None
    return t.data_ptr()


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _i32(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


class Plan:
    """A jagged attention plan: validated problem plus longest-first work lists on the device."""

    def __init__(self, q_offsets, kv_offsets, num_heads: int, head_dim: int, *, mask: str = "none",
                 act: str = "softmax", bias: str = "none", scale: float = 0.0, out_dtype: str = "bf16",
                 grad_dtype: str = "bf16", num_slots: int = 0, host_only: bool = False, no_split: bool = False,
                 window: int = 0, block: int = 0, shared_q: bool = False, mxfp8: bool = False, stream=None):
        self._q_off = _i32(q_offsets)
        self._kv_off = _i32(kv_offsets)
        self.B = len(self._q_off) - 1
        self.H, self.D = int(num_heads), int(head_dim)
        self.mask, self.act, self.bias_kind = mask, act, bias
        self.window, self.block = int(window), int(block)
        self.out_dtype, self.grad_dtype = out_dtype, grad_dtype
        self.Tq = int(self._q_off[-1]) if self.B >= 0 and len(self._q_off) else 0
        self.Tkv = int(self._kv_off[-1]) if len(self._kv_off) else 0
        p = Problem()
        p.num_seqs = self.B
        p.num_heads = self.H
        p.head_dim = self.D
        p.q_offsets_host = self._q_off.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        p.kv_offsets_host = self._kv_off.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        p.mask = MASKS[mask]
        p.act = ACTS[act]
        p.bias = BIASES[bias]
        p.scale = float(scale)
        p.out_dtype = DTYPES[out_dtype]
        p.grad_dtype = DTYPES[grad_dtype]
        p.num_slots = int(num_slots)
        p.flags = (PLAN_HOST_ONLY if host_only else 0) | (PLAN_NO_SPLIT if no_split else 0) | \
            (PLAN_SHARED_Q if shared_q else 0) | (PLAN_MXFP8 if mxfp8 else 0)
        self.shared_q = bool(shared_q)
        self.mxfp8 = bool(mxfp8)
        # rows of q and dq: one shared set of Ls rows, or one set per sequence
        self.Tq_src = (int(self._q_off[1]) if self.B >= 1 else 0) if shared_q else self.Tq
        p.window = self.window
        p.block = self.block
        handle = ctypes.c_void_p()
        s = None if host_only else _stream_handle(stream)
        _check(LIB.jfa_plan(ctypes.byref(p), s, ctypes.byref(handle)))
        self._h = handle

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and LIB is not None:  # LIB is None during interpreter shutdown
            LIB.jfa_plan_destroy(h)
            self._h = None

    # ------------------------------------------------------------------ inspection
    def workspace_bytes(self) -> tuple[int, int]:
        f, b = ctypes.c_size_t(), ctypes.c_size_t()
        _check(LIB.jfa_workspace_bytes(self._h, ctypes.byref(f), ctypes.byref(b)))
        return f.value, b.value

    def schedule(self, which: int) -> np.ndarray:
        n = ctypes.c_size_t()
        _check(LIB.jfa_plan_schedule(self._h, which, None, 0, ctypes.byref(n)))
        per = 5 if which in (1, 3, 5) else 6  # 6..8: items in dispatch order
        out = np.zeros(n.value * per, dtype=np.int32)
        _check(LIB.jfa_plan_schedule(self._h, which, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), n.value,
                                     ctypes.byref(n)))
        return out.reshape(n.value, per)

    def info(self) -> dict:
        buf = (ctypes.c_int32 * 10)()
        _check(LIB.jfa_plan_info(self._h, buf, 10))
        keys = ["fwd_bm", "fwd_bn", "dq_bm", "dq_bn", "kv_bm", "kv_bn", "fwd_slots", "dq_slots", "kv_slots",
                "fused_bwd"]
        return dict(zip(keys, list(buf)))

    def timing_enable(self, on: bool = True):
        _check(LIB.jfa_timing_enable(self._h, 1 if on else 0))

    def timing_read(self, kernel: str) -> tuple[float, int]:
        ms, n = ctypes.c_float(), ctypes.c_int32()
        _check(LIB.jfa_timing_read(self._h, KERNELS[kernel], ctypes.byref(ms), ctypes.byref(n)))
        return ms.value, n.value

    # ------------------------------------------------------------------ compute
    def _workspace(self, nbytes: int, ws):
        if nbytes == 0:
            return None
        if ws is None:
            ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        return ws

    # ------------------------------------------------------------------ argument checks
    def _dtype(self, name: str):
        return torch.float32 if name == "f32" else torch.bfloat16

    def _common_specs(self, q, k, v, q_offsets, kv_offsets, bias):
        bf = torch.bfloat16
        specs = [("q", q, (self.Tq_src, self.H, self.D), bf), ("k", k, (self.Tkv, self.H, self.D), bf),
                 ("v", v, (self.Tkv, self.H, self.D), bf)]
        for name, off in (("q_offsets", q_offsets), ("kv_offsets", kv_offsets)):
            if off is not None:
                specs.append((name, off, (self.B + 1,), torch.int32))
        if self.bias_kind == "none":
            if bias is not None:
                raise ValueError("bias given to a plan without bias")
        else:
            specs.append(("bias", bias, (self.H, 64) if self.bias_kind == "bucket" else (self.H,), torch.float32))
        return specs

    def _check_workspace(self, ws, nbytes: int, dev):
        if nbytes == 0 or ws is None:
            return
        if not isinstance(ws, torch.Tensor) or not ws.is_contiguous() or ws.device != dev:
            raise ValueError("workspace must be a contiguous tensor on the inputs' device")
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError(f"workspace holds {ws.numel() * ws.element_size()} bytes, the plan needs {nbytes}")

    def forward(self, q, k, v, q_offsets, kv_offsets, bias=None, out=None, lse=None, workspace=None, stream=None):
        """Forward pass; returns (out, lse). Tensors are torch device tensors in the ABI layouts.

        ``q_offsets`` / ``kv_offsets`` are optional device copies of the planned offsets (checked
        against the plan only with JFA_DEBUG=1); every tensor is checked for shape, dtype, layout and
        device before the library is called."""
        specs = self._common_specs(q, k, v, q_offsets, kv_offsets, bias)
        if out is not None:
            specs.append(("out", out, (self.Tq, self.H, self.D), self._dtype(self.out_dtype)))
        if lse is not None:
            if self.act != "softmax":
                raise ValueError("lse is defined for softmax only")
            specs.append(("lse", lse, (self.H, self.Tq), torch.float32))
        dev = _check_tensors(specs)
        if out is None:
            out = torch.empty((self.Tq, self.H, self.D), device=q.device,
                              dtype=torch.float32 if self.out_dtype == "f32" else torch.bfloat16)
        if lse is None and self.act == "softmax":
            lse = torch.empty((self.H, self.Tq), device=q.device, dtype=torch.float32)
        fwd_bytes, _ = self.workspace_bytes()
        self._check_workspace(workspace, fwd_bytes, dev)
        ws = self._workspace(fwd_bytes, workspace)
        _check(LIB.jfa_forward(self._h, _ptr(q), _ptr(k), _ptr(v), _ptr(q_offsets), _ptr(kv_offsets), _ptr(bias),
                               _ptr(out), _ptr(lse), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                               _stream_handle(stream)))
        return out, lse

    def backward(self, q, k, v, q_offsets, kv_offsets, bias, out, lse, dout, dq=None, dk=None, dv=None,
                 workspace=None, stream=None, dbias=None):
        """Backward pass; returns (dq, dk, dv), or (dq, dk, dv, dbias) when ``dbias`` is given.

        ``dbias`` is None (no bias gradient), True (allocate it) or an fp32 device tensor of the
        bias shape that receives the gradient.
        """
        specs = self._common_specs(q, k, v, q_offsets, kv_offsets, bias)
        specs.append(("dout", dout, (self.Tq, self.H, self.D), torch.bfloat16))
        if self.act == "softmax":
            specs += [("out", out, (self.Tq, self.H, self.D), self._dtype(self.out_dtype)),
                      ("lse", lse, (self.H, self.Tq), torch.float32)]
        gdt = self._dtype(self.grad_dtype)
        for name, t, T in (("dq", dq, self.Tq_src), ("dk", dk, self.Tkv), ("dv", dv, self.Tkv)):
            if t is not None:
                specs.append((name, t, (T, self.H, self.D), gdt))
        if dbias is not None and dbias is not False:
            if self.bias_kind == "none":
                raise ValueError("dbias requested from a plan without bias")
            if isinstance(dbias, torch.Tensor):
                specs.append(("dbias", dbias, (self.H, 64) if self.bias_kind == "bucket" else (self.H,),
                              torch.float32))
        dev = _check_tensors(specs)
        if dq is None:
            dq = torch.empty((self.Tq_src, self.H, self.D), device=q.device, dtype=gdt)
        if dk is None:
            dk = torch.empty((self.Tkv, self.H, self.D), device=q.device, dtype=gdt)
        if dv is None:
            dv = torch.empty((self.Tkv, self.H, self.D), device=q.device, dtype=gdt)
        want_db = dbias is not None and dbias is not False
        if dbias is True:
            shape = (self.H, 64) if self.bias_kind == "bucket" else (self.H,)
            dbias = torch.empty(shape, device=q.device, dtype=torch.float32)
        _, bwd_bytes = self.workspace_bytes()
        self._check_workspace(workspace, bwd_bytes, dev)
        ws = self._workspace(bwd_bytes, workspace)
        _check(LIB.jfa_backward(self._h, _ptr(q), _ptr(k), _ptr(v), _ptr(q_offsets), _ptr(kv_offsets), _ptr(bias),
                                _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                                _ptr(dbias) if want_db else None, _ptr(ws),
                                0 if ws is None else ws.numel() * ws.element_size(), _stream_handle(stream)))
        return (dq, dk, dv, dbias) if want_db else (dq, dk, dv)


def _backward_noalloc(plan: "Plan", q, k, v, q_offsets, kv_offsets, bias, out, lse, dout, dq=None, dk=None, dv=None,
                      stream=None, dbias=None):
    specs = plan._common_specs(q, k, v, q_offsets, kv_offsets, bias)
    specs.append(("dout", dout, (plan.Tq, plan.H, plan.D), torch.bfloat16))
    if plan.act == "softmax":
        specs += [("out", out, (plan.Tq, plan.H, plan.D), plan._dtype(plan.out_dtype)),
                  ("lse", lse, (plan.H, plan.Tq), torch.float32)]
    gdt = plan._dtype(plan.grad_dtype)
    for name, t, T in (("dq", dq, plan.Tq_src), ("dk", dk, plan.Tkv), ("dv", dv, plan.Tkv)):
        specs.append((name, t, (T, plan.H, plan.D), gdt))
    if dbias is not None:
        if plan.bias_kind == "none":
            raise ValueError("dbias requested from a plan without bias")
        specs.append(("dbias", dbias, (plan.H, 64) if plan.bias_kind == "bucket" else (plan.H,), torch.float32))
    _check_tensors(specs)
    _check(LIB.jfa_backward_noalloc(plan._h, _ptr(q), _ptr(k), _ptr(v), _ptr(q_offsets), _ptr(kv_offsets), _ptr(bias),
                                    _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbias),
                                    _stream_handle(stream)))
    return (dq, dk, dv, dbias) if dbias is not None else (dq, dk, dv)


# ---------------------------------------------------------------------- C-named entry points
def jfa_plan(q_offsets, kv_offsets, num_heads: int, head_dim: int, **kw) -> Plan:
    """``jfa_plan``: validate the problem and build the device work lists (see :class:`Plan`)."""
    return Plan(q_offsets, kv_offsets, num_heads, head_dim, **kw)


def jfa_forward(plan: Plan, q, k, v, q_offsets, kv_offsets, bias=None, out=None, lse=None, workspace=None,
                stream=None):
    """``jfa_forward``: returns (out, lse)."""
    return plan.forward(q, k, v, q_offsets, kv_offsets, bias, out, lse, workspace, stream)


def jfa_backward(plan: Plan, q, k, v, q_offsets, kv_offsets, bias, out, lse, dout, dq=None, dk=None, dv=None,
                 workspace=None, stream=None, dbias=None):
    """``jfa_backward``: returns (dq, dk, dv), plus dbias when it is requested."""
    return plan.backward(q, k, v, q_offsets, kv_offsets, bias, out, lse, dout, dq, dk, dv, workspace, stream, dbias)


def jfa_backward_noalloc(plan: Plan, q, k, v, q_offsets, kv_offsets, bias, out, lse, dout, dq, dk, dv, stream=None,
                         dbias=None):
    """``jfa_backward_noalloc``: the backward pass into caller-given dq / dk / dv (and dbias) with the
    library's static scratch array as workspace; allocates nothing. Returns (dq, dk, dv[, dbias])."""
    return _backward_noalloc(plan, q, k, v, q_offsets, kv_offsets, bias, out, lse, dout, dq, dk, dv, stream, dbias)
