"""ctypes binding of libgdr.so (the C ABI declared in include/gdr.h).

Argument marshalling only: tensors are passed as device pointers, the workspace and outputs
are allocated with torch, and every computation runs in the library's HIP kernels.  There
is no fallback: if the library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
# GDR_LIBRARY selects another build of the same C ABI (the host-sanitized one for the ABI tests)
LIB_PATH = os.environ.get("GDR_LIBRARY") or os.path.join(PKG, "libgdr.so")

GDR_OK, GDR_ERR_INVALID_ARG, GDR_ERR_UNSUPPORTED, GDR_ERR_WORKSPACE, GDR_ERR_HIP = range(5)
VARIANTS = {"deltanet": 0, "gated": 1, "kda": 2, "gdn2": 3, "gla": 4}
DTYPES = {"f32": 0, "bf16": 1}

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32


class GdrProblem(ctypes.Structure):
    _fields_ = [("variant", _i32), ("dtype", _i32), ("B", _i32), ("H", _i32), ("T", _i32),
                ("dk", _i32), ("dv", _i32), ("chunk", _i32), ("n_seqs", _i32),
                ("cu_seqlens_host", ctypes.POINTER(_i32)), ("cu_seqlens_dev", _vp),
                ("scale", ctypes.c_float), ("gates", _i32), ("qk_norm", _i32)]


class GdrInputs(ctypes.Structure):
    _fields_ = [("q", _vp), ("k", _vp), ("v", _vp), ("beta", _vp), ("alpha", _vp),
                ("erase", _vp), ("write", _vp), ("h0", _vp)]


class GdrGrads(ctypes.Structure):
    _fields_ = [("dq", _vp), ("dk", _vp), ("dv", _vp), ("dbeta", _vp), ("dalpha", _vp),
                ("derase", _vp), ("dwrite", _vp), ("dh0", _vp)]


class GdrError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


_LIB = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libgdr.so once.  Raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m gated_delta_rule_73_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    lib.gdr_workspace_size.argtypes = [P(GdrProblem), ctypes.c_int, P(ctypes.c_size_t)]
    lib.gdr_saved_size.argtypes = [P(GdrProblem), P(ctypes.c_size_t)]
    lib.gdr_forward.argtypes = [P(GdrProblem), P(GdrInputs), _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    lib.gdr_backward.argtypes = [P(GdrProblem), P(GdrInputs), _vp, _vp, _vp, P(GdrGrads), _vp,
                                 ctypes.c_size_t, _vp]
    lib.gdr_decode.argtypes = [P(GdrProblem), P(GdrInputs), _vp, _vp, _vp]
    lib.gdr_forward_residual.argtypes = [P(GdrProblem), P(GdrInputs), _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    lib.gdr_backward_residual.argtypes = [P(GdrProblem), P(GdrInputs), _vp, _vp, _vp, _vp, P(GdrGrads), _vp,
                                          ctypes.c_size_t, _vp]
    lib.gdr_forward_noalloc.argtypes = [P(GdrProblem), P(GdrInputs), _vp, _vp, _vp, _vp]
    for f in ("gdr_workspace_size", "gdr_saved_size", "gdr_forward", "gdr_backward", "gdr_decode",
              "gdr_forward_residual", "gdr_backward_residual", "gdr_forward_noalloc"):
        getattr(lib, f).restype = ctypes.c_int
    lib.gdr_status_string.argtypes = [ctypes.c_int]
    lib.gdr_status_string.restype = ctypes.c_char_p
    lib.gdr_last_error.argtypes = []
    lib.gdr_last_error.restype = ctypes.c_char_p
    lib.gdr_trace_launches.argtypes = [_vp, ctypes.c_int]
    lib.gdr_trace_launches.restype = ctypes.c_int
    lib.gdr_traced_launches.argtypes = []
    lib.gdr_traced_launches.restype = ctypes.c_int
    lib.gdr_traced_launch_name.argtypes = [ctypes.c_int]
    lib.gdr_traced_launch_name.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def _check(lib, status: int):
    if status != GDR_OK:
        raise GdrError(status, f"{lib.gdr_status_string(status).decode()}: {lib.gdr_last_error().decode()}")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def make_problem(q, v, *, variant: str, cu_seqlens=None, scale: float = 1.0, chunk: int = 64,
                 gate_logits: bool = False, qk_norm: bool = False):
    """Build a GdrProblem from the query and value tensors ([B,H,T,dk], [B,H,T,dv]).
    gate_logits: beta and alpha are logits (beta = sigmoid(x), alpha = exp(-softplus(x))).
    qk_norm: q and k are scaled to unit length per token inside the library.

    cu_seqlens: None, or a sequence / CPU tensor of n+1 int offsets.  Returns (problem,
    keepalive) where keepalive holds the host and device copies of the offsets."""
    import torch
    B, H, T, dk = q.shape
    dtype = {torch.bfloat16: "bf16", torch.float32: "f32"}[q.dtype]
    keep = []
    p = GdrProblem(variant=VARIANTS[variant], dtype=DTYPES[dtype], B=B, H=H, T=T, dk=dk,
                   dv=v.shape[-1], chunk=chunk, n_seqs=0, cu_seqlens_host=None, cu_seqlens_dev=None,
                   scale=float(scale), gates=int(bool(gate_logits)), qk_norm=int(bool(qk_norm)))
    if cu_seqlens is not None:
        host = torch.as_tensor(cu_seqlens, dtype=torch.int32).cpu().contiguous()
        dev = host.to(q.device)
        keep += [host, dev]
        p.n_seqs = host.numel() - 1
        p.cu_seqlens_host = ctypes.cast(host.data_ptr(), ctypes.POINTER(_i32))
        p.cu_seqlens_dev = dev.data_ptr()
    return p, keep


def _stream(t):
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def gdr_workspace_size(problem: GdrProblem, backward: bool) -> int:
    lib = load_library()
    n = ctypes.c_size_t(0)
    _check(lib, lib.gdr_workspace_size(ctypes.byref(problem), int(bool(backward)), ctypes.byref(n)))
    return n.value


def gdr_saved_size(problem: GdrProblem) -> int:
    lib = load_library()
    n = ctypes.c_size_t(0)
    _check(lib, lib.gdr_saved_size(ctypes.byref(problem), ctypes.byref(n)))
    return n.value


def _inputs(q, k, v, beta, alpha, erase, write, h0) -> GdrInputs:
    return GdrInputs(q=_ptr(q), k=_ptr(k), v=_ptr(v), beta=_ptr(beta), alpha=_ptr(alpha),
                     erase=_ptr(erase), write=_ptr(write), h0=_ptr(h0))


def _expect(name, t, shape, dtype, device):
    """Raise ValueError unless t is a contiguous tensor of this shape and dtype on `device`
    (None passes: presence is checked by the library)."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device} (the device of q)")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _token_shapes(p: GdrProblem, variant: str) -> dict:
    """Shapes of every tensor the ABI reads or writes, by input name (gradients share them)."""
    B, H, T, dk, dv = p.B, p.H, p.T, p.dk, p.dv
    N = p.n_seqs if p.n_seqs > 0 else B
    return {"q": (B, H, T, dk), "k": (B, H, T, dk), "v": (B, H, T, dv), "beta": (B, H, T),
            "alpha": (B, H, T, dk) if variant in ("kda", "gla") else (B, H, T), "erase": (B, H, T, dk),
            "write": (B, H, T, dv), "h0": (N, H, dv, dk), "o": (B, H, T, dv), "state": (N, H, dv, dk)}


def _validate(p: GdrProblem, variant: str, tensors: dict, require_gpu: bool = True):
    """Checks every tensor handed to the library (shape, dtype, contiguity, device) before any
    call: token tensors in q's dtype, states (h0, ht, dht, dh0) in float32."""
    import torch
    q = tensors["q"]
    if q is None or q.dim() != 4:
        raise ValueError("q must be a [B, H, T, d_k] tensor")
    if require_gpu and q.device.type != "cuda":
        raise ValueError(f"tensors must be on the GPU (q is on {q.device})")
    shapes = _token_shapes(p, variant)
    state_like = {"h0", "ht", "dht", "dh0", "state"}
    base = {"dq": "q", "dk": "k", "dv": "v", "dbeta": "beta", "dalpha": "alpha", "derase": "erase",
            "dwrite": "write", "do": "o", "r": "o", "dr": "o", "ht": "h0", "dht": "h0", "dh0": "h0"}
    for name, t in tensors.items():
        if name == "saved" or t is None:
            continue
        key = base.get(name, name)
        dtype = torch.float32 if name in state_like else q.dtype
        _expect(name, t, shapes[key], dtype, q.device)


def _check_saved(saved, p: GdrProblem, device):
    import torch
    if saved is None:
        return
    need = gdr_saved_size(p)
    if saved.dtype != torch.uint8 or saved.numel() != need or not saved.is_contiguous() or saved.device != device:
        raise ValueError(f"saved must be the contiguous uint8 buffer of {need} bytes that gdr_forward(save=True) "
                         f"returned for this problem (got {saved.dtype}, {saved.numel()} bytes, {saved.device})")


def gdr_forward(q, k, v, beta=None, alpha=None, erase=None, write=None, h0=None, *, variant: str,
                cu_seqlens=None, scale: float = 1.0, chunk: int = 64, output_final_state: bool = True,
                save: bool = False, workspace=None, residual=None, gate_logits: bool = False,
                qk_norm: bool = False, out: Optional[dict] = None):
    """Forward.  Returns (o, ht or None, saved or None).  Tensors must be contiguous and on
    the GPU; the call is asynchronous on torch's current stream.  `residual`: an optional
    [B,H,T,dv] tensor (I/O dtype) that receives r_t = v_t - v_bar_t (gdr_forward_residual).
    `out`: optional preallocated results by name ("o", "ht", "saved"), written in place."""
    import torch
    lib = load_library()
    p, keep = make_problem(q, v, variant=variant, cu_seqlens=cu_seqlens, scale=scale, chunk=chunk,
                           gate_logits=gate_logits, qk_norm=qk_norm)
    out = dict(out or {})
    N = p.n_seqs if p.n_seqs > 0 else p.B
    o = out.get("o")
    if o is None:
        o = torch.empty(q.shape[:3] + (p.dv,), dtype=q.dtype, device=q.device)
    ht = out.get("ht")
    if ht is None and output_final_state:
        ht = torch.empty((N, p.H, p.dv, p.dk), dtype=torch.float32, device=q.device)
    saved = out.get("saved")
    if saved is None and save:
        saved = torch.empty(gdr_saved_size(p), dtype=torch.uint8, device=q.device)
    _validate(p, variant, dict(q=q, k=k, v=v, beta=beta, alpha=alpha, erase=erase, write=write, h0=h0, o=o,
                               ht=ht, r=residual))
    _check_saved(saved, p, q.device)
    need = gdr_workspace_size(p, False)
    ws = workspace if workspace is not None and workspace.numel() >= need else \
        torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ins = _inputs(q, k, v, beta, alpha, erase, write, h0)
    st = lib.gdr_forward_residual(ctypes.byref(p), ctypes.byref(ins), _ptr(o), _ptr(residual), _ptr(ht),
                                  _ptr(saved), _ptr(ws), ws.numel(), _stream(q))
    _check(lib, st)
    del keep
    return o, ht, saved


def gdr_forward_noalloc(q, k, v, beta=None, alpha=None, erase=None, write=None, h0=None, *, variant: str,
                        o, ht=None, saved=None, cu_seqlens=None, scale: float = 1.0, chunk: int = 64,
                        gate_logits: bool = False, qk_norm: bool = False):
    """Forward through gdr_forward_noalloc: the caller passes the outputs (o, and optionally ht
    and saved), and the library's own scratch replaces the workspace, so the call allocates
    nothing (neither here nor in the library).  Asynchronous on torch's current stream."""
    lib = load_library()
    p, keep = make_problem(q, v, variant=variant, cu_seqlens=cu_seqlens, scale=scale, chunk=chunk,
                           gate_logits=gate_logits, qk_norm=qk_norm)
    _validate(p, variant, dict(q=q, k=k, v=v, beta=beta, alpha=alpha, erase=erase, write=write, h0=h0, o=o, ht=ht))
    _check_saved(saved, p, q.device)
    ins = _inputs(q, k, v, beta, alpha, erase, write, h0)
    st = lib.gdr_forward_noalloc(ctypes.byref(p), ctypes.byref(ins), _ptr(o), _ptr(ht), _ptr(saved), _stream(q))
    _check(lib, st)
    del keep
    return o, ht, saved


def gdr_backward(q, k, v, beta=None, alpha=None, erase=None, write=None, h0=None, do=None, dht=None, *,
                 variant: str, cu_seqlens=None, scale: float = 1.0, chunk: int = 64, saved=None,
                 want_dh0: bool = True, workspace=None, dr=None, gate_logits: bool = False,
                 qk_norm: bool = False, out: Optional[dict] = None) -> dict:
    """Backward of sum(o * do) + sum(ht * dht) [+ sum(r * dr) with the residual's gradient dr,
    gdr_backward_residual].  Returns a dict of gradients (None where the input is absent).
    `saved` is the third result of gdr_forward(save=True), or None.  `out`: optional
    preallocated gradients by name (dq, dk, dv, dbeta, dalpha, derase, dwrite, dh0)."""
    import torch
    lib = load_library()
    p, keep = make_problem(q, v, variant=variant, cu_seqlens=cu_seqlens, scale=scale, chunk=chunk,
                           gate_logits=gate_logits, qk_norm=qk_norm)
    N = p.n_seqs if p.n_seqs > 0 else p.B
    given = dict(out or {})
    e = lambda name, x: None if x is None else (given[name] if given.get(name) is not None else torch.empty_like(x))
    res = {"dq": e("dq", q), "dk": e("dk", k), "dv": e("dv", v), "dbeta": e("dbeta", beta),
           "dalpha": e("dalpha", alpha), "derase": e("derase", erase), "dwrite": e("dwrite", write)}
    res["dh0"] = given.get("dh0")
    if res["dh0"] is None and want_dh0:
        res["dh0"] = torch.empty((N, p.H, p.dv, p.dk), dtype=torch.float32, device=q.device)
    _validate(p, variant, dict(q=q, k=k, v=v, beta=beta, alpha=alpha, erase=erase, write=write, h0=h0, do=do,
                               dht=dht, dr=dr, **res))
    _check_saved(saved, p, q.device)
    g = GdrGrads(**{name: _ptr(t) for name, t in res.items()})
    need = gdr_workspace_size(p, True)
    ws = workspace if workspace is not None and workspace.numel() >= need else \
        torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ins = _inputs(q, k, v, beta, alpha, erase, write, h0)
    st = lib.gdr_backward_residual(ctypes.byref(p), ctypes.byref(ins), _ptr(do), _ptr(dr), _ptr(dht), _ptr(saved),
                                   ctypes.byref(g), _ptr(ws), ws.numel(), _stream(q))
    _check(lib, st)
    del keep
    return res


def gdr_decode(q, k, v, beta=None, alpha=None, erase=None, write=None, *, state, variant: str,
               cu_seqlens=None, scale: float = 1.0, out=None, gate_logits: bool = False):
    """Recurrent form (decoding): runs every sequence's tokens in order through its memory.
    `state` ([N,H,dv,dk] float32) is updated in place; returns o ([B,H,T,dv]).  The call is
    asynchronous on torch's current stream."""
    import torch
    lib = load_library()
    p, keep = make_problem(q, v, variant=variant, cu_seqlens=cu_seqlens, scale=scale, gate_logits=gate_logits)
    o = out if out is not None else torch.empty(q.shape[:3] + (p.dv,), dtype=q.dtype, device=q.device)
    _validate(p, variant, dict(q=q, k=k, v=v, beta=beta, alpha=alpha, erase=erase, write=write, o=o, state=state))
    ins = _inputs(q, k, v, beta, alpha, erase, write, None)
    st = lib.gdr_decode(ctypes.byref(p), ctypes.byref(ins), _ptr(state), _ptr(o), _stream(q))
    _check(lib, st)
    del keep
    return o
