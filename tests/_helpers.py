"""Shared helpers for the parity tests: moving seeded inputs to the GPU, running the HIP path
through the C ABI binding, running the oracle, and comparing."""
from __future__ import annotations

import numpy as np

GRAD_NAMES = ("dq", "dk", "dv", "dbeta", "dalpha", "derase", "dwrite", "dh0")
INPUT_NAMES = ("q", "k", "v", "beta", "alpha", "erase", "write", "h0")


def to_gpu(x, dtype: str):
    import torch
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def gpu_inputs(inp: dict, dtype: str) -> dict:
    """Token tensors in the I/O dtype; states (h0) always float32."""
    out = {}
    for name in INPUT_NAMES:
        out[name] = to_gpu(inp.get(name), "f32" if name == "h0" else dtype)
    return out


def to_np(t):
    return None if t is None else t.float().cpu().numpy().astype(np.float64)


def run_hip(inp: dict, variant: str, dtype: str, *, backward: bool, scale: float = 1.0, dht=None,
            use_saved: bool = True):
    import torch
    from gated_delta_rule_73_amd import gdr_backward, gdr_forward
    g = gpu_inputs(inp, dtype)
    cu = inp.get("cu_seqlens")
    o, ht, saved = gdr_forward(**g, variant=variant, cu_seqlens=cu, scale=scale, save=backward and use_saved)
    res = {"o": to_np(o), "ht": to_np(ht)}
    if backward:
        do = to_gpu(inp["do"], dtype)
        dh = None if dht is None else to_gpu(dht, "f32")
        grads = gdr_backward(**g, do=do, dht=dh, variant=variant, cu_seqlens=cu, scale=scale,
                             saved=saved if use_saved else None)
        for name, t in grads.items():
            res[name] = to_np(t)
    torch.cuda.synchronize()
    return res


def run_oracle(inp: dict, variant: str, *, backward: bool, scale: float = 1.0, dht=None):
    from oracle import recurrence as R
    kw = {name: inp.get(name) for name in INPUT_NAMES}
    cu = inp.get("cu_seqlens")
    o, ht = R.forward(**kw, variant=variant, cu_seqlens=cu, scale=scale)
    res = {"o": o, "ht": ht}
    if backward:
        g = R.backward(**kw, do=inp["do"], dht=dht, variant=variant, cu_seqlens=cu, scale=scale)
        res.update(g)
    return res


RELRMS_TOL = {"f32": 1e-4, "bf16": 1e-2}


def compare(got: dict, ref: dict, dtype: str, names=None, report=None):
    """Per-tensor parity, two bounds that must both hold.
    Largest error: float32 I/O max|err| / max|ref| <= 1e-4 (normwise); bfloat16 I/O
    max|err| <= 2e-2 * max(1, max|ref|) (the absolute 2e-2 bound wherever the reference stays
    within [-1, 1]; relative to the tensor's largest value beyond that).
    Relative RMS error ||err||_2 / ||ref||_2 <= 1e-4 (float32) or 1e-2 (bfloat16), so that an
    error spread over the small entries of a tensor is not hidden by the slack its largest
    entry gives the max bound (skipped for an all-zero reference, where the max bound is
    absolute)."""
    failures = []
    for name in names or ref.keys():
        r = ref.get(name)
        g = got.get(name)
        if r is None:
            continue
        assert g is not None, f"{name}: missing from the HIP result"
        assert g.shape == r.shape, f"{name}: shape {g.shape} vs {r.shape}"
        assert np.all(np.isfinite(g)), f"{name}: non-finite values"
        err = np.max(np.abs(g - r)) if r.size else 0.0
        mref = np.max(np.abs(r)) if r.size else 0.0
        rrms = (np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30)) if r.size else 0.0
        if dtype == "f32":
            tol = 1e-4 * mref
        else:
            tol = 2e-2 * max(1.0, mref)
        rtol = RELRMS_TOL[dtype]
        rms_ok = (not r.size) or np.linalg.norm(r) == 0 or rrms <= rtol
        line = (f"{name:7s} max|err|={err:.3e} max|ref|={mref:.3e} relrms={rrms:.3e} tol={tol:.3e} "
                f"relrms_tol={rtol:.0e}")
        if report is not None:
            report.append(line)
        if not (err <= tol and rms_ok):
            failures.append(line)
    assert not failures, "parity failures:\n" + "\n".join(failures)
