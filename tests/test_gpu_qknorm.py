"""GPU parity of in-library q/k L2-normalisation (gdr_problem.qk_norm = 1) against the float64
oracle run with the same option: q and k of arbitrary per-token scale in, outputs and gradients
(w.r.t. the raw q and k) out."""
import numpy as np
import pytest

import synth
from tests._helpers import compare, gpu_inputs, to_gpu, to_np

pytestmark = pytest.mark.gpu


def _inputs(variant, dtype, d, T, B=2, H=2, cu=None, seed=71, alpha_mode="weak"):
    w = synth.Workload("qkn", variant, dtype, B, H, T, d, d, seed=seed, h0_std=0.1,
                       cu_seqlens=None if cu is None else tuple(cu))
    inp = synth.make_inputs(w, alpha_mode=alpha_mode)
    rng = np.random.default_rng(seed + 1)
    for name in ("q", "k"):  # the generator's rows have unit length: give each its own scale
        x = np.asarray(inp[name], np.float64)
        inp[name] = synth.to_io(x * rng.uniform(0.3, 3.0, size=x.shape[:-1] + (1,)), dtype)
    return inp


def _oracle(inp, variant):
    from oracle import recurrence as R
    kw = {n: inp.get(n) for n in ("q", "k", "v", "beta", "alpha", "erase", "write", "h0")}
    cu = inp.get("cu_seqlens")
    o, ht = R.forward(**kw, variant=variant, cu_seqlens=cu, qk_l2norm=True)
    ref = {"o": o, "ht": ht}
    ref.update(R.backward(**kw, do=inp["do"], variant=variant, cu_seqlens=cu, qk_l2norm=True))
    return ref


def _hip(inp, variant, dtype, use_saved):
    import torch
    from gated_delta_rule_73_amd import gdr_backward, gdr_forward
    g = gpu_inputs(inp, dtype)
    cu = inp.get("cu_seqlens")
    o, ht, saved = gdr_forward(**g, variant=variant, cu_seqlens=cu, save=use_saved, qk_norm=True)
    gr = gdr_backward(**g, do=to_gpu(inp["do"], dtype), variant=variant, cu_seqlens=cu,
                      saved=saved if use_saved else None, qk_norm=True)
    torch.cuda.synchronize()
    return {"o": to_np(o), "ht": to_np(ht), **{k: to_np(v) for k, v in gr.items()}}


CASES = [(v, dt, d, s) for v in ("deltanet", "gated", "kda", "gdn2", "gla") for dt, d in (("bf16", 128), ("f32", 64))
         for s in (True, False)]


@pytest.mark.parametrize("variant,dtype,d,use_saved", CASES,
                         ids=[f"{v}-{dt}-{d}-{'saved' if s else 'recompute'}" for v, dt, d, s in CASES])
def test_qk_norm(variant, dtype, d, use_saved):
    inp = _inputs(variant, dtype, d, T=150)
    rep = []
    compare(_hip(inp, variant, dtype, use_saved), _oracle(inp, variant), dtype, report=rep)
    print("\n".join(rep))


def test_qk_norm_packed_pipelined(monkeypatch):
    """Packed sequences (one empty, ragged tails), through the backward's per-sequence pipelines."""
    monkeypatch.setenv("GDR_PIPELINE", "1")
    cu = [0, 70, 70, 200, 333]
    inp = _inputs("gated", "bf16", 128, T=333, B=1, H=3, cu=cu)
    compare(_hip(inp, "gated", "bf16", True), _oracle(inp, "gated"), "bf16")


@pytest.mark.parametrize("variant,dtype,d", [("gated", "bf16", 128), ("deltanet", "f32", 64), ("gdn2", "bf16", 128)])
def test_qk_norm_segmented_scans(monkeypatch, variant, dtype, d):
    """Fused normalisation through the segmented scans (map pass, combine, rerun forced on),
    packed sequences with an empty one and ragged tails."""
    monkeypatch.setenv("GDR_SEG_CHUNKS", "1")
    cu = [0, 150, 150, 347]
    inp = _inputs(variant, dtype, d, T=347, B=1, H=2, cu=cu)
    compare(_hip(inp, variant, dtype, False), _oracle(inp, variant), dtype)


@pytest.mark.parametrize("variant", ["deltanet", "gated", "kda"])
def test_qk_norm_with_residual(variant):
    """Normalised q and k with the residual output and its gradient (bf16: the beta gradient's
    second pass forms A again from the normalised keys)."""
    import torch
    from gated_delta_rule_73_amd import gdr_backward, gdr_forward
    from oracle import recurrence as R
    inp = _inputs(variant, "bf16", 128, T=200)
    dr = synth.to_io(np.random.default_rng(5).standard_normal(inp["v"].shape), "bf16")
    g = gpu_inputs(inp, "bf16")
    r = torch.empty_like(g["v"])
    o, ht, saved = gdr_forward(**g, variant=variant, save=True, residual=r, qk_norm=True)
    gr = gdr_backward(**g, do=to_gpu(inp["do"], "bf16"), dr=to_gpu(dr, "bf16"), variant=variant, saved=saved,
                      qk_norm=True)
    torch.cuda.synchronize()
    got = {"o": to_np(o), "ht": to_np(ht), "r": to_np(r), **{k: to_np(v) for k, v in gr.items()}}
    kw = {n: inp.get(n) for n in ("q", "k", "v", "beta", "alpha", "erase", "write", "h0")}
    oo, hh, rr = R.forward(**kw, variant=variant, residual=True, qk_l2norm=True)
    ref = {"o": oo, "ht": hh, "r": rr}
    ref.update(R.backward(**kw, do=inp["do"], dr=dr, variant=variant, qk_l2norm=True))
    compare(got, ref, "bf16")


@pytest.mark.parametrize("env", [{"GDR_SCAN_BV": "32"}, {"GDR_PIPELINE": "1", "GDR_TSPLIT_CHUNKS": "3"}],
                         ids=["bv32", "time-split"])
def test_qk_norm_scan_tiles_and_time_split(monkeypatch, env):
    """The normalisation factors through the 32-row value-tile scans (the instantiation the
    32k-token workloads run) and through the time-split backward (one long sequence whose chunk
    gradients run part by part)."""
    for k_, v_ in env.items():
        monkeypatch.setenv(k_, v_)
    for variant in ("gated", "gdn2"):
        inp = _inputs(variant, "bf16", 128, T=600, B=1, H=2)
        compare(_hip(inp, variant, "bf16", True), _oracle(inp, variant), "bf16")


@pytest.mark.parametrize("variant", ["kda", "gla"])
def test_qk_norm_per_channel_strong_decay_packed(variant):
    """Per-channel decay strong enough that some 16-token blocks take the exact in-block sums
    (their query rows scaled inside the preparation's exact path), packed sequences with an
    empty one and ragged tails."""
    cu = [0, 70, 70, 200, 333]
    inp = _inputs(variant, "bf16", 128, T=333, B=1, H=2, cu=cu, alpha_mode="strong")
    compare(_hip(inp, variant, "bf16", True), _oracle(inp, variant), "bf16")
