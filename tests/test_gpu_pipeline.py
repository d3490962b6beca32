"""Per-sequence pipelines in the backward (GDR_PIPELINE=1): packed sequences cut into contiguous
ranges whose reverse scans and chunk-parallel gradients run as sub-problems on separate streams
(with the forward's recompute when nothing was saved).  Every unit is computed by the same kernels from the same
operands either way, so the results must equal the single-stream results bit for bit (whose
parity with the float64 oracle the other GPU tests establish); the gradient residual case is
checked against the oracle as well."""
import numpy as np
import pytest

import synth
from tests._helpers import compare, gpu_inputs, to_gpu, to_np

pytestmark = pytest.mark.gpu


def _run(inp, variant, dtype, use_saved, scale, dr=None):
    import torch
    from gated_delta_rule_73_amd import gdr_backward, gdr_forward
    g = gpu_inputs(inp, dtype)
    cu = inp["cu_seqlens"]
    r = torch.empty_like(g["v"]) if dr is not None else None
    o, ht, saved = gdr_forward(**g, variant=variant, cu_seqlens=cu, scale=scale, save=use_saved, residual=r)
    gr = gdr_backward(**g, do=to_gpu(inp["do"], dtype), variant=variant, cu_seqlens=cu, scale=scale,
                      saved=saved if use_saved else None, dr=None if dr is None else to_gpu(dr, dtype))
    torch.cuda.synchronize()
    out = {"o": to_np(o), "ht": to_np(ht), **{k: to_np(v) for k, v in gr.items() if v is not None}}
    if r is not None:
        out["r"] = to_np(r)
    return out


# lengths: ragged tails, one long sequence among short ones, more sequences than streams
CASES = [
    ("gated", "bf16", 128, (0, 64 * 5 + 17, 64 * 7, 64 * 19 + 3, 64 * 22), True),
    ("gated", "bf16", 128, (0, 100, 64 * 12), False),
    ("deltanet", "bf16", 64, (0, 30, 64 * 3, 64 * 3 + 1, 64 * 9, 64 * 10 + 50, 64 * 16, 64 * 17), True),
    ("gated", "f32", 64, (0, 64 * 2 + 5, 64 * 9, 64 * 10, 64 * 13 + 33), False),
]


@pytest.mark.parametrize("variant,dtype,d,cu,use_saved", CASES,
                         ids=[f"{c[0]}-{c[1]}-{c[2]}-n{len(c[3]) - 1}-{'saved' if c[4] else 'recompute'}"
                              for c in CASES])
def test_pipelined_equals_single_stream(monkeypatch, variant, dtype, d, cu, use_saved):
    w = synth.Workload("pipe", variant, dtype, 1, 3, cu[-1], d, d, seed=61, h0_std=0.1, cu_seqlens=cu)
    inp = synth.make_inputs(w, alpha_mode="weak")
    monkeypatch.delenv("GDR_PIPELINE", raising=False)
    ref = _run(inp, variant, dtype, use_saved, 0.9)
    monkeypatch.setenv("GDR_PIPELINE", "1")
    got = _run(inp, variant, dtype, use_saved, 0.9)
    assert set(got) == set(ref)
    for k in ref:
        assert np.array_equal(got[k], ref[k], equal_nan=True), k


@pytest.mark.parametrize("variant", ["deltanet", "gated"])
def test_pipelined_residual_bf16_equals_single_stream(monkeypatch, variant):
    """bfloat16 residual gradient (its beta gradient formed in a second pass from dR without the
    residual's term, recorded per range) through the pipelines: bitwise the single-stream result."""
    cu = (0, 64 * 3 + 7, 64 * 5, 64 * 11 + 40)
    w = synth.Workload("pipe", variant, "bf16", 1, 2, cu[-1], 128, 128, seed=64, h0_std=0.1, cu_seqlens=cu)
    inp = synth.make_inputs(w, alpha_mode="weak")
    dr = synth.to_io(np.random.default_rng(65).standard_normal(inp["v"].shape), "bf16")
    monkeypatch.delenv("GDR_PIPELINE", raising=False)
    ref = _run(inp, variant, "bf16", True, 1.0, dr=dr)
    monkeypatch.setenv("GDR_PIPELINE", "1")
    got = _run(inp, variant, "bf16", True, 1.0, dr=dr)
    for k in ref:
        assert np.array_equal(got[k], ref[k], equal_nan=True), k


def test_pipelined_residual_against_oracle(monkeypatch):
    from oracle import recurrence as R
    cu = (0, 64 + 9, 64 * 4, 64 * 6 + 2)
    w = synth.Workload("pipe", "gated", "f32", 1, 2, cu[-1], 64, 64, seed=62, h0_std=0.1, cu_seqlens=cu)
    inp = synth.make_inputs(w, alpha_mode="weak")
    dr = synth.to_io(np.random.default_rng(63).standard_normal(inp["v"].shape), "f32")
    monkeypatch.setenv("GDR_PIPELINE", "1")
    got = _run(inp, "gated", "f32", True, 1.0, dr=dr)
    kw = {n: inp.get(n) for n in ("q", "k", "v", "beta", "alpha", "erase", "write", "h0")}
    o, ht, r = R.forward(**kw, variant="gated", cu_seqlens=inp["cu_seqlens"], residual=True)
    ref = {"o": o, "ht": ht, "r": r}
    ref.update(R.backward(**kw, do=inp["do"], dr=dr, variant="gated", cu_seqlens=inp["cu_seqlens"]))
    rep = []
    compare(got, ref, "f32", report=rep)
    print("\n".join(rep))


# Time-split backward (ScanSeg mode 3): the reverse scan in parts of GDR_TSPLIT_CHUNKS chunks,
# each finished part's chunk gradients on a side stream.  Parts of three chunks give several
# parts with a ragged last one; the carried state crosses parts in float32, so the results are
# bitwise the single-stream ones.  GDR_PIPELINE=2 takes the time split also for packed
# sequences (whose part counts then differ, one of them empty).
TS_CASES = [
    ("gated", "bf16", 128, 1, 64 * 13 + 21, None, True),
    ("gated", "bf16", 128, 1, 64 * 10, None, False),
    ("deltanet", "bf16", 64, 2, 64 * 9 + 5, None, True),
    ("gated", "f32", 64, 1, 64 * 11, (0, 64 * 3 + 5, 64 * 3 + 5, 64 * 11), True),
    ("deltanet", "bf16", 128, 1, 64 * 12 + 7, (0, 64 * 8 + 7, 64 * 12 + 7), False),
]


@pytest.mark.parametrize("variant,dtype,d,B,T,cu,use_saved", TS_CASES,
                         ids=[f"{c[0]}-{c[1]}-{c[2]}-B{c[3]}-T{c[4]}-{'packed' if c[5] else 'dense'}-"
                              f"{'saved' if c[6] else 'recompute'}" for c in TS_CASES])
def test_time_split_equals_single_stream(monkeypatch, variant, dtype, d, B, T, cu, use_saved):
    w = synth.Workload("tsplit", variant, dtype, B, 2, T, d, d, seed=71, h0_std=0.5, cu_seqlens=cu)
    inp = synth.make_inputs(w, alpha_mode="weak")
    monkeypatch.delenv("GDR_PIPELINE", raising=False)
    monkeypatch.delenv("GDR_TSPLIT_CHUNKS", raising=False)
    ref = _run(inp, variant, dtype, use_saved, 0.9)
    monkeypatch.setenv("GDR_PIPELINE", "2" if cu else "1")
    monkeypatch.setenv("GDR_TSPLIT_CHUNKS", "3")
    got = _run(inp, variant, dtype, use_saved, 0.9)
    assert set(got) == set(ref)
    for k in ref:
        assert np.array_equal(got[k], ref[k], equal_nan=True), k
