"""GPU parity of the erase-free memory with a decay per key channel (variant "gla",
W <- W diag(alpha) + beta v k^T): no key Gram and no triangular solve in its kernels.  Against the
float64 oracle for both I/O types and head sizes, with strong, weak and very strong decay, with
and without beta, an initial memory and a final-memory gradient; packed sequences through forced
segmented scans and both scan tile heights; logit gates; decoding; the full-size workload."""
import numpy as np
import pytest

import synth
from tests._helpers import compare, run_hip, run_oracle

pytestmark = pytest.mark.gpu


def _w(dtype, d, *, B=2, H=2, T=190, seed=91, has_beta=True, cu=None, h0=0.5):
    return synth.Workload("gla", "gla", dtype, B, H, T, d, d, seed=seed, has_beta=has_beta, h0_std=h0,
                          cu_seqlens=cu)


CASES = [(dt, d, m, b) for dt, d in (("bf16", 128), ("f32", 64), ("bf16", 64)) for m in ("config", "weak", "strong")
         for b in (True, False)]


@pytest.mark.parametrize("dtype,d,alpha_mode,with_beta", CASES,
                         ids=[f"{dt}-{d}-{m}-{'beta' if b else 'nobeta'}" for dt, d, m, b in CASES])
def test_gla_fwd_bwd(dtype, d, alpha_mode, with_beta):
    w = _w(dtype, d, has_beta=with_beta)
    inp = synth.make_inputs(w, alpha_mode=alpha_mode)
    dht = np.random.default_rng(3).standard_normal((2, 2, d, d)).astype(np.float32) * 0.2
    rep = []
    compare(run_hip(inp, "gla", dtype, backward=True, dht=dht, scale=0.8),
            run_oracle(inp, "gla", backward=True, dht=dht, scale=0.8), dtype, report=rep)
    print("\n".join(rep))


def test_gla_saved_and_recomputed_agree_bitwise():
    inp = synth.make_inputs(_w("bf16", 128, T=200), alpha_mode="weak")
    a = run_hip(inp, "gla", "bf16", backward=True, use_saved=True)
    b = run_hip(inp, "gla", "bf16", backward=True, use_saved=False)
    for name in a:
        if a[name] is not None:
            assert np.array_equal(a[name], b[name]), name


@pytest.mark.parametrize("bv", [16, 32])
@pytest.mark.parametrize("lseg", [0, 1])
def test_gla_packed_segmented(monkeypatch, bv, lseg):
    """Packed sequences (an empty one, ragged tails); segmented scans forced on or off; both
    value-tile heights."""
    monkeypatch.setenv("GDR_SCAN_BV", str(bv))
    monkeypatch.setenv("GDR_SEG_CHUNKS", str(lseg))
    cu = (0, 70, 70, 200, 333)
    inp = synth.make_inputs(_w("bf16", 128, B=1, H=3, T=333, cu=cu), alpha_mode="weak")
    dht = np.random.default_rng(4).standard_normal((4, 3, 128, 128)).astype(np.float32) * 0.1
    compare(run_hip(inp, "gla", "bf16", backward=True, dht=dht), run_oracle(inp, "gla", backward=True, dht=dht),
            "bf16")


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_gla_gate_logits(dtype, d):
    import torch
    from gated_delta_rule_73_amd import gdr_backward, gdr_forward
    from oracle import recurrence as R
    from tests._helpers import gpu_inputs, to_gpu, to_np
    inp = synth.make_inputs(_w(dtype, d, T=150, h0=0.1), alpha_mode="weak", gate_logits=True)
    g = gpu_inputs(inp, dtype)
    o, ht, saved = gdr_forward(**g, variant="gla", save=True, gate_logits=True)
    gr = gdr_backward(**g, do=to_gpu(inp["do"], dtype), variant="gla", saved=saved, gate_logits=True)
    torch.cuda.synchronize()
    got = {"o": to_np(o), "ht": to_np(ht), **{k: to_np(v) for k, v in gr.items()}}
    kw = {n: inp.get(n) for n in ("q", "k", "v", "beta", "alpha", "erase", "write", "h0")}
    oo, hh = R.forward(**kw, variant="gla", gate_logits=True)
    ref = {"o": oo, "ht": hh, **R.backward(**kw, do=inp["do"], variant="gla", gate_logits=True)}
    compare(got, ref, dtype)


def test_gla_decode_continues_a_prefill():
    """Prefill through the chunked forward, then decode the next tokens from its ht: equal to
    one oracle run over all the tokens."""
    import torch
    from gated_delta_rule_73_amd import gdr_decode, gdr_forward
    from tests._helpers import gpu_inputs, to_np
    w = _w("bf16", 128, B=2, H=2, T=133)
    inp = synth.make_inputs(w, alpha_mode="weak")
    pre = {n: (None if inp.get(n) is None or n in ("h0", "cu_seqlens", "do") else inp[n][:, :, :128])
           for n in inp}
    pre["h0"] = inp["h0"]
    g = gpu_inputs(pre, "bf16")
    o1, ht, _ = gdr_forward(**g, variant="gla")
    post = {n: (None if inp.get(n) is None or n in ("h0", "cu_seqlens", "do") else inp[n][:, :, 128:]) for n in inp}
    gp = gpu_inputs(post, "bf16")
    gp.pop("h0")
    o2 = gdr_decode(**gp, state=ht, variant="gla")
    torch.cuda.synchronize()
    ref = run_oracle(inp, "gla", backward=False)
    got = {"o": np.concatenate([to_np(o1), to_np(o2)], axis=2), "ht": to_np(ht)}
    compare(got, ref, "bf16")


def test_gla_rejects_a_residual():
    import torch
    from gated_delta_rule_73_amd import GdrError, gdr_forward
    from tests._helpers import gpu_inputs
    inp = synth.make_inputs(_w("bf16", 128, T=64), alpha_mode="weak")
    g = gpu_inputs(inp, "bf16")
    with pytest.raises(GdrError):
        gdr_forward(**g, variant="gla", residual=torch.empty_like(g["v"]))


def test_gla_qk_norm():
    from tests.test_gpu_qknorm import _hip, _inputs, _oracle
    inp = _inputs("gla", "bf16", 128, T=150)
    compare(_hip(inp, "gla", "bf16", True), _oracle(inp, "gla"), "bf16")


def test_gla_fullsize_sampled():
    """The B=4 H=16 T=8192 erase-free workload at full size, in the bench's launch configuration,
    every output NaN-prefilled; sampled (sequence, head) pairs against the oracle."""
    from tests.test_gpu_fullsize import _check_samples, _run_full
    w = synth.EXTRA_WORKLOADS["gla_B4H16T8192"]
    inp = synth.make_inputs(w)
    got = _run_full(w, inp)
    _check_samples(w.name, w, inp, got, [(0, 0), (3, 15)])
