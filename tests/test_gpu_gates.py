"""GPU parity with the gates given as logits (gdr_problem.gates = 1): beta = sigmoid(x) and
alpha = exp(-softplus(x)) are applied inside the kernels and the gradients come back w.r.t.
the logits.  The float64 reference is the oracle run on the same (rounded) logits with
gate_logits=True: it applies the same maps and carries its gate gradients to the logits by the
chain rule (both pinned against closed forms and finite differences in the oracle's tests)."""
import numpy as np
import pytest

import synth
from tests._helpers import compare, run_hip

pytestmark = pytest.mark.gpu


def _oracle(inp, variant, backward, cu=None, scale=1.0):
    from oracle import recurrence as R
    kw = {n: inp.get(n) for n in ("q", "k", "v", "beta", "alpha", "erase", "write", "h0")}
    o, ht = R.forward(**kw, variant=variant, cu_seqlens=cu, scale=scale, gate_logits=True)
    ref = {"o": o, "ht": ht}
    if backward:
        ref.update(R.backward(**kw, do=inp["do"], variant=variant, cu_seqlens=cu, scale=scale, gate_logits=True))
    return ref


def _hip(inp, variant, dtype, backward, use_saved=True, scale=1.0):
    import torch
    from gated_delta_rule_73_amd import gdr_backward, gdr_forward
    from tests._helpers import gpu_inputs, to_gpu, to_np
    g = gpu_inputs(inp, dtype)
    cu = inp.get("cu_seqlens")
    o, ht, saved = gdr_forward(**g, variant=variant, cu_seqlens=cu, scale=scale, save=backward and use_saved,
                               gate_logits=True)
    res = {"o": to_np(o), "ht": to_np(ht)}
    if backward:
        gr = gdr_backward(**g, do=to_gpu(inp["do"], dtype), variant=variant, cu_seqlens=cu, scale=scale,
                          saved=saved if use_saved else None, gate_logits=True)
        res.update({k: to_np(v) for k, v in gr.items()})
    torch.cuda.synchronize()
    return res


CASES = [(v, dt, d, m, s) for v in ("deltanet", "gated", "kda", "gdn2") for dt, d in (("bf16", 128), ("f32", 64))
         for m in ("config", "weak") for s in (True, False)]


@pytest.mark.parametrize("variant,dtype,d,alpha_mode,use_saved", CASES,
                         ids=[f"{v}-{dt}-{d}-{m}-{'saved' if s else 'recompute'}" for v, dt, d, m, s in CASES])
def test_gate_logits_fwd_bwd(variant, dtype, d, alpha_mode, use_saved):
    w = synth.Workload("lg", variant, dtype, 2, 2, 150, d, d, seed=61, h0_std=0.1)
    inp = synth.make_inputs(w, alpha_mode=alpha_mode, gate_logits=True)
    rep = []
    compare(_hip(inp, variant, dtype, True, use_saved, scale=0.9), _oracle(inp, variant, True, scale=0.9), dtype,
            report=rep)
    print("\n".join(rep))


def test_gate_logits_packed_bench_shape_sample():
    """The packed long-context workload with logits, one (sequence, head) sample checked."""
    w = synth.WORKLOADS["gated_varlen_T32768"]
    inp = synth.make_inputs(w, gate_logits=True)
    got = _hip(inp, "gated", "bf16", True)
    cu = inp["cu_seqlens"]
    s, h = 1, 7
    t0, t1 = int(cu[s]), int(cu[s + 1])
    sub = {n: (None if inp.get(n) is None else inp[n][:, h:h + 1, t0:t1]) for n in ("q", "k", "v", "beta", "alpha", "do")}
    sub["h0"] = inp["h0"][s:s + 1, h:h + 1]
    ref = _oracle(sub, "gated", True)
    mine = {"o": got["o"][:, h:h + 1, t0:t1], "ht": got["ht"][s:s + 1, h:h + 1], "dh0": got["dh0"][s:s + 1, h:h + 1]}
    for n in ("dq", "dk", "dv", "dbeta", "dalpha"):
        mine[n] = got[n][:, h:h + 1, t0:t1]
    compare(mine, ref, "bf16")


@pytest.mark.parametrize("variant", ["deltanet", "gated", "kda", "gdn2"])
def test_gate_logits_decode(variant):
    import torch
    from gated_delta_rule_73_amd import gdr_decode
    from tests._helpers import to_gpu, to_np
    w = synth.Workload("lgd", variant, "bf16", 3, 2, 5, 128, 128, seed=62, backward=False, h0_std=0.3)
    inp = synth.make_inputs(w, alpha_mode="weak", gate_logits=True)
    g = {n: to_gpu(inp.get(n), "bf16") for n in ("q", "k", "v", "beta", "alpha", "erase", "write")}
    state = torch.from_numpy(inp["h0"]).cuda()
    o = gdr_decode(**g, state=state, variant=variant, gate_logits=True)
    torch.cuda.synchronize()
    ref = _oracle(inp, variant, False)
    compare({"o": to_np(o), "ht": to_np(state)}, ref, "bf16")


def test_gate_logits_gdn2_without_beta():
    """Gated DeltaNet-2 as in its workload (no beta), erase/write/alpha as logits."""
    w = synth.Workload("lg2", "gdn2", "bf16", 1, 2, 200, 128, 128, seed=63, h0_std=0.1, has_beta=False)
    inp = synth.make_inputs(w, alpha_mode="weak", gate_logits=True)
    compare(_hip(inp, "gdn2", "bf16", True), _oracle(inp, "gdn2", True), "bf16")


@pytest.mark.parametrize("variant", ["gated", "kda", "gdn2"])
def test_gate_logits_segmented_scans(variant):
    """Logit gates through the segmented scans (map pass, combine, rerun forced on), packed
    sequences with ragged tails and an empty one; Gated DeltaNet-2 runs its logit scan variant."""
    import os
    cu = [0, 150, 150, 347]
    w = synth.Workload("lgs", variant, "bf16", 1, 2, 347, 128, 128, seed=64, h0_std=0.1,
                       cu_seqlens=tuple(cu))
    inp = synth.make_inputs(w, alpha_mode="weak", gate_logits=True)
    os.environ["GDR_SEG_CHUNKS"] = "1"
    try:
        got = _hip(inp, variant, "bf16", True)
    finally:
        del os.environ["GDR_SEG_CHUNKS"]
    compare(got, _oracle(inp, variant, True, cu=np.asarray(cu)), "bf16")


def test_gate_logits_decode_d64_f32():
    import torch
    from gated_delta_rule_73_amd import gdr_decode
    from tests._helpers import to_gpu, to_np
    w = synth.Workload("lgd64", "kda", "f32", 2, 3, 4, 64, 64, seed=65, backward=False, h0_std=0.3)
    inp = synth.make_inputs(w, alpha_mode="weak", gate_logits=True)
    g = {n: to_gpu(inp.get(n), "f32") for n in ("q", "k", "v", "beta", "alpha")}
    state = torch.from_numpy(inp["h0"]).cuda()
    o = gdr_decode(**g, state=state, variant="kda", gate_logits=True)
    torch.cuda.synchronize()
    compare({"o": to_np(o), "ht": to_np(state)}, _oracle(inp, "kda", False), "f32")
