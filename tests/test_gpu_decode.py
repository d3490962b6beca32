"""GPU parity of the recurrent (decoding) entry point gdr_decode against the float64 oracle.

The oracle is the same token-by-token recurrence that defines the operator: decoding T tokens
from a memory h0 must give the oracle's outputs for those tokens and its final memory.  A
prefill through the chunked gdr_forward followed by decoding from its ht must equal one oracle
run over all the tokens."""
import numpy as np
import pytest

import synth
from tests._helpers import compare, to_gpu, to_np

pytestmark = pytest.mark.gpu

TOKENS = ("q", "k", "v", "beta", "alpha", "erase", "write")


def _oracle(inp, variant, h0, cu=None, scale=1.0):
    from oracle import recurrence as R
    kw = {n: inp.get(n) for n in TOKENS}
    return R.forward(**kw, h0=h0, variant=variant, cu_seqlens=cu, scale=scale)


def _decode(inp, variant, dtype, h0, cu=None, scale=1.0):
    import torch
    from gated_delta_rule_73_amd import gdr_decode
    g = {n: to_gpu(inp.get(n), dtype) for n in TOKENS}
    state = torch.from_numpy(np.ascontiguousarray(h0, dtype=np.float32)).cuda()
    o = gdr_decode(**g, state=state, variant=variant, cu_seqlens=cu, scale=scale)
    torch.cuda.synchronize()
    return to_np(o), to_np(state)


CASES = [(v, dt, d) for v in synth.VARIANTS for dt, d in (("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128))]


@pytest.mark.parametrize("variant,dtype,d", CASES, ids=[f"{v}-{dt}-{d}" for v, dt, d in CASES])
@pytest.mark.parametrize("T", [1, 7])
def test_decode_matches_oracle(variant, dtype, d, T):
    w = synth.Workload("dec", variant, dtype, 3, 2, T, d, d, seed=11 + T, backward=False, h0_std=0.3,
                       has_beta=variant != "gdn2")
    inp = synth.make_inputs(w, alpha_mode="weak")
    o, ht = _decode(inp, variant, dtype, inp["h0"], scale=0.7)
    ro, rht = _oracle(inp, variant, inp["h0"], scale=0.7)
    rep = []
    compare({"o": o, "ht": ht}, {"o": ro, "ht": rht}, dtype, report=rep)
    print("\n".join(rep))


@pytest.mark.parametrize("variant", synth.VARIANTS)
def test_prefill_then_decode(variant):
    """Chunked forward over 150 tokens returns ht; decoding the next 3 tokens from it matches one
    oracle run over all 153 tokens."""
    import torch
    from gated_delta_rule_73_amd import gdr_forward
    T0, T1 = 150, 3
    w = synth.Workload("pd", variant, "bf16", 2, 3, T0 + T1, 128, 128, seed=21, backward=False, h0_std=0.1,
                       has_beta=variant != "gdn2")
    inp = synth.make_inputs(w, alpha_mode="weak")
    pre = {n: (None if inp.get(n) is None else inp[n][:, :, :T0]) for n in TOKENS}
    post = {n: (None if inp.get(n) is None else np.ascontiguousarray(inp[n][:, :, T0:])) for n in TOKENS}
    g = {n: to_gpu(pre[n], "bf16") for n in TOKENS}
    h0 = to_gpu(inp["h0"], "f32")
    o_pre, ht, _ = gdr_forward(**g, h0=h0, variant=variant)
    torch.cuda.synchronize()
    o_post, h_end = _decode(post, variant, "bf16", to_np(ht))
    ro, rht = _oracle(inp, variant, inp["h0"])
    rep = []
    compare({"o_pre": to_np(o_pre), "o_post": o_post, "ht": h_end},
            {"o_pre": ro[:, :, :T0], "o_post": ro[:, :, T0:], "ht": rht}, "bf16", report=rep)
    print("\n".join(rep))


@pytest.mark.parametrize("variant", ["gated", "kda"])
def test_decode_packed_sequences(variant):
    """Packed sequences of 2, 0, 1 and 3 new tokens: each continues its own memory; the empty
    one keeps it unchanged."""
    cu = np.array([0, 2, 2, 3, 6], np.int32)
    w = synth.Workload("pk", variant, "bf16", 1, 4, 6, 128, 128, seed=31, backward=False, h0_std=0.3,
                       cu_seqlens=tuple(int(c) for c in cu))
    inp = synth.make_inputs(w, alpha_mode="weak")
    o, ht = _decode(inp, variant, "bf16", inp["h0"], cu=cu)
    ro, rht = _oracle(inp, variant, inp["h0"], cu=cu)
    compare({"o": o, "ht": ht}, {"o": ro, "ht": rht}, "bf16")
    assert np.array_equal(ht[1], inp["h0"][1]), "an empty sequence must leave its memory untouched"


def test_decode_zero_tokens_is_a_no_op():
    import torch
    from gated_delta_rule_73_amd import gdr_decode
    h0 = torch.randn(2, 3, 128, 128, device="cuda")
    ref = h0.clone()
    z = torch.empty(2, 3, 0, 128, device="cuda", dtype=torch.bfloat16)
    b = torch.empty(2, 3, 0, device="cuda", dtype=torch.bfloat16)
    o = gdr_decode(z, z, z, b, b, state=h0, variant="gated")
    torch.cuda.synchronize()
    assert o.shape == (2, 3, 0, 128)
    assert torch.equal(h0, ref)


def test_decode_fullsize():
    """The timed decoding workload (B=512 sequences x 16 heads, one token each, d=128), every
    memory and output compared with the oracle."""
    w = synth.DECODE_WORKLOADS["gated_decode_B512H16"]
    inp = synth.make_inputs(w)
    o, ht = _decode(inp, w.variant, w.dtype, inp["h0"])
    ro, rht = _oracle(inp, w.variant, inp["h0"])
    rep = []
    compare({"o": o, "ht": ht}, {"o": ro, "ht": rht}, w.dtype, report=rep)
    print("\n".join(rep))
