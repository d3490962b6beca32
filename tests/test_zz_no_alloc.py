"""gdr_forward_noalloc (the forward whose workspace is the library's own device scratch) against
gdr_forward with a caller workspace: the same kernels and plan, so the results must be bitwise
equal.  Two calls in a row on one GPU, the second with a smaller problem (the scratch keeps the
first call's contents), with and without a saved buffer; a problem too large for the scratch is
refused before anything is launched."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


def _pair(w, alpha_mode, use_saved):
    import torch
    from gated_delta_rule_73_amd import gdr_forward, gdr_forward_noalloc, gdr_saved_size, make_problem
    from tests._helpers import gpu_inputs
    inp = synth.make_inputs(w, alpha_mode=alpha_mode)
    g = gpu_inputs(inp, w.dtype)
    cu = inp.get("cu_seqlens")
    o_ref, ht_ref, saved_ref = gdr_forward(**g, variant=w.variant, cu_seqlens=cu, save=use_saved)
    p, _keep = make_problem(g["q"], g["v"], variant=w.variant, cu_seqlens=cu)
    o = torch.full_like(o_ref, float("nan"))
    ht = torch.full_like(ht_ref, float("nan"))
    saved = torch.full((gdr_saved_size(p),), 255, dtype=torch.uint8, device=o.device) if use_saved else None
    gdr_forward_noalloc(**g, variant=w.variant, cu_seqlens=cu, o=o, ht=ht, saved=saved)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref), "o differs from gdr_forward"
    assert torch.equal(ht, ht_ref), "ht differs from gdr_forward"
    if use_saved:
        assert torch.equal(saved, saved_ref), "saved differs from gdr_forward"
    # and to the tolerance against the oracle, on a sample (the parity bar of every forward)
    from tests._helpers import compare, run_oracle, to_np
    if w.T <= 400:
        compare({"o": to_np(o), "ht": to_np(ht)}, run_oracle(inp, w.variant, backward=False), w.dtype)


@pytest.mark.parametrize("use_saved", [False, True], ids=["scratch-cache", "saved"])
def test_noalloc_matches_forward_twice(use_saved):
    big = synth.Workload("na1", "gated", "bf16", 2, 4, 1000, 128, 128, seed=81, h0_std=0.5)
    small = synth.Workload("na2", "gated", "bf16", 1, 2, 300, 128, 128, seed=82, h0_std=0.5)
    _pair(big, "weak", use_saved)
    _pair(small, "weak", use_saved)


def test_noalloc_packed_kda_then_smaller_deltanet():
    cu = (0, 70, 70, 200, 333)
    _pair(synth.Workload("na3", "kda", "bf16", 1, 3, 333, 128, 128, seed=83, cu_seqlens=cu, h0_std=0.5),
          "weak", False)
    _pair(synth.Workload("na4", "deltanet", "f32", 1, 2, 130, 64, 64, seed=84, h0_std=0.5), "config", False)


def test_noalloc_refuses_a_problem_beyond_the_scratch():
    import torch
    from gated_delta_rule_73_amd import GdrError, gdr_forward_noalloc
    B, H, T, d = 1, 16, 8192, 128  # 2048 (chunk, head) units x about 104 KiB each: over 64 MiB
    q = torch.zeros(B, H, T, d, dtype=torch.bfloat16, device="cuda")
    gates = torch.full((B, H, T), 0.5, dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    with pytest.raises(GdrError) as e:
        gdr_forward_noalloc(q, q, q, gates, gates, variant="gated", o=o)
    assert e.value.status == 3  # GDR_ERR_WORKSPACE
    assert "scratch" in str(e.value)
