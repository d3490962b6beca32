"""GPU parity: the HIP path (through the C ABI) against the float64 oracle on the same seeded
inputs.  Shapes span several chunks with a ragged tail; companions with weak or no decay make
the inter-chunk carry and the initial memory visible at the tolerance."""
import numpy as np
import pytest

import synth
from tests._helpers import compare, run_hip, run_oracle

pytestmark = pytest.mark.gpu


def _small(variant, dtype, *, B=2, H=2, T=200, d=128, alpha_mode="config", h0=False, seed=11,
           cu=None, backward=True):
    w = synth.Workload("t", variant, dtype, B, H, T, d, d, seed=seed, backward=backward,
                       cu_seqlens=cu, h0_std=0.5 if h0 else 0.0)
    return w, synth.make_inputs(w, alpha_mode=alpha_mode)


def test_deltanet_f32_T256_d64_forward():
    """The float32 DeltaNet workload (B=1 H=1 T=256 d=64, seed 0), forward only."""
    w = synth.WORKLOADS["deltanet_f32_T256"]
    inp = synth.make_inputs(w)
    rep = []
    compare(run_hip(inp, w.variant, w.dtype, backward=False), run_oracle(inp, w.variant, backward=False),
            w.dtype, report=rep)
    print("\n".join(rep))


@pytest.fixture(params=[16, 32], ids=["bv16", "bv32"])
def scan_bv(request, monkeypatch):
    """Value-tile height of the scans, forced: 32-row tiles are what the planner picks at the
    benchmarked sizes (many memories), 16 what it picks for small problems; both are tested
    with a long memory (weak or no decay) and a visible initial memory."""
    monkeypatch.setenv("GDR_SCAN_BV", str(request.param))
    return request.param


@pytest.mark.parametrize("alpha_mode", ["config", "weak", "one"])
def test_gated_bf16_small(alpha_mode, scan_bv):
    w, inp = _small("gated", "bf16", alpha_mode=alpha_mode, h0=True)
    dht = np.random.default_rng(5).standard_normal((2, 2, 128, 128)).astype(np.float32)
    rep = []
    got = run_hip(inp, "gated", "bf16", backward=True, dht=dht, scale=0.75)
    ref = run_oracle(inp, "gated", backward=True, dht=dht, scale=0.75)
    compare(got, ref, "bf16", report=rep)
    print("\n".join(rep))


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("f32", 64)])
def test_deltanet_fwd_bwd(dtype, d):
    w, inp = _small("deltanet", dtype, d=d, T=130, h0=True)
    rep = []
    compare(run_hip(inp, "deltanet", dtype, backward=True), run_oracle(inp, "deltanet", backward=True),
            dtype, report=rep)
    print("\n".join(rep))


def test_gated_f32_d64_fwd_bwd():
    w, inp = _small("gated", "f32", d=64, T=150, h0=True, alpha_mode="weak")
    rep = []
    compare(run_hip(inp, "gated", "f32", backward=True), run_oracle(inp, "gated", backward=True), "f32",
            report=rep)
    print("\n".join(rep))


def test_gated_varlen_with_initial_state(scan_bv):
    cu = (0, 100, 164, 165, 300)
    w, inp = _small("gated", "bf16", B=1, H=3, T=300, cu=cu, h0=True, alpha_mode="weak")
    dht = np.random.default_rng(6).standard_normal((4, 3, 128, 128)).astype(np.float32) * 0.1
    rep = []
    compare(run_hip(inp, "gated", "bf16", backward=True, dht=dht),
            run_oracle(inp, "gated", backward=True, dht=dht), "bf16", report=rep)
    print("\n".join(rep))


def test_saved_and_recomputed_backward_agree_bitwise():
    w, inp = _small("gated", "bf16", T=190)
    a = run_hip(inp, "gated", "bf16", backward=True, use_saved=True)
    b = run_hip(inp, "gated", "bf16", backward=True, use_saved=False)
    for name in ("dq", "dk", "dv", "dbeta", "dalpha", "dh0"):
        assert np.array_equal(a[name], b[name]), name


def test_run_to_run_bitwise_determinism():
    w, inp = _small("gated", "bf16", T=256, alpha_mode="weak")
    a = run_hip(inp, "gated", "bf16", backward=True)
    b = run_hip(inp, "gated", "bf16", backward=True)
    for name in a:
        if a[name] is not None:
            assert np.array_equal(a[name], b[name]), name


def test_initial_state_is_visible(scan_bv):
    """With weak decay the initial memory changes the outputs by far more than the tolerance,
    so the parity of test_gated_bf16_small[weak] also pins the h0 path."""
    w, inp = _small("gated", "bf16", alpha_mode="weak", h0=True)
    a = run_hip(inp, "gated", "bf16", backward=False)
    inp0 = dict(inp, h0=None)
    b = run_hip(inp0, "gated", "bf16", backward=False)
    assert np.max(np.abs(a["o"] - b["o"])) > 0.2


def test_empty_sequences_and_empty_input():
    cu = (0, 0, 70, 70, 70)
    w, inp = _small("gated", "bf16", B=1, H=2, T=70, cu=cu, h0=True)
    compare(run_hip(inp, "gated", "bf16", backward=True), run_oracle(inp, "gated", backward=True), "bf16")
    w0, inp0 = _small("gated", "bf16", B=2, H=2, T=0, h0=True)
    got = run_hip(inp0, "gated", "bf16", backward=True)
    assert got["o"].shape == (2, 2, 0, 128)
    np.testing.assert_array_equal(got["ht"], inp0["h0"])
    np.testing.assert_array_equal(got["dh0"], np.zeros_like(inp0["h0"]))


@pytest.mark.parametrize("alpha_mode,with_beta", [("config", False), ("weak", False), ("one", True),
                                                   ("config", True)])
def test_gdn2_bf16_small(alpha_mode, with_beta, scan_bv):
    """Gated DeltaNet-2: separate erase (key channels) and write (value channels) gates."""
    w = synth.Workload("t", "gdn2", "bf16", 2, 2, 190, 128, 128, seed=21, has_beta=with_beta, h0_std=0.5)
    inp = synth.make_inputs(w, alpha_mode=alpha_mode)
    dht = np.random.default_rng(7).standard_normal((2, 2, 128, 128)).astype(np.float32) * 0.2
    rep = []
    compare(run_hip(inp, "gdn2", "bf16", backward=True, dht=dht, scale=0.9),
            run_oracle(inp, "gdn2", backward=True, dht=dht, scale=0.9), "bf16", report=rep)
    print("\n".join(rep))


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("f32", 64)])
def test_gdn2_small_heads(dtype, d):
    w = synth.Workload("t", "gdn2", dtype, 1, 3, 140, d, d, seed=22, has_beta=True, h0_std=0.3)
    inp = synth.make_inputs(w, alpha_mode="weak")
    rep = []
    compare(run_hip(inp, "gdn2", dtype, backward=True), run_oracle(inp, "gdn2", backward=True), dtype, report=rep)
    print("\n".join(rep))


def test_gdn2_varlen_saved_vs_recomputed():
    cu = (0, 70, 71, 200)
    w = synth.Workload("t", "gdn2", "bf16", 1, 2, 200, 128, 128, seed=23, cu_seqlens=cu, h0_std=0.4,
                       has_beta=False)
    inp = synth.make_inputs(w, alpha_mode="weak")
    a = run_hip(inp, "gdn2", "bf16", backward=True, use_saved=True)
    b = run_hip(inp, "gdn2", "bf16", backward=True, use_saved=False)
    for name in ("o", "dq", "dk", "dv", "dalpha", "derase", "dwrite", "dh0"):
        assert np.array_equal(a[name], b[name]), name
    compare(a, run_oracle(inp, "gdn2", backward=True), "bf16")


@pytest.mark.parametrize("alpha_mode", ["config", "weak", "strong"])
def test_kda_bf16_small(alpha_mode, scan_bv):
    """Kimi Delta Attention: decay per key channel.  "strong" decays by more than e^-60 within
    16 tokens, so every diagonal block takes the exact path."""
    w = synth.Workload("t", "kda", "bf16", 2, 2, 190, 128, 128, seed=31, h0_std=0.5)
    inp = synth.make_inputs(w, alpha_mode=alpha_mode)
    dht = np.random.default_rng(8).standard_normal((2, 2, 128, 128)).astype(np.float32) * 0.2
    rep = []
    compare(run_hip(inp, "kda", "bf16", backward=True, dht=dht, scale=0.8),
            run_oracle(inp, "kda", backward=True, dht=dht, scale=0.8), "bf16", report=rep)
    print("\n".join(rep))


@pytest.mark.parametrize("dtype,alpha_mode", [("bf16", "config"), ("f32", "config"), ("f32", "weak"),
                                              ("f32", "strong")])
def test_kda_small_heads(dtype, alpha_mode):
    w = synth.Workload("t", "kda", dtype, 1, 3, 150, 64, 64, seed=32, h0_std=0.3)
    inp = synth.make_inputs(w, alpha_mode=alpha_mode)
    rep = []
    compare(run_hip(inp, "kda", dtype, backward=True), run_oracle(inp, "kda", backward=True), dtype, report=rep)
    print("\n".join(rep))


def test_kda_mixed_decay_channels():
    """A quarter of the key channels decay strongly: exact diagonal blocks sit next to
    blocks that use the block-start reference, in the same chunk."""
    w = synth.Workload("t", "kda", "f32", 1, 2, 130, 64, 64, seed=33, h0_std=0.3)
    inp = synth.make_inputs(w, alpha_mode="config")
    strong = synth.make_inputs(w, alpha_mode="strong")
    inp["alpha"][..., :16] = strong["alpha"][..., :16]
    rep = []
    compare(run_hip(inp, "kda", "f32", backward=True), run_oracle(inp, "kda", backward=True), "f32", report=rep)
    print("\n".join(rep))


def test_kda_varlen_saved_vs_recomputed():
    cu = (0, 70, 71, 200)
    w = synth.Workload("t", "kda", "bf16", 1, 2, 200, 128, 128, seed=34, cu_seqlens=cu, h0_std=0.4)
    inp = synth.make_inputs(w, alpha_mode="weak")
    a = run_hip(inp, "kda", "bf16", backward=True, use_saved=True)
    b = run_hip(inp, "kda", "bf16", backward=True, use_saved=False)
    for name in ("o", "dq", "dk", "dv", "dbeta", "dalpha", "dh0"):
        assert np.array_equal(a[name], b[name]), name
    compare(a, run_oracle(inp, "kda", backward=True), "bf16")


@pytest.fixture
def segments(monkeypatch):
    """Force segmented scans (segments of the given number of chunks) for small problems."""
    def force(n):
        monkeypatch.setenv("GDR_SEG_CHUNKS", str(n))
    return force


@pytest.mark.parametrize("variant,dtype,lseg", [("gated", "bf16", 2), ("gated", "f32", 3), ("deltanet", "f32", 2),
                                                ("kda", "f32", 2), ("gdn2", "bf16", 3)])
def test_segmented_scans(segments, variant, dtype, lseg):
    """Sequences cut into segments whose affine maps are composed: same results as the oracle,
    with packed sequences of 1..5 segments, an initial memory and a final-memory gradient."""
    cu = (0, 40, 300, 301, 620)
    d = 64 if dtype == "f32" else 128
    w = synth.Workload("t", variant, dtype, 1, 2, 620, d, d, seed=41, cu_seqlens=cu, h0_std=0.4,
                       has_beta=variant != "gdn2")
    inp = synth.make_inputs(w, alpha_mode="weak")
    dht = np.random.default_rng(9).standard_normal((4, 2, d, d)).astype(np.float32) * 0.3
    segments(lseg)
    rep = []
    compare(run_hip(inp, variant, dtype, backward=True, dht=dht), run_oracle(inp, variant, backward=True, dht=dht),
            dtype, report=rep)
    print("\n".join(rep))


def test_segmented_matches_unsegmented(segments):
    w = synth.Workload("t", "gated", "f32", 2, 2, 500, 64, 64, seed=42, h0_std=0.3)
    inp = synth.make_inputs(w, alpha_mode="one")
    segments(0)
    a = run_hip(inp, "gated", "f32", backward=True)
    segments(2)
    b = run_hip(inp, "gated", "f32", backward=True)
    for name in a:
        if a[name] is not None:
            err = np.max(np.abs(a[name] - b[name]))
            assert err <= 1e-4 * max(1e-30, np.max(np.abs(a[name]))), (name, err)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_gdn2_erase_free_is_decayed_linear_attention(dtype, d):
    """Gated DeltaNet-2 with the erase gate closed (e = 0) is the erase-free decayed memory
    W <- alpha W + (beta w*v) k^T (RetNet-style scalar decay with a per-value write gate).  The
    HIP path is checked against the float64 recurrence and, independently, against the closed
    form of causal decayed linear attention computed here in float64."""
    w = synth.Workload("g2e0", "gdn2", dtype, 2, 2, 150, d, d, seed=51, h0_std=0.1)
    inp = synth.make_inputs(w, alpha_mode="weak")
    inp["erase"] = np.zeros_like(inp["erase"])
    got = run_hip(inp, "gdn2", dtype, backward=True)
    ref = run_oracle(inp, "gdn2", backward=True)
    compare(got, ref, dtype)
    # closed form: o_t = Gamma_t W0 q_t + sum_{s<=t} (gamma_t/gamma_s) (k_s . q_t) beta_s (w_s*v_s)
    for b in range(2):
        for h in range(2):
            logg = np.cumsum(np.log(inp["alpha"][b, h].astype(np.float64)))
            Q = inp["q"][b, h].astype(np.float64)
            K = inp["k"][b, h].astype(np.float64)
            Bv = (inp["beta"][b, h][:, None] * inp["write"][b, h] * inp["v"][b, h]).astype(np.float64)
            Dm = np.tril(np.exp(logg[:, None] - logg[None, :]))
            want = (Dm * (Q @ K.T)) @ Bv + np.exp(logg)[:, None] * (Q @ inp["h0"][b, h].astype(np.float64).T)
            tol = 1e-4 * np.max(np.abs(want)) if dtype == "f32" else 2e-2 * max(1.0, np.max(np.abs(want)))
            assert np.max(np.abs(got["o"][b, h] - want)) <= tol


@pytest.mark.parametrize("variant", ["gated", "kda"])
def test_many_ragged_packed_sequences(variant):
    """300 packed sequences of ragged lengths (0 to 160 tokens: empty ones, single tokens,
    ragged tails, several chunks) in one call: every sequence restarts from its own initial
    memory, found by the kernels' wave-parallel lookup of the chunk's sequence."""
    rng = np.random.default_rng(77)
    lens = rng.integers(0, 161, size=300)
    lens[:6] = [0, 1, 64, 0, 65, 128]
    cu = tuple(int(x) for x in np.concatenate([[0], np.cumsum(lens)]))
    w = synth.Workload("t", variant, "bf16", 1, 2, cu[-1], 128, 128, seed=71, cu_seqlens=cu, h0_std=0.5)
    inp = synth.make_inputs(w, alpha_mode="weak")
    dht = np.random.default_rng(78).standard_normal((300, 2, 128, 128)).astype(np.float32) * 0.1
    rep = []
    compare(run_hip(inp, variant, "bf16", backward=True, dht=dht),
            run_oracle(inp, variant, backward=True, dht=dht), "bf16", report=rep)
    print("\n".join(rep))
