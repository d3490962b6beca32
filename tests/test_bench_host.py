"""Host-side checks of bench.py (no GPU): it refuses more than one GPU, and its byte models
give the operator's minima quoted for the workloads and agree with the recorded counters."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_byte_models():
    sys.path.insert(0, ROOT)
    import bench
    import synth
    # Gated DeltaNet, d = 128, bf16: forward q,k,v,beta,alpha -> o (1028 B) + backward (1800 B)
    assert bench.path_bytes_per_head_token("gated", 128, 2, True) == 2828
    assert bench.path_bytes_per_head_token("kda", 128, 2, True) == 3590
    assert bench.path_bytes_per_head_token("gdn2", 128, 2, False) == 4358
    w = synth.DECODE_WORKLOADS["gated_decode_B512H16"]
    # 512 x 16 float32 memories read and written, plus q, k, v, o, beta, alpha per head-token
    assert bench.decode_bytes(w, 2) == 2 * 512 * 16 * 128 * 128 * 4 + 512 * 16 * (4 * 128 * 2 + 2 + 2)


def test_operator_bytes_attribution():
    """Each kernel is charged the operator tensors it reads or writes (no intermediates): the
    delta family's chunk-parallel backward reads every token tensor of the backward and writes
    every gradient (1800 B per head-token at d = 128, bf16), the preparation reads the
    forward's inputs, the forward scan writes o (reading q and k), the reverse scan reads dO."""
    import bench
    tok = 256
    assert bench.kernel_operator_bytes("gated", "bwd_chunk") == 1800
    assert bench.kernel_operator_bytes("gated", "fwd_prep") == 3 * tok + 4
    assert bench.kernel_operator_bytes("gated", "fwd_scan") == 3 * tok
    assert bench.kernel_operator_bytes("gated", "bwd_scan") == 3 * tok
    assert bench.kernel_operator_bytes("deltanet", "bwd_chunk") == 7 * tok + 4
    # every operator tensor of the Gated path is charged to some kernel
    fwd = bench.kernel_operator_bytes("gated", "fwd_prep") + tok  # + o, written by the scan
    assert fwd + bench.kernel_operator_bytes("gated", "bwd_chunk") == bench.path_bytes_per_head_token("gated")
    # Kimi Delta Attention's backward stages together write every gradient and read every input
    k = sum(bench.kernel_operator_bytes("kda", s) for s in ("bwd_kda_wy", "bwd_kda_gram"))
    assert k == (2 * tok + 2 + tok + tok) + (2 * tok + tok) * 2 + 2
    assert bench.kernel_state_bytes("fwd_scan", 128, True) == 2 * 128 * 128 * 4


def test_traced_steps_counts_the_sampled_steps():
    import bench
    for steps in (1, 3, 4, 5, 20, 21):
        want = sum(1 for i in range(steps) if (steps - 1 - i) % bench.TRACE_EVERY == 0)
        assert bench.traced_steps(steps) == want
    assert bench.traced_steps(20) == 5


def test_byte_models_agree_with_recorded_counters():
    """The algorithmic bytes the roofline uses agree (within 2%) with the calibrated HBM counters
    committed under profiles/, whenever those were taken on the current kernel sources."""
    import bench
    import synth
    w = synth.WORKLOADS["gated_varlen_T32768"]
    cu = w.cu_seqlens
    units = sum((b - a + 63) // 64 for a, b in zip(cu[:-1], cu[1:])) * w.H
    measured = bench.measured_traffic("bwd_chunk", w.name)
    if measured is None:
        pytest.skip("counters were taken on other kernel sources")
    model = bench.kernel_bytes_per_unit(w.variant, "bwd_chunk", w.dk, 2, w.has_beta) * units
    assert abs(model - measured) / measured < 0.02
    d = synth.DECODE_WORKLOADS["gated_decode_B512H16"]
    measured = bench.measured_traffic("decode", d.name)
    if measured is not None:
        model = bench.decode_bytes(d, 2)
        assert abs(model - measured) / measured < 0.02
