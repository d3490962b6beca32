"""GPU parity at the workloads' full sizes, in the launch configuration bench.py times
(gdr_forward keeping the per-chunk cache, then gdr_backward reading it).

The whole problem runs on the GPU; the float64 oracle then recomputes sampled (sequence, head)
pairs end to end.  Sequences and heads are independent in the recurrence, so each sample's
forward outputs, final memory and every gradient depend only on that sample's own inputs:
the comparison is exact in scope, not an approximation of the full run.  Samples include
the first and the last (sequence, head) of each workload."""
import numpy as np
import pytest

import synth
from tests._helpers import compare, run_hip

pytestmark = pytest.mark.gpu

TOKEN = ("q", "k", "v", "beta", "alpha", "erase", "write", "do")
GRADS = {"dq": "q", "dk": "k", "dv": "v", "dbeta": "beta", "dalpha": "alpha", "derase": "erase", "dwrite": "write"}


def _span(w, inp, s):
    """(batch row, first token, end token) of sequence s."""
    cu = inp.get("cu_seqlens")
    if cu is None:
        return s, 0, w.T
    return 0, int(cu[s]), int(cu[s + 1])


def _oracle_sample(w, inp, s, h):
    from oracle import recurrence as R
    b, t0, t1 = _span(w, inp, s)
    kw = {}
    for name in TOKEN:
        x = inp.get(name)
        kw[name] = None if x is None else x[b:b + 1, h:h + 1, t0:t1]
    h0 = inp.get("h0")
    kw["h0"] = None if h0 is None else h0[s:s + 1, h:h + 1]
    do = kw.pop("do")
    o, ht = R.forward(**kw, variant=w.variant)
    ref = {"o": o, "ht": ht}
    ref.update(R.backward(**kw, do=do, variant=w.variant))
    return ref


def _hip_sample(w, inp, got, s, h):
    b, t0, t1 = _span(w, inp, s)
    out = {"o": got["o"][b:b + 1, h:h + 1, t0:t1], "ht": got["ht"][s:s + 1, h:h + 1],
           "dh0": got["dh0"][s:s + 1, h:h + 1]}
    for g in GRADS:
        if got.get(g) is not None:
            out[g] = got[g][b:b + 1, h:h + 1, t0:t1]
    return out


CASES = [
    ("gated_B8H8T4096", [(0, 0), (7, 7), (3, 5)]),
    ("kda_B4H16T8192", [(0, 0), (3, 15)]),
    ("gdn2_B2H16T16384", [(0, 0), (1, 15)]),
    ("gated_varlen_T32768", [(0, 0), (3, 15), (2, 9)]),
    ("gated_B1H16T32768", [(0, 0), (0, 15)]),
]


@pytest.mark.parametrize("name,samples", CASES, ids=[c[0] for c in CASES])
def test_fullsize_sampled(name, samples):
    w = synth.WORKLOADS.get(name) or {x.name: x for x in synth.SWEEP}[name]
    inp = synth.make_inputs(w)
    print(f"\n{name}: HIP path on the full problem", flush=True)
    got = run_hip(inp, w.variant, w.dtype, backward=True, use_saved=True)
    for name_ in got:
        assert got[name_] is None or np.all(np.isfinite(got[name_])), name_
    for s, h in samples:
        rep = []
        ref = _oracle_sample(w, inp, s, h)
        sub = _hip_sample(w, inp, got, s, h)
        compare(sub, ref, w.dtype, report=rep)
        lit = {k: float(np.max(np.abs(sub[k] - ref[k]))) for k in ref if ref[k] is not None and ref[k].size}
        print(f"sample (sequence {s}, head {h}):\n" + "\n".join(rep), flush=True)
        print("  literal max|err| <= 2e-2 holds for: "
              + ", ".join(k for k, e in lit.items() if e <= 2e-2)
              + " | exceeds (scaled rule applies): " + ", ".join(k for k, e in lit.items() if e > 2e-2), flush=True)
