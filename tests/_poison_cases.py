"""Cases run through both the release library and the LDS-poisoning debug build
(libgdr_poison.so); see test_gpu_lds_poison.py.

As a script (the child process the test starts, with GDR_LIBRARY naming the debug build):
    python -m tests._poison_cases OUT.npz
runs every case and writes its results to OUT.npz, keyed "<case>/<tensor>".
"""
from __future__ import annotations

import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

PACK = (0, 5, 70, 70, 200, 330)  # an empty sequence, a short one, ragged tails

# name, variant, I/O type, head size, B, H, T, cu_seqlens, and options: gate logits, q/k
# normalisation, residual output (with its gradient), decode, alpha law, environment (scan
# planning switches: 32-row value tiles, forced segments, the time-split backward)
CASES = [
    dict(name="gated_bf16_packed", variant="gated", dtype="bf16", d=128, B=1, H=2, T=330, cu=PACK),
    dict(name="gated_bf16_bv32", variant="gated", dtype="bf16", d=128, B=2, H=2, T=200, env={"GDR_SCAN_BV": "32"}),
    dict(name="gated_bf16_segments", variant="gated", dtype="bf16", d=128, B=1, H=2, T=330, cu=PACK,
         env={"GDR_SEG_CHUNKS": "2"}),
    dict(name="gated_bf16_time_split", variant="gated", dtype="bf16", d=128, B=1, H=2, T=600,
         env={"GDR_PIPELINE": "1", "GDR_TSPLIT_CHUNKS": "3"}),
    dict(name="gated_bf16_logits_qknorm", variant="gated", dtype="bf16", d=128, B=1, H=2, T=330, cu=PACK,
         logits=True, qk_norm=True),
    dict(name="gated_bf16_residual", variant="gated", dtype="bf16", d=128, B=2, H=2, T=150, residual=True),
    dict(name="gated_f32", variant="gated", dtype="f32", d=64, B=2, H=2, T=150),
    dict(name="deltanet_bf16_qknorm", variant="deltanet", dtype="bf16", d=128, B=2, H=2, T=150, qk_norm=True),
    dict(name="deltanet_f32_residual", variant="deltanet", dtype="f32", d=64, B=1, H=2, T=330, cu=PACK,
         residual=True),
    dict(name="kda_bf16_packed", variant="kda", dtype="bf16", d=128, B=1, H=2, T=330, cu=PACK),
    dict(name="kda_bf16_logits", variant="kda", dtype="bf16", d=128, B=2, H=2, T=150, logits=True),
    dict(name="kda_bf16_residual", variant="kda", dtype="bf16", d=128, B=2, H=2, T=150, residual=True),
    dict(name="kda_bf16_strong_decay", variant="kda", dtype="bf16", d=128, B=1, H=2, T=200, alpha="strong"),
    dict(name="kda_f32", variant="kda", dtype="f32", d=64, B=2, H=2, T=150),
    dict(name="kda_bf16_strong_qknorm", variant="kda", dtype="bf16", d=128, B=1, H=2, T=330, cu=PACK,
         alpha="strong", qk_norm=True),
    dict(name="gla_bf16", variant="gla", dtype="bf16", d=128, B=1, H=2, T=330, cu=PACK),
    dict(name="gla_f32_qknorm", variant="gla", dtype="f32", d=64, B=2, H=2, T=150, qk_norm=True),
    dict(name="gdn2_bf16_packed", variant="gdn2", dtype="bf16", d=128, B=1, H=2, T=330, cu=PACK),
    dict(name="gdn2_bf16_logits", variant="gdn2", dtype="bf16", d=128, B=2, H=2, T=150, logits=True),
    dict(name="gdn2_f32", variant="gdn2", dtype="f32", d=64, B=2, H=2, T=150),
    dict(name="gdn2_bf16_logits_qknorm", variant="gdn2", dtype="bf16", d=128, B=1, H=2, T=330, cu=PACK,
         logits=True, qk_norm=True),
    dict(name="gated_decode", variant="gated", dtype="bf16", d=128, B=3, H=2, T=5, decode=True),
]


def case_inputs(c: dict) -> dict:
    w = synth.Workload(c["name"], c["variant"], c["dtype"], c["B"], c["H"], c["T"], c["d"], c["d"], seed=17,
                       h0_std=0.1, cu_seqlens=c.get("cu"))
    inp = synth.make_inputs(w, alpha_mode=c.get("alpha", "weak"), gate_logits=c.get("logits", False))
    if c.get("residual"):
        rng = np.random.default_rng(18)
        inp["dr"] = synth.to_io(rng.standard_normal(inp["v"].shape), c["dtype"])
    return inp


def run_case(c: dict) -> dict:
    """The case's results through whichever build this process loaded (numpy arrays)."""
    import torch
    from gated_delta_rule_73_amd import gdr_backward, gdr_decode, gdr_forward
    from tests._helpers import gpu_inputs, to_gpu, to_np

    saved_env = {k: os.environ.get(k) for k in c.get("env", {})}
    os.environ.update(c.get("env", {}))
    try:
        inp = case_inputs(c)
        g = gpu_inputs(inp, c["dtype"])
        cu = inp.get("cu_seqlens")
        kw = dict(variant=c["variant"], cu_seqlens=cu, gate_logits=c.get("logits", False))
        if c.get("decode"):
            st = torch.zeros(c["B"], c["H"], c["d"], c["d"], dtype=torch.float32, device="cuda")
            g.pop("h0")
            o = gdr_decode(**g, state=st, **kw)
            torch.cuda.synchronize()
            return {"o": to_np(o), "state": to_np(st)}
        r = torch.empty_like(g["v"]) if c.get("residual") else None
        o, ht, saved = gdr_forward(**g, save=True, residual=r, qk_norm=c.get("qk_norm", False), **kw)
        res = {"o": to_np(o), "ht": to_np(ht)}
        if r is not None:
            res["r"] = to_np(r)
        dr = to_gpu(inp["dr"], c["dtype"]) if c.get("residual") else None
        grads = gdr_backward(**g, do=to_gpu(inp["do"], c["dtype"]), saved=saved, dr=dr,
                             qk_norm=c.get("qk_norm", False), **kw)
        res.update({k: to_np(v) for k, v in grads.items() if v is not None})
        torch.cuda.synchronize()
        return res
    finally:
        for k, v in saved_env.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def main(out_path: str) -> None:
    import torch
    torch.cuda.set_device(0)
    arrays = {}
    for c in CASES:
        print("case", c["name"], flush=True)
        for k, v in run_case(c).items():
            arrays[f"{c['name']}/{k}"] = v
    np.savez(out_path, **arrays)


if __name__ == "__main__":
    main(sys.argv[1])
