"""Seeded synthetic inputs for the delta-rule memory operator.

This module only draws random numbers and rounds them to the I/O precision.
It holds none of the operator's arithmetic, so both the CPU oracle and the
HIP path can consume its output without sharing any computation.

The workloads stand in for the training activations of the pages' 350M-param
DeltaNet-family language models ("Linear Attention Architectures: Mechanisms,
Trade-offs, and Cross-Layer Routing", section "Configuracion Experimental"):
there is no dataset or trained model here, so every input is drawn from the
distributions below.

Draw order (fixed, one ``numpy.random.default_rng(seed)`` stream per call):
q, k, v, beta-logits, alpha-logits, erase-logits, write-logits, h0, dO.
Only the tensors a variant uses are drawn.

Values are drawn in float64, transformed in float64 (L2 normalisation,
sigmoid, exp(-softplus)), then rounded to nearest-even in the I/O precision
(bfloat16 or float32).  The returned arrays are float32 holding exactly those
rounded values; initial states and output gradients of the state are float32.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

VARIANTS = ("deltanet", "gated", "kda", "gdn2", "gla")


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    variant: str
    dtype: str            # "bf16" or "f32": precision of every token-indexed tensor
    B: int
    H: int
    T: int
    dk: int
    dv: int
    chunk: int = 64
    seed: int = 0
    backward: bool = True
    cu_seqlens: Optional[tuple] = None
    h0_std: float = 0.0   # 0 -> no initial state
    has_beta: bool = True

    @property
    def n_seqs(self) -> int:
        return 0 if self.cu_seqlens is None else len(self.cu_seqlens) - 1

    @property
    def n_states(self) -> int:
        return self.B if self.cu_seqlens is None else len(self.cu_seqlens) - 1

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads of the operator study plus the sequence-length sweep.
WORKLOADS = {
    "deltanet_f32_T256": Workload("deltanet_f32_T256", "deltanet", "f32", 1, 1, 256, 64, 64,
                                  seed=0, backward=False),
    "gated_B8H8T4096": Workload("gated_B8H8T4096", "gated", "bf16", 8, 8, 4096, 128, 128, seed=1),
    "kda_B4H16T8192": Workload("kda_B4H16T8192", "kda", "bf16", 4, 16, 8192, 128, 128, seed=2),
    "gdn2_B2H16T16384": Workload("gdn2_B2H16T16384", "gdn2", "bf16", 2, 16, 16384, 128, 128,
                                 seed=3, has_beta=False),
    "gated_varlen_T32768": Workload("gated_varlen_T32768", "gated", "bf16", 1, 16, 32768, 128, 128,
                                    seed=4, cu_seqlens=(0, 4096, 12288, 24576, 32768),
                                    h0_std=0.02),
}
# The erase-free memory with a decay per key channel (GLA form), at the Kimi Delta Attention
# workload's shape and laws (no workload of the operator study uses it; timed with --workload).
EXTRA_WORKLOADS = {
    "gla_B4H16T8192": Workload("gla_B4H16T8192", "gla", "bf16", 4, 16, 8192, 128, 128, seed=6),
}
# Decoding: one new token per sequence against a batch of memories (the recurrent form).  Not
# a workload of the operator study (the pages give no inference benchmark); sized so the
# float32 memories (512 MiB) are twice the GPU's 256 MiB last-level cache.
DECODE_WORKLOADS = {
    "gated_decode_B512H16": Workload("gated_decode_B512H16", "gated", "bf16", 512, 16, 1, 128, 128,
                                     seed=5, backward=False, h0_std=0.02),
}
SWEEP = [Workload(f"gated_B{b}H16T{t}", "gated", "bf16", b, 16, t, 128, 128, seed=1)
         for b, t in ((8, 4096), (4, 8192), (2, 16384), (1, 32768))]


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64/float32 values to the nearest bfloat16 (ties to even).

    Returns float32 holding the rounded values (a bfloat16 is the top half of
    a float32).  Rounds float64 -> float32 first (nearest-even), then keeps
    the top 16 bits with nearest-even rounding on the bit pattern.
    """
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    nan = np.isnan(f)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32)
    out = np.where(nan, np.float32(np.nan), out)
    return out.astype(np.float32)


def to_io(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    raise ValueError(dtype)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _softplus(x):
    return np.logaddexp(0.0, x)


def _l2norm(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def make_inputs(w: Workload, *, alpha_mode: str = "config", with_grad: Optional[bool] = None,
                seed: Optional[int] = None, T: Optional[int] = None, gate_logits: bool = False) -> dict:
    """Draw one workload's inputs.

    gate_logits: return beta, alpha (and the erase/write gates) as the logits drawn for them
    (N(0,1), and N(0,1) plus the alpha_mode's shift for alpha), rounded to the I/O precision,
    instead of the gate values; the consumer applies sigmoid / exp(-softplus).  Same draws,
    same order.

    alpha_mode: "config" -> alpha = exp(-softplus(N(0,1) + 2)) (the workloads' law);
                "weak"   -> alpha = exp(-softplus(N(0,1) - 5)) (about 0.99: long memory);
                "strong" -> alpha = exp(-softplus(N(0,1) + 6)) (about 0.0025: memory of a few tokens);
                "one"    -> alpha = 1 exactly.
    Returns a dict of float32 arrays: q, k [B,H,T,dk]; v [B,H,T,dv]; beta [B,H,T] or None;
    alpha [B,H,T] (scalar decay) or [B,H,T,dk] (per-channel decay) or None; erase [B,H,T,dk];
    write [B,H,T,dv]; h0 [N,H,dv,dk] or None; do [B,H,T,dv] (if with_grad); cu_seqlens (int32).
    """
    seed = w.seed if seed is None else seed
    T = w.T if T is None else T
    with_grad = w.backward if with_grad is None else with_grad
    rng = np.random.default_rng(seed)
    B, H, dk, dv = w.B, w.H, w.dk, w.dv
    out = {}
    out["q"] = to_io(_l2norm(rng.standard_normal((B, H, T, dk))), w.dtype)
    out["k"] = to_io(_l2norm(rng.standard_normal((B, H, T, dk))), w.dtype)
    out["v"] = to_io(rng.standard_normal((B, H, T, dv)), w.dtype)
    act_b = (lambda x: x) if gate_logits else _sigmoid
    out["beta"] = to_io(act_b(rng.standard_normal((B, H, T))), w.dtype) if w.has_beta else None
    if w.variant == "deltanet":
        out["alpha"] = None
    else:
        shape = (B, H, T, dk) if w.variant in ("kda", "gla") else (B, H, T)
        if alpha_mode == "one":
            if gate_logits:
                raise ValueError("alpha = 1 has no finite logit")
            out["alpha"] = np.ones(shape, np.float32)
        else:
            shift = {"config": 2.0, "weak": -5.0, "strong": 6.0}[alpha_mode]
            x = rng.standard_normal(shape) + shift
            out["alpha"] = to_io(x if gate_logits else np.exp(-_softplus(x)), w.dtype)
    if w.variant == "gdn2":
        out["erase"] = to_io(act_b(rng.standard_normal((B, H, T, dk))), w.dtype)
        out["write"] = to_io(act_b(rng.standard_normal((B, H, T, dv))), w.dtype)
    else:
        out["erase"] = out["write"] = None
    if w.h0_std > 0:
        out["h0"] = (rng.standard_normal((w.n_states, H, dv, dk)) * w.h0_std).astype(np.float32)
    else:
        out["h0"] = None
    if with_grad:
        out["do"] = to_io(rng.standard_normal((B, H, T, dv)), w.dtype)
    out["cu_seqlens"] = None if w.cu_seqlens is None else np.asarray(w.cu_seqlens, np.int32)
    return out


def random_cu_seqlens(rng: np.random.Generator, total: int, n: int, multiple: int = 1) -> np.ndarray:
    """Strictly increasing offsets [0, ..., total] splitting `total` tokens into `n` pieces."""
    cuts = np.sort(rng.choice(np.arange(1, total // multiple), size=n - 1, replace=False)) * multiple
    return np.concatenate([[0], cuts, [total]]).astype(np.int32)
