"""Token-by-token float64 recurrence of the delta-rule memory (oracle; test infrastructure).

Only tests, the smoke check and the benchmark's CPU-baseline leg may use this
file.  It shares no code with the HIP path.

Source: "Linear Attention Architectures: Mechanisms, Trade-offs, and
Cross-Layer Routing" (gist.science summary, section "Metodologia y Marco de
Trabajo", item 1 "Notacion Unificada", and the English abstract on the
chatpaper.ai page of the same paper).  The pages describe one recurrent
memory matrix W per (sequence, head), a residual r = v - v_bar between the
incoming value and the memory's own prediction v_bar, and four ways of
controlling decay, erasing and writing:

  DeltaNet          -- only the residual is written (no decay);
  Gated DeltaNet    -- a learned scalar decay alpha scales the memory before
                       the residual is formed;
  Kimi Delta Attn.  -- the decay is a vector alpha, one rate per channel;
  Gated DeltaNet-2  -- separate per-channel erase and write gates: one picks
                       which key channels are erased, the other which value
                       channels are stored.

The erase-free decayed memories of the earlier generation of matrix-state
models (RetNet with a fixed decay, GLA with data-dependent gates: page "Resumen
Tecnico: Un Analisis Sistematico de la Atencion Lineal Hibrida" (gist.science),
section "Metodologia", list "Modelos Evaluados", item 2; the same page's
"Olvido Controlado" bullet calls GLA's update purely additive) are the same
memory with nothing erased: Gated DeltaNet-2 with a closed erase gate (scalar
decay), and here variant "gla", a decay per key channel:
W <- W diag(alpha) + beta v k^T (beta optional, 1 when absent).

The pages print no formula beyond r = v - v_bar.  Readings taken here (each is
listed with its justification in the design notes):

  * W is d_v x d_k; a key k addresses the memory, the prediction is
    v_bar = W' k, where W' is the memory after this token's decay.
  * Decay happens before the residual is formed (Gated DeltaNet bullet):
    W' = W * alpha (scalar) or W' = W diag(alpha) over KEY channels (Kimi).
  * Delta family write: W <- W' + beta * r k^T with r = v - v_bar and a
    write strength beta in (0,1) per token.
  * Gated DeltaNet-2: erase along gated key channels, write gated value
    channels:  W <- W' - v_bar (beta e*k)^T + (beta w*v) k^T.  beta is 1 when
    the workload has none.  With e = w = 1 this is the Gated DeltaNet update.
  * Output o_t = scale * W_t q_t with the memory after token t's write.
  * Optionally the residual itself, r_t = v_t - v_bar_t (the delta rule's write
    error, which the pages' cross-layer error routing passes to another layer),
    for the delta family; Gated DeltaNet-2 and the erase-free "gla" have no
    single residual.

Everything is float64.  Heads are independent memories; the per-token update
is applied to all heads of one sequence at once (numpy batching over the head
axis, no reordering of the per-token steps).
"""
from __future__ import annotations

import numpy as np

_VARIANTS = ("deltanet", "gated", "kda", "gdn2", "gla")


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def _sequences(B, T, cu_seqlens):
    """Yield (batch index, begin, end, state index) for every independent sequence.

    A packed sequence may be empty; its memory then stays at its initial value."""
    if cu_seqlens is None:
        for b in range(B):
            yield b, 0, T, b
    else:
        cu = [int(c) for c in cu_seqlens]
        if B != 1:
            raise ValueError("packed variable-length sequences need B == 1")
        if cu[0] != 0 or cu[-1] != T or any(b < a for a, b in zip(cu[:-1], cu[1:])):
            raise ValueError("cu_seqlens must run from 0 to T without decreasing")
        for n in range(len(cu) - 1):
            yield 0, cu[n], cu[n + 1], n


class _Seq:
    """One sequence of every head: the token tensors sliced to [H, L, ...]."""

    def __init__(self, variant, q, k, v, beta, alpha, erase, write, b, t0, t1):
        sl = (b, slice(None), slice(t0, t1))
        self.variant = variant
        self.q = q[sl]
        self.k = k[sl]
        self.v = v[sl]
        self.L = t1 - t0
        H = self.k.shape[0]
        self.beta = beta[sl] if beta is not None else np.ones((H, self.L))
        self.alpha = alpha[sl] if alpha is not None else None
        self.erase = erase[sl] if erase is not None else None
        self.write = write[sl] if write is not None else None

    # -- the pieces of one token's step -------------------------------------------------
    def decay(self, W, t):
        """W' = W D_t: no decay, a scalar per head, or one factor per key channel (columns)."""
        if self.variant == "deltanet":
            return W.copy()
        if self.variant in ("kda", "gla"):
            return W * self.alpha[:, t][:, None, :]
        return W * self.alpha[:, t][:, None, None]

    def write_step(self, Wd, t):
        """Memory after token t's write, given the decayed memory Wd = W'.

        Returns (W_t, v_bar) with v_bar = W' k_t the memory's prediction."""
        k = self.k[:, t]
        v = self.v[:, t]
        beta = self.beta[:, t]
        v_bar = np.einsum("hij,hj->hi", Wd, k)
        if self.variant == "gdn2":
            erase_dir = beta[:, None] * self.erase[:, t] * k          # which key channels lose v_bar
            stored = beta[:, None] * self.write[:, t] * v             # which value channels are stored
            Wt = Wd - v_bar[:, :, None] * erase_dir[:, None, :] + stored[:, :, None] * k[:, None, :]
        elif self.variant == "gla":
            Wt = Wd + (beta[:, None] * v)[:, :, None] * k[:, None, :]  # nothing erased, v written at k
        else:
            r = v - v_bar                                             # the delta-rule residual
            Wt = Wd + (beta[:, None] * r)[:, :, None] * k[:, None, :]
        return Wt, v_bar

    def step(self, W, t):
        Wt, _ = self.write_step(self.decay(W, t), t)
        return Wt


def _check(variant, q, k, v, beta, alpha, erase, write):
    if variant not in _VARIANTS:
        raise ValueError(f"unknown variant {variant!r}")
    if (alpha is None) != (variant == "deltanet"):
        raise ValueError("alpha is required by every variant except deltanet")
    if variant in ("kda", "gla") and alpha.shape != k.shape:
        raise ValueError(f"{variant} takes one decay per key channel: alpha must be [B,H,T,dk]")
    if variant in ("gated", "gdn2") and alpha.shape != k.shape[:3]:
        raise ValueError("scalar decay alpha must be [B,H,T]")
    if (erase is None or write is None) != (variant != "gdn2"):
        raise ValueError("erase/write gates are used by gdn2 only")
    if beta is None and variant not in ("gdn2", "gla"):
        raise ValueError("beta is required by the delta family")


def l2_normalize(x):
    """x / ||x||_2 over the last axis (a zero row stays zero): queries and keys of unit length,
    so that the delta rule's rank-1 factor I - beta k k^T has its eigenvalue 1 - beta in (0, 1)."""
    x = _f64(x)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return np.divide(x, n, out=np.zeros_like(x), where=n > 0)


def l2_normalize_backward(x, dy):
    """Gradient w.r.t. x of sum(y * dy), y = l2_normalize(x): (dy - y (y . dy)) / ||x||."""
    x, dy = _f64(x), _f64(dy)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    y = np.divide(x, n, out=np.zeros_like(x), where=n > 0)
    g = dy - y * np.sum(y * dy, axis=-1, keepdims=True)
    return np.divide(g, n, out=np.zeros_like(g), where=n > 0)


# -- gates given as logits -----------------------------------------------------------------
# The workloads draw every gate from a standard-normal logit x: the write strength beta and
# GDN-2's erase and write gates as the logistic sigmoid of x, the decay as alpha = exp(-softplus(x))
# (so log alpha = -softplus(x) < 0 and alpha lies in (0, 1)).  A caller may pass the logits and
# receive gradients with respect to them.
def sigmoid(x):
    """1 / (1 + e^-x), evaluated without overflow for either sign of x."""
    x = _f64(x)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def neg_softplus(x):
    """-log(1 + e^x), the log of the decay alpha = exp(-softplus(x))."""
    return -np.logaddexp(0.0, _f64(x))


def gates_from_logits(beta=None, alpha=None, erase=None, write=None):
    """Gate values from logits: beta, erase, write = sigmoid(x); alpha = exp(-softplus(x)).
    None stays None."""
    f = lambda x, m: None if x is None else m(x)
    return (f(beta, sigmoid), f(alpha, lambda x: np.exp(neg_softplus(x))), f(erase, sigmoid),
            f(write, sigmoid))


def logit_gradients(g, beta=None, alpha=None, erase=None, write=None):
    """Carries gradients w.r.t. the gate values (dbeta, dalpha, derase, dwrite in g) to the
    logits they came from, in place: d/dx sigmoid(x) = s (1 - s), and
    d/dx exp(-softplus(x)) = alpha * (-sigmoid(x))."""
    for x, name in ((beta, "dbeta"), (erase, "derase"), (write, "dwrite")):
        if x is not None:
            s = sigmoid(x)
            g[name] = g[name] * s * (1.0 - s)
    if alpha is not None:
        g["dalpha"] = g["dalpha"] * np.exp(neg_softplus(alpha)) * (-sigmoid(alpha))
    return g


def forward(q, k, v, beta=None, alpha=None, erase=None, write=None, h0=None, *,
            variant, cu_seqlens=None, scale=1.0, residual=False, qk_l2norm=False, gate_logits=False):
    """Run the recurrence.  Returns (o [B,H,T,dv], ht [N,H,dv,dk]) in float64, and with
    residual=True also r [B,H,T,dv], r_t = v_t - v_bar_t (delta family only).
    qk_l2norm: q and k are first scaled to unit length per token (l2_normalize).
    gate_logits: beta, alpha, erase and write are logits, mapped by gates_from_logits first.

    q, k: [B,H,T,dk]; v: [B,H,T,dv]; beta: [B,H,T] (None -> 1, gdn2 and gla only);
    alpha: None (deltanet), [B,H,T] (gated, gdn2) or [B,H,T,dk] (kda, gla);
    erase: [B,H,T,dk], write: [B,H,T,dv] (gdn2 only); h0: [N,H,dv,dk] or None (zeros),
    where N = B, or the number of packed sequences when cu_seqlens is given (then B == 1).
    """
    q, k, v, beta, alpha, erase, write, h0 = map(_f64, (q, k, v, beta, alpha, erase, write, h0))
    if qk_l2norm:
        q, k = l2_normalize(q), l2_normalize(k)
    if gate_logits:
        beta, alpha, erase, write = gates_from_logits(beta, alpha, erase, write)
    _check(variant, q, k, v, beta, alpha, erase, write)
    if residual and variant in ("gdn2", "gla"):
        raise ValueError(f"{variant} writes without a residual (no single residual)")
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    seqs = list(_sequences(B, T, cu_seqlens))
    o = np.zeros((B, H, T, dv))
    r = np.zeros((B, H, T, dv))
    ht = np.zeros((len(seqs), H, dv, dk))
    for b, t0, t1, n in seqs:
        s = _Seq(variant, q, k, v, beta, alpha, erase, write, b, t0, t1)
        W = np.zeros((H, dv, dk)) if h0 is None else h0[n].copy()
        for t in range(s.L):
            W, v_bar = s.write_step(s.decay(W, t), t)
            r[b, :, t0 + t] = s.v[:, t] - v_bar
            o[b, :, t0 + t] = scale * np.einsum("hij,hj->hi", W, s.q[:, t])
        ht[n] = W
    return (o, ht, r) if residual else (o, ht)


def backward(q, k, v, beta=None, alpha=None, erase=None, write=None, h0=None, do=None,
             dht=None, *, variant, cu_seqlens=None, scale=1.0, checkpoint_every=64, dr=None,
             qk_l2norm=False, gate_logits=False):
    """Gradients of sum(o * do) + sum(ht * dht) [+ sum(r * dr), r the residual output of
    forward(residual=True), when dr is given] by manual reverse mode through the recurrence.

    The memory is checkpointed every `checkpoint_every` tokens; each segment's
    per-token memories are recomputed from its checkpoint (the same float64
    steps, so the result does not depend on the checkpoint spacing).
    Returns a dict with dq, dk, dv, dbeta, dalpha, derase, dwrite, dh0 (None where
    the input is absent).  dalpha is the gradient with respect to alpha itself.
    qk_l2norm: as in forward; dq and dk are then w.r.t. the raw q and k.
    gate_logits: as in forward; the gate gradients are then w.r.t. the logits (logit_gradients).
    """
    q, k, v, beta, alpha, erase, write, h0, do, dht, dr = map(
        _f64, (q, k, v, beta, alpha, erase, write, h0, do, dht, dr))
    if gate_logits:
        vals = gates_from_logits(beta, alpha, erase, write)
        g = backward(q, k, v, *vals, h0, do, dht, variant=variant, cu_seqlens=cu_seqlens, scale=scale,
                     checkpoint_every=checkpoint_every, dr=dr, qk_l2norm=qk_l2norm)
        return logit_gradients(g, beta, alpha, erase, write)
    if qk_l2norm:
        g = backward(l2_normalize(q), l2_normalize(k), v, beta, alpha, erase, write, h0, do, dht,
                     variant=variant, cu_seqlens=cu_seqlens, scale=scale,
                     checkpoint_every=checkpoint_every, dr=dr)
        g["dq"], g["dk"] = l2_normalize_backward(q, g["dq"]), l2_normalize_backward(k, g["dk"])
        return g
    _check(variant, q, k, v, beta, alpha, erase, write)
    if dr is not None and variant in ("gdn2", "gla"):
        raise ValueError(f"{variant} writes without a residual (no single residual)")
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    seqs = list(_sequences(B, T, cu_seqlens))
    g = {name: np.zeros_like(x) if x is not None else None
         for name, x in (("dq", q), ("dk", k), ("dv", v), ("dbeta", beta), ("dalpha", alpha),
                         ("derase", erase), ("dwrite", write))}
    dh0 = np.zeros((len(seqs), H, dv, dk))
    S = max(1, int(checkpoint_every))
    for b, t0, t1, n in seqs:
        s = _Seq(variant, q, k, v, beta, alpha, erase, write, b, t0, t1)
        # forward pass keeping only checkpoints (memory before token c, c = 0, S, 2S, ...)
        W = np.zeros((H, dv, dk)) if h0 is None else h0[n].copy()
        ckpt = {}
        for t in range(s.L):
            if t % S == 0:
                ckpt[t] = W.copy()
            W = s.step(W, t)
        dW = np.zeros((H, dv, dk)) if dht is None else dht[n].copy()
        for c0 in sorted(ckpt, reverse=True):
            c1 = min(c0 + S, s.L)
            before = []                       # memory before each token of the segment
            W = ckpt[c0].copy()
            for t in range(c0, c1):
                before.append(W)
                W = s.step(W, t)
            for t in range(c1 - 1, c0 - 1, -1):
                _token_backward(s, t, before[t - c0], dW, do[b, :, t0 + t] * scale, g, b, t0,
                                None if dr is None else dr[b, :, t0 + t])
                dW = s.last_dW_prev
        dh0[n] = dW
    g["dh0"] = dh0
    return g


def _token_backward(s, t, W_prev, dW, do_t, g, b, t0, dr_t=None):
    """Reverse mode through token t.  dW is the gradient w.r.t. W_t (post-write memory),
    do_t the (scaled) output gradient, dr_t the gradient w.r.t. the residual r_t = v_t - v_bar
    (or None).  Leaves the gradient w.r.t. W_{t-1} in s.last_dW_prev."""
    k = s.k[:, t]
    v = s.v[:, t]
    beta = s.beta[:, t]
    Wd = s.decay(W_prev, t)
    Wt, v_bar = s.write_step(Wd, t)
    tt = t0 + t
    # output o_t = W_t q_t (scale already folded into do_t)
    dW = dW + do_t[:, :, None] * s.q[:, t][:, None, :]
    g["dq"][b, :, tt] += np.einsum("hij,hi->hj", Wt, do_t)
    # write step: W_t = Wd - v_bar a^T + b_vec k^T  (a, b_vec as in write_step)
    if s.variant == "gdn2":
        e = s.erase[:, t]
        w = s.write[:, t]
        a = beta[:, None] * e * k
        bvec = beta[:, None] * w * v
    elif s.variant == "gla":
        a = np.zeros_like(k)                  # nothing erased
        bvec = beta[:, None] * v
    else:
        a = beta[:, None] * k
        bvec = beta[:, None] * v
    d_vbar = -np.einsum("hij,hj->hi", dW, a)
    if dr_t is not None:                      # r_t = v_t - v_bar
        d_vbar = d_vbar - dr_t
        g["dv"][b, :, tt] += dr_t
    d_a = -np.einsum("hij,hi->hj", dW, v_bar)
    d_b = np.einsum("hij,hj->hi", dW, k)
    dk_t = np.einsum("hij,hi->hj", dW, bvec)
    # v_bar = Wd k
    dWd = dW + d_vbar[:, :, None] * k[:, None, :]
    dk_t += np.einsum("hij,hi->hj", Wd, d_vbar)
    if s.variant == "gdn2":
        g["derase"][b, :, tt] += beta[:, None] * d_a * k
        dk_t += beta[:, None] * d_a * e
        g["dwrite"][b, :, tt] += beta[:, None] * d_b * v
        g["dv"][b, :, tt] += beta[:, None] * d_b * w
        if g["dbeta"] is not None:
            g["dbeta"][b, :, tt] += np.sum(d_a * e * k, -1) + np.sum(d_b * w * v, -1)
    elif s.variant == "gla":
        g["dv"][b, :, tt] += beta[:, None] * d_b
        if g["dbeta"] is not None:
            g["dbeta"][b, :, tt] += np.sum(d_b * v, -1)
    else:
        dk_t += beta[:, None] * d_a
        g["dv"][b, :, tt] += beta[:, None] * d_b
        g["dbeta"][b, :, tt] += np.sum(d_a * k, -1) + np.sum(d_b * v, -1)
    g["dk"][b, :, tt] += dk_t
    # decay: Wd = W_prev D_t
    if s.variant == "deltanet":
        s.last_dW_prev = dWd
    elif s.variant in ("kda", "gla"):
        al = s.alpha[:, t]
        g["dalpha"][b, :, tt] += np.einsum("hij,hij->hj", dWd, W_prev)
        s.last_dW_prev = dWd * al[:, None, :]
    else:
        al = s.alpha[:, t]
        g["dalpha"][b, :, tt] += np.einsum("hij,hij->h", dWd, W_prev)
        s.last_dW_prev = dWd * al[:, None, None]
