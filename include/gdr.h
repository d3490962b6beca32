/*
 * gdr.h -- C ABI of the chunked delta-rule memory operator on AMD MI355X (gfx950).
 *
 * The operator is the recurrent matrix memory of "Linear Attention Architectures:
 * Mechanisms, Trade-offs, and Cross-Layer Routing" (section "Metodologia y Marco de
 * Trabajo", item 1 "Notacion Unificada"): per (sequence, head) a memory W (d_v x d_k)
 * is updated once per token.  With D_t the token's decay, v_bar = (W D_t) k the memory's
 * prediction and r = v - v_bar the residual:
 *
 *   DeltaNet        W <- W + beta r k^T                         (no decay)
 *   Gated DeltaNet  W <- alpha W; then the DeltaNet write       (scalar alpha per token)
 *   Kimi Delta Att. W <- W diag(alpha); then the DeltaNet write (alpha per key channel)
 *   Gated DeltaNet-2 W <- alpha W; W <- W - v_bar (beta e*k)^T + (beta w*v) k^T
 *                                    (e: per-key-channel erase gate, w: per-value-channel
 *                                     write gate; beta may be absent, meaning 1)
 *   erase-free (GLA) W <- W diag(alpha) + beta v k^T  (alpha per key channel, nothing
 *                                    erased, beta may be absent: the purely additive memory
 *                                    of the earlier generation of matrix-state models, page
 *                                    "Resumen Tecnico: Un Analisis Sistematico de la Atencion
 *                                    Lineal Hibrida", section "Metodologia", list "Modelos
 *                                    Evaluados", item 2)
 *   output          o_t = scale * W_t q_t   (memory after token t's write)
 *
 * The library computes it in chunkwise-parallel form (chunks of 64 tokens: per-chunk
 * WY/UT factors of the products of (I - beta k k^T), a triangular solve, an
 * inter-chunk state carry), forward and backward.
 *
 * Conventions (all entry points):
 *  - Token tensors are contiguous [B, H, T, d] in the problem's I/O dtype (float32 or
 *    bfloat16), gates included; states (h0, ht, dh0, dht) are float32 [N, H, d_v, d_k].
 *    N = B for a dense batch, N = n_seqs for packed variable-length sequences (then B == 1
 *    and sequence n covers tokens [cu_seqlens[n], cu_seqlens[n+1]) of every head).
 *  - Every pointer is owned by the caller.  The library allocates no device memory and
 *    keeps no state between calls; scratch lives in the caller's workspace (the exception is
 *    gdr_forward_noalloc, whose scratch is a device array the library holds).
 *  - Calls are asynchronous on the given stream (a hipStream_t passed as void*; NULL is the
 *    default stream).  cu_seqlens_host is read on the host for checking and planning only.
 *  - Every argument is checked before anything is launched.  On any non-OK return nothing
 *    was launched and no output was written; gdr_last_error() gives a thread-local message.
 *  - Device pointers must be 16-byte aligned, the workspace 256-byte aligned.
 *  - NaN and Inf inputs are not checked; they propagate.
 *  - The entry points are reentrant; calls that share a workspace must be ordered.
 */
#ifndef GDR_H_
#define GDR_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDR_OK = 0,
  GDR_ERR_INVALID_ARG = 1,  /* a pointer, size, flag or cu_seqlens entry is wrong */
  GDR_ERR_UNSUPPORTED = 2,  /* valid, but not built here (e.g. head size or chunk size) */
  GDR_ERR_WORKSPACE = 3,    /* workspace NULL, misaligned or smaller than required */
  GDR_ERR_HIP = 4           /* a HIP launch failed; see gdr_last_error() */
} gdr_status;

typedef enum {
  GDR_DELTANET = 0, /* alpha absent */
  GDR_GATED = 1,    /* alpha [B,H,T] */
  GDR_KDA = 2,      /* alpha [B,H,T,d_k] */
  GDR_GDN2 = 3,     /* alpha [B,H,T]; erase [B,H,T,d_k]; write [B,H,T,d_v]; beta optional */
  GDR_GLA = 4       /* alpha [B,H,T,d_k]; beta optional; no erase/write; no residual output */
} gdr_variant;

typedef enum { GDR_F32 = 0, GDR_BF16 = 1 } gdr_dtype;

typedef struct {
  int32_t variant;                /* gdr_variant */
  int32_t dtype;                  /* gdr_dtype of every token-indexed tensor */
  int32_t B, H, T;                /* batch, heads, tokens (T >= 0) */
  int32_t dk, dv;                 /* head sizes; supported: dk == dv, 64 or 128 (float32: 64) */
  int32_t chunk;                  /* chunk length; supported: 64 */
  int32_t n_seqs;                 /* 0: dense batch; > 0: packed sequences, needs B == 1 */
  const int32_t *cu_seqlens_host; /* n_seqs+1 offsets: [0] = 0, [n_seqs] = T, non-decreasing */
  const int32_t *cu_seqlens_dev;  /* the same offsets in device memory (read by kernels) */
  float scale;                    /* o = scale * W q; finite */
  int32_t gates;                  /* 0: beta, alpha are the gate values.  1: they are logits x,
                                     beta = sigmoid(x), alpha = exp(-softplus(x)) (the gate laws of
                                     the operator's workloads), applied inside the kernels, and
                                     dbeta, dalpha are gradients w.r.t. x; for GDR_GDN2 the
                                     erase and write gates too (e = sigmoid(x), w = sigmoid(x),
                                     derase, dwrite w.r.t. x).  Built for every variant in
                                     gdr_forward, gdr_backward and gdr_decode; not with a
                                     residual output or gradient */
  int32_t qk_norm;                /* 0: q and k are used as given.  1: each token's q and k are
                                     first scaled to unit length over d_k (x / ||x||_2, a zero
                                     row left zero) and dq, dk are gradients w.r.t. the raw q, k.
                                     Done inside the kernels (the inverse norms, 2 floats per
                                     token and head, are part of the saved cache); the backward
                                     maps dq, dk back to the raw rows inside its last kernel.
                                     Every
                                     variant in gdr_forward and gdr_backward; gdr_decode returns
                                     UNSUPPORTED (normalise there before the call) */
} gdr_problem;

typedef struct {
  const void *q, *k, *v;   /* [B,H,T,dk], [B,H,T,dk], [B,H,T,dv]; required */
  const void *beta;        /* [B,H,T]; required except for GDR_GDN2 and GDR_GLA, where NULL means 1 */
  const void *alpha;       /* NULL for GDR_DELTANET, else see gdr_variant; values in (0,1] */
  const void *erase;       /* GDR_GDN2 only: [B,H,T,dk]; NULL otherwise */
  const void *write;       /* GDR_GDN2 only: [B,H,T,dv]; NULL otherwise */
  const float *h0;         /* [N,H,dv,dk] float32 initial memory, or NULL for zeros */
} gdr_inputs;

typedef struct {           /* same shape and dtype as the matching input */
  void *dq, *dk, *dv;      /* required */
  void *dbeta;             /* required iff inputs->beta != NULL */
  void *dalpha;            /* required iff inputs->alpha != NULL; gradient w.r.t. alpha */
  void *derase, *dwrite;   /* required iff the variant is GDR_GDN2 */
  float *dh0;              /* optional [N,H,dv,dk] float32 */
} gdr_grads;

/* Bytes of workspace gdr_forward (backward == 0) or gdr_backward (backward != 0) needs.
 * The backward figure assumes saved == NULL (it recomputes the forward memories); with a
 * saved buffer the same size is accepted.  Errors: INVALID_ARG, UNSUPPORTED. */
gdr_status gdr_workspace_size(const gdr_problem *p, int backward, size_t *bytes);

/* Bytes of the optional forward->backward buffer: the forward's per-chunk WY factor X, the
 * decayed causal Gram M, the in-chunk cumulative log decay, the memory at the start of every
 * chunk, the scaled residuals R (all in the I/O dtype except the log decay, float32), and the
 * float32 inverse L^{-1} of the chunk's triangular factor (Kimi Delta Attention and Gated
 * DeltaNet-2 also keep their key Grams and per-channel or erase-gate factors).
 * Errors: INVALID_ARG, UNSUPPORTED. */
gdr_status gdr_saved_size(const gdr_problem *p, size_t *bytes);

/* Forward.  o: [B,H,T,dv] I/O dtype (required).  ht: [N,H,dv,dk] float32 final memory,
 * or NULL.  saved: gdr_saved_size() bytes or NULL; when given, the per-chunk results the
 * backward needs are written there for a later gdr_backward.  ws: gdr_workspace_size(p, 0) bytes. */
gdr_status gdr_forward(const gdr_problem *p, const gdr_inputs *in, void *o, float *ht,
                       void *saved, void *ws, size_t ws_bytes, void *stream);

/* Forward that allocates nothing, for callers that cannot call hipMalloc (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation) and so cannot provide a
 * workspace.  The workspace comes from a scratch array the library holds in device memory,
 * GDR_NOALLOC_SCRATCH_BYTES bytes per GPU (every GPU the library is loaded on holds its own copy
 * until the process ends).  Everything else is as for gdr_forward: o, ht and saved are the
 * caller's; with saved given the per-chunk results go there and the scratch holds only the
 * scan's own buffers (about 16 KiB per chunk and head at d = 128, bfloat16), without it the
 * scratch also holds them (about 104 KiB per chunk and head).
 *  - Returns GDR_ERR_WORKSPACE, launching nothing, when the problem needs more scratch than the
 *    library holds (call gdr_forward with a workspace instead).
 *  - The stream must belong to the current device (NULL: the default stream); INVALID_ARG if not.
 *  - Every call on one GPU uses that GPU's one scratch array and leaves its contents behind
 *    (nothing in it needs to start at zero).  Calls that overlap on one GPU race: order them,
 *    e.g. on one stream.
 *  - The first call on a device looks up that device's scratch address (no allocation);
 *    no call allocates device or pinned host memory.
 * Errors: as gdr_forward, plus WORKSPACE as above. */
#define GDR_NOALLOC_SCRATCH_BYTES (64u << 20)
gdr_status gdr_forward_noalloc(const gdr_problem *p, const gdr_inputs *in, void *o, float *ht,
                               void *saved, void *stream);

/* Backward of sum(o * dO) + sum(ht * dht).  dO: [B,H,T,dv] I/O dtype (required).
 * dht: [N,H,dv,dk] float32 or NULL (zeros).  saved: the buffer a gdr_forward with the same
 * problem and inputs filled, or NULL to recompute it inside the workspace.
 * ws: gdr_workspace_size(p, 1) bytes.  Gradients are overwritten, not accumulated.
 * With the environment variable GDR_PIPELINE=1, a packed call of the delta family (GDR_DELTANET,
 * GDR_GATED) whose scans are not segmented runs up to four contiguous ranges of its sequences
 * on separate streams: the caller's and three side streams the library creates once per device
 * and keeps (default priority, non-blocking), forked from and joined back into the caller's
 * stream with events, so the call stays ordered on the caller's stream.  Results are bitwise
 * those of the single-stream path.  Calls from several host threads are serialised while they
 * enqueue. */
gdr_status gdr_backward(const gdr_problem *p, const gdr_inputs *in, const void *dO,
                        const float *dht, const void *saved, gdr_grads *g, void *ws,
                        size_t ws_bytes, void *stream);

/* Forward that also returns the delta-rule residual r_t = v_t - v_bar_t of every token: the
 * "write error" of item 1 "Notacion Unificada" (page "Linear Attention Architectures:
 * Mechanisms, Trade-offs, and Cross-Layer Routing", section "Metodologia y Marco de Trabajo"),
 * which the cross-layer error routing of item 3 of the same section (CLER, CLER-H) passes on
 * to another layer.  v_bar_t is the prediction of the decayed memory before token t's write.
 *  - r: [B,H,T,d_v] in the I/O dtype, or NULL (then this is gdr_forward).  Every other
 *    argument as for gdr_forward.
 *  - Defined for GDR_DELTANET, GDR_GATED and GDR_KDA; GDR_GDN2 with r != NULL returns
 *    UNSUPPORTED (its update has separate erase and write terms, not one residual).
 *  - The chunk form writes R_t = beta_t r_t into the memory; r_t is returned as R_t / beta_t
 *    from the float32 R_t, so it needs beta_t > 0: a token with beta_t == 0 gets r_t = 0.
 * Errors: as gdr_forward. */
gdr_status gdr_forward_residual(const gdr_problem *p, const gdr_inputs *in, void *o, void *r, float *ht,
                                void *saved, void *ws, size_t ws_bytes, void *stream);

/* Backward of sum(o * dO) + sum(r * dr) + sum(ht * dht), r the residual output of
 * gdr_forward_residual.  dr: [B,H,T,d_v] in the I/O dtype, or NULL (then this is
 * gdr_backward).  Built for GDR_DELTANET, GDR_GATED and GDR_KDA with gate values (gates == 0);
 * GDR_GDN2, and logit gates, with dr != NULL return UNSUPPORTED.  With bfloat16 I/O (and for
 * GDR_KDA always) the beta gradient is formed in a second pass from dR without the residual's
 * term plus the residual's own term (no two large terms left to cancel); the workspace size is
 * that of gdr_backward.
 * Needs beta_t > 0 as above.  Every other argument as for gdr_backward. */
gdr_status gdr_backward_residual(const gdr_problem *p, const gdr_inputs *in, const void *dO, const void *dr,
                                 const float *dht, const void *saved, gdr_grads *g, void *ws,
                                 size_t ws_bytes, void *stream);

/* Recurrent (token-by-token) form, for decoding.  The page "Linear Attention Architectures:
 * Mechanisms, Trade-offs, and Cross-Layer Routing" (section "Declaracion del Problema") gives
 * linear attention a constant-size memory updated once per token, hence constant inference
 * work per token; the update is the one of item 1 "Notacion Unificada" written out at the top
 * of this file.  For every sequence n and head h, the memory
 * state[n,h] (float32 [d_v, d_k]) takes the sequence's T tokens (or its packed span) in order
 * with the update above and o receives scale * W_t q_t after each token; state is read once
 * and overwritten in place with the memory after the last token (an empty sequence leaves it
 * unchanged).  A memory that gdr_forward returned as ht continues here exactly as if the
 * tokens had been part of that forward call.
 *  - p: as for gdr_forward, except that chunk is not used (it must still be positive) and
 *    head sizes dk == dv in {64, 128} are built for both dtypes.
 *  - in: q, k, v, beta, alpha, erase, write as for gdr_forward; in->h0 must be NULL (the
 *    initial memory is state).
 *  - state: [N,H,d_v,d_k] float32, required, 16-byte aligned; read, then overwritten.
 *  - o: [B,H,T,d_v] in the I/O dtype, required when T > 0.
 * No workspace; nothing is allocated.  There is no backward for this entry point.
 * Errors: INVALID_ARG, UNSUPPORTED (as for gdr_forward), HIP. */
gdr_status gdr_decode(const gdr_problem *p, const gdr_inputs *in, float *state, void *o, void *stream);

/* Name of a status code.  Takes any int, so a code from a newer or foreign caller is safe:
 * values that are not a gdr_status give "GDR_UNKNOWN_STATUS".  The string is static. */
const char *gdr_status_string(int s);

/* Per-launch timing, for profiling tools.  After gdr_trace_launches(events, capacity), the
 * next gdr_forward or gdr_backward call made by the same thread records events[2i] on its
 * stream just before its i-th kernel launch and events[2i+1] just after it (i < capacity/2),
 * then tracing switches itself off.  events: hipEvent_t handles created by the caller.
 * gdr_traced_launches() gives the number of launches that call made (also those beyond the
 * capacity) and gdr_traced_launch_name(i) the kernel of launch i ("" when out of range).
 * Errors: INVALID_ARG when events is NULL or capacity < 2. */
gdr_status gdr_trace_launches(void **events, int capacity);
int gdr_traced_launches(void);
const char *gdr_traced_launch_name(int i);

/* Thread-local description of the last non-OK return of this thread ("" if none). */
const char *gdr_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H_ */
