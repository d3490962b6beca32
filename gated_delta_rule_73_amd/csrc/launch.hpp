// Host-side plan shared by the C ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/gdr.h"
#include "common.hpp"

namespace gdr {

// One call's geometry and the carve-up of the forward cache / workspace.
// Per-chunk buffers are indexed by unit u = global_chunk * H + head.
struct Plan {
  Geo geo;
  int variant, dtype, D, bv;
  int gates;          // 1: beta and alpha are logits (Delta family)
  int qkn;            // 1: q and k scaled to unit length per token (every variant but Gated
                      //    DeltaNet-2): the preparation keeps 1/||q||, 1/||k|| (Rn) and every later
                      //    kernel applies them to the raw rows
  int lseg, max_seg;      // forward segmented scans: chunks per segment (0: off), largest segment count
  int lseg_b, max_seg_b;  // the same for the backward scans
  // time-split backward (ScanSeg mode 3; delta family): parts of ts_lseg chunks, ts_parts of
  // them (0: off); the chained states live in seg_maps.  Used only with a side stream, on which
  // each part's chunk gradients run (ts_fork / ts_join order it against the caller's stream).
  int ts_lseg, ts_parts;
  hipStream_t ts_side;
  hipEvent_t ts_fork, ts_join;
  float* seg_maps;        // [memories][max_seg][2][D][D] float32 (workspace; max_seg of the pass)
  float* seg_starts;      // [memories][max_seg][D][D] float32 (workspace)
  // forward cache (in the caller's saved buffer or in the workspace)
  void* X;    // [units][64][D]  WY factor X = T (e^g K)
  void* M;    // [units][64][64] decayed causal Q K^T
  float* G;   // [units][64]     in-chunk cumulative log decay
  void* Hs;   // [units][D][D]   memory at the start of each chunk
  void* R;    // [units][64][D]  scaled residuals R = U - X W0^T
  void* M2;   // Gated DeltaNet-2: [units][64][64] decayed causal Q K^T (M holds Q A^T)
  void* U2;   // Gated DeltaNet-2: [units][64][D]  -L^{-1} A_kk B
  float* Li;  // [units][64][64] L^{-1} (float32) of the chunk's unit lower-triangular L
  float* A1;  // [units][64][64] the chunk's strictly lower Gram (float32): KDA's A or GDN-2's A_kk
              // (NULL for the delta family, whose backward forms A again from K)
  float* A2;  // Gated DeltaNet-2: [units][64][64] A_ak (float32)
  void* Kb;   // Kimi Delta Attention: [units][64][D] Kbar = e^{g_n - g} K
  void* Qh;   // Kimi Delta Attention: [units][64][D] Qhat = e^g Q
  float* Gn;  // Kimi Delta Attention: [units][D]     e^{g_n} per key channel
  float* Rn;  // q/k normalisation (qkn): [units][2][64] 1/||q||, 1/||k|| per token (zero past the end)
  // workspace only
  void* Ub;   // [units][64][D]  WY factor U = T V
  void* dHs;  // [units][D][D]   gradient w.r.t. the memory at the end of each chunk
  void* dR;   // [units][64][D]  gradient w.r.t. R
  // Gated DeltaNet-2 backward intermediates (float32): per unit 64 x D partial gradients of
  // q, k, the erase direction a and the write vector b, the gradient of X', then 64 x 64
  // gradients of the four chunk matrices, and per-token sums.
  float *g2_dq, *g2_dk, *g2_da, *g2_db, *g2_dx;
  float *g2_dakk, *g2_daak, *g2_dmqk, *g2_dmqa;
  float* g2_rows;  // [units][4][64]: prefix-type sums, Khat.dKhat, dbeta from b, gamma term
  // Kimi Delta Attention backward intermediates (the same workspace region): per unit 64 x D
  // float32 gradients w.r.t. Qhat, X, Kbar, Khat; 64 x 64 gradients w.r.t. M and A in the I/O
  // type (the Gram stage uses them only as matrix-core operands, rounded to that type; their
  // slots keep the float32 size); D float32 values e^{g_n} <W0, dW> per key channel.
  float *kd_dqh, *kd_dx, *kd_dkb, *kd_dkh, *kd_gam;
  void *kd_dm, *kd_da;
};

// Optional per-launch event recording (see gdr_trace_launches in gdr.h).
struct LaunchTrace {
  void** ev = nullptr;
  int cap = 0;      // events available (pairs = cap / 2)
  int n = 0;        // launches seen in the traced call
  bool armed = false;
  const char* names[64] = {};
};
LaunchTrace& launch_trace();

// Records the "before" event on construction and the "after" event on destruction.
struct TraceScope {
  hipStream_t st;
  int idx = -1;
  TraceScope(const char* name, hipStream_t s) : st(s) {
    LaunchTrace& t = launch_trace();
    if (!t.armed) return;
    idx = t.n++;
    if (idx < 64) t.names[idx] = name;
    if (2 * idx + 1 < t.cap) (void)hipEventRecord(static_cast<hipEvent_t>(t.ev[2 * idx]), st);
    else idx = -1;
  }
  ~TraceScope() {
    if (idx < 0) return;
    (void)hipEventRecord(static_cast<hipEvent_t>(launch_trace().ev[2 * idx + 1]), st);
  }
};

template <typename E, int D>
hipError_t launch_fwd_prep_gdn2(const Plan& p, const gdr_inputs& in, hipStream_t st);
template <typename E, int D>
hipError_t launch_bwd_gdn2(const Plan& p, const gdr_inputs& in, const void* dO, const gdr_grads& gr, hipStream_t st);
template <typename E, int D>
hipError_t launch_fwd_prep_kda(const Plan& p, const gdr_inputs& in, hipStream_t st);
template <typename E, int D>
hipError_t launch_bwd_kda(const Plan& p, const gdr_inputs& in, const void* dO, const gdr_grads& gr, hipStream_t st);

hipError_t launch_seg_combine(const Plan& p, const ScanSeg& sg, const float* init, bool reverse, hipStream_t st);


// Recurrent form over every sequence's tokens, memory updated in place (decoding).
hipError_t run_decode(const Geo& g, int variant, int gates, int dtype, int D, const gdr_inputs& in, float* state,
                      void* o, hipStream_t st);
// r: optional residual output (Delta family and Kimi Delta Attention); dr: optional gradient
// w.r.t. it (Delta family).  Both may be NULL.
hipError_t run_forward(const Plan& p, const gdr_inputs& in, void* o, void* r, float* ht, bool want_out,
                       hipStream_t st);
hipError_t run_backward(const Plan& p, const gdr_inputs& in, const void* dO, const void* dr, const float* dht,
                        const gdr_grads& gr, hipStream_t st);

}  // namespace gdr
