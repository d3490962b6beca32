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
  // forward cache (in the caller's saved buffer or in the workspace)
  void* X;    // [units][64][D]  WY factor X = T (e^g K)
  void* M;    // [units][64][64] decayed causal Q K^T
  float* G;   // [units][64]     in-chunk cumulative log decay
  void* Hs;   // [units][D][D]   memory at the start of each chunk
  void* R;    // [units][64][D]  scaled residuals R = U - X W0^T
  // workspace only
  void* Ub;   // [units][64][D]  WY factor U = T V
  void* dHs;  // [units][D][D]   gradient w.r.t. the memory at the end of each chunk
  void* dR;   // [units][64][D]  gradient w.r.t. R
};

hipError_t run_forward(const Plan& p, const gdr_inputs& in, void* o, float* ht, bool want_out, hipStream_t st);
hipError_t run_backward(const Plan& p, const gdr_inputs& in, const void* dO, const float* dht, const gdr_grads& gr,
                        hipStream_t st);

}  // namespace gdr
