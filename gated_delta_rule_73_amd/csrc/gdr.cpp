// C ABI of the chunked delta-rule operator: argument checks, planning, workspace carving and
// kernel dispatch.  Everything here runs on the host; nothing is launched before every
// argument has been checked.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/gdr.h"
#include "launch.hpp"

namespace {

thread_local std::string g_last_error;

gdr_status fail(gdr_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Sizes {
  long long units = 0;   // chunks * heads
  int total_chunks = 0;
  int nstates = 0;
  size_t esz = 0;
  int bv = 16, lseg = 0, max_seg = 1;  // scan value tile; forward segmented scans (see plan_scans)
  int lseg_b = 0, max_seg_b = 1;       // backward segmented scans
  int ts_lseg = 0, ts_parts = 0;       // time-split backward (see ts_length)
  size_t X, M, G, Hs, R, M2, U2, Li, A1, A2, Kb, Qh, Gn, Ub, dHs, dR, g2, seg;
  size_t Rn = 0;  // q/k normalisation of the delta family: the inverse norms
  bool qkn = false;  // with qk_norm: the kernels normalise q and k as they load them
  size_t cache() const { return X + M + G + Hs + R + M2 + U2 + Li + A1 + A2 + Kb + Qh + Gn + Rn; }
  size_t fwd_ws() const { return Ub + seg; }                   // workspace before the cache
  size_t bwd_ws() const { return Ub + dHs + dR + g2 + seg; }
};

// Scan shape.  Value tiles of 32 rows when the memories give at least one per CU, else 16
// (always 16 for float32 I/O, whose operand tiles take twice the LDS).
// Segmented scans (see ScanSeg) shorten the sequential chain at the price of a map pass and a
// combine.  Measured on one MI355X at 16 memories x 512 chunks (128 value tiles): the forward
// gains with segments that give about 512 workgroups (128 chunks: 0.72 ms against 0.85 ms
// unsegmented; 64 chunks 0.78, 32 chunks 0.84, since the combine grows with the segment count),
// while the backward's map pass costs more than it saves (0.83 ms against 0.75 unsegmented).
// So the forward segments when its value tiles leave CUs idle (fewer than 256), aiming at about
// 512 workgroups with at least 16 chunks per segment, and the backward only when fewer than 64
// tiles would run.  GDR_SEG_CHUNKS, if set, forces the segment length of both (0: never
// segment) and GDR_SCAN_BV the value tile (16 or 32); they exist for tuning and tests and
// change nothing but speed.
int seg_length(long long tiles, long long min_tiles, int max_chunks) {
  if (const char* env = std::getenv("GDR_SEG_CHUNKS")) {
    const int l = std::atoi(env);
    return (l <= 0 || l >= max_chunks) ? 0 : l;
  }
  if (tiles >= min_tiles || max_chunks < 32) return 0;
  const long long want = (512 + tiles - 1) / tiles;
  const int l = (int)std::max<long long>(16, (max_chunks + want - 1) / want);
  return l >= max_chunks ? 0 : l;
}

// Time-split backward of the delta family (ScanSeg mode 3): when the reverse scan's value tiles
// leave CUs idle (fewer than 256) and it is not segmented, it runs in two parts, so that the
// later half's chunk gradients overlap the earlier half's scan (on a side stream; see the
// backward entry point).  Measured on one MI355X at 16 memories x 512 chunks: 2.09 ms per
// training step in two parts, 2.14 in four, 2.17 in sixteen, 2.18 unsplit; more parts lose
// because each part's gradient kernel, one workgroup per CU, holds the CUs the next part's scan
// waits for.  GDR_TSPLIT_CHUNKS, if set, forces the part length (0: never split); like the other
// planning variables it changes nothing but speed.
int ts_length(long long tiles, int max_chunks) {
  if (const char* env = std::getenv("GDR_TSPLIT_CHUNKS")) {
    const int l = std::atoi(env);
    return (l <= 0 || l >= max_chunks) ? 0 : l;
  }
  if (tiles >= 256 || max_chunks < 64) return 0;
  return (max_chunks + 1) / 2;
}

void plan_scans(long long memories, int d, int max_chunks, bool f32, Sizes* s) {
  s->bv = (!f32 && memories * (d / 32) >= 256) ? 32 : 16;
  if (const char* env = std::getenv("GDR_SCAN_BV")) {
    const int bv = std::atoi(env);
    if (bv == 16 || (bv == 32 && !f32)) s->bv = bv;
  }
  const long long tiles = memories * (d / s->bv);
  s->lseg = seg_length(tiles, 256, max_chunks);
  s->lseg_b = seg_length(tiles, 64, max_chunks);
  s->max_seg = s->lseg ? (max_chunks + s->lseg - 1) / s->lseg : 1;
  s->max_seg_b = s->lseg_b ? (max_chunks + s->lseg_b - 1) / s->lseg_b : 1;
}

// Checks the fields every entry point reads (variant, dtype, sizes, scale, packed offsets) and
// counts the chunks of 64 tokens over all sequences.
gdr_status check_shape(const gdr_problem* p, long long* total_chunks_out, int* max_chunks_out) {
  if (!p) return fail(GDR_ERR_INVALID_ARG, "problem is NULL");
  if (p->variant < GDR_DELTANET || p->variant > GDR_GLA)
    return fail(GDR_ERR_INVALID_ARG, "variant %d is not a gdr_variant", p->variant);
  if (p->dtype != GDR_F32 && p->dtype != GDR_BF16)
    return fail(GDR_ERR_INVALID_ARG, "dtype %d is not a gdr_dtype", p->dtype);
  if (p->B < 1 || p->H < 1 || p->T < 0)
    return fail(GDR_ERR_INVALID_ARG, "need B >= 1, H >= 1, T >= 0 (got B=%d H=%d T=%d)", p->B, p->H, p->T);
  if (p->dk < 1 || p->dv < 1) return fail(GDR_ERR_INVALID_ARG, "head sizes must be positive");
  if (p->chunk < 1) return fail(GDR_ERR_INVALID_ARG, "chunk must be positive");
  if (!std::isfinite(p->scale)) return fail(GDR_ERR_INVALID_ARG, "scale must be finite");
  if (p->n_seqs < 0) return fail(GDR_ERR_INVALID_ARG, "n_seqs must be >= 0");
  if (p->H > 65535) return fail(GDR_ERR_UNSUPPORTED, "H > 65535 is not supported");
  if (p->gates != 0 && p->gates != 1) return fail(GDR_ERR_INVALID_ARG, "gates must be 0 (values) or 1 (logits)");
  if (p->qk_norm != 0 && p->qk_norm != 1) return fail(GDR_ERR_INVALID_ARG, "qk_norm must be 0 or 1");
  long long total_chunks = 0;
  int max_chunks = 0;
  if (p->n_seqs > 0) {
    if (p->B != 1) return fail(GDR_ERR_INVALID_ARG, "packed sequences need B == 1 (got %d)", p->B);
    if (!p->cu_seqlens_host || !p->cu_seqlens_dev)
      return fail(GDR_ERR_INVALID_ARG, "packed sequences need cu_seqlens_host and cu_seqlens_dev");
    const int32_t* cu = p->cu_seqlens_host;
    if (cu[0] != 0) return fail(GDR_ERR_INVALID_ARG, "cu_seqlens[0] must be 0 (got %d)", cu[0]);
    if (cu[p->n_seqs] != p->T)
      return fail(GDR_ERR_INVALID_ARG, "cu_seqlens[%d] must equal T=%d (got %d)", p->n_seqs, p->T, cu[p->n_seqs]);
    for (int i = 0; i < p->n_seqs; ++i) {
      if (cu[i + 1] < cu[i]) return fail(GDR_ERR_INVALID_ARG, "cu_seqlens must be non-decreasing (index %d)", i + 1);
      const int nc = (cu[i + 1] - cu[i] + gdr::CH - 1) / gdr::CH;
      total_chunks += nc;
      max_chunks = std::max(max_chunks, nc);
    }
  } else {
    if (p->cu_seqlens_host || p->cu_seqlens_dev)
      return fail(GDR_ERR_INVALID_ARG, "cu_seqlens given but n_seqs == 0");
    max_chunks = (p->T + gdr::CH - 1) / gdr::CH;
    total_chunks = (long long)p->B * max_chunks;
  }
  if ((long long)p->B * p->H * (long long)p->T * p->dk > (1LL << 40))
    return fail(GDR_ERR_UNSUPPORTED, "tensor too large");
  *total_chunks_out = total_chunks;
  *max_chunks_out = max_chunks;
  return GDR_OK;
}

// Checks the problem description for the chunked entry points and computes the buffer sizes.
gdr_status check_problem(const gdr_problem* p, Sizes* sz) {
  long long total_chunks = 0;
  int max_chunks = 0;
  const gdr_status st0 = check_shape(p, &total_chunks, &max_chunks);
  if (st0 != GDR_OK) return st0;
  if (p->chunk != gdr::CH) return fail(GDR_ERR_UNSUPPORTED, "chunk=%d: only 64 is built", p->chunk);
  if (p->dk != p->dv) return fail(GDR_ERR_UNSUPPORTED, "dk=%d != dv=%d is not built", p->dk, p->dv);
  if (p->dtype == GDR_BF16 && p->dk != 64 && p->dk != 128)
    return fail(GDR_ERR_UNSUPPORTED, "bf16 head size %d: only 64 and 128 are built", p->dk);
  if (p->dtype == GDR_F32 && p->dk != 64)
    return fail(GDR_ERR_UNSUPPORTED, "float32 head size %d: only 64 is built", p->dk);
  if (total_chunks > 0x7fffffffLL) return fail(GDR_ERR_UNSUPPORTED, "too many chunks");
  Sizes s;
  s.total_chunks = (int)total_chunks;
  s.units = total_chunks * p->H;
  s.nstates = p->n_seqs > 0 ? p->n_seqs : p->B;
  s.esz = p->dtype == GDR_BF16 ? 2 : 4;
  const size_t D = (size_t)p->dk, C = gdr::CH, U = (size_t)s.units, A = 256;
  s.X = align_up(U * C * D * s.esz, A);
  s.M = align_up(U * C * C * s.esz, A);
  s.G = align_up(U * C * 4, A);
  s.Hs = align_up(U * D * D * s.esz, A);
  s.R = align_up(U * C * D * s.esz, A);
  s.Ub = align_up(U * C * D * s.esz, A);
  s.dHs = align_up(U * D * D * s.esz, A);
  s.dR = align_up(U * C * D * s.esz, A);
  const bool g2 = p->variant == GDR_GDN2, kda = p->variant == GDR_KDA, gla = p->variant == GDR_GLA;
  s.M2 = g2 ? align_up(U * C * C * s.esz, A) : 0;
  s.U2 = g2 ? align_up(U * C * D * s.esz, A) : 0;
  s.Li = gla ? 0 : align_up(U * C * C * 4, A);  // nothing erased: L = I, no inverse kept
  // the delta family's backward forms A again from K (see k_bwd_chunk); the others keep it
  s.A1 = (g2 || kda) ? align_up(U * C * C * 4, A) : 0;
  s.A2 = g2 ? align_up(U * C * C * 4, A) : 0;
  s.Kb = (kda || gla) ? align_up(U * C * D * s.esz, A) : 0;
  s.Qh = (kda || gla) ? align_up(U * C * D * s.esz, A) : 0;
  s.Gn = (kda || gla) ? align_up(U * D * 4, A) : 0;
  // float32 backward intermediates per unit -- GDN-2: 5 of 64xD, 4 of 64x64, 4x64;
  // KDA: 4 of 64xD, 2 of 64x64, D
  if (g2) s.g2 = align_up(U * (5 * C * D + 4 * C * C + 4 * C) * 4, A);
  else if (kda || gla) s.g2 = align_up(U * (4 * C * D + 2 * C * C + D) * 4, A);
  else s.g2 = 0;
  plan_scans((long long)s.nstates * p->H, p->dk, max_chunks, p->dtype == GDR_F32, &s);
  if ((p->variant == GDR_DELTANET || p->variant == GDR_GATED) && s.lseg_b == 0) {
    s.ts_lseg = ts_length((long long)s.nstates * p->H * (p->dk / s.bv), max_chunks);
    s.ts_parts = s.ts_lseg ? (max_chunks + s.ts_lseg - 1) / s.ts_lseg : 0;
  }
  // segmented scans: two maps and a start per segment; the time-split backward: one state per part
  const size_t ms = (size_t)std::max(s.lseg ? s.max_seg : 0, s.lseg_b ? s.max_seg_b : 0);
  const size_t nst = std::max(3 * ms, (size_t)s.ts_parts);
  s.seg = nst ? align_up((size_t)s.nstates * p->H * nst * D * D * 4, A) : 0;
  // q/k normalisation: the preparation kernel normalises the rows it loads and keeps the inverse
  // norms in the cache, with which the later kernels scale the raw rows themselves; the backward's
  // last stage also maps dq, dk back to the raw rows
  s.qkn = p->qk_norm != 0;
  if (s.qkn) s.Rn = align_up(U * 2 * C * 4, A);
  *sz = s;
  return GDR_OK;
}

gdr_status check_inputs(const gdr_problem* p, const gdr_inputs* in) {
  if (!in) return fail(GDR_ERR_INVALID_ARG, "inputs is NULL");
  const void* ptrs[] = {in->q, in->k, in->v, in->beta, in->alpha, in->erase, in->write, in->h0};
  for (const void* x : ptrs)
    if (x && !aligned(x, 16)) return fail(GDR_ERR_INVALID_ARG, "input pointers must be 16-byte aligned");
  if (p->T == 0) return GDR_OK;  // no token is read: token tensors may be empty (NULL)
  if (!in->q || !in->k || !in->v) return fail(GDR_ERR_INVALID_ARG, "q, k and v are required");
  const bool gdn2 = p->variant == GDR_GDN2;
  if (!in->beta && !gdn2 && p->variant != GDR_GLA) return fail(GDR_ERR_INVALID_ARG, "beta is required for this variant");
  if ((in->alpha != nullptr) != (p->variant != GDR_DELTANET))
    return fail(GDR_ERR_INVALID_ARG, p->variant == GDR_DELTANET ? "alpha must be NULL for DeltaNet"
                                                                 : "alpha is required for this variant");
  if ((in->erase != nullptr) != gdn2 || (in->write != nullptr) != gdn2)
    return fail(GDR_ERR_INVALID_ARG, "erase/write gates are given iff the variant is GDR_GDN2");
  return GDR_OK;
}

gdr_status check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return GDR_OK;
  if (!ws) return fail(GDR_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (!aligned(ws, 256)) return fail(GDR_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (have < need) return fail(GDR_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", have, need);
  return GDR_OK;
}

gdr::Plan make_plan(const gdr_problem* p, const Sizes& s, char* cache, char* ws, bool backward) {
  gdr::Plan pl{};
  pl.geo.B = p->B;
  pl.geo.H = p->H;
  pl.geo.T = p->T;
  pl.geo.nseq = s.nstates;
  pl.geo.varlen = p->n_seqs > 0;
  pl.geo.cu = p->cu_seqlens_dev;
  pl.geo.total_chunks = s.total_chunks;
  pl.geo.scale = p->scale;
  pl.variant = p->variant;
  pl.dtype = p->dtype;
  pl.gates = p->gates;
  pl.qkn = s.qkn ? 1 : 0;
  pl.D = p->dk;
  pl.bv = s.bv;
  pl.lseg = s.lseg;
  pl.max_seg = s.max_seg;
  pl.lseg_b = s.lseg_b;
  pl.max_seg_b = s.max_seg_b;
  pl.ts_lseg = s.ts_lseg;  // used only once a side stream is given (ts_side)
  pl.ts_parts = s.ts_parts;
  char* c = cache;
  pl.X = c; c += s.X;
  pl.M = c; c += s.M;
  pl.G = reinterpret_cast<float*>(c); c += s.G;
  pl.Hs = c; c += s.Hs;
  pl.R = c; c += s.R;
  pl.M2 = c; c += s.M2;
  pl.U2 = c; c += s.U2;
  pl.Li = reinterpret_cast<float*>(c); c += s.Li;
  pl.A1 = s.A1 ? reinterpret_cast<float*>(c) : nullptr; c += s.A1;
  pl.A2 = reinterpret_cast<float*>(c); c += s.A2;
  pl.Kb = c; c += s.Kb;
  pl.Qh = c; c += s.Qh;
  pl.Gn = reinterpret_cast<float*>(c); c += s.Gn;
  pl.Rn = s.Rn ? reinterpret_cast<float*>(c) : nullptr; c += s.Rn;
  char* w = ws;
  pl.Ub = w; w += s.Ub;
  pl.seg_maps = reinterpret_cast<float*>(w);
  pl.seg_starts = pl.seg_maps + (size_t)s.nstates * p->H * std::max(s.max_seg, s.max_seg_b) * 2 * p->dk * p->dk;
  w += s.seg;
  pl.dHs = pl.dR = nullptr;
  if (backward) {
    pl.dHs = w; w += s.dHs;
    pl.dR = w; w += s.dR;
    // float32 backward intermediates: GDN-2 and KDA carve the same region differently
    const size_t U = (size_t)s.units, C = gdr::CH, D = (size_t)p->dk;
    float* fk = reinterpret_cast<float*>(w);
    pl.kd_dqh = fk; fk += U * C * D;
    pl.kd_dx = fk; fk += U * C * D;
    pl.kd_dkb = fk; fk += U * C * D;
    pl.kd_dkh = fk; fk += U * C * D;
    pl.kd_dm = fk; fk += U * C * C;
    pl.kd_da = fk; fk += U * C * C;
    pl.kd_gam = fk;
    float* f = reinterpret_cast<float*>(w);
    pl.g2_dq = f; f += U * C * D;
    pl.g2_dk = f; f += U * C * D;
    pl.g2_da = f; f += U * C * D;
    pl.g2_db = f; f += U * C * D;
    pl.g2_dx = f; f += U * C * D;
    pl.g2_dakk = f; f += U * C * C;
    pl.g2_daak = f; f += U * C * C;
    pl.g2_dmqk = f; f += U * C * C;
    pl.g2_dmqa = f; f += U * C * C;
    pl.g2_rows = f;
  }
  return pl;
}

gdr_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return GDR_OK;
  return fail(GDR_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}


// Arms/disarms the per-launch trace around one public call.
struct TraceCall {
  TraceCall() {
    gdr::LaunchTrace& t = gdr::launch_trace();
    if (t.armed) t.n = 0;
  }
  ~TraceCall() { gdr::launch_trace().armed = false; }
};

// Per-sequence pipelines in the backward.  Packed sequences are independent, and the reverse
// scan's time is set by the longest one, whose value tiles keep a few CUs busy while the rest of
// the chip idles.  Cut into contiguous ranges of sequences, each range is a problem of its own
// (the same kernels with cu_seqlens, the per-unit buffers and the per-sequence states offset to
// the range) and runs its reverse scan and chunk-parallel gradients on a stream of its own, so
// the short ranges' gradient kernels fill the CUs the long range's scan leaves idle.  (The
// forward gains nothing this way: what could fill those CUs is the other ranges' chunk
// preparation, whose HBM and L2 traffic slows the long scan by as much as it saves.)  Only the
// delta family with unsegmented scans takes this path (its per-unit buffers are the ones offset
// here).  GDR_PIPELINE=1 turns it on (see pipeline_mode).
constexpr int kSide = 3;  // side streams: with the caller's, four hardware queues
struct Pipes {
  hipStream_t side[kSide] = {};
  hipEvent_t fork = nullptr, join[kSide] = {};
  bool ready = false;
};
std::mutex g_pipe_mu;
Pipes g_pipes[64];

// GDR_PIPELINE: 1 = per-sequence ranges, else the time split (below); 2 = the time split only
// (for tests of it with packed sequences); unset or other values = neither.
int pipeline_mode() {
  const char* env = std::getenv("GDR_PIPELINE");
  const int m = env ? std::atoi(env) : 0;
  return (m == 1 || m == 2) ? m : 0;
}

bool pipeline_wanted(const gdr_problem* p, const Sizes& s) {
  return pipeline_mode() == 1 && p->n_seqs >= 2 && (p->variant == GDR_DELTANET || p->variant == GDR_GATED) &&
         s.lseg == 0 && s.lseg_b == 0;
}

// The time-split backward (see ts_length) where the per-sequence ranges do not apply.
bool tsplit_wanted(const gdr_problem* p, const Sizes& s) {
  return pipeline_mode() != 0 && s.ts_lseg > 0 && !pipeline_wanted(p, s);
}

// Streams and events of the calling thread's current device, created on first use and kept
// for the life of the process.  Caller holds g_pipe_mu.  NULL if the caller's stream belongs to
// another device or creation fails (the call then runs on the caller's stream alone).
Pipes* pipes_for(hipStream_t caller) {
  int dev = -1, sdev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  if (hipStreamGetDevice(caller, &sdev) != hipSuccess || sdev != dev) return nullptr;
  Pipes& pp = g_pipes[dev];
  if (!pp.ready) {
    for (int i = 0; i < kSide; ++i) {
      if (hipStreamCreateWithFlags(&pp.side[i], hipStreamNonBlocking) != hipSuccess) return nullptr;
      if (hipEventCreateWithFlags(&pp.join[i], hipEventDisableTiming) != hipSuccess) return nullptr;
    }
    if (hipEventCreateWithFlags(&pp.fork, hipEventDisableTiming) != hipSuccess) return nullptr;
    pp.ready = true;
  }
  return &pp;
}

struct SeqRange {
  int s0, s1;  // sequences [s0, s1)
  int c0, nc;  // their first global chunk and chunk count
  int longest;  // chunks of the longest sequence in the range
};

// Up to kSide + 1 contiguous ranges of about equal sequence counts, longest range first.
std::vector<SeqRange> seq_ranges(const gdr_problem* p) {
  const int n = p->n_seqs, G = std::min(n, kSide + 1);
  std::vector<SeqRange> r;
  int c = 0;
  for (int g = 0; g < G; ++g) {
    SeqRange x{g * n / G, (g + 1) * n / G, c, 0, 0};
    for (int i = x.s0; i < x.s1; ++i) {
      const int len = p->cu_seqlens_host[i + 1] - p->cu_seqlens_host[i];
      const int ch = (len + gdr::CH - 1) / gdr::CH;
      x.nc += ch;
      x.longest = std::max(x.longest, ch);
    }
    c += x.nc;
    r.push_back(x);
  }
  std::stable_sort(r.begin(), r.end(), [](const SeqRange& a, const SeqRange& b) { return a.longest > b.longest; });
  return r;
}

// The plan of one range: every buffer indexed by unit (chunk * H + head) starts at the range's
// first chunk, the states at its first sequence.
gdr::Plan sub_plan(const gdr::Plan& pl, const gdr_problem* p, const Sizes& s, const SeqRange& x) {
  gdr::Plan q = pl;
  q.geo.cu = p->cu_seqlens_dev + x.s0;
  q.geo.nseq = x.s1 - x.s0;
  q.geo.total_chunks = x.nc;
  const size_t u = (size_t)x.c0 * p->H, C = gdr::CH, D = (size_t)p->dk, e = s.esz;
  auto adv = [u](auto* ptr, size_t per_unit_bytes) {
    using P = decltype(ptr);
    return ptr ? reinterpret_cast<P>(reinterpret_cast<char*>(ptr) + u * per_unit_bytes) : ptr;
  };
  q.X = adv(q.X, C * D * e);
  q.M = adv(q.M, C * C * e);
  q.G = adv(q.G, C * 4);
  q.Hs = adv(q.Hs, D * D * e);
  q.R = adv(q.R, C * D * e);
  q.Li = adv(q.Li, C * C * 4);
  q.A1 = adv(q.A1, C * C * 4);
  q.Ub = adv(q.Ub, C * D * e);
  q.dHs = adv(q.dHs, D * D * e);
  q.dR = adv(q.dR, C * D * e);
  q.Rn = adv(q.Rn, 2 * C * 4);
  return q;
}

float* state_at(const float* st, const gdr_problem* p, int s0) {
  return st ? const_cast<float*>(st) + (size_t)s0 * p->H * p->dk * p->dv : nullptr;
}

// Runs body(range plan, range, stream) for every range, the first (longest) on the caller's
// stream and the others on side streams forked from it and joined back into it.  Without side
// streams, body runs once on the whole problem on the caller's stream.
template <typename Body>
hipError_t run_ranges(const gdr::Plan& pl, const gdr_problem* p, const Sizes& s, hipStream_t caller, Body body) {
  std::lock_guard<std::mutex> lock(g_pipe_mu);
  Pipes* pp = pipes_for(caller);
  if (!pp) return body(pl, SeqRange{0, s.nstates, 0, s.total_chunks, 0}, caller);
  const std::vector<SeqRange> rs = seq_ranges(p);
  hipError_t e = hipEventRecord(pp->fork, caller);
  if (e != hipSuccess) return e;
  // Side streams that wait on the fork are joined back into the caller's stream whatever
  // happens after it, so that no work already enqueued on them outlives the call unordered
  // (the caller may free the workspace and gradients as soon as an error is returned).
  size_t forked = 1;
  for (; forked < rs.size(); ++forked)
    if ((e = hipStreamWaitEvent(pp->side[forked - 1], pp->fork, 0)) != hipSuccess) break;
  for (size_t i = 0; i < forked && e == hipSuccess; ++i) {
    const hipStream_t st = i == 0 ? caller : pp->side[i - 1];
    e = body(sub_plan(pl, p, s, rs[i]), rs[i], st);
  }
  for (size_t i = 1; i < forked; ++i) {
    hipError_t j = hipEventRecord(pp->join[i - 1], pp->side[i - 1]);
    if (j == hipSuccess) j = hipStreamWaitEvent(caller, pp->join[i - 1], 0);
    if (j != hipSuccess) {
      // the ordering could not be expressed through the caller's stream: wait on the host
      (void)hipStreamSynchronize(pp->side[i - 1]);
      if (e == hipSuccess) e = j;
    }
  }
  return e;
}

// The forward behind gdr_forward_residual and gdr_forward_noalloc.  Workspace layout: the scan
// workspace (fwd_ws), then the per-chunk cache when it is not in `saved` (the layout
// gdr_workspace_size describes).
gdr_status forward_impl(const gdr_problem* p, const gdr_inputs* in, void* o, void* r, float* ht, void* saved,
                        const Sizes& s, char* ws, void* stream) {
  char* cache = saved ? static_cast<char*>(saved) : ws + s.fwd_ws();
  gdr::Plan pl = make_plan(p, s, cache, ws, false);
  g_last_error.clear();
  TraceCall tc;
  return hip_status(gdr::run_forward(pl, *in, o, r, ht, true, static_cast<hipStream_t>(stream)), "gdr_forward launch");
}

// Checks shared by the forward entry points (everything but the workspace).
gdr_status check_forward(const gdr_problem* p, const gdr_inputs* in, void* o, void* r, float* ht, void* saved,
                         Sizes* s) {
  gdr_status st = check_problem(p, s);
  if (st != GDR_OK) return st;
  if ((st = check_inputs(p, in)) != GDR_OK) return st;
  if (!o && p->T > 0) return fail(GDR_ERR_INVALID_ARG, "o is required");
  if ((o && !aligned(o, 16)) || (r && !aligned(r, 16)) || (ht && !aligned(ht, 16)) || (saved && !aligned(saved, 256)))
    return fail(GDR_ERR_INVALID_ARG, "o/r/ht must be 16-byte and saved 256-byte aligned");
  if (r && (p->variant == GDR_GDN2 || p->variant == GDR_GLA))
    return fail(GDR_ERR_UNSUPPORTED, "the residual output is defined for the delta family and Kimi Delta Attention");
  if (r && p->gates) return fail(GDR_ERR_UNSUPPORTED, "the residual output takes gate values, not logits");
  return GDR_OK;
}

// ---------------------------------------------------------------------------------------
// Library-held scratch for gdr_forward_noalloc.  `scratch` is a device array: every GPU the
// library runs on holds its own copy (at its own address) from the moment the code object is
// loaded there until the process ends.  In host code its name is only a stand-in for the
// symbol; the device address is looked up once per device (hipGetSymbolAddress, with that
// device current) and only that address is ever passed to kernels or copies.
// ---------------------------------------------------------------------------------------
constexpr size_t kScratchBytes = (size_t)GDR_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of the current device's scratch (looked up on the first call there).
gdr_status scratch_on_current_device(void* stream, char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(GDR_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  if (stream) {  // the stream must belong to the current device, whose scratch is used
    int sdev = -1;
    if ((e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev)) != hipSuccess)
      return hip_status(e, "hipStreamGetDevice");
    if (sdev != dev)
      return fail(GDR_ERR_INVALID_ARG, "the stream belongs to device %d, the current device is %d", sdev, dev);
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if ((e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch))) != hipSuccess)
      return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!ptr || !aligned(ptr, 256)) return fail(GDR_ERR_HIP, "scratch has no usable device address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = static_cast<char*>(g_scratch_ptr[dev]);
  return GDR_OK;
}

}  // namespace

namespace gdr {
LaunchTrace& launch_trace() {
  static thread_local LaunchTrace t;
  return t;
}
}  // namespace gdr

extern "C" {

gdr_status gdr_workspace_size(const gdr_problem* p, int backward, size_t* bytes) {
  Sizes s;
  gdr_status st = check_problem(p, &s);
  if (st != GDR_OK) return st;
  if (!bytes) return fail(GDR_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = s.cache() + (backward ? s.bwd_ws() : s.fwd_ws());
  return GDR_OK;
}

gdr_status gdr_saved_size(const gdr_problem* p, size_t* bytes) {
  Sizes s;
  gdr_status st = check_problem(p, &s);
  if (st != GDR_OK) return st;
  if (!bytes) return fail(GDR_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = s.cache();
  return GDR_OK;
}

gdr_status gdr_forward_residual(const gdr_problem* p, const gdr_inputs* in, void* o, void* r, float* ht, void* saved,
                                void* ws, size_t ws_bytes, void* stream) {
  Sizes s;
  gdr_status st = check_forward(p, in, o, r, ht, saved, &s);
  if (st != GDR_OK) return st;
  if ((st = check_ws(ws, ws_bytes, s.cache() + s.fwd_ws())) != GDR_OK) return st;
  return forward_impl(p, in, o, r, ht, saved, s, static_cast<char*>(ws), stream);
}

gdr_status gdr_forward(const gdr_problem* p, const gdr_inputs* in, void* o, float* ht, void* saved, void* ws,
                       size_t ws_bytes, void* stream) {
  return gdr_forward_residual(p, in, o, nullptr, ht, saved, ws, ws_bytes, stream);
}

gdr_status gdr_forward_noalloc(const gdr_problem* p, const gdr_inputs* in, void* o, float* ht, void* saved,
                               void* stream) {
  Sizes s;
  gdr_status st = check_forward(p, in, o, nullptr, ht, saved, &s);
  if (st != GDR_OK) return st;
  const size_t need = s.fwd_ws() + (saved ? 0 : s.cache());
  if (need > kScratchBytes)
    return fail(GDR_ERR_WORKSPACE, "gdr_forward_noalloc: this problem needs %zu bytes of scratch, more than the "
                "%zu the library holds; pass a saved buffer or call gdr_forward with a workspace",
                need, kScratchBytes);
  char* ws = nullptr;
  if ((st = scratch_on_current_device(stream, &ws)) != GDR_OK) return st;
  return forward_impl(p, in, o, nullptr, ht, saved, s, ws, stream);
}

gdr_status gdr_backward_residual(const gdr_problem* p, const gdr_inputs* in, const void* dO, const void* dr,
                                 const float* dht, const void* saved, gdr_grads* g, void* ws, size_t ws_bytes,
                                 void* stream) {
  Sizes s;
  gdr_status st = check_problem(p, &s);
  if (st != GDR_OK) return st;
  if ((st = check_inputs(p, in)) != GDR_OK) return st;
  if (!g) return fail(GDR_ERR_INVALID_ARG, "grads is NULL");
  if (dr && (p->variant == GDR_GDN2 || p->variant == GDR_GLA))
    return fail(GDR_ERR_UNSUPPORTED, "this variant has no residual output, hence no residual gradient");
  if (dr && p->gates) return fail(GDR_ERR_UNSUPPORTED, "the residual gradient takes gate values, not logits");
  if (dr && !aligned(dr, 16)) return fail(GDR_ERR_INVALID_ARG, "dr must be 16-byte aligned");
  if (p->T > 0) {
    if (!dO) return fail(GDR_ERR_INVALID_ARG, "dO is required");
    if (!g->dq || !g->dk || !g->dv) return fail(GDR_ERR_INVALID_ARG, "dq, dk and dv are required");
    if ((g->dbeta != nullptr) != (in->beta != nullptr))
      return fail(GDR_ERR_INVALID_ARG, "dbeta is required iff beta is given");
    if ((g->dalpha != nullptr) != (in->alpha != nullptr))
      return fail(GDR_ERR_INVALID_ARG, "dalpha is required iff alpha is given");
    if ((g->derase != nullptr) != (in->erase != nullptr) || (g->dwrite != nullptr) != (in->write != nullptr))
      return fail(GDR_ERR_INVALID_ARG, "derase/dwrite are required iff the gates are given");
  }
  const void* ptrs[] = {dO, dht, g->dq, g->dk, g->dv, g->dbeta, g->dalpha, g->derase, g->dwrite, g->dh0};
  for (const void* x : ptrs)
    if (x && !aligned(x, 16)) return fail(GDR_ERR_INVALID_ARG, "gradient pointers must be 16-byte aligned");
  if (saved && !aligned(saved, 256)) return fail(GDR_ERR_INVALID_ARG, "saved must be 256-byte aligned");
  if ((st = check_ws(ws, ws_bytes, s.cache() + s.bwd_ws())) != GDR_OK) return st;
  char* base = static_cast<char*>(ws);
  char* cache = saved ? const_cast<char*>(static_cast<const char*>(saved)) : base + s.bwd_ws();
  gdr::Plan pl = make_plan(p, s, cache, base, true);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  g_last_error.clear();
  TraceCall tc;
  const gdr_inputs ins = *in;
  if (pipeline_wanted(p, s)) {
    st = hip_status(run_ranges(pl, p, s, hs, [&](const gdr::Plan& q, const SeqRange& x, hipStream_t sq) {
      gdr_inputs sub = ins;
      sub.h0 = state_at(in->h0, p, x.s0);
      if (!saved) {
        const hipError_t e = gdr::run_forward(q, sub, nullptr, nullptr, nullptr, false, sq);
        if (e != hipSuccess) return e;
      }
      gdr_grads gs = *g;
      gs.dh0 = state_at(g->dh0, p, x.s0);
      return gdr::run_backward(q, sub, dO, dr, state_at(dht, p, x.s0), gs, sq);
    }), "gdr_backward launch");
  } else {
    if (!saved) {
      st = hip_status(gdr::run_forward(pl, ins, nullptr, nullptr, nullptr, false, hs), "gdr_backward recompute launch");
      if (st != GDR_OK) return st;
    }
    // the side stream and its events are shared by every call on this device: held while used
    std::unique_lock<std::mutex> lock;
    if (tsplit_wanted(p, s)) {
      lock = std::unique_lock<std::mutex>(g_pipe_mu);
      if (Pipes* pp = pipes_for(hs)) {
        pl.ts_side = pp->side[0];
        pl.ts_fork = pp->fork;
        pl.ts_join = pp->join[0];
      }
    }
    st = hip_status(gdr::run_backward(pl, ins, dO, dr, dht, *g, hs), "gdr_backward launch");
  }
  return st;
}

gdr_status gdr_backward(const gdr_problem* p, const gdr_inputs* in, const void* dO, const float* dht,
                        const void* saved, gdr_grads* g, void* ws, size_t ws_bytes, void* stream) {
  return gdr_backward_residual(p, in, dO, nullptr, dht, saved, g, ws, ws_bytes, stream);
}

gdr_status gdr_decode(const gdr_problem* p, const gdr_inputs* in, float* state, void* o, void* stream) {
  if (p && p->qk_norm) return fail(GDR_ERR_UNSUPPORTED, "gdr_decode takes normalised q and k (qk_norm must be 0)");
  long long total_chunks = 0;
  int max_chunks = 0;
  gdr_status st = check_shape(p, &total_chunks, &max_chunks);
  if (st != GDR_OK) return st;
  if (p->dk != p->dv) return fail(GDR_ERR_UNSUPPORTED, "dk=%d != dv=%d is not built", p->dk, p->dv);
  if (p->dk != 64 && p->dk != 128) return fail(GDR_ERR_UNSUPPORTED, "head size %d: only 64 and 128 are built", p->dk);
  if ((st = check_inputs(p, in)) != GDR_OK) return st;
  if (in->h0) return fail(GDR_ERR_INVALID_ARG, "decode takes the memory through state; h0 must be NULL");
  if (!state) return fail(GDR_ERR_INVALID_ARG, "state is required");
  if (!o && p->T > 0) return fail(GDR_ERR_INVALID_ARG, "o is required");
  if (!aligned(state, 16) || (o && !aligned(o, 16)))
    return fail(GDR_ERR_INVALID_ARG, "state and o must be 16-byte aligned");
  gdr::Geo g{};
  g.B = p->B;
  g.H = p->H;
  g.T = p->T;
  g.nseq = p->n_seqs > 0 ? p->n_seqs : p->B;
  g.varlen = p->n_seqs > 0;
  g.cu = p->cu_seqlens_dev;
  g.total_chunks = (int)std::min<long long>(total_chunks, 0x7fffffffLL);
  g.scale = p->scale;
  g_last_error.clear();
  TraceCall tc;
  return hip_status(gdr::run_decode(g, p->variant, p->gates, p->dtype, p->dk, *in, state, o,
                                    static_cast<hipStream_t>(stream)),
                    "gdr_decode launch");
}

const char* gdr_status_string(int s) {
  switch (s) {
    case GDR_OK: return "GDR_OK";
    case GDR_ERR_INVALID_ARG: return "GDR_ERR_INVALID_ARG";
    case GDR_ERR_UNSUPPORTED: return "GDR_ERR_UNSUPPORTED";
    case GDR_ERR_WORKSPACE: return "GDR_ERR_WORKSPACE";
    case GDR_ERR_HIP: return "GDR_ERR_HIP";
  }
  return "GDR_UNKNOWN_STATUS";
}

const char* gdr_last_error(void) { return g_last_error.c_str(); }

gdr_status gdr_trace_launches(void** events, int capacity) {
  if (!events || capacity < 2) return fail(GDR_ERR_INVALID_ARG, "trace needs events and capacity >= 2");
  gdr::LaunchTrace& t = gdr::launch_trace();
  t.ev = events;
  t.cap = capacity;
  t.n = 0;
  t.armed = true;
  return GDR_OK;
}

int gdr_traced_launches(void) { return gdr::launch_trace().n; }

const char* gdr_traced_launch_name(int i) {
  const gdr::LaunchTrace& t = gdr::launch_trace();
  if (i < 0 || i >= t.n || i >= 64 || !t.names[i]) return "";
  return t.names[i];
}

}  // extern "C"
