// C ABI of libgka.so: argument checks, segment plan, workspace layout and kernel launches.
// Every check runs on the host before anything is enqueued, so a rejected call writes nothing.
#include <algorithm>
#include <cmath>
#include <cstdint>

#include "gka.h"
#include "gka_internal.hpp"

namespace {

using gka::ChebConsts;
using gka::FwdPlan;

constexpr int kAbiVersion = 8;
constexpr int kCUs = 256;  // MI355X compute units: the segment plan aims at one workgroup per CU
// A call from the zero state with at most this many segments skips the segment scan: the token
// walk of segment s composes its start state from the s summaries before it (s x 2 D^2 floats
// read by that workgroup, against a separate scan over every segment state)
constexpr int kComposeMaxSegments = 4;

bool dims_supported(int dtype, int D) {
  (void)dtype;
  return D == 16 || D == 32 || D == 64 || D == 128;
}
bool chunk_supported(int dtype, int D, int C) {
  // bf16 with chunks of 16 (D >= 32: a chunk's rows must fill whole waves of 16-byte loads)
  // takes float32 operands, as float32 inputs do (fp16 products need blocks of 32 tokens)
  if (dtype == GKA_BF16) return C == 32 || C == 64 || (C == 16 && D >= 32);
  if (D == 128) return C == 16;  // float32 operands of D = 128 fit the LDS of a CU at C = 16
  return C == 16 || C == 32 || C == 64;
}
size_t elem_bytes(int dtype) { return dtype == GKA_BF16 ? 2 : 4; }

// The kernels address the rows of one chunk (at most 64 tokens) of one head with 32-bit byte
// offsets from the chunk's first row, across the H heads of a token: the D-element rows of q, k,
// v, o and, in the residual mode, the (iters + 1)-float residual rows. Those spans must stay
// below 2^31 bytes (an offset of 2^31 or more is the kernels' marker for a dropped store).
bool row_spans_fit(const gka_params* p) {
  return 64LL * p->H * p->D * (long long)elem_bytes(p->dtype) < (1LL << 31);
}
bool resid_rows_fit(const gka_params* p) {
  return 64LL * p->H * (p->iters + 1) * 4LL < (1LL << 31);
}

gka_status check_common(const gka_params* p) {
  if (!p) return GKA_ERR_NULL;
  if (p->dtype != GKA_BF16 && p->dtype != GKA_FP32) return GKA_ERR_DTYPE;
  if (p->B < 1 || p->H < 1 || !dims_supported(p->dtype, p->D)) return GKA_ERR_SHAPE;
  if ((long long)p->B * p->H > (1LL << 30)) return GKA_ERR_SHAPE;
  if (!row_spans_fit(p)) return GKA_ERR_SHAPE;
  if (!(p->a > 0.0f) || !std::isfinite(p->a)) return GKA_ERR_VALUE;
  if (p->iters < 1 || p->iters > GKA_MAX_ITERS) return GKA_ERR_VALUE;
  return GKA_OK;
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Chebyshev constants of the system divided by ||H_t||_F: spectrum in [mu, L] = [a, 1 + a],
// c = 2 / (L + mu), rho = (L - mu) / (L + mu), omega_0 = 2, omega_i = 4 / (4 - rho^2 omega_{i-1})
// (weight schedule of Lemma 3 / Lemma 4 on the pith.science page of arXiv 2511.21016).
double w_of(int i, const double* om) { return i == 0 ? 1.0 : om[i]; }

ChebConsts cheb_consts(float a, int iters) {
  ChebConsts cc{};
  const double ad = a;
  const double mu = ad, L = 1.0 + ad;
  const double rho = (L - mu) / (L + mu);
  cc.a = a;
  cc.c = (float)(2.0 / (L + mu));
  cc.iters = iters;
  double om[GKA_MAX_ITERS];
  om[0] = 2.0;
  for (int i = 1; i < iters; ++i) om[i] = 4.0 / (4.0 - rho * rho * om[i - 1]);
  // x_{i+1} = (1 - omega_i) x_{i-1} + omega_i x_i + omega_i c r_i with x_0 = 0, x_1 = c r_0,
  // so every iterate is a fixed combination of the residuals: x_i = sum_j b^(i)_j r_j.
  double prev[GKA_MAX_ITERS] = {0.0}, cur[GKA_MAX_ITERS] = {0.0}, nxt[GKA_MAX_ITERS];
  cur[0] = 2.0 / (L + mu);
  for (int i = 1; i < iters; ++i) {
    for (int j = 0; j < i; ++j) nxt[j] = (1.0 - om[i]) * prev[j] + om[i] * cur[j];
    nxt[i] = om[i] * 2.0 / (L + mu);
    for (int j = 0; j <= i; ++j) {
      prev[j] = cur[j];
      cur[j] = nxt[j];
    }
  }
  for (int i = 0; i < iters; ++i) {
    cc.omega[i] = (float)om[i];
    cc.beta[i] = (float)cur[i];
  }
  // R_{i+1} = R_{i-1} + omega_i (R_i - R_{i-1} - c (Y + a R_i)) = kp R_{i-1} + kr R_i + ky Y,
  // and the first step R_1 = R_0 - c (Y + a R_0)
  const double c = 2.0 / (L + mu);
  for (int i = 0; i < iters; ++i) {
    const double w = i == 0 ? 1.0 : om[i];
    cc.kp[i] = (float)(i == 0 ? 0.0 : 1.0 - w);
    cc.kr[i] = (float)(w * (1.0 - c * ad));
    cc.ky[i] = (float)(-w * c);
  }
  // The iterate's coefficients (beta, bts) carry the power of two xsc (exact scaling): for
  // large a the iterate is about |q| / a, below the normal range of fp16 operands
  double xsc = 1.0;
  while (xsc * 2.0 <= ad) xsc *= 2.0;
  cc.inv_xsc = (float)(1.0 / xsc);
  for (int i = 0; i < iters; ++i) cc.beta[i] = (float)(cur[i] * xsc);
  // Rescaled form: ratio r = s_i / s_{i-1} of consecutive scales, s_i itself only for bts
  // (where underflow to 0 only drops terms far below the rounding of the rest)
  constexpr double kS0 = 0.7390851332151607;  // the fixed point of cos
  cc.iters_rs = iters;
  cc.inv_s0 = (float)(1.0 / kS0);
  // The coefficients of step iters - 1 (which gives R_iters) are used by the residual mode only.
  double r = 1.0, s = kS0;
  for (int i = 0; i < iters; ++i) {
    cc.bts[i] = (float)(cur[i] * s * xsc);
    cc.sres[i] = (float)s;
    const double kp = i == 0 ? 0.0 : 1.0 - om[i];
    if (i >= 1 && std::fabs(kp) < 0x1p-64) {
      if (i + 1 < iters) cc.iters_rs = i + 1;
      break;
    }
    const double rn = i == 0 ? 1.0 : kp / r;  // s_{i+1} / s_i
    cc.krs[i] = (float)(w_of(i, om) * (1.0 - c * ad) / rn);
    cc.kys[i] = (float)(-w_of(i, om) * c / rn);
    s *= rn;
    r = rn;
    if (i + 1 == iters) {
      cc.sres[iters] = (float)s;
      cc.res_extra = 1;
    }
  }
  return cc;
}

// Segment plan: N chunks per head cut into S segments of J chunks; more segments give more
// workgroups (B*H*S) at the price of a summary pass over the keys and values.
bool make_plan(const gka_params* p, FwdPlan& pl, bool packed = false) {
  pl.B = p->B;
  pl.T = p->T;
  pl.H = p->H;
  pl.D = p->D;
  pl.C = p->chunk;
  pl.dtype = p->dtype;
  pl.N = (p->T + p->chunk - 1) / p->chunk;
  pl.order_off = 0;
  if (pl.N == 0) {
    pl.S = pl.J = 0;
    pl.ws_bytes = 0;
    return true;
  }
  int S = p->segments;
  if (S <= 0 && packed) {
    // packed batches: lengths differ, so the plan aims at the longest sequence -- about 12
    // chunks per segment (the sequences are dispatched longest first). Fewer, longer segments
    // leave compute units to the short sequences while the long ones run: on 8 prompts of up
    // to 2048 tokens and 56 decode rows (x 8 heads) 12 chunks per segment measured best.
    S = std::max(1, (pl.N + 11) / 12);
  } else if (S <= 0) {
    const long long bh = (long long)p->B * p->H;
    // aim at one fused-walk workgroup per CU (its LDS, and for D = 128 its registers, fill
    // one), two for the token walk of D <= 64; more segments only add summary and scan work
    const long long per_cu = p->dtype == GKA_BF16 && p->chunk == 64 && p->D <= 64 ? 2 : 1;
    const long long want = (kCUs * per_cu + bh - 1) / bh;
    S = (int)std::min<long long>(want, pl.N);
    if (pl.N / S < 2 && pl.N >= 2) S = std::max(1, pl.N / 2);  // keep >= 2 chunks per segment
  }
  if (S > pl.N) S = pl.N;
  pl.J = (pl.N + S - 1) / S;
  pl.S = (pl.N + pl.J - 1) / pl.J;  // no empty segments
  pl.order_off = 0;
  if (pl.S == 1) {
    pl.ws_bytes = 0;
  } else {
    const size_t bh = (size_t)p->B * p->H;
    const size_t DD = (size_t)p->D * p->D;
    pl.ws_bytes = bh * pl.S * 2 * DD * sizeof(float)  // per-segment (dH, dU), then start states
                  + bh * pl.S * sizeof(float)          // per-segment log2 gate product
                  + bh * sizeof(float);                // ||H||^2 at the start of segment 0
    pl.ws_bytes = (pl.ws_bytes + 255) & ~(size_t)255;
  }
  if (packed && p->B <= gka::kMaxOrdered) {  // the dispatch order, after the segment states
    pl.order_off = pl.ws_bytes;
    pl.ws_bytes += ((size_t)p->B * sizeof(int32_t) + 255) & ~(size_t)255;
  }
  return true;
}

gka_status check_fwd(const gka_params* p) {
  gka_status st = check_common(p);
  if (st != GKA_OK) return st;
  if (p->T < 0 || !chunk_supported(p->dtype, p->D, p->chunk)) return GKA_ERR_SHAPE;
  if (p->segments < 0) return GKA_ERR_SHAPE;
  if ((long long)p->B * p->T * p->H * p->D > (1LL << 40)) return GKA_ERR_SHAPE;
  return GKA_OK;
}

// Backward: chunks of 64 tokens (16 for float32 with D = 128, as the forward), one chunk per
// segment; workspace regions in floats, each rounded up to 64 floats (256 bytes).
int bwd_chunk(const gka_params* p) { return p->dtype == GKA_FP32 && p->D == 128 ? 16 : 64; }

FwdPlan bwd_plan(const gka_params* p) {
  FwdPlan pl{};
  pl.B = p->B;
  pl.T = p->T;
  pl.H = p->H;
  pl.D = p->D;
  pl.C = bwd_chunk(p);
  pl.dtype = p->dtype;
  pl.N = (p->T + pl.C - 1) / pl.C;
  pl.S = pl.N;
  pl.J = 1;
  return pl;
}

// The matrix-core path's segment plan for the chunk-state walk: the forward's plan of the same
// shape with chunks of 64.
FwdPlan bwd_seg_plan(const gka_params* p) {
  gka_params q = *p;
  q.chunk = 64;
  q.segments = 0;
  FwdPlan ps{};
  make_plan(&q, ps);
  return ps;
}

struct BwdLayoutHost {
  bool tok;  // the matrix-core path: no snapshots, per-token results of the solve kernel
  size_t snap, xs, ys, cs, dkh, tokv, fstates, flog2, fn2, rstates, rlog2, rn2;
  size_t sstates, slog2, sn2;  // matrix-core path: the segment summaries and start states
  size_t rs16, rexp;           // matrix-core path: the reverse scan's fp16 outputs
  size_t rd16, rdx;            // matrix-core path: the chunk gradients it scans (fp16)
  size_t fs16, fexp;           // matrix-core path: every chunk's start state (fp16)
  size_t total;
};

BwdLayoutHost bwd_layout(const gka_params* p) {
  auto up = [](size_t x) { return (x + 63) & ~(size_t)63; };
  const size_t n = (size_t)p->B * p->H * p->T, D = (size_t)p->D, bh = (size_t)p->B * p->H;
  const size_t N = (size_t)((p->T + bwd_chunk(p) - 1) / bwd_chunk(p));
  BwdLayoutHost l{};
  l.tok = gka::bwd_tok_supported(bwd_plan(p));
  size_t o = 0;
  if (!l.tok) {
    l.snap = o;
    o += up(n * 2 * D * D);
  }
  l.xs = o; o += up(n * D);
  l.ys = o; o += up(n * D);
  if (l.tok) {
    l.dkh = o; o += up(n * D);
    l.tokv = o; o += up(n * 4);
    const size_t S = (size_t)bwd_seg_plan(p).S;
    l.sstates = o; o += up(bh * S * 2 * D * D);
    l.slog2 = o; o += up(bh * S);
    l.sn2 = o; o += up(bh);
    l.rs16 = o; o += up(bh * N * D * D);  // (2 D^2 fp16 per slot)
    l.rexp = o; o += up(bh * N * 2 * D);
  } else {
    l.cs = o; o += up(n);
  }
  if (l.tok) {
    l.fs16 = o; o += up(bh * N * D * D);  // (2 D^2 fp16 per chunk)
    l.fexp = o; o += up(bh * N * 2);
  } else {
    l.fstates = o; o += up(bh * N * 2 * D * D);
    l.flog2 = o; o += up(bh * N);
    l.fn2 = o; o += up(bh);
  }
  if (l.tok) {
    l.rd16 = o; o += up(bh * N * D * D);      // (2 D^2 fp16 per slot)
    l.rdx = o; o += up(bh * N * D * D / 32);  // (2 D (D / 16) bytes per slot)
  } else {
    l.rstates = o; o += up(bh * N * 2 * D * D);
  }
  l.rlog2 = o; o += up(bh * N);
  l.rn2 = o; o += up(bh);
  l.total = o * sizeof(float);
  return l;
}

gka_status fwd_impl(const gka_params* p, const int32_t* cu, int64_t total, const void* q,
                    const void* k, const void* v, const float* gamma, const float* beta, void* o,
                    float* h_state, float* u_state, float* hnorm2, float* hnorm_t, float* resid,
                    void* workspace, size_t workspace_bytes, void* stream,
                    void* const* phase_events, bool static_ws = false);

}  // namespace

extern "C" {

int gka_abi_version(void) { return kAbiVersion; }

const char* gka_status_str(int s) {
  switch (s) {
    case GKA_OK: return "ok";
    case GKA_ERR_NULL: return "required pointer is NULL (or state pointers mixed NULL / non-NULL)";
    case GKA_ERR_SHAPE: return "unsupported shape, chunk, segment count or misaligned pointer";
    case GKA_ERR_VALUE: return "a must be finite and > 0; iters in [1, GKA_MAX_ITERS]";
    case GKA_ERR_DTYPE: return "unknown dtype";
    case GKA_ERR_WORKSPACE: return "workspace missing or too small";
    case GKA_ERR_HIP: return "HIP launch failed";
    case GKA_ERR_ALIAS: return "output overlaps an input";
    case GKA_ERR_SCRATCH:
      return "segment plan needs more workspace than the static scratch (GKA_STATIC_SCRATCH_BYTES)";
  }
  return "unknown status";
}

size_t gka_fwd_workspace_bytes(const gka_params* p) {
  if (check_fwd(p) != GKA_OK) return 0;
  FwdPlan pl;
  make_plan(p, pl);
  return pl.ws_bytes;
}

size_t gka_fwd_varlen_workspace_bytes(const gka_params* p) {
  if (check_fwd(p) != GKA_OK) return 0;
  FwdPlan pl;
  make_plan(p, pl, true);
  return pl.ws_bytes;
}

gka_status gka_fwd_chunked(const gka_params* p, const void* q, const void* k, const void* v,
                           const float* gamma, void* o, float* h_state, float* u_state,
                           float* hnorm2, float* hnorm_t, void* workspace,
                           size_t workspace_bytes, void* stream, void* const* phase_events) {
  return gka_fwd_chunked_beta(p, q, k, v, gamma, nullptr, o, h_state, u_state, hnorm2, hnorm_t,
                              workspace, workspace_bytes, stream, phase_events);
}

gka_status gka_fwd_chunked_beta(const gka_params* p, const void* q, const void* k, const void* v,
                                const float* gamma, const float* beta, void* o, float* h_state,
                                float* u_state, float* hnorm2, float* hnorm_t, void* workspace,
                                size_t workspace_bytes, void* stream, void* const* phase_events) {
  return fwd_impl(p, nullptr, -1, q, k, v, gamma, beta, o, h_state, u_state, hnorm2, hnorm_t,
                  nullptr, workspace, workspace_bytes, stream, phase_events);
}

gka_status gka_fwd_chunked_residuals(const gka_params* p, const void* q, const void* k,
                                     const void* v, const float* gamma, const float* beta,
                                     void* o, float* h_state, float* u_state, float* hnorm2,
                                     float* hnorm_t, float* resid, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  gka_status st = check_fwd(p);
  if (st != GKA_OK) return st;
  if (!resid_rows_fit(p)) return GKA_ERR_SHAPE;
  if (p->T > 0 && !resid) return GKA_ERR_NULL;
  return fwd_impl(p, nullptr, -1, q, k, v, gamma, beta, o, h_state, u_state, hnorm2, hnorm_t,
                  resid, workspace, workspace_bytes, stream, nullptr);
}

gka_status gka_fwd_chunked_static(const gka_params* p, const void* q, const void* k,
                                  const void* v, const float* gamma, const float* beta, void* o,
                                  float* h_state, float* u_state, float* hnorm2, float* hnorm_t,
                                  void* stream) {
  return fwd_impl(p, nullptr, -1, q, k, v, gamma, beta, o, h_state, u_state, hnorm2, hnorm_t,
                  nullptr, nullptr, 0, stream, nullptr, /*static_ws=*/true);
}

gka_status gka_fwd_varlen(const gka_params* p, const int32_t* cu_seqlens, int64_t total,
                          const void* q, const void* k, const void* v, const float* gamma,
                          const float* beta, void* o, float* h_state, float* u_state,
                          float* hnorm2, float* hnorm_t, void* workspace, size_t workspace_bytes,
                          void* stream) {
  gka_status st = check_fwd(p);
  if (st != GKA_OK) return st;
  if (!cu_seqlens) return GKA_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) return GKA_ERR_SHAPE;
  if (total < 0 || total > (int64_t)p->B * p->T) return GKA_ERR_SHAPE;
  return fwd_impl(p, cu_seqlens, total, q, k, v, gamma, beta, o, h_state, u_state, hnorm2,
                  hnorm_t, nullptr, workspace, workspace_bytes, stream, nullptr);
}

}  // extern "C"

namespace {

gka_status fwd_impl(const gka_params* p, const int32_t* cu, int64_t total, const void* q,
                    const void* k, const void* v, const float* gamma, const float* beta, void* o,
                    float* h_state, float* u_state, float* hnorm2, float* hnorm_t, float* resid,
                    void* workspace, size_t workspace_bytes, void* stream,
                    void* const* phase_events, bool static_ws) {
  gka_status st = check_fwd(p);
  if (st != GKA_OK) return st;
  const bool any_state = h_state || u_state || hnorm2;
  const bool all_state = h_state && u_state && hnorm2;
  if (any_state && !all_state) return GKA_ERR_NULL;
  // rows of the token axis: B T (dense) or the packed total
  const int64_t rows = cu ? total : (int64_t)p->B * p->T;
  if (p->T == 0 || rows == 0) return GKA_OK;  // nothing to do; the state is unchanged
  if (!q || !k || !v || !gamma || !o) return GKA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return GKA_ERR_SHAPE;
  if (h_state && (!aligned16(h_state) || !aligned16(u_state))) return GKA_ERR_SHAPE;
  const size_t n_io = (size_t)rows * p->H * p->D * elem_bytes(p->dtype);
  if (overlap(o, n_io, q, n_io) || overlap(o, n_io, k, n_io) || overlap(o, n_io, v, n_io))
    return GKA_ERR_ALIAS;
  if (beta && (reinterpret_cast<uintptr_t>(beta) & 3u)) return GKA_ERR_SHAPE;
  if (beta && overlap(o, n_io, beta, (size_t)rows * p->H * sizeof(float))) return GKA_ERR_ALIAS;
  if (resid && (reinterpret_cast<uintptr_t>(resid) & 3u)) return GKA_ERR_SHAPE;
  if (resid && overlap(o, n_io, resid, (size_t)rows * p->H * (p->iters + 1) * sizeof(float)))
    return GKA_ERR_ALIAS;
  FwdPlan pl;
  make_plan(p, pl, cu != nullptr);
  if (static_ws && pl.ws_bytes > 0) {  // the library's static scratch replaces the workspace
    if (pl.ws_bytes > (size_t)GKA_STATIC_SCRATCH_BYTES) return GKA_ERR_SCRATCH;
    if (gka::static_scratch(&workspace) != hipSuccess) return GKA_ERR_HIP;
    workspace_bytes = GKA_STATIC_SCRATCH_BYTES;
  }
  if (pl.ws_bytes > 0 && (!workspace || workspace_bytes < pl.ws_bytes || !aligned16(workspace)))
    return GKA_ERR_WORKSPACE;

  const ChebConsts cc = cheb_consts(p->a, p->iters);
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto mark = [&](int i) {
    if (phase_events && phase_events[i])
      return hipEventRecord(static_cast<hipEvent_t>(phase_events[i]), s) == hipSuccess;
    return true;
  };
  const long long DD = (long long)p->D * p->D;
  gka::WalkArgs wa{};
  wa.q = q;
  wa.k = k;
  wa.v = v;
  wa.gamma = gamma;
  wa.beta = beta;
  wa.resid = resid;
  wa.cu = cu;
  if (cu && p->B <= gka::kMaxOrdered) {
    int* order = reinterpret_cast<int*>(static_cast<char*>(workspace) + pl.order_off);
    if (gka::launch_order(cu, p->B, p->T, order, s) != hipSuccess) return GKA_ERR_HIP;
    wa.order = order;
  }
  wa.o = o;
  wa.hnorm_t = hnorm_t;
  // the fused chunk walk from the segment-start states in (in_h, in_u, n2_in, with strides
  // in_bh, in_seg)
  auto walk = [&](const float* in_h, const float* in_u, long long in_bh, long long in_seg,
                  const float* n2_in, const float* in_log2g) -> gka_status {
    wa.in_log2g = in_log2g;
    wa.in_h = in_h;
    wa.in_u = in_u;
    wa.in_bh = in_bh;
    wa.in_seg = in_seg;
    wa.n2_in = n2_in;
    wa.out_h = h_state;
    wa.out_u = u_state;
    wa.n2_out = hnorm2;
    if (gka::launch_walk(pl, false, wa, cc, s) != hipSuccess) return GKA_ERR_HIP;
    if (!mark(3)) return GKA_ERR_HIP;
    return GKA_OK;
  };
  if (pl.S == 1) {
    if (!mark(0) || !mark(1) || !mark(2)) return GKA_ERR_HIP;
    return walk(h_state, u_state, DD, 0, hnorm2, nullptr);
  }
  const size_t bh = (size_t)p->B * p->H;
  float* ws_states = static_cast<float*>(workspace);
  float* ws_log2g = ws_states + bh * pl.S * 2 * DD;
  float* ws_n2 = ws_log2g + bh * pl.S;
  gka::WalkArgs sa = wa;
  sa.sum_h = ws_states;
  sa.sum_u = ws_states + DD;
  sa.sum_bh = (long long)pl.S * 2 * DD;
  sa.sum_seg = 2 * DD;
  sa.log2g_out = ws_log2g;
  if (!mark(0)) return GKA_ERR_HIP;
  if (gka::launch_walk(pl, true, sa, cc, s) != hipSuccess) return GKA_ERR_HIP;
  if (!mark(1)) return GKA_ERR_HIP;
  if (!cu && !h_state && pl.S <= kComposeMaxSegments && gka::walk_tok_supported(pl)) {
    if (!mark(2)) return GKA_ERR_HIP;
    return walk(ws_states, ws_states + DD, (long long)pl.S * 2 * DD, 2 * DD, nullptr, ws_log2g);
  }
  if (gka::launch_scan(pl, ws_states, ws_log2g, h_state, u_state, hnorm2, ws_n2, cu, s) !=
      hipSuccess)
    return GKA_ERR_HIP;
  if (!mark(2)) return GKA_ERR_HIP;
  return walk(ws_states, ws_states + DD, (long long)pl.S * 2 * DD, 2 * DD, ws_n2, nullptr);
}

gka_status step_impl(const gka_params* p, const void* q, const void* k, const void* v,
                     const float* gamma, const float* beta, void* o, float* h_state,
                     float* u_state, float* hnorm2, float* resid, void* stream) {
  gka_status st = check_common(p);
  if (st != GKA_OK) return st;
  if (!q || !k || !v || !gamma || !o || !h_state || !u_state || !hnorm2) return GKA_ERR_NULL;
  if (!aligned16(h_state) || !aligned16(u_state)) return GKA_ERR_SHAPE;
  const size_t n_io = (size_t)p->B * p->H * p->D * elem_bytes(p->dtype);
  if (overlap(o, n_io, q, n_io) || overlap(o, n_io, k, n_io) || overlap(o, n_io, v, n_io))
    return GKA_ERR_ALIAS;
  if (beta && (reinterpret_cast<uintptr_t>(beta) & 3u)) return GKA_ERR_SHAPE;
  if (beta && overlap(o, n_io, beta, (size_t)p->B * p->H * sizeof(float))) return GKA_ERR_ALIAS;
  if (resid && (reinterpret_cast<uintptr_t>(resid) & 3u)) return GKA_ERR_SHAPE;
  if (resid && overlap(o, n_io, resid, (size_t)p->B * p->H * (p->iters + 1) * sizeof(float)))
    return GKA_ERR_ALIAS;
  const ChebConsts cc = cheb_consts(p->a, p->iters);
  if (gka::launch_step(p->dtype, p->D, p->B * p->H, q, k, v, gamma, beta, o, h_state, u_state,
                       hnorm2, resid, cc, static_cast<hipStream_t>(stream)) != hipSuccess)
    return GKA_ERR_HIP;
  return GKA_OK;
}

}  // namespace

extern "C" {

gka_status gka_step(const gka_params* p, const void* q, const void* k, const void* v,
                    const float* gamma, void* o, float* h_state, float* u_state, float* hnorm2,
                    void* stream) {
  return step_impl(p, q, k, v, gamma, nullptr, o, h_state, u_state, hnorm2, nullptr, stream);
}

gka_status gka_step_beta(const gka_params* p, const void* q, const void* k, const void* v,
                         const float* gamma, const float* beta, void* o, float* h_state,
                         float* u_state, float* hnorm2, void* stream) {
  return step_impl(p, q, k, v, gamma, beta, o, h_state, u_state, hnorm2, nullptr, stream);
}

size_t gka_bwd_workspace_bytes(const gka_params* p) {
  if (check_common(p) != GKA_OK || p->T < 0) return 0;
  return bwd_layout(p).total;
}

gka_status gka_bwd(const gka_params* p, const void* q, const void* k, const void* v,
                   const float* gamma, const float* beta, const void* dout, void* dq, void* dk,
                   void* dv, float* dgamma, float* dbeta, void* workspace,
                   size_t workspace_bytes, void* stream) {
  gka_status st = check_common(p);
  if (st != GKA_OK) return st;
  if (p->T < 0) return GKA_ERR_SHAPE;
  if ((long long)p->B * p->T * p->H * p->D > (1LL << 40)) return GKA_ERR_SHAPE;
  if (p->T == 0) return GKA_OK;
  if (!q || !k || !v || !gamma || !dout || !dq || !dk || !dv || !dgamma) return GKA_ERR_NULL;
  const size_t rows = (size_t)p->B * p->T * p->H;
  const size_t n_io = rows * p->D * elem_bytes(p->dtype);
  const void* ins[] = {q, k, v, dout};
  void* outs[] = {dq, dk, dv};
  for (void* o : outs) {
    for (const void* i : ins)
      if (overlap(o, n_io, i, n_io)) return GKA_ERR_ALIAS;
    if (overlap(o, n_io, gamma, rows * 4) || (beta && overlap(o, n_io, beta, rows * 4)))
      return GKA_ERR_ALIAS;
  }
  if (overlap(dq, n_io, dk, n_io) || overlap(dq, n_io, dv, n_io) || overlap(dk, n_io, dv, n_io))
    return GKA_ERR_ALIAS;
  if ((reinterpret_cast<uintptr_t>(dgamma) & 3u) || (dbeta && (reinterpret_cast<uintptr_t>(dbeta) & 3u)) ||
      (beta && (reinterpret_cast<uintptr_t>(beta) & 3u)))
    return GKA_ERR_SHAPE;
  const BwdLayoutHost lay = bwd_layout(p);
  if (!workspace || workspace_bytes < lay.total || !aligned16(workspace)) return GKA_ERR_WORKSPACE;
  const ChebConsts cc = cheb_consts(p->a, p->iters);
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* ws = static_cast<float*>(workspace);
  // the plan of one chunk per segment
  const FwdPlan pl = bwd_plan(p);
  const long long DD = (long long)p->D * p->D;
  // every chunk's starting state from the zero state. Matrix-core path: the forward's segment
  // summaries and scan, then a walk over each segment's chunks. Vector sweeps: the summaries and
  // scan with one chunk per segment.
  if (lay.tok) {
    const FwdPlan ps = bwd_seg_plan(p);
    if (ps.S > 1) {
      gka::WalkArgs sa{};
      sa.q = q;
      sa.k = k;
      sa.v = v;
      sa.gamma = gamma;
      sa.beta = beta;
      sa.sum_h = ws + lay.sstates;
      sa.sum_u = ws + lay.sstates + DD;
      sa.sum_bh = (long long)ps.S * 2 * DD;
      sa.sum_seg = 2 * DD;
      sa.log2g_out = ws + lay.slog2;
      if (gka::launch_walk(ps, true, sa, cc, s) != hipSuccess) return GKA_ERR_HIP;
    }
    if (gka::launch_scan(ps, ws + lay.sstates, ws + lay.slog2, nullptr, nullptr, nullptr,
                         ws + lay.sn2, nullptr, s) != hipSuccess)
      return GKA_ERR_HIP;
    gka::BwdArgs sb{};
    sb.k = k;
    sb.v = v;
    sb.gamma = gamma;
    sb.beta = beta;
    sb.fs16 = ws + lay.fs16;
    sb.fexp = ws + lay.fexp;
    if (gka::launch_bwd_states(ps, sb, ws + lay.sstates, s) != hipSuccess) return GKA_ERR_HIP;
  } else if (pl.S > 1) {
    gka::WalkArgs sa{};
    sa.q = q;
    sa.k = k;
    sa.v = v;
    sa.gamma = gamma;
    sa.beta = beta;
    sa.sum_h = ws + lay.fstates;
    sa.sum_u = ws + lay.fstates + DD;
    sa.sum_bh = (long long)pl.S * 2 * DD;
    sa.sum_seg = 2 * DD;
    sa.log2g_out = ws + lay.flog2;
    if (gka::launch_walk(pl, true, sa, cc, s) != hipSuccess) return GKA_ERR_HIP;
  }
  if (!lay.tok && gka::launch_scan(pl, ws + lay.fstates, ws + lay.flog2, nullptr, nullptr,
                                   nullptr, ws + lay.fn2, nullptr, s) != hipSuccess)
    return GKA_ERR_HIP;
  gka::BwdArgs ba{};
  ba.q = q;
  ba.k = k;
  ba.v = v;
  ba.gamma = gamma;
  ba.beta = beta;
  ba.dout = dout;
  ba.dq = dq;
  ba.dk = dk;
  ba.dv = dv;
  ba.dgamma = dgamma;
  ba.dbeta = dbeta;
  ba.xs = ws + lay.xs;
  ba.ys = ws + lay.ys;
  ba.fstates = lay.tok ? nullptr : ws + lay.fstates;
  ba.fs16 = lay.tok ? ws + lay.fs16 : nullptr;
  ba.fexp = lay.tok ? ws + lay.fexp : nullptr;
  ba.rstates = lay.tok ? nullptr : ws + lay.rstates;
  ba.rd16 = lay.tok ? ws + lay.rd16 : nullptr;
  ba.rdx = lay.tok ? reinterpret_cast<signed char*>(ws + lay.rdx) : nullptr;
  ba.rlog2 = ws + lay.rlog2;
  ba.rn2 = ws + lay.rn2;
  if (lay.tok) {
    ba.dkh = ws + lay.dkh;
    ba.tokv = ws + lay.tokv;
    ba.rs16 = ws + lay.rs16;
    ba.rexp = ws + lay.rexp;
    if (gka::launch_bwd_tok(pl, ba, cc, s) != hipSuccess) return GKA_ERR_HIP;
  } else {
    ba.snap = ws + lay.snap;
    ba.cs = ws + lay.cs;
    if (gka::launch_bwd(pl, ba, cc, s) != hipSuccess) return GKA_ERR_HIP;
  }
  return GKA_OK;
}

gka_status gka_step_residuals(const gka_params* p, const void* q, const void* k, const void* v,
                              const float* gamma, const float* beta, void* o, float* h_state,
                              float* u_state, float* hnorm2, float* resid, void* stream) {
  if (p && check_common(p) == GKA_OK && !resid_rows_fit(p)) return GKA_ERR_SHAPE;
  if (!resid && p) {
    const gka_status st = check_common(p);
    return st != GKA_OK ? st : GKA_ERR_NULL;
  }
  return step_impl(p, q, k, v, gamma, beta, o, h_state, u_state, hnorm2, resid, stream);
}

}  // extern "C"
