// Host-side launchers of the GKA kernels (internal to libgka.so; the public ABI is gka.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

#include "gka_common.hpp"

namespace gka {

// Raises a kernel's dynamic LDS limit, once per device: the attribute persists, and setting it on
// every launch costs host time between the launches of one call. `done` holds one bit per
// device (devices >= 64 are set every time).
inline hipError_t ensure_dynamic_lds(const void* kern, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t)1 << dev : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
  return e;
}

// Decode step: one workgroup per (batch row, head).
// resid (optional, [BH][iters + 1]): the residual mode's ||q - A x_i|| for i = 0..iters.
hipError_t launch_step(int dtype, int D, int BH, const void* q, const void* k, const void* v,
                       const float* gamma, const float* beta, void* o, float* h, float* u,
                       float* n2, float* resid, const ChebConsts& cc, hipStream_t stream);

// Prefill. Segment plan of one call: N chunks split into S segments of J chunks each.
struct FwdPlan {
  int B, T, H, D, C, dtype;
  int N;  // chunks = ceil(T / C)
  int S;  // segments
  int J;  // chunks per segment
  size_t ws_bytes;
  size_t order_off;  // packed batches: byte offset of the dispatch order in the workspace
};

// Arguments of the fused chunk walk (one workgroup per (segment, batch row x head)).
// State matrices are float32 D x D, row-major; head bh, segment sg lives at
// base + bh * *_bh + sg * *_seg (floats).
struct WalkArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* gamma;
  const float* beta;      // optional per-token write gate [B, T, H] (NULL: 1)
  void* o;
  float* hnorm_t;         // optional per-token ||H_t||_F [B, T, H]
  const float* in_h;      // segment-start H (NULL: zero state)
  const float* in_u;      // segment-start U
  long long in_bh, in_seg;
  const float* n2_in;     // [BH] ||H||_F^2 at the start of segment 0 (NULL: from in_h / zero)
  const float* in_log2g;  // token walk, a call from the zero state: the segment summaries'
                          // log2 gate products [BH][S]; in_h / in_u then hold the summaries of
                          // segments 0 .. S-2 and every segment composes its own start state
  float* out_h;           // optional final state, [BH][D][D], written by the last segment
  float* out_u;
  float* n2_out;          // optional final ||H||_F^2, written by the last segment
  float* sum_h;           // summary mode: per-segment (dH, dU) from a zero start
  float* sum_u;
  long long sum_bh, sum_seg;
  float* log2g_out;       // summary mode: per-segment log2 of the gate product [BH][S]
  float* resid;           // optional residual norms ||q_t - A_t x_i||, [B, T, H, iters + 1]
  const int* cu;          // packed batches: sequence b is rows [cu[b], cu[b+1]) (NULL: dense)
  const int* order;       // packed batches: sequences by decreasing length (NULL: in order)
};

// The last segment holding tokens of a sequence of len tokens (segments of J chunks of C): -1
// for an empty sequence. Segments past it have nothing to do; it writes the final state. For a
// dense batch it is S - 1.
__host__ __device__ inline int last_segment(int len, int J, int C) {
  return (len + J * C - 1) / (J * C) - 1;
}

// Sequence b and head h of grid row y: with an order, rows go to the longest sequences first,
// so that their workgroups are dispatched first.
__device__ inline void head_of(const WalkArgs& A, int y, int Hn, int& b, int& h) {
  const int slot = y / Hn;
  b = A.order ? A.order[slot] : slot;
  h = y % Hn;
}

// Rows of sequence b on the token axis: [s0, s0 + len). Dense batches: s0 = b Tmax, len = Tmax;
// packed batches: from the offsets, the length clamped to [0, Tmax] (rows past Tmax are not
// part of the call).
__device__ inline void seq_range(const WalkArgs& A, int b, int Tmax, long long& s0, int& len) {
  if (A.cu) {
    const int a0 = A.cu[b], a1 = A.cu[b + 1];
    s0 = a0;
    len = min(max(a1 - a0, 0), Tmax);
  } else {
    s0 = (long long)b * Tmax;
    len = Tmax;
  }
}

hipError_t launch_walk(const FwdPlan& pl, bool summary, const WalkArgs& a, const ChebConsts& cc,
                       hipStream_t stream);

// Packed batches: order[rank] = b, the sequences by decreasing length (ties by index), from
// the offsets cu [B + 1] with lengths clamped to [0, Tmax]. B <= kMaxOrdered.
constexpr int kMaxOrdered = 4096;
hipError_t launch_order(const int* cu, int B, int Tmax, int* order, hipStream_t stream);

// The chunk walk with token-owning waves (bf16 inputs, chunks of 64 tokens, D = 32, 64, 128):
// same arguments and results as the feature-split walk of launch_walk.
bool walk_tok_supported(const FwdPlan& pl);
hipError_t launch_walk_tok(const FwdPlan& pl, const WalkArgs& a, const ChebConsts& cc,
                           hipStream_t stream);

// Segment summaries of the token-owning walk's configurations (bf16, chunks of 64, D = 64, 128),
// for segments 0 .. S-2; same arguments and results as launch_walk with summary = true.
bool summary_tok_supported(const FwdPlan& pl);
hipError_t launch_summary_tok(const FwdPlan& pl, const WalkArgs& a, hipStream_t stream);

// Affine scan over segments: start[0] = (h, u) (zero when NULL), start[s] = G_{s-1} start[s-1] +
// d_{s-1} for s >= 1, written in place over the summaries d_0 .. d_{S-2} (slot S-1 receives
// start[S-1]); also copies hnorm2 to n2_seg0. The final state comes from the last segment's walk.
hipError_t launch_scan(const FwdPlan& pl, float* ws_states, const float* ws_log2g, float* h,
                       float* u, const float* hnorm2, float* n2_seg0, const int* cu,
                       hipStream_t stream);

// Device address of the static scratch array (GKA_STATIC_SCRATCH_BYTES) on the current device,
// looked up on the first call there and kept.
hipError_t static_scratch(void** out);

// Backward pass (gka_bwd): arguments of its kernels. Workspace of the vector sweeps: snap
// [BH][T][2][D][D] (H_t, U_t after every token), xs, ys [BH][T][D] (the solves of the forward
// sweep), cs [BH][T], and the chunk states of the two scans. The matrix-core path (bf16, chunks
// of 64) has no snapshots: xs, ys, dkh [BH][T][D] and tokv [BH][T][4] carry the solve kernel's
// per-token results to the gradient kernel.
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* gamma;
  const float* beta;  // optional write gate (NULL: 1)
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* dgamma;
  float* dbeta;  // optional
  float* snap;
  float* xs;
  float* ys;
  float* cs;
  float* dkh;   // [BH][T][D] 2 Gam_t E_t H0 k_t (matrix-core path)
  float* tokv;  // [BH][T][4] (c_t, sigma_t, k_t^T H0 k_t, -) (matrix-core path)
  float* fstates;  // [BH][N][2][D][D] every chunk's starting H and U (forward scan or the
                   // matrix-core path's state walk)
  float* rstates;        // [BH][N][2][D][D] chunk gradients (Gb, Wb), slot N - 1 - chunk
  void* rd16;            // matrix-core path: the same in fp16, [BH][N][2][D][D], each run of 16
  signed char* rdx;      // columns of a row times 2^-rdx[BH][N][2][D][D / 16]
  float* rlog2;          // [BH][N] log2 of each chunk's gate product P_c, same slots
  void* rs16;            // matrix-core path: the scan's outputs, fp16 [BH][N][2][D][D], each
  float* rexp;           // row times 2^-rexp[BH][N][2][D]
  void* fs16;            // matrix-core path: every chunk's start state, fp16 [BH][N][2][D][D],
  float* fexp;           // each matrix times 2^-fexp[BH][N][2]
  float* rn2;            // [BH] scratch of the reverse scan
};

// Backward of a dense batch; pl: the plan of one chunk per segment (S = N, J = 1).
hipError_t launch_bwd(const FwdPlan& pl, const BwdArgs& a, const ChebConsts& cc,
                      hipStream_t stream);

// The backward on the matrix cores (bf16, chunks of 64, D = 32, 64, 128): the solve kernel, the
// reverse scan and the gradient kernel, after the forward's scan has filled fstates.
bool bwd_tok_supported(const FwdPlan& pl);
// Every chunk's start state into a.fstates [BH][N][2][D][D] for the matrix-core backward: a walk
// over the chunks of each segment of the plan ps (chunks of 64) from seg_states [BH][S][2][D][D],
// the segment scan's start states.
hipError_t launch_bwd_states(const FwdPlan& ps, const BwdArgs& a, const float* seg_states,
                             hipStream_t stream);
hipError_t launch_bwd_tok(const FwdPlan& pl, const BwdArgs& a, const ChebConsts& cc,
                          hipStream_t stream);

}  // namespace gka
