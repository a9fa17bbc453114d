/*
 * gka.h -- C ABI of the MI355X (gfx950) Gated KalmaNet forward library, libgka.so.
 *
 * The layer (arXiv 2511.21016, "Gated KalmaNet: A Fading Memory Layer Through Test-Time Ridge
 * Regression"). For every batch row b, head h and token t it keeps the gated statistics
 *     H_t = gamma_t H_{t-1} + k_t k_t^T          (D x D, symmetric PSD)
 *     U_t = gamma_t U_{t-1} + v_t k_t^T          (D x D, indexed [value dim][key dim])
 * (pith.science page, appendix fragment "Adaptive weighting (gating)": eta_{t,i} is the
 * product of gamma_j for j = i+1..t), sets the adaptive ridge lambda_t = a ||H_t||_F (ai.info
 * summary, "Key Contributions" 2: the condition number is then at most (a+1)/a), solves
 * (H_t + lambda_t I) x_t = q_t with `iters` Chebyshev iterations on the interval
 * [lambda_t, lambda_t + ||H_t||_F] (ai.info summary, "Methodology in Plain English"; weight
 * schedule of Lemma 3/4 on the pith.science page) and emits o_t = U_t x_t.
 *
 * Conventions shared by both entry points
 *   - Every data pointer is a DEVICE pointer owned by the caller, and the library allocates no
 *     memory. Its only global state: per device, which kernels have had their LDS limit raised
 *     (a kernel attribute, set once per device), and the static scratch array of
 *     gka_fwd_chunked_static with its device address. `stream` is a hipStream_t (NULL = the
 *     default stream); all work is enqueued on it and the call returns without synchronising.
 *   - Tensors are dense, contiguous, row-major: q, k, v, o are [B, T, H, D] (prefill) or
 *     [B, H, D] (decode) in `dtype`; gamma is float32 [B, T, H] / [B, H] with values in [0, 1];
 *     h_state and u_state are float32 [B, H, D, D]; hnorm2 is float32 [B, H] holding
 *     ||H||_F^2 of the carried state.
 *   - q and k are used as given (the caller l2-normalises them, caption of Figure 2 on the
 *     pith.science page). gamma = 0 is allowed.
 *   - Chebyshev convention: x_0 = 0, x_1 = 2 q / (L + mu), three-term recurrence with
 *     omega_0 = 2; `iters` = r returns x_r (r - 1 products with the system matrix).
 *     If ||H_t||_F = 0 the output o_t is 0.
 *   - o is rounded to `dtype` (round to nearest even for bf16). Results are deterministic
 *     run to run (no atomics in any reduction).
 *   - Errors: every argument is checked on the host before anything is enqueued; on an error
 *     the call returns its status and writes nothing. GKA_ERR_HIP reports a failed launch;
 *     faults inside a kernel surface at the caller's next synchronisation of `stream`.
 *   - Accepted range. The bf16 prefill with chunks of 64 (the token-owning walk) rescales its
 *     16-bit matrix operands by exact powers of two: the keys and values per chunk, the queries
 *     and the iterate per token, the value state per wave. At its largest each operand then lies
 *     in [1, 2), and the scales are undone in float32. Any bf16 inputs are therefore accepted
 *     whose float32 intermediates stay finite and normal: in practice |q| and |v| within 2^+-60
 *     of unit scale and |k| within 2^+-25 (||H_t||_F^2 grows like |k|^4).
 *     Tested with q scaled by 2^-12 .. 2^10, k by 2^-12 .. 2^8 and v by 2^-20 .. 2^17 at D = 32,
 *     64 and 128. Elsewhere the operands are used as they are. The bf16 prefill with chunks of 32
 *     converts q, k and v to fp16 operands, so there they must lie within fp16's range
 *     (|x| < 65504, and above 2^-14 for full precision). bf16 with chunks of 16 or D = 16, the
 *     float32 prefill and the decode step compute on float32 throughout.
 *   - Interface choices: `stream` is a void* (a hipStream_t) so that this header needs no HIP
 *     include; gka_params.segments lets a caller fix the segment plan (results depend on it only
 *     through rounding order); gka_fwd_chunked's phase_events is a timing hook;
 *     GKA_ERR_ALIAS rejects outputs that overlap inputs.
 */
#ifndef GKA_H
#define GKA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GKA_OK = 0,
  GKA_ERR_NULL = 1,      /* a required pointer is NULL, or the state pointers are mixed  */
  GKA_ERR_SHAPE = 2,     /* B, T, H, D, chunk or segments outside the supported set        */
  GKA_ERR_VALUE = 3,     /* a <= 0 or not finite, iters outside [1, GKA_MAX_ITERS]           */
  GKA_ERR_DTYPE = 4,     /* dtype not one of gka_dtype                                       */
  GKA_ERR_WORKSPACE = 5, /* workspace missing or smaller than gka_fwd_workspace_bytes()      */
  GKA_ERR_HIP = 6,       /* a kernel launch failed                                           */
  GKA_ERR_ALIAS = 7,     /* o overlaps an input tensor                                       */
  GKA_ERR_SCRATCH = 8    /* gka_fwd_chunked_static: plan needs more than the static scratch   */
} gka_status;

typedef enum { GKA_BF16 = 0, GKA_FP32 = 1 } gka_dtype;

#define GKA_MAX_ITERS 64
#define GKA_PHASE_EVENTS 4
#define GKA_STATIC_SCRATCH_BYTES (64u << 20) /* per GPU, held by gka_fwd_chunked_static */

/*
 * Problem description shared by both entry points.
 *   B, H     batch rows and heads, >= 1
 *   T        tokens per sequence (prefill; ignored by gka_step), >= 0; any T is allowed, a
 *            last partial chunk is handled exactly
 *   D        head dimension (key dim = value dim): {16, 32, 64, 128}
 *   chunk    tokens per chunk for the chunk-wise form (prefill; ignored by gka_step):
 *            bf16 {32, 64}, and 16 for D >= 32 (float32 matrix operands); fp32 {16, 32, 64}
 *            for D <= 64 and {16} for D = 128. The result does not depend on it beyond
 *            rounding (N = ceil(T / chunk) chunks).
 *   iters    Chebyshev iterations r, 1 <= r <= GKA_MAX_ITERS
 *   a        ridge scale, a > 0 and finite
 *   dtype    element type of q, k, v, o (gka_dtype)
 *   segments prefill only: sequence segments scanned in parallel; 0 = chosen by the library,
 *            otherwise 1 <= segments (clamped to the number of chunks)
 */
typedef struct {
  int32_t B, T, H, D, chunk, iters;
  float a;
  int32_t dtype;
  int32_t segments;
} gka_params;

/* Bytes of device workspace gka_fwd_chunked needs for *p (0 when none), or 0 for bad *p. */
size_t gka_fwd_workspace_bytes(const gka_params* p);

/*
 * Chunk-wise forward over whole sequences (prefill / training forward). The chunk-wise form
 * follows "Methodology in Plain English" on the ai.info summary: chunks of C tokens, only the
 * chunk-initial states are carried sequentially, and ||H_t||_F comes from a closed form over the
 * chunk's key Gram matrix ("Key Contributions" 3).
 *   q, k, v   [B, T, H, D] dtype, read
 *   gamma     [B, T, H] float32, read
 *   o         [B, T, H, D] dtype, written; must not overlap q, k or v
 *   h_state, u_state, hnorm2
 *             all NULL: start from the zero state and return no final state; or all non-NULL:
 *             read as the initial state and overwritten with the final state (in place)
 *   hnorm_t   optional [B, T, H] float32: ||H_t||_F of every token, written
 *   workspace device scratch of at least gka_fwd_workspace_bytes(p) bytes (NULL if that is 0):
 *             the per-segment states of a multi-segment plan
 *   phase_events
 *             optional (NULL = none): GKA_PHASE_EVENTS (4) caller-created hipEvent_t recorded on
 *             `stream` at the phase boundaries -- [0] before the segment summaries, [1] before
 *             the segment scan, [2] before the fused chunk walk, [3] after it. With one segment
 *             the first three are recorded back to back. For per-phase timing only; nothing else
 *             changes. (A timing hook in the signature: it exists so that the kernels' own times
 *             can be measured on the launch stream.)
 */
gka_status gka_fwd_chunked(const gka_params* p, const void* q, const void* k, const void* v,
                           const float* gamma, void* o, float* h_state, float* u_state,
                           float* hnorm2, float* hnorm_t, void* workspace,
                           size_t workspace_bytes, void* stream, void* const* phase_events);

/*
 * One recurrent decode step for B x H independent heads (the inference path, ai.info summary
 * "Key Contributions" 4). The token first updates the carried state, then the system of the
 * updated state is solved: o uses H_t and U_t including token t, and
 * ||H_t||_F^2 = gamma^2 ||H_{t-1}||_F^2 + 2 gamma k^T H_{t-1} k + ||k||^4.
 *   q, k, v   [B, H, D] dtype, read
 *   gamma     [B, H] float32, read
 *   o         [B, H, D] dtype, written
 *   h_state, u_state [B, H, D, D] float32 and hnorm2 [B, H] float32: required, updated in place
 */
gka_status gka_step(const gka_params* p, const void* q, const void* k, const void* v,
                    const float* gamma, void* o, float* h_state, float* u_state, float* hnorm2,
                    void* stream);

/*
 * Write-gated variants (ai.info summary, "Main Findings": the variant whose recurrence carries a
 * per-token write strength beta_t next to the forget gate gamma_t). Every token's write into the
 * statistics is scaled by beta_t:
 *     H_t = gamma_t H_{t-1} + beta_t k_t k_t^T,   U_t = gamma_t U_{t-1} + beta_t v_t k_t^T
 * and, for the decode step, ||H_t||_F^2 = gamma^2 ||H_{t-1}||_F^2 + 2 gamma beta k^T H_{t-1} k
 * + beta^2 ||k||^4. Everything else (ridge, solver, output) is as in gka_fwd_chunked / gka_step.
 *   beta      float32 [B, T, H] (prefill) or [B, H] (decode), values in [0, 1], read; NULL means
 *             beta = 1 for every token, which gives results identical to the base entry points
 *             (they are these calls with beta = NULL)
 * Other arguments, layouts, ownership and errors are those of the base entry point; in addition
 * a beta that is not 4-byte aligned gives GKA_ERR_SHAPE and one that overlaps o GKA_ERR_ALIAS.
 * Internally
 * the bf16 prefill with chunks of 64 applies beta through float32 weights (the carry weights,
 * the intra-chunk mask and the norm terms), so its carried state is as accurate as without a
 * gate. The other prefill paths apply sqrt(beta_t) on the token's key and value rows where they
 * become matrix operands (bf16 with chunks of 32: fp16 operands, so the state is accurate to
 * about 1e-3 relative). The per-segment summaries take beta_t as a factor of the token's
 * weight. In exact arithmetic all of these give the recurrence above.
 */
gka_status gka_fwd_chunked_beta(const gka_params* p, const void* q, const void* k, const void* v,
                                const float* gamma, const float* beta, void* o, float* h_state,
                                float* u_state, float* hnorm2, float* hnorm_t, void* workspace,
                                size_t workspace_bytes, void* stream, void* const* phase_events);

gka_status gka_step_beta(const gka_params* p, const void* q, const void* k, const void* v,
                         const float* gamma, const float* beta, void* o, float* h_state,
                         float* u_state, float* hnorm2, void* stream);

/*
 * Solver-convergence mode: the calls above (with the optional write gate beta, NULL = 1), which
 * also record how the Chebyshev iteration converges on every token's system. The pages compare
 * solvers by the residual norm per iteration (pith.science page, caption of Figure 1 (a);
 * ai.info summary, "Main Findings", the bullet comparing CH with CG); this is that quantity
 * for the layer's own solver, at the layer's own precision.
 *   resid     required, float32 [B, T, H, iters + 1] (prefill) or [B, H, iters + 1] (decode),
 *             written: resid[..., i] = ||q_t - A_t x_i||_2 for i = 0..iters, A_t = H_t + a
 *             ||H_t||_F I and x_i the i-th Chebyshev iterate (x_0 = 0, so resid[..., 0] =
 *             ||q_t||). The prefill reports the residual that its iteration carries (equal to
 *             q_t - A_t x_i in exact arithmetic, computed with the same matrix-core operands as
 *             the solve; R_iters takes one extra product), the decode step recomputes it from
 *             x_i. Tokens with ||H_t||_F = 0 have x_i = 0 for every i and report ||q_t||
 *             throughout; residuals past the point where the iteration's own coefficients
 *             vanish (|1 - omega_i| < 2^-64, only for a of order 1e9 and more) are below 2^-64
 *             ||q_t|| and are reported as 0.
 * Everything else, o, the state and hnorm_t included, is exactly what the base call computes
 * (the same kernels plus the residual output), so a call here replaces the base call. resid
 * must be 4-byte aligned (GKA_ERR_SHAPE) and must not overlap o (GKA_ERR_ALIAS); NULL resid is
 * GKA_ERR_NULL (for T > 0). The residual mode runs slower than the base call.
 */
gka_status gka_fwd_chunked_residuals(const gka_params* p, const void* q, const void* k,
                                     const void* v, const float* gamma, const float* beta,
                                     void* o, float* h_state, float* u_state, float* hnorm2,
                                     float* hnorm_t, float* resid, void* workspace,
                                     size_t workspace_bytes, void* stream);

gka_status gka_step_residuals(const gka_params* p, const void* q, const void* k, const void* v,
                              const float* gamma, const float* beta, void* o, float* h_state,
                              float* u_state, float* hnorm2, float* resid, void* stream);

/*
 * Packed variable-length batches (serving): B sequences of different lengths concatenated on
 * the token axis, each with its own carried state. Every sequence is the recurrence of
 * gka_fwd_chunked_beta on its own rows. A decode row is a sequence of length 1 continuing its
 * carried state, so one call can serve a batch that mixes prompts being prefilled and
 * sequences being decoded (the chunked-prefill / decode hand-off inside one call).
 *   p          B = number of sequences, T = an upper bound on every sequence length (it sizes
 *              the segment plan); other fields as for gka_fwd_chunked. segments = 0 chooses
 *              about 12 chunks of T per segment.
 *   workspace  at least gka_fwd_varlen_workspace_bytes(p) bytes (it also holds the dispatch
 *              order: the workgroups of the longest sequences are started first, for B <= 4096)
 *   cu_seqlens DEVICE int32 [B + 1], 4-byte aligned: sequence b is rows [cu[b], cu[b+1]) of
 *              the token axis, cu[0] = 0, non-decreasing, cu[B] = total. A length above T counts
 *              as T (the rows past it are not read, written or carried); an empty sequence
 *              leaves its state unchanged.
 *   total      number of rows (host copy of cu[B]), 0 <= total <= B T; it sizes the alias
 *              checks only
 *   q, k, v, o [total, H, D] dtype; gamma, optional beta (NULL = 1) and optional hnorm_t
 *              [total, H] float32
 *   h_state, u_state [B, H, D, D], hnorm2 [B, H]: per sequence, as for gka_fwd_chunked (all
 *              NULL: every sequence starts from the zero state and no final state is returned)
 * Errors as for gka_fwd_chunked_beta; NULL cu_seqlens is GKA_ERR_NULL, a misaligned one or a
 * total outside [0, B T] GKA_ERR_SHAPE. total = 0 (or T = 0) is a no-op.
 */
size_t gka_fwd_varlen_workspace_bytes(const gka_params* p);

gka_status gka_fwd_varlen(const gka_params* p, const int32_t* cu_seqlens, int64_t total,
                          const void* q, const void* k, const void* v, const float* gamma,
                          const float* beta, void* o, float* h_state, float* u_state,
                          float* hnorm2, float* hnorm_t, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * Backward pass: the gradients of L = sum_t <do_t, o_t> for the forward of gka_fwd_chunked_beta
 * from the zero initial state, by implicit differentiation of the solve (ai.info summary,
 * "Methodology in Plain English" and "Main Findings": the backward re-runs the solver on the
 * upstream gradient; Lemma 2: the query gradient is that solve). With x_t the Chebyshev iterate
 * of the forward, y_t = A_t^-1 U_t^T do_t (the same Chebyshev iteration) and
 * c_t = -a (y_t . x_t) / ||H_t||_F:
 *   dq_t = y_t; the statistics' local gradients G_t = -y_t x_t^T + c_t H_t, W_t = do_t x_t^T
 *   run back through the gated recurrences (Gb_t = G_t + gamma_{t+1} Gb_{t+1}, Wb likewise);
 *   dk_t = beta_t ((Gb_t + Gb_t^T) k_t + Wb_t^T v_t), dv_t = beta_t Wb_t k_t,
 *   dgamma_t = <Gb_t, H_{t-1}> + <Wb_t, U_{t-1}>, dbeta_t = k_t^T Gb_t k_t + v_t^T Wb_t k_t.
 * A token with ||H_t||_F = 0 has x_t = 0 by definition and contributes nothing (dq_t = 0).
 *   q, k, v, dout  [B, T, H, D] dtype, read; gamma, optional beta (NULL = 1) [B, T, H] float32
 *   dq, dk, dv     [B, T, H, D] dtype, written; dgamma [B, T, H] float32, written; dbeta
 *                  optional [B, T, H] float32 (the gradient at the given beta, or at beta = 1)
 *   workspace      at least gka_bwd_workspace_bytes(p) bytes. bf16 with D = 32, 64, 128: per
 *                  chunk of 64 tokens and head, the start state, the chunk's own gradient and
 *                  the incoming gradient, each in fp16 (12 D^2 bytes and their exponents); per
 *                  token 4 (3 D + 4) bytes; one float32 D x D pair per segment of the forward's
 *                  plan. Otherwise: two float32 D x D pairs per chunk and 4 (2 D^2 + 2 D + 1)
 *                  bytes per token (every H_t and U_t)
 * Two paths. Every chunk's start state comes from the forward's segment summaries and scan (then,
 * on the matrix-core path, a walk over each segment's chunks), every chunk's incoming gradient
 * from the same scan run over the chunks in reverse order:
 *   bf16 with D = 32, 64, 128: the chunk form on the matrix cores (chunks of 64). Per chunk, the
 *     two Chebyshev solves (x for q, y for U^T do) on the forward walk's scheme, then every
 *     gradient from C x C token-pair products with the decay mask and the dense interaction mask
 *     M diag(c Gam^2) M^T (ai.info summary, "Main Findings", the backward's full interaction
 *     mask). fp16 operands with exact power-of-two scales and float32 accumulation, as the
 *     forward: every gradient within the forward's bf16 tolerance.
 *   float32, and bf16 with D = 16: chunks of 64 tokens (16 for float32 with D = 128) swept in
 *     parallel, token by token, in float32 on the vector units.
 * Errors as for gka_fwd_chunked; outputs must not overlap the inputs or each other
 * (GKA_ERR_ALIAS). T = 0 is a no-op.
 */
size_t gka_bwd_workspace_bytes(const gka_params* p);

gka_status gka_bwd(const gka_params* p, const void* q, const void* k, const void* v,
                   const float* gamma, const float* beta, const void* dout, void* dq, void* dk,
                   void* dv, float* dgamma, float* dbeta, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * Allocation-free prefill, for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc). It is gka_fwd_chunked_beta
 * (beta may be NULL) with the segment workspace in a static device array of the library,
 * GKA_STATIC_SCRATCH_BYTES (64 MiB) on every GPU the library runs on, held until the process
 * ends; it calls no allocating routine. Arguments, layouts and results are those of
 * gka_fwd_chunked_beta (the same kernels: identical output for the same parameters), without
 * the workspace and the phase events.
 *   Errors: those of gka_fwd_chunked_beta; GKA_ERR_SCRATCH when the segment plan of *p needs
 *   more than GKA_STATIC_SCRATCH_BYTES (gka_fwd_workspace_bytes(p) says how much: 2 D^2 floats
 *   per segment and head; set p->segments lower, 1 needs none); GKA_ERR_HIP when the array's
 *   address cannot be obtained on the current device (looked up once per device, on the first
 *   call there that needs it).
 *   Concurrency: all calls on one GPU share its array, which keeps the last call's contents.
 *   Calls on one stream are ordered and safe; calls that overlap in time on one GPU (several
 *   streams or host threads without ordering between them) race and give wrong results.
 */
gka_status gka_fwd_chunked_static(const gka_params* p, const void* q, const void* k,
                                  const void* v, const float* gamma, const float* beta, void* o,
                                  float* h_state, float* u_state, float* hnorm2, float* hnorm_t,
                                  void* stream);

/* Static description of a status code. */
const char* gka_status_str(int status);

/* ABI version of this header (bumped on any signature change). */
int gka_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GKA_H */
