// gka_bwd: backward pass of the Gated KalmaNet layer by implicit differentiation.
//
// For L = sum_t <do_t, o_t> (ai.info summary, "Methodology in Plain English" and "Main Findings":
// the backward re-runs the solver on the upstream gradient; Lemma 2 for the query):
//   x_t = A_t^-1 q_t, g_t = U_t^T do_t, y_t = A_t^-1 g_t (Chebyshev on the normalised system, as
//   the forward), dq_t = y_t, c_t = -a (y_t . x_t) / ||H_t||_F,
//   G_t = -y_t x_t^T + c_t H_t,  W_t = do_t x_t^T,
//   Gb_t = G_t + gamma_{t+1} Gb_{t+1},  Wb_t = W_t + gamma_{t+1} Wb_{t+1},
//   dk_t = beta_t ((Gb_t + Gb_t^T) k_t + Wb_t^T v_t),  dv_t = beta_t Wb_t k_t,
//   dbeta_t = k_t^T Gb_t k_t + v_t^T Wb_t k_t,  dgamma_t = <Gb_t, H_{t-1}> + <Wb_t, U_{t-1}>.
//
// Chunk-parallel sweeps: the D x D matrices are held in registers with the decode step's layout
// (thread tid owns the float4 column group c4 = tid % (D/4) and rows r0 + j RS), one workgroup
// per (chunk, head) of 2D threads (one wave for D <= 32): the per-token block reductions then
// span fewer waves, and the lower register count lets several workgroups share a compute unit.
//   1. The forward's segment summaries and scan with one chunk per segment give every chunk's
//      starting H and U.
//   2. The forward sweep runs each chunk token by token from its starting state: H_t and U_t
//      are written to the workspace (the reverse sweep needs them in reverse order, and the
//      recurrence cannot be run backwards stably: it divides by gamma), the two solves give
//      x_t, y_t, c_t and dq_t.
//   3. The same sweep accumulates the chunk's part of (Gb, Wb) at its first token, a forward
//      sum: Gb_local(c) = sum_t (gamma_{t0+1} .. gamma_t) G_t, likewise Wb, and the product
//      P_c of the gates that carry the next chunk's gradients into it.
//   4. The forward's segment scan over the chunks in reverse order combines them into every
//      chunk's incoming (Gb, Wb): Gb_first(c) = Gb_local(c) + P_c Gb_first(c + 1).
//   5. The final reverse sweep per chunk starts from its incoming gradients and writes dk, dv,
//      dgamma, dbeta.
// Each sweep is sequential over its chunk's tokens (block reductions per token): correct, and
// parallel over chunks and heads, but far from the matrix cores.
#include "gka_internal.hpp"

namespace gka {

namespace {

template <int D, int NT>
struct BwdLayout {
  static constexpr int C4 = D / 4;    // float4 groups per row
  static constexpr int RS = NT / C4;  // rows covered by one pass of the workgroup
  static constexpr int F = D / RS;    // rows per thread
  static constexpr int NW = NT / kWave;
  static_assert(NT % C4 == 0 && D % RS == 0 && kWave % C4 == 0, "bad tiling");
};

// Reductions of the decode-step layout. Every thread of the workgroup calls them (they hold
// barriers); LDS scratch: part [NW][D], red [NW].
template <int D, int NT>
struct BwdReduce {
  using L = BwdLayout<D, NT>;
  float (*part)[D];
  float* red;
  int tid, lane, wave, c4, r0;
  // sum over the workgroup of x
  __device__ float sum(float x) {
    x = wave_sum(x);
    __syncthreads();  // earlier readers of red are done
    if (lane == 0) red[wave] = x;
    __syncthreads();
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < L::NW; ++w) s += red[w];
    return s;
  }
  // column sums: thread c < D receives sum_r M[r][c] w[r] (w in LDS, D floats)
  __device__ float colsum(const f32x4 (&M)[L::F], const float* w) {
    f32x4 y = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < L::F; ++j) y += M[j] * w[r0 + j * L::RS];
#pragma unroll
    for (int m = L::C4; m < kWave; m <<= 1) {
      y[0] += __shfl_xor(y[0], m, kWave);
      y[1] += __shfl_xor(y[1], m, kWave);
      y[2] += __shfl_xor(y[2], m, kWave);
      y[3] += __shfl_xor(y[3], m, kWave);
    }
    __syncthreads();  // earlier readers of part are done
    if (lane < L::C4) *reinterpret_cast<f32x4*>(&part[wave][4 * c4]) = y;
    __syncthreads();
    float s = 0.0f;
    if (tid < D) {
#pragma unroll
      for (int w = 0; w < L::NW; ++w) s += part[w][tid];
    }
    return s;
  }
  // a column sum (as colsum) and a sum over the workgroup of x at once (one pair of barriers)
  __device__ void colsum_sum(const f32x4 (&M)[L::F], const float* w, float x, float& cs,
                             float& s) {
    f32x4 y = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < L::F; ++j) y += M[j] * w[r0 + j * L::RS];
#pragma unroll
    for (int m = L::C4; m < kWave; m <<= 1) {
      y[0] += __shfl_xor(y[0], m, kWave);
      y[1] += __shfl_xor(y[1], m, kWave);
      y[2] += __shfl_xor(y[2], m, kWave);
      y[3] += __shfl_xor(y[3], m, kWave);
    }
    x = wave_sum(x);
    __syncthreads();  // earlier readers of part and red are done
    if (lane < L::C4) *reinterpret_cast<f32x4*>(&part[wave][4 * c4]) = y;
    if (lane == 0) red[wave] = x;
    __syncthreads();
    cs = 0.0f;
    if (tid < D) {
#pragma unroll
      for (int w = 0; w < L::NW; ++w) cs += part[w][tid];
    }
    s = 0.0f;
#pragma unroll
    for (int w = 0; w < L::NW; ++w) s += red[w];
  }
  // two column sums of one matrix at once: thread c < D receives s1 = sum_r M[r][c] w1[r] and
  // s2 = sum_r M[r][c] w2[r]; part2 is a second [NW][D] scratch. The caller guarantees a barrier
  // between the previous reads of part / part2 and this call (the one that publishes w1, w2).
  __device__ void colsum2(const f32x4 (&M)[L::F], const float* w1, const float* w2,
                          float (*part2)[D], float& s1, float& s2) {
    f32x4 y1 = {0.0f, 0.0f, 0.0f, 0.0f}, y2 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < L::F; ++j) {
      y1 += M[j] * w1[r0 + j * L::RS];
      y2 += M[j] * w2[r0 + j * L::RS];
    }
#pragma unroll
    for (int m = L::C4; m < kWave; m <<= 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        y1[i] += __shfl_xor(y1[i], m, kWave);
        y2[i] += __shfl_xor(y2[i], m, kWave);
      }
    }
    if (lane < L::C4) {
      *reinterpret_cast<f32x4*>(&part[wave][4 * c4]) = y1;
      *reinterpret_cast<f32x4*>(&part2[wave][4 * c4]) = y2;
    }
    __syncthreads();
    s1 = s2 = 0.0f;
    if (tid < D) {
#pragma unroll
      for (int w = 0; w < L::NW; ++w) {
        s1 += part[w][tid];
        s2 += part2[w][tid];
      }
    }
  }
  // two sums over the workgroup at once (red2 is a second [NW] scratch)
  __device__ void sum2(float& a, float& b, float* red2) {
    a = wave_sum(a);
    b = wave_sum(b);
    __syncthreads();
    if (lane == 0) {
      red[wave] = a;
      red2[wave] = b;
    }
    __syncthreads();
    a = b = 0.0f;
#pragma unroll
    for (int w = 0; w < L::NW; ++w) {
      a += red[w];
      b += red2[w];
    }
  }
  // column sums of two matrices at once: s1 = sum_r M1[r][c] w1[r], s2 = sum_r M2[r][c] w2[r]
  __device__ void colsum_mm(const f32x4 (&M1)[L::F], const float* w1, const f32x4 (&M2)[L::F],
                            const float* w2, float (*part2)[D], float& s1, float& s2) {
    f32x4 y1 = {0.0f, 0.0f, 0.0f, 0.0f}, y2 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < L::F; ++j) {
      y1 += M1[j] * w1[r0 + j * L::RS];
      y2 += M2[j] * w2[r0 + j * L::RS];
    }
#pragma unroll
    for (int m = L::C4; m < kWave; m <<= 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        y1[i] += __shfl_xor(y1[i], m, kWave);
        y2[i] += __shfl_xor(y2[i], m, kWave);
      }
    }
    __syncthreads();
    if (lane < L::C4) {
      *reinterpret_cast<f32x4*>(&part[wave][4 * c4]) = y1;
      *reinterpret_cast<f32x4*>(&part2[wave][4 * c4]) = y2;
    }
    __syncthreads();
    s1 = s2 = 0.0f;
    if (tid < D) {
#pragma unroll
      for (int w = 0; w < L::NW; ++w) {
        s1 += part[w][tid];
        s2 += part2[w][tid];
      }
    }
  }
  // row sums of two matrices with one vector, written to LDS out1, out2 (one barrier)
  __device__ void rowsum2(const f32x4 (&M1)[L::F], const f32x4 (&M2)[L::F], const float* w,
                          float* out1, float* out2) {
    const f32x4 wc = *reinterpret_cast<const f32x4*>(w + 4 * c4);
#pragma unroll
    for (int j = 0; j < L::F; ++j) {
      float p1 = M1[j][0] * wc[0] + M1[j][1] * wc[1] + M1[j][2] * wc[2] + M1[j][3] * wc[3];
      float p2 = M2[j][0] * wc[0] + M2[j][1] * wc[1] + M2[j][2] * wc[2] + M2[j][3] * wc[3];
#pragma unroll
      for (int m = 1; m < L::C4; m <<= 1) {
        p1 += __shfl_xor(p1, m, kWave);
        p2 += __shfl_xor(p2, m, kWave);
      }
      if (c4 == 0) {
        out1[r0 + j * L::RS] = p1;
        out2[r0 + j * L::RS] = p2;
      }
    }
    __syncthreads();
  }
  // row sums: out[r] = sum_c M[r][c] w[c] for every row r (w in LDS), written to LDS out
  __device__ void rowsum(const f32x4 (&M)[L::F], const float* w, float* out) {
    const f32x4 wc = *reinterpret_cast<const f32x4*>(w + 4 * c4);
#pragma unroll
    for (int j = 0; j < L::F; ++j) {
      float p = M[j][0] * wc[0] + M[j][1] * wc[1] + M[j][2] * wc[2] + M[j][3] * wc[3];
#pragma unroll
      for (int m = 1; m < L::C4; m <<= 1) p += __shfl_xor(p, m, kWave);
      if (c4 == 0) out[r0 + j * L::RS] = p;
    }
    __syncthreads();
  }
};

template <typename T, int D, int NT>
__global__ __launch_bounds__(NT) void bwd_forward_kernel(BwdArgs A, int Tlen, int Hn, int C,
                                                         ChebConsts cc) {
  using L = BwdLayout<D, NT>;
  constexpr int F = L::F, RS = L::RS, NW = L::NW;
  __shared__ float ks[D], vs[D], qv[D], dv_[D], ws[D], ws2[D], xl[D], yl[D];
  __shared__ float part[NW][D], part2[NW][D];
  __shared__ float red[NW];
  const int ch = blockIdx.x, N = gridDim.x;
  const int bh = blockIdx.y;
  const int b = bh / Hn, h = bh % Hn;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int c4 = tid % L::C4, r0 = tid / L::C4;
  BwdReduce<D, NT> R{part, red, tid, lane, wave, c4, r0};
  const T* q = static_cast<const T*>(A.q);
  const T* k = static_cast<const T*>(A.k);
  const T* v = static_cast<const T*>(A.v);
  const T* dout = static_cast<const T*>(A.dout);
  T* dq = static_cast<T*>(A.dq);

  // the chunk's starting state (row-major H and U of the forward's segment scan)
  f32x4 Hr[F], Ur[F];
  const float* st0 = A.fstates + ((size_t)bh * N + ch) * 2 * D * D;
#pragma unroll
  for (int j = 0; j < F; ++j) {
    const int r = r0 + j * RS;
    Hr[j] = *reinterpret_cast<const f32x4*>(st0 + (size_t)r * D + 4 * c4);
    Ur[j] = *reinterpret_cast<const f32x4*>(st0 + (size_t)D * D + (size_t)r * D + 4 * c4);
  }
  // the chunk's part of the statistics' gradients at its first token, weighted by the gate
  // products w_t = gamma_{t0+1} .. gamma_t
  f32x4 Gl[F], Wl[F];
#pragma unroll
  for (int j = 0; j < F; ++j) {
    Gl[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    Wl[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float w = 1.0f, l2p = 0.0f;
  const int t0 = ch * C, t_end = min(Tlen, (ch + 1) * C);
  for (int t = t0; t < t_end; ++t) {
    const long long tok = (b * (long long)Tlen + t) * Hn + h;
    if (tid < D) {
      ks[tid] = to_f32(k[tok * D + tid]);
      vs[tid] = to_f32(v[tok * D + tid]);
      qv[tid] = to_f32(q[tok * D + tid]);
      dv_[tid] = to_f32(dout[tok * D + tid]);
    }
    const float g = A.gamma[tok];
    const float bt = A.beta ? A.beta[tok] : 1.0f;
    if (t > t0) {
      w *= g;
      l2p += log2_gate(g);
    }
    __syncthreads();
    // H_t, U_t, and their snapshot (the reverse sweep reads them back)
    const f32x4 kc = *reinterpret_cast<const f32x4*>(ks + 4 * c4);
    float* snap = A.snap + ((size_t)bh * Tlen + t) * 2 * D * D;
    float sq = 0.0f;
#pragma unroll
    for (int j = 0; j < F; ++j) {
      const int r = r0 + j * RS;
      Hr[j] = g * Hr[j] + (bt * ks[r]) * kc;
      Ur[j] = g * Ur[j] + (bt * vs[r]) * kc;
      *reinterpret_cast<f32x4*>(snap + (size_t)r * D + 4 * c4) = Hr[j];
      *reinterpret_cast<f32x4*>(snap + (size_t)D * D + (size_t)r * D + 4 * c4) = Ur[j];
      sq += Hr[j][0] * Hr[j][0] + Hr[j][1] * Hr[j][1] + Hr[j][2] * Hr[j][2] + Hr[j][3] * Hr[j][3];
    }
    float n2, gu;  // ||H_t||^2 and (U^T do)[c]
    R.colsum_sum(Ur, dv_, sq, gu, n2);
    const bool live = n2 > 0.0f;
    const float n = sqrtf(n2), inv_n = live ? 1.0f / n : 0.0f;
    // the two Chebyshev solves on (H / ||H|| + a I) side by side, x for q and y for U^T do
    // (thread c < D holds element c of both); x = xh / ||H||, y = yh / ||H||
    const float bq = tid < D ? qv[tid] : 0.0f, bg = tid < D ? gu : 0.0f;
    float x = cc.c * bq, xp = 0.0f, y = cc.c * bg, yp = 0.0f;
    for (int i = 1; i < cc.iters; ++i) {
      if (tid < D) {
        ws[tid] = x;
        ws2[tid] = y;
      }
      __syncthreads();
      float hx, hy;
      R.colsum2(Hr, ws, ws2, part2, hx, hy);
      if (tid < D) {
        const float ax = hx * inv_n + cc.a * x, ay = hy * inv_n + cc.a * y;
        const float xn = xp + cc.omega[i] * (x - xp + cc.c * (bq - ax));
        const float yn = yp + cc.omega[i] * (y - yp + cc.c * (bg - ay));
        xp = x;
        x = xn;
        yp = y;
        y = yn;
      }
    }
    x *= inv_n;
    y *= inv_n;
    const float yx = R.sum(tid < D ? y * x : 0.0f);
    const float c = live ? -cc.a * yx * inv_n : 0.0f;
    if (tid < D) {
      const size_t o = ((size_t)bh * Tlen + t) * D + tid;
      A.xs[o] = xl[tid] = live ? x : 0.0f;
      A.ys[o] = yl[tid] = live ? y : 0.0f;
      dq[tok * D + tid] = from_f32<T>(live ? y : 0.0f);
    }
    if (tid == 0) A.cs[(size_t)bh * Tlen + t] = c;
    __syncthreads();
    // G_t = -y x^T + c H_t and W_t = do x^T, into the chunk's weighted sums
    {
      const f32x4 xc = *reinterpret_cast<const f32x4*>(xl + 4 * c4);
#pragma unroll
      for (int j = 0; j < F; ++j) {
        const int r = r0 + j * RS;
        Gl[j] += w * (c * Hr[j] - yl[r] * xc);
        Wl[j] += w * (dv_[r] * xc);
      }
    }
    __syncthreads();  // the token vectors are read
  }
  // slot N - 1 - c of the reverse scan: the chunk's (Gb, Wb) and log2 P_c, P_c = w_{t_end-1}
  // gamma_{t_end} (the next chunk's first gate)
  float* slot = A.rstates + ((size_t)bh * N + (N - 1 - ch)) * 2 * D * D;
#pragma unroll
  for (int j = 0; j < F; ++j) {
    const int r = r0 + j * RS;
    *reinterpret_cast<f32x4*>(slot + (size_t)r * D + 4 * c4) = Gl[j];
    *reinterpret_cast<f32x4*>(slot + (size_t)D * D + (size_t)r * D + 4 * c4) = Wl[j];
  }
  if (tid == 0) {
    const long long tnext = (b * (long long)Tlen + t_end) * Hn + h;
    A.rlog2[(size_t)bh * N + (N - 1 - ch)] = l2p + (t_end < Tlen ? log2_gate(A.gamma[tnext]) : 0.0f);
  }
}

// From the incoming gradients of slot N - 1 - c (as the reverse scan left them), writing the
// gradients of the inputs.
template <typename T, int D, int NT>
__global__ __launch_bounds__(NT) void bwd_reverse_kernel(BwdArgs A, int Tlen, int Hn, int C) {
  using L = BwdLayout<D, NT>;
  constexpr int F = L::F, RS = L::RS, NW = L::NW;
  __shared__ float ks[D], vs[D], xv[D], yv[D], dv_[D], rgk[D], rwk[D];
  __shared__ float part[NW][D], part2[NW][D];
  __shared__ float red[NW], red2[NW];
  const int ch = blockIdx.x, N = gridDim.x;
  const int bh = blockIdx.y;
  const int b = bh / Hn, h = bh % Hn;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int c4 = tid % L::C4, r0 = tid / L::C4;
  BwdReduce<D, NT> R{part, red, tid, lane, wave, c4, r0};
  const T* k = static_cast<const T*>(A.k);
  const T* v = static_cast<const T*>(A.v);
  const T* dout = static_cast<const T*>(A.dout);
  T* dk = static_cast<T*>(A.dk);
  T* dvo = static_cast<T*>(A.dv);

  const float* slot = A.rstates + ((size_t)bh * N + (N - 1 - ch)) * 2 * D * D;
  f32x4 Gb[F], Wb[F];
#pragma unroll
  for (int j = 0; j < F; ++j) {
    const int r = r0 + j * RS;
    Gb[j] = *reinterpret_cast<const f32x4*>(slot + (size_t)r * D + 4 * c4);
    Wb[j] = *reinterpret_cast<const f32x4*>(slot + (size_t)D * D + (size_t)r * D + 4 * c4);
  }
  const int t0 = ch * C, t_end = min(Tlen, (ch + 1) * C);
  // H_{t-1} is read for dgamma at step t and kept as H_t of step t - 1
  f32x4 Hc[F];
  {
    const float* snap_last = A.snap + ((size_t)bh * Tlen + (t_end - 1)) * 2 * D * D;
#pragma unroll
    for (int j = 0; j < F; ++j)
      Hc[j] = *reinterpret_cast<const f32x4*>(snap_last + (size_t)(r0 + j * RS) * D + 4 * c4);
  }
  for (int t = t_end - 1; t >= t0; --t) {
    const long long tok = (b * (long long)Tlen + t) * Hn + h;
    const size_t row = ((size_t)bh * Tlen + t) * D;
    if (tid < D) {
      ks[tid] = to_f32(k[tok * D + tid]);
      vs[tid] = to_f32(v[tok * D + tid]);
      dv_[tid] = to_f32(dout[tok * D + tid]);
      xv[tid] = A.xs[row + tid];
      yv[tid] = A.ys[row + tid];
    }
    const float c = A.cs[(size_t)bh * Tlen + t];
    // gamma_{t+1} (past the chunk's last token it carries the incoming gradients)
    const float gn = t + 1 < Tlen ? A.gamma[tok + Hn] : 0.0f;
    const float bt = A.beta ? A.beta[tok] : 1.0f;
    __syncthreads();
    // Gb_t = -y x^T + c H_t + gamma_{t+1} Gb_{t+1},  Wb_t = do x^T + gamma_{t+1} Wb_{t+1}
    const f32x4 xc = *reinterpret_cast<const f32x4*>(xv + 4 * c4);
    const float* snap = A.snap + ((size_t)bh * Tlen + t) * 2 * D * D;
    const float* prev = t > 0 ? snap - 2 * D * D : nullptr;  // H_{t-1}, U_{t-1} (zero at t = 0)
    float dg = 0.0f;
#pragma unroll
    for (int j = 0; j < F; ++j) {
      const int r = r0 + j * RS;
      Gb[j] = c * Hc[j] - yv[r] * xc + gn * Gb[j];
      Wb[j] = dv_[r] * xc + gn * Wb[j];
      if (prev) {
        const f32x4 Hp = *reinterpret_cast<const f32x4*>(prev + (size_t)r * D + 4 * c4);
        const f32x4 Up = *reinterpret_cast<const f32x4*>(prev + (size_t)D * D + (size_t)r * D + 4 * c4);
        dg += Gb[j][0] * Hp[0] + Gb[j][1] * Hp[1] + Gb[j][2] * Hp[2] + Gb[j][3] * Hp[3];
        dg += Wb[j][0] * Up[0] + Wb[j][1] * Up[1] + Wb[j][2] * Up[2] + Wb[j][3] * Up[3];
        Hc[j] = Hp;  // H_t of step t - 1
      }
    }
    {
      R.rowsum2(Gb, Wb, ks, rgk, rwk);  // (Gb k)[r], (Wb k)[r]
      float gtk, wtv;
      R.colsum_mm(Gb, ks, Wb, vs, part2, gtk, wtv);  // (Gb^T k)[c], (Wb^T v)[c]
      float db = 0.0f;
      if (tid < D) {
        dk[tok * D + tid] = from_f32<T>(bt * (rgk[tid] + gtk + wtv));
        dvo[tok * D + tid] = from_f32<T>(bt * rwk[tid]);
        db = ks[tid] * rgk[tid] + vs[tid] * rwk[tid];
      }
      R.sum2(dg, db, red2);
      if (tid == 0) {
        A.dgamma[tok] = dg;
        if (A.dbeta) A.dbeta[tok] = db;
      }
    }
    __syncthreads();  // the token vectors are read
  }
}

// NT threads for the forward sweep (it holds four D x D matrices), NTR for the reverse (two)
template <typename T, int D, int NT, int NTR>
hipError_t launch_bwd_t(const FwdPlan& pl, const BwdArgs& a, const ChebConsts& cc,
                        hipStream_t stream) {
  const dim3 grid(pl.N, pl.B * pl.H);
  hipLaunchKernelGGL((bwd_forward_kernel<T, D, NT>), grid, dim3(NT), 0, stream, a, pl.T, pl.H,
                     pl.C, cc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // incoming gradients of every chunk: the segment scan over the chunks in reverse order
  if ((e = launch_scan(pl, a.rstates, a.rlog2, nullptr, nullptr, nullptr, a.rn2, nullptr,
                       stream)) != hipSuccess)
    return e;
  hipLaunchKernelGGL((bwd_reverse_kernel<T, D, NTR>), grid, dim3(NTR), 0, stream, a, pl.T,
                     pl.H, pl.C);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const FwdPlan& pl, const BwdArgs& a, const ChebConsts& cc,
                      hipStream_t stream) {
  if (pl.dtype == 0) {
    switch (pl.D) {
      case 16: return launch_bwd_t<bf16, 16, 64, 64>(pl, a, cc, stream);
      case 32: return launch_bwd_t<bf16, 32, 64, 64>(pl, a, cc, stream);
      case 64: return launch_bwd_t<bf16, 64, 128, 128>(pl, a, cc, stream);
      case 128: return launch_bwd_t<bf16, 128, 512, 256>(pl, a, cc, stream);
    }
  } else {
    switch (pl.D) {
      case 16: return launch_bwd_t<float, 16, 64, 64>(pl, a, cc, stream);
      case 32: return launch_bwd_t<float, 32, 64, 64>(pl, a, cc, stream);
      case 64: return launch_bwd_t<float, 64, 128, 128>(pl, a, cc, stream);
      case 128: return launch_bwd_t<float, 128, 512, 256>(pl, a, cc, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace gka
