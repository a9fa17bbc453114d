// gka_step: one recurrent decode step of the Gated KalmaNet layer for B x H independent heads.
//
// Per head (arXiv 2511.21016; recurrences from the gating fragment and the adaptive ridge of
// "Key Contributions" 2 on the ai.info summary; solver of Lemma 3/4 on the pith.science page):
//   n2  <- gamma^2 n2 + 2 gamma beta k^T H k + beta^2 ||k||^4   (uses H before the update)
//   H   <- gamma H + beta k k^T,   U <- gamma U + beta v k^T
// with the optional write gate beta of the variant in "Main Findings" on the ai.info summary
// (beta = 1 without it)
//   Chebyshev on (H / ||H||_F + a I) xh = q (spectrum in [a, 1+a]), x = xh / ||H||_F
//   o   =  U x
//
// The step is bound by HBM traffic: the float32 H and U (8 D^2 bytes each) are read once and
// written once; everything else is on chip. Layout of the work: one workgroup per head,
// NT threads; thread tid owns the float4 column group c4 = tid % (D/4) and rows
// r0 + j*RS (r0 = tid / (D/4), RS = 4 NT / D, j < D/RS) of both H and U, held in registers for
// the whole step. H is symmetric, so H x is formed as column sums
// y[c] = sum_r H[r][c] x[r]: each thread reduces over its own rows, lanes sharing a column
// group are combined with cross-lane swaps and the waves through LDS. o = U x needs row sums,
// which are reduced across the D/4 consecutive lanes that share a row.
#include "gka_internal.hpp"

namespace gka {

// RES: residual mode, which also writes ||q - A x_i|| for i = 0..iters to resid[head][i]
template <typename T, int D, int NT, bool RES>
__global__ __launch_bounds__(NT) void step_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                  const T* __restrict__ v,
                                                  const float* __restrict__ gamma,
                                                  const float* __restrict__ beta,
                                                  T* __restrict__ o, float* __restrict__ hs,
                                                  float* __restrict__ us,
                                                  float* __restrict__ n2s,
                                                  float* __restrict__ resid, ChebConsts cc) {
  constexpr int C4 = D / 4;    // float4 groups per row
  constexpr int RS = NT / C4;  // rows covered by one pass of the workgroup
  constexpr int F = D / RS;    // rows per thread
  constexpr int NW = NT / kWave;
  static_assert(NT % C4 == 0 && D % RS == 0 && kWave % C4 == 0, "bad step tiling");

  __shared__ float ks[D], vs[D], xs[D];
  __shared__ float part[NW][D];
  __shared__ float red[2][NW];

  const int head = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid % kWave, wave = tid / kWave;
  const int c4 = tid % C4, r0 = tid / C4;
  const size_t mat = (size_t)head * D * D;

  // state loads first: they are the whole cost of the step
  f32x4 Hr[F], Ur[F];
#pragma unroll
  for (int j = 0; j < F; ++j)
    Hr[j] = *reinterpret_cast<const f32x4*>(hs + mat + (size_t)(r0 + j * RS) * D + 4 * c4);
#pragma unroll
  for (int j = 0; j < F; ++j)
    Ur[j] = *reinterpret_cast<const f32x4*>(us + mat + (size_t)(r0 + j * RS) * D + 4 * c4);

  const float g = gamma[head];
  const float bt = beta ? beta[head] : 1.0f;
  const float n2_old = n2s[head];
  float q_own = 0.0f;
  if (tid < D) {
    ks[tid] = to_f32(k[(size_t)head * D + tid]);
    vs[tid] = to_f32(v[(size_t)head * D + tid]);
    q_own = to_f32(q[(size_t)head * D + tid]);
  }
  __syncthreads();

  const f32x4 kc = *reinterpret_cast<const f32x4*>(ks + 4 * c4);
  float kHk = 0.0f;
#pragma unroll
  for (int j = 0; j < F; ++j) {
    const float kr = ks[r0 + j * RS];
    const float vr = vs[r0 + j * RS];
    const float bkr = bt * kr, bvr = bt * vr;
    kHk += kr * (Hr[j][0] * kc[0] + Hr[j][1] * kc[1] + Hr[j][2] * kc[2] + Hr[j][3] * kc[3]);
    Hr[j] = g * Hr[j] + bkr * kc;
    Ur[j] = g * Ur[j] + bvr * kc;
  }
#pragma unroll
  for (int j = 0; j < F; ++j) {
    *reinterpret_cast<f32x4*>(hs + mat + (size_t)(r0 + j * RS) * D + 4 * c4) = Hr[j];
    *reinterpret_cast<f32x4*>(us + mat + (size_t)(r0 + j * RS) * D + 4 * c4) = Ur[j];
  }

  float kk = tid < D ? ks[tid] * ks[tid] : 0.0f;
  kHk = wave_sum(kHk);
  kk = wave_sum(kk);
  if (lane == 0) {
    red[0][wave] = kHk;
    red[1][wave] = kk;
  }
  __syncthreads();
  kHk = 0.0f;
  kk = 0.0f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    kHk += red[0][w];
    kk += red[1][w];
  }
  const float bkk = bt * kk;
  const float n2 = g * g * n2_old + 2.0f * g * bt * kHk + bkk * bkk;
  if (tid == 0) n2s[head] = n2;

  // Chebyshev iteration on the normalised system; thread c < D owns element c of the iterates
  const bool degenerate = !(n2 > 0.0f);
  const float inv_n = degenerate ? 0.0f : 1.0f / sqrtf(n2);
  // residual mode: sqrt of the sum over the D threads of r^2 (every thread takes part)
  auto block_norm = [&](float r) {
    float s2 = wave_sum(r * r);
    __syncthreads();  // the previous readers of red are done
    if (lane == 0) red[0][wave] = s2;
    __syncthreads();
    s2 = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) s2 += red[0][w];
    return sqrtf(s2);
  };
  // ||H_t|| = 0: x_i = 0 for every i, so every residual is ||q||
  float qn = 0.0f;
  if constexpr (RES) {
    qn = block_norm(q_own);
    if (tid == 0) resid[(size_t)head * (cc.iters + 1)] = qn;  // x_0 = 0
  }
  if (degenerate) q_own = 0.0f;  // ||H_t|| = 0: x = 0 and o = 0
  // A x_i of the normalised system (threads c < D; y = H x as column sums, H symmetric)
  auto apply = [&](float xv) {
    if (tid < D) xs[tid] = xv;
    __syncthreads();
    f32x4 y = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < F; ++j) y += Hr[j] * xs[r0 + j * RS];
#pragma unroll
    for (int m = C4; m < kWave; m <<= 1) {
      y[0] += __shfl_xor(y[0], m, kWave);
      y[1] += __shfl_xor(y[1], m, kWave);
      y[2] += __shfl_xor(y[2], m, kWave);
      y[3] += __shfl_xor(y[3], m, kWave);
    }
    if (lane < C4) *reinterpret_cast<f32x4*>(&part[wave][4 * c4]) = y;
    __syncthreads();
    float ax = 0.0f;
    if (tid < D) {
      float yc = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) yc += part[w][tid];
      ax = yc * inv_n + cc.a * xv;
    }
    return ax;
  };
  auto put_res = [&](int i, float r) {
    const float nr = block_norm(tid < D ? r : 0.0f);
    if (tid == 0) resid[(size_t)head * (cc.iters + 1) + i] = degenerate ? qn : nr;
  };
  float x = cc.c * q_own, xp = 0.0f;
  for (int i = 1; i < cc.iters; ++i) {
    const float ax = apply(x);
    if constexpr (RES) put_res(i, q_own - ax);  // every thread: it holds barriers
    if (tid < D) {
      const float xn = xp + cc.omega[i] * (x - xp + cc.c * (q_own - ax));
      xp = x;
      x = xn;
    }
  }
  if constexpr (RES) put_res(cc.iters, q_own - apply(x));

  // o = U x = (U xh) / ||H||_F
  if (tid < D) xs[tid] = x;
  __syncthreads();
  const f32x4 xc = *reinterpret_cast<const f32x4*>(xs + 4 * c4);
#pragma unroll
  for (int j = 0; j < F; ++j) {
    float pr = Ur[j][0] * xc[0] + Ur[j][1] * xc[1] + Ur[j][2] * xc[2] + Ur[j][3] * xc[3];
#pragma unroll
    for (int m = 1; m < C4; m <<= 1) pr += __shfl_xor(pr, m, kWave);
    if (c4 == 0) o[(size_t)head * D + r0 + j * RS] = from_f32<T>(pr * inv_n);
  }
}

template <typename T, int D, int NT>
static hipError_t launch_step_t(int BH, const void* q, const void* k, const void* v,
                                const float* gamma, const float* beta, void* o, float* h,
                                float* u, float* n2, float* resid, const ChebConsts& cc,
                                hipStream_t stream) {
  if (resid)
    hipLaunchKernelGGL((step_kernel<T, D, NT, true>), dim3(BH), dim3(NT), 0, stream,
                       static_cast<const T*>(q), static_cast<const T*>(k),
                       static_cast<const T*>(v), gamma, beta, static_cast<T*>(o), h, u, n2, resid,
                       cc);
  else
    hipLaunchKernelGGL((step_kernel<T, D, NT, false>), dim3(BH), dim3(NT), 0, stream,
                       static_cast<const T*>(q), static_cast<const T*>(k),
                       static_cast<const T*>(v), gamma, beta, static_cast<T*>(o), h, u, n2,
                       nullptr, cc);
  return hipGetLastError();
}

hipError_t launch_step(int dtype, int D, int BH, const void* q, const void* k, const void* v,
                       const float* gamma, const float* beta, void* o, float* h, float* u,
                       float* n2, float* resid, const ChebConsts& cc, hipStream_t stream) {
  if (dtype == 0) {
    switch (D) {
      case 16: return launch_step_t<bf16, 16, 64>(BH, q, k, v, gamma, beta, o, h, u, n2, resid, cc, stream);
      case 32: return launch_step_t<bf16, 32, 128>(BH, q, k, v, gamma, beta, o, h, u, n2, resid, cc, stream);
      case 64: return launch_step_t<bf16, 64, 256>(BH, q, k, v, gamma, beta, o, h, u, n2, resid, cc, stream);
      case 128: return launch_step_t<bf16, 128, 512>(BH, q, k, v, gamma, beta, o, h, u, n2, resid, cc, stream);
    }
  } else {
    switch (D) {
      case 16: return launch_step_t<float, 16, 64>(BH, q, k, v, gamma, beta, o, h, u, n2, resid, cc, stream);
      case 32: return launch_step_t<float, 32, 128>(BH, q, k, v, gamma, beta, o, h, u, n2, resid, cc, stream);
      case 64: return launch_step_t<float, 64, 256>(BH, q, k, v, gamma, beta, o, h, u, n2, resid, cc, stream);
      case 128: return launch_step_t<float, 128, 512>(BH, q, k, v, gamma, beta, o, h, u, n2, resid, cc, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace gka
