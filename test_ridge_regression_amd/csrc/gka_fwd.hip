// gka_fwd_chunked: chunk-wise forward of the Gated KalmaNet layer (prefill / training forward).
//
// The chunk-wise form follows "Methodology in Plain English" on the ai.info summary of
// arXiv 2511.21016: the sequence is cut into chunks of C tokens, only the chunk-initial states
// are carried from chunk to chunk, everything inside a chunk is parallel, and ||H_t||_F comes
// from a closed form over the chunk's key Gram matrix ("Key Contributions" 3). The algebra used
// here, for a chunk starting from (H0, U0, ||H0||^2) with in-chunk log2-gate prefix cl_t,
// Gam_t = 2^cl_t and the causal decay mask M_ts = 2^(cl_t - cl_s) [s <= t]:
//
//   H_t x     = Gam_t H0 x + sum_s M_ts (k_s . x) k_s
//   ||H_t||^2 = Gam_t^2 ||H0||^2 + 2 Gam_t sum_s M_ts k_s^T H0 k_s + sum_{s,u} M_ts M_tu (k_s.k_u)^2
//   U_t x     = Gam_t U0 x + sum_s M_ts (k_s . x) v_s
//   carry       H0 <- Gam_C H0 + K^T diag(w) K,  U0 <- Gam_C U0 + V^T diag(w) K, w_s = 2^(cl_C - cl_s)
//
// The Chebyshev iteration runs on the system divided by ||H_t||_F, whose spectrum lies in
// [a, 1 + a] for every token, so the step 2/(1+2a) and the weights omega_i are launch constants
// and only the per-token scales s_t = Gam_t / ||H_t|| and M_ts / ||H_t|| change. With X the
// C x D block of normalised iterates (one row per token), one application of the system is
//   A(X) = diag(s) X H0 + ((X K^T) o Mhat) K + a X,      and   O = diag(s) X U0^T + ((X K^T) o Mhat) V.
// All products are computed transposed (feature x token outputs), so that the matrix-core
// accumulator layout (4 consecutive rows per lane) maps to 4 consecutive features of one token.
//
// Kernels of one call:
//   1. summary walk (only with S > 1 segments): per (segment, head), the state reached from a zero
//      state over the segment's chunks, and the segment's total gate (log2);
//   2. segment scan: elementwise affine scan over segments -> segment-start states, final state;
//   3. fused walk: per (segment, head), from the segment-start state, chunk by chunk:
//      gate prologue, norms, Chebyshev loop, output, state carry. The float32 state lives in
//      matrix-core accumulators for the whole walk; bf16 (or fp32) copies of H0, U0, K, K^T, V^T,
//      the iterate and the masked product are staged in LDS.
#include "gka_internal.hpp"

namespace gka {

template <typename T, int D, int C>
struct WalkCfg {
  static constexpr int NW = 4;
  static constexpr int NT = NW * kWave;
  static constexpr int PAD = 16 / (int)sizeof(T);  // 16 bytes of row padding
  static constexpr int LDD = D + PAD;              // row stride of [*][D] tiles (elements)
  static constexpr int LDC = C + PAD;              // row stride of [*][C] tiles (elements)
  static constexpr int LDF = C + 4;                // row stride of [C][C] float tiles
  static constexpr int FT = D / 16;                // feature tiles
  static constexpr int CT = C / 16;                // token tiles
  static constexpr int FPW = (FT + NW - 1) / NW;   // feature tiles per wave
  static constexpr int PT = CT * CT;               // C x C tiles
  static constexpr int PPW = (PT + NW - 1) / NW;
  static constexpr int ST = FT * FT;               // D x D tiles
  static constexpr int SPW = (ST + NW - 1) / NW;
  static constexpr int K = Mma<T>::K;
  static constexpr int E = Mma<T>::E;
  static_assert(D % K == 0 && C % K == 0 && C <= kWave, "unsupported D / C");
  static_assert(NT == 256, "walk_kernel is declared with __launch_bounds__(256)");

  // bf16 operands of the intra-chunk pair and of the output are split into hi + lo parts
  static constexpr bool SPLIT = sizeof(T) == 2;

  // LDS layout (bytes)
  static constexpr size_t szHs = (size_t)D * LDD * sizeof(T);  // H0 (then U0) copy, [D][LDD]
  static constexpr size_t szKs = (size_t)C * LDD * sizeof(T);  // K, [C][LDD]
  static constexpr size_t szKT = (size_t)D * LDC * sizeof(T);  // K^T, [D][LDC]
  static constexpr size_t szVT = szKT;                         // V^T, [D][LDC]
  static constexpr size_t szXs = (size_t)C * LDD * sizeof(T);  // operand (hi), [C][LDD]
  static constexpr size_t szG2 = (size_t)C * LDF * sizeof(float);  // (K K^T)^2, aliases Xs
  static constexpr size_t szMf = (size_t)C * LDF * sizeof(float);  // decay mask M, [C][LDF]
  static constexpr size_t szPs = (size_t)C * LDC * sizeof(T);  // masked product (hi), [C][LDC]
  static constexpr size_t mx(size_t a, size_t b) { return a > b ? a : b; }
  static constexpr size_t szXG = mx(szXs, szG2);
  // with SPLIT the mask shares its buffer with the lo part of the operand (the mask is moved to
  // registers before the operand is first written)
  static constexpr size_t szXl = SPLIT ? mx(szXs, szMf) : szMf;
  static constexpr size_t szPl = SPLIT ? szPs : 0;
  static constexpr size_t szVec = (size_t)(8 * C + 2 * NW * C + 16) * sizeof(float);
  static constexpr size_t oHs = 0;
  static constexpr size_t oKs = oHs + szHs;
  static constexpr size_t oKT = oKs + szKs;
  static constexpr size_t oVT = oKT + szKT;
  static constexpr size_t oXs = oVT + szVT;
  static constexpr size_t oXl = oXs + szXG;  // lo operand (SPLIT) and the mask
  static constexpr size_t oMf = oXl;
  static constexpr size_t oPs = oXl + szXl;
  static constexpr size_t oPl = oPs + szPs;
  static constexpr size_t oVec = oPl + szPl;
  static constexpr size_t bytes = oVec + szVec;
  static_assert(bytes <= 160 * 1024, "LDS budget of one CU exceeded");
};

template <typename T>
__device__ inline void split_hi_lo(float x, T& hi, T& lo);
template <>
__device__ inline void split_hi_lo<bf16>(float x, bf16& hi, bf16& lo) {
  hi = (bf16)x;
  lo = (bf16)(x - (float)hi);
}

template <typename T, int D, int C, bool SUMMARY>
__global__ __launch_bounds__(256) void walk_kernel(WalkArgs A, int B, int Tlen,
                                                                   int Hn, int N, int S, int J,
                                                                   ChebConsts cc) {
  using Cfg = WalkCfg<T, D, C>;
  using M = Mma<T>;
  using MF = Mma<float>;
  constexpr int NW = Cfg::NW, LDD = Cfg::LDD, LDC = Cfg::LDC, LDF = Cfg::LDF;
  constexpr int FT = Cfg::FT, CT = Cfg::CT, FPW = Cfg::FPW, PPW = Cfg::PPW, SPW = Cfg::SPW;
  constexpr int K = Cfg::K, E = Cfg::E;
  constexpr bool SPLIT = Cfg::SPLIT;

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  T* Hs = reinterpret_cast<T*>(smem + Cfg::oHs);
  T* Ks = reinterpret_cast<T*>(smem + Cfg::oKs);
  T* KT = reinterpret_cast<T*>(smem + Cfg::oKT);
  T* VT = reinterpret_cast<T*>(smem + Cfg::oVT);
  T* Xs = reinterpret_cast<T*>(smem + Cfg::oXs);
  T* Xl = reinterpret_cast<T*>(smem + Cfg::oXl);
  float* G2 = reinterpret_cast<float*>(smem + Cfg::oXs);
  T* Ps = reinterpret_cast<T*>(smem + Cfg::oPs);
  T* Pl = reinterpret_cast<T*>(smem + Cfg::oPl);
  float* Mf = reinterpret_cast<float*>(smem + Cfg::oMf);
  float* vec = reinterpret_cast<float*>(smem + Cfg::oVec);
  float* v_cl = vec;            // [C] in-chunk log2 gate prefix
  float* v_gam = v_cl + C;      // [C] 2^cl
  float* v_w = v_gam + C;       // [C] carry weights 2^(cl_C - cl_s)
  float* v_ninv = v_w + C;      // [C] 1 / ||H_t|| (0 when ||H_t|| = 0)
  float* v_s = v_ninv + C;      // [C] Gam_t / ||H_t||
  float* v_u = v_s + C;         // [C] k_s^T H0 k_s
  float* v_n2 = v_u + C;        // [C] ||H_t||^2
  float* v_t3 = v_n2 + C;       // [C] quadratic term of ||H_t||^2
  float* p_u = v_t3 + C;        // [NW][C] per-wave partials
  float* p_t3 = p_u + NW * C;   // [NW][C]
  float* v_sc = p_t3 + NW * C;  // scalars: [0] n0^2, [1] reduction scratch (NW)

  const int seg = blockIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / Hn, h = bh % Hn;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int lr = lane % 16;  // row (A) / column (B, accumulator) index inside a tile
  const int lg = lane / 16;  // lane group: K offset E*lg in operands, rows 4*lg.. in accumulators
  const int c_begin = seg * J;
  const int c_end = min(N, c_begin + J);
  const long long tok_stride = (long long)Hn * D;  // elements between consecutive tokens
  const T* qg = static_cast<const T*>(A.q);
  const T* kg = static_cast<const T*>(A.k);
  const T* vg = static_cast<const T*>(A.v);
  T* og = static_cast<T*>(A.o);

  // ---- float32 state in accumulator tiles -----------------------------------------------
  // state tile p = wave + NW*j covers rows 16*(p/FT).., columns 16*(p%FT)..; the H tile holds
  // H[row][col], the U tile holds U^T[row][col] = U[col][row].
  f32x4 Hst[SPW], Ust[SPW];
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    Hst[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    Ust[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float n0sq = 0.0f;
  if (!SUMMARY) {
    if (A.in_h) {
      const float* ih = A.in_h + bh * A.in_bh + seg * A.in_seg;
      const float* iu = A.in_u + bh * A.in_bh + seg * A.in_seg;
      float sq = 0.0f;
#pragma unroll
      for (int j = 0; j < SPW; ++j) {
        const int p = wave + NW * j;
        if (p < Cfg::ST) {
          const int r = 16 * (p / FT) + 4 * lg, c = 16 * (p % FT) + lr;
          // H is symmetric: H[r..r+3][c] is read as H[c][r..r+3]
          Hst[j] = *reinterpret_cast<const f32x4*>(ih + (size_t)c * D + r);
          Ust[j] = *reinterpret_cast<const f32x4*>(iu + (size_t)c * D + r);
          sq += Hst[j][0] * Hst[j][0] + Hst[j][1] * Hst[j][1] + Hst[j][2] * Hst[j][2] +
                Hst[j][3] * Hst[j][3];
        }
      }
      sq = wave_sum(sq);
      if (lane == 0) v_sc[1 + wave] = sq;
      __syncthreads();
      if (seg == 0 && A.n2_in) {
        n0sq = A.n2_in[bh];
      } else {
        n0sq = 0.0f;
        for (int w = 0; w < NW; ++w) n0sq += v_sc[1 + w];
      }
    } else if (seg == 0 && A.n2_in) {
      n0sq = A.n2_in[bh];
    }
  }
  float log2g_seg = 0.0f;  // summary mode: running log2 of the segment's gate product

  for (int ch = c_begin; ch < c_end; ++ch) {
    const int t0 = ch * C;
    const int nv = min(C, Tlen - t0);  // valid tokens of this chunk (last chunk may be partial)
    __syncthreads();  // LDS of the previous chunk is free

    // ---- stage K (row-major), K^T, V^T in LDS; tokens past the end are zero ----------------
    {
      constexpr int VEC = 16 / (int)sizeof(T);
      constexpr int NV = C * D / VEC;
      typedef T vecT __attribute__((ext_vector_type(VEC)));
      for (int e = tid; e < NV; e += Cfg::NT) {
        const int t = e / (D / VEC), d0 = (e % (D / VEC)) * VEC;
        vecT kv, vv;
        if (t < nv) {
          const long long off = ((long long)(b * (long long)Tlen + t0 + t)) * tok_stride + (long long)h * D + d0;
          kv = *reinterpret_cast<const vecT*>(kg + off);
          vv = *reinterpret_cast<const vecT*>(vg + off);
        } else {
#pragma unroll
          for (int i = 0; i < VEC; ++i) { kv[i] = (T)0.0f; vv[i] = (T)0.0f; }
        }
        if (!SUMMARY) *reinterpret_cast<vecT*>(Ks + t * LDD + d0) = kv;
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          KT[(d0 + i) * LDC + t] = kv[i];
          VT[(d0 + i) * LDC + t] = vv[i];
        }
      }
    }
    // ---- gate prologue (wave 0): in-chunk prefix of log2 gamma, Gam, carry weights --------
    if (wave == 0) {
      float l2 = 0.0f;  // tokens past the end behave as gamma = 1 with k = v = q = 0
      if (lane < nv) l2 = log2_gate(A.gamma[(b * (long long)Tlen + t0 + lane) * Hn + h]);
      float cl = l2;
#pragma unroll
      for (int m = 1; m < kWave; m <<= 1) {
        const float o = __shfl_up(cl, m, kWave);
        if (lane >= m) cl += o;
      }
      const float clast = __shfl(cl, C - 1, kWave);
      if (lane < C) {
        v_cl[lane] = cl;
        v_gam[lane] = exp2f(cl);
        v_w[lane] = exp2f(fminf(clast - cl, 0.0f));
      }
      log2g_seg += clast;
    }
    if (!SUMMARY) {
      // bf16 / fp32 copy of H0 for the matrix cores: Hs[c][r..r+3] = H[r..r+3][c] (symmetric)
#pragma unroll
      for (int j = 0; j < SPW; ++j) {
        const int p = wave + NW * j;
        if (p < Cfg::ST) {
          const int r = 16 * (p / FT) + 4 * lg, c = 16 * (p % FT) + lr;
          store4<T>(Hs + c * LDD + r, Hst[j]);
        }
      }
    }
    __syncthreads();

    if (!SUMMARY) {
      // ---- decay mask M[t][s] ----------------------------------------------------------------
      for (int e = tid; e < C * C; e += Cfg::NT) {
        const int t = e / C, s = e % C;
        Mf[t * LDF + s] = s <= t ? exp2f(fminf(v_cl[t] - v_cl[s], 0.0f)) : 0.0f;
      }
      // ---- (K K^T)^2 into G2 (aliases the iterate buffer, unused until the solve) ------------
#pragma unroll
      for (int j = 0; j < PPW; ++j) {
        const int p = wave + NW * j;
        if (p < Cfg::PT) {
          const int sb = p / CT, ub = p % CT;
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < D; kk += K)
            acc = M::mma(M::load(Ks, LDD, 16 * sb + lr, kk + E * lg),
                         M::load(Ks, LDD, 16 * ub + lr, kk + E * lg), acc);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            G2[(16 * sb + 4 * lg + i) * LDF + 16 * ub + lr] = acc[i] * acc[i];
        }
      }
      // ---- u_s = k_s^T H0 k_s from Y = H0 K^T (own feature tiles x all token tiles) ---------
      {
        float up[CT];
#pragma unroll
        for (int tb = 0; tb < CT; ++tb) up[tb] = 0.0f;
#pragma unroll
        for (int jf = 0; jf < FPW; ++jf) {
          const int fb = wave + NW * jf;
          if (fb < FT) {
#pragma unroll
            for (int tb = 0; tb < CT; ++tb) {
              f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int kk = 0; kk < D; kk += K)
                acc = M::mma(M::load(Hs, LDD, 16 * fb + lr, kk + E * lg),
                             M::load(Ks, LDD, 16 * tb + lr, kk + E * lg), acc);
              const f32x4 kf = load4<T>(Ks + (16 * tb + lr) * LDD + 16 * fb + 4 * lg);
              up[tb] += acc[0] * kf[0] + acc[1] * kf[1] + acc[2] * kf[2] + acc[3] * kf[3];
            }
          }
        }
#pragma unroll
        for (int tb = 0; tb < CT; ++tb) {
          float x = up[tb];
          x += __shfl_xor(x, 16, kWave);
          x += __shfl_xor(x, 32, kWave);
          if (lg == 0) p_u[wave * C + 16 * tb + lr] = x;
        }
      }
      __syncthreads();
      // ---- quadratic term: t3_t = sum_s M_ts Z[s][t], Z = G2 M^T (float32 matrix cores) ------
      for (int e = tid; e < NW * C; e += Cfg::NT) p_t3[e] = 0.0f;
      if (tid < C) {
        float u = 0.0f;
        for (int w = 0; w < NW; ++w) u += p_u[w * C + tid];
        v_u[tid] = u;
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < PPW; ++j) {
        const int p = wave + NW * j;
        if (p < Cfg::PT) {
          const int sb = p / CT, tb = p % CT;
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < C; kk += MF::K)
            acc = MF::mma(MF::load(G2, LDF, 16 * sb + lr, kk + lg),
                          MF::load(Mf, LDF, 16 * tb + lr, kk + lg), acc);
          const int t = 16 * tb + lr;
          const f32x4 mts = *reinterpret_cast<const f32x4*>(Mf + t * LDF + 16 * sb + 4 * lg);
          float x = acc[0] * mts[0] + acc[1] * mts[1] + acc[2] * mts[2] + acc[3] * mts[3];
          x += __shfl_xor(x, 16, kWave);
          x += __shfl_xor(x, 32, kWave);
          if (lg == 0) p_t3[wave * C + t] += x;
        }
      }
      __syncthreads();
      // ---- per-token norm and scales ------------------------------------------------------------
      if (tid < C) {
        const int t = tid;
        float t2 = 0.0f;
        for (int s = 0; s <= t; ++s) t2 += Mf[t * LDF + s] * v_u[s];
        float t3 = 0.0f;
        for (int w = 0; w < NW; ++w) t3 += p_t3[w * C + t];
        const float gam = v_gam[t];
        const float n2 = gam * gam * n0sq + 2.0f * gam * t2 + t3;
        const bool zero = !(n2 > 0.0f);
        const float ninv = zero ? 0.0f : 1.0f / sqrtf(n2);
        v_n2[t] = n2;
        v_ninv[t] = ninv;
        v_s[t] = gam * ninv;
        if (A.hnorm_t && t < nv) A.hnorm_t[(b * (long long)Tlen + t0 + t) * Hn + h] = sqrtf(n2);
      }
      __syncthreads();

      // ---- Chebyshev loop, residual form --------------------------------------------------------
      // The iteration is run on the residuals R_i = Q - A X_i (same iterates in exact arithmetic):
      //   R_0 = Q,  R_1 = R_0 - c A R_0,  R_{i+1} = R_{i-1} + omega_i (R_i - R_{i-1} - c A R_i),
      // and X_r = sum_i beta_i R_i with host-computed beta. The products act on the shrinking
      // residual instead of the iterate, whose large components in the null space of H_t would
      // otherwise leak bf16 rounding error into the key directions (amplified by up to
      // kappa = (1+a)/a). For bf16 the operand of the intra-chunk pair (R K^T, then P' K) and of
      // the output products is split into hi + lo bf16 parts.
      // Own tiles of R^T / X^T: feature tiles fb = wave + NW*jf, all token tiles tb; lane holds
      // features 16 fb + 4 lg + i of token 16 tb + lr.
      f32x4 R[FPW][CT], Rp[FPW][CT], Xa[FPW][CT], Y[FPW][CT];
      float sv[CT];
#pragma unroll
      for (int tb = 0; tb < CT; ++tb) sv[tb] = v_s[16 * tb + lr];
#pragma unroll
      for (int jf = 0; jf < FPW; ++jf) {
        const int fb = wave + NW * jf;
#pragma unroll
        for (int tb = 0; tb < CT; ++tb) {
          const int t = 16 * tb + lr;
          f32x4 qv = {0.f, 0.f, 0.f, 0.f};
          if (fb < FT && t < nv && v_ninv[t] > 0.0f) {  // ||H_t|| = 0: x_t = 0
            const long long off = ((long long)(b * (long long)Tlen + t0 + t)) * tok_stride + (long long)h * D + 16 * fb + 4 * lg;
            qv = load4<T>(qg + off);
          }
          R[jf][tb] = qv;
          Rp[jf][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
          Xa[jf][tb] = cc.beta[0] * qv;
        }
      }
      // masked-product tiles P^T (s x t): p = wave + NW*jp; Mhat^T[s][t] = M[t][s] / ||H_t||
      f32x4 Mh[PPW];
#pragma unroll
      for (int jp = 0; jp < PPW; ++jp) {
        const int p = wave + NW * jp;
        Mh[jp] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (p < Cfg::PT) {
          const int sb = p / CT, tb = p % CT;
          const int t = 16 * tb + lr;
          const f32x4 m4 = *reinterpret_cast<const f32x4*>(Mf + t * LDF + 16 * sb + 4 * lg);
          Mh[jp] = m4 * v_ninv[t];
        }
      }
      if (SPLIT) __syncthreads();  // the mask buffer is reused as the lo part of the operand

      // operand V (own tiles) -> Xs (hi) and Xl (lo), token-major
      auto write_operand = [&](f32x4 (&V)[FPW][CT]) {
#pragma unroll
        for (int jf = 0; jf < FPW; ++jf) {
          const int fb = wave + NW * jf;
          if (fb < FT) {
#pragma unroll
            for (int tb = 0; tb < CT; ++tb) {
              const int o = (16 * tb + lr) * LDD + 16 * fb + 4 * lg;
              if constexpr (SPLIT) {
                store4_split<T>(Xs + o, Xl + o, V[jf][tb]);
              } else {
                store4<T>(Xs + o, V[jf][tb]);
              }
            }
          }
        }
      };
      // P'^T = (K V^T) o Mhat^T, stored token-major (hi in Ps, lo in Pl)
      auto masked_product = [&]() {
#pragma unroll
        for (int jp = 0; jp < PPW; ++jp) {
          const int p = wave + NW * jp;
          if (p < Cfg::PT) {
            const int sb = p / CT, tb = p % CT;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < D; kk += K) {
              const typename M::frag ka = M::load(Ks, LDD, 16 * sb + lr, kk + E * lg);
              acc = M::mma(ka, M::load(Xs, LDD, 16 * tb + lr, kk + E * lg), acc);
              if constexpr (SPLIT) acc = M::mma(ka, M::load(Xl, LDD, 16 * tb + lr, kk + E * lg), acc);
            }
            const int o = (16 * tb + lr) * LDC + 16 * sb + 4 * lg;
            if constexpr (SPLIT) store4_split<T>(Ps + o, Pl + o, acc * Mh[jp]);
            else store4<T>(Ps + o, acc * Mh[jp]);
          }
        }
      };
      // Y = Mat V^T for own tiles, Mat = the H0 copy (hi part of V only) or the U0 copy (hi + lo)
      auto state_product = [&](bool with_lo) {
#pragma unroll
        for (int jf = 0; jf < FPW; ++jf) {
          const int fb = wave + NW * jf;
          if (fb < FT) {
#pragma unroll
            for (int tb = 0; tb < CT; ++tb) Y[jf][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < D; kk += K) {
              const typename M::frag af = M::load(Hs, LDD, 16 * fb + lr, kk + E * lg);
#pragma unroll
              for (int tb = 0; tb < CT; ++tb) {
                Y[jf][tb] = M::mma(af, M::load(Xs, LDD, 16 * tb + lr, kk + E * lg), Y[jf][tb]);
                if constexpr (SPLIT) {
                  if (with_lo)
                    Y[jf][tb] = M::mma(af, M::load(Xl, LDD, 16 * tb + lr, kk + E * lg), Y[jf][tb]);
                }
              }
            }
          }
        }
      };
      // Y = diag(s) Y + Mat2 P'^T, Mat2 = K^T (system) or V^T (output)
      auto intra_product = [&](const T* Mat2) {
#pragma unroll
        for (int jf = 0; jf < FPW; ++jf) {
          const int fb = wave + NW * jf;
          if (fb < FT) {
#pragma unroll
            for (int tb = 0; tb < CT; ++tb) Y[jf][tb] = Y[jf][tb] * sv[tb];
#pragma unroll
            for (int kk = 0; kk < C; kk += K) {
              const typename M::frag af = M::load(Mat2, LDC, 16 * fb + lr, kk + E * lg);
#pragma unroll
              for (int tb = 0; tb < CT; ++tb) {
                Y[jf][tb] = M::mma(af, M::load(Ps, LDC, 16 * tb + lr, kk + E * lg), Y[jf][tb]);
                if constexpr (SPLIT)
                  Y[jf][tb] = M::mma(af, M::load(Pl, LDC, 16 * tb + lr, kk + E * lg), Y[jf][tb]);
              }
            }
          }
        }
      };

      for (int it = 0; it + 1 < cc.iters; ++it) {
        write_operand(R);
        __syncthreads();
        state_product(false);
        masked_product();
        __syncthreads();
        intra_product(KT);
        const float om = cc.omega[it], bn = cc.beta[it + 1];
#pragma unroll
        for (int jf = 0; jf < FPW; ++jf) {
#pragma unroll
          for (int tb = 0; tb < CT; ++tb) {
            const f32x4 ar = Y[jf][tb] + cc.a * R[jf][tb];  // A R_i
            const f32x4 rn = it == 0 ? R[jf][tb] - cc.c * ar
                                     : Rp[jf][tb] + om * (R[jf][tb] - Rp[jf][tb] - cc.c * ar);
            Rp[jf][tb] = R[jf][tb];
            R[jf][tb] = rn;
            Xa[jf][tb] += bn * rn;
          }
        }
      }

      // ---- output O^T = diag(s) U0 X^T + V^T P'^T -----------------------------------------------
      write_operand(Xa);
#pragma unroll
      for (int j = 0; j < SPW; ++j) {  // U0 copy into the H0 buffer: Hs[v][k..k+3] = U^T[k..k+3][v]
        const int p = wave + NW * j;
        if (p < Cfg::ST) {
          const int r = 16 * (p / FT) + 4 * lg, c = 16 * (p % FT) + lr;
          store4<T>(Hs + c * LDD + r, Ust[j]);
        }
      }
      __syncthreads();
      state_product(true);
      masked_product();
      __syncthreads();
      intra_product(VT);
#pragma unroll
      for (int jf = 0; jf < FPW; ++jf) {
        const int fb = wave + NW * jf;
        if (fb < FT) {
#pragma unroll
          for (int tb = 0; tb < CT; ++tb) {
            const int t = 16 * tb + lr;
            if (t < nv) {
              const long long off = ((long long)(b * (long long)Tlen + t0 + t)) * tok_stride + (long long)h * D + 16 * fb + 4 * lg;
              store4<T>(og + off, Y[jf][tb]);
            }
          }
        }
      }
    }

    // ---- state carry: H <- Gam_C H + K^T diag(w) K, U^T <- Gam_C U^T + K^T diag(w) V ----------
    {
      const float gC = v_gam[C - 1];
#pragma unroll
      for (int j = 0; j < SPW; ++j) {
        const int p = wave + NW * j;
        if (p < Cfg::ST) {
          const int rb = p / FT, cb = p % FT;
          f32x4 hacc = Hst[j] * gC, uacc = Ust[j] * gC;
#pragma unroll
          for (int kk = 0; kk < C; kk += K) {
            // A[f][s] = K[s][f] w_s (row f = 16 rb + lr), split into hi + lo parts for bf16
            const typename M::frag kt = M::load(KT, LDC, 16 * rb + lr, kk + E * lg);
            const typename M::frag bk = M::load(KT, LDC, 16 * cb + lr, kk + E * lg);
            const typename M::frag bv = M::load(VT, LDC, 16 * cb + lr, kk + E * lg);
            if constexpr (E == 1) {
              const float aw = kt * v_w[kk + lg];
              hacc = M::mma(aw, bk, hacc);
              uacc = M::mma(aw, bv, uacc);
            } else {
              typename M::frag ahi, alo;
#pragma unroll
              for (int e = 0; e < E; ++e) {
                T hi, lo;
                split_hi_lo<T>(to_f32(kt[e]) * v_w[kk + E * lg + e], hi, lo);
                ahi[e] = hi;
                alo[e] = lo;
              }
              hacc = M::mma(ahi, bk, hacc);
              hacc = M::mma(alo, bk, hacc);
              uacc = M::mma(ahi, bv, uacc);
              uacc = M::mma(alo, bv, uacc);
            }
          }
          Hst[j] = hacc;
          Ust[j] = uacc;
        }
      }
      n0sq = SUMMARY ? 0.0f : v_n2[C - 1];
    }
  }

  // ---- results of the walk ------------------------------------------------------------------
  if (SUMMARY) {
    float* oh = A.sum_h + bh * A.sum_bh + seg * A.sum_seg;
    float* ou = A.sum_u + bh * A.sum_bh + seg * A.sum_seg;
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const int p = wave + NW * j;
      if (p < Cfg::ST) {
        const int r = 16 * (p / FT) + 4 * lg, c = 16 * (p % FT) + lr;
        *reinterpret_cast<f32x4*>(oh + (size_t)c * D + r) = Hst[j];
        *reinterpret_cast<f32x4*>(ou + (size_t)c * D + r) = Ust[j];
      }
    }
    if (tid == 0) A.log2g_out[(long long)bh * S + seg] = log2g_seg;
  } else {
    if (A.out_h) {
      float* oh = A.out_h + (size_t)bh * D * D;
      float* ou = A.out_u + (size_t)bh * D * D;
#pragma unroll
      for (int j = 0; j < SPW; ++j) {
        const int p = wave + NW * j;
        if (p < Cfg::ST) {
          const int r = 16 * (p / FT) + 4 * lg, c = 16 * (p % FT) + lr;
          *reinterpret_cast<f32x4*>(oh + (size_t)c * D + r) = Hst[j];
          *reinterpret_cast<f32x4*>(ou + (size_t)c * D + r) = Ust[j];
        }
      }
    }
    if (A.n2_out && seg == S - 1 && tid == 0) A.n2_out[bh] = n0sq;
  }
}

// Affine scan over segments, elementwise over the D x D entries of H and U.
__global__ __launch_bounds__(256) void scan_kernel(float* __restrict__ st,
                                                   const float* __restrict__ log2g,
                                                   float* __restrict__ h, float* __restrict__ u,
                                                   const float* __restrict__ hnorm2,
                                                   float* __restrict__ n2_seg0, int S, int DD) {
  const int bh = blockIdx.y;
  const int e4 = blockIdx.x * blockDim.x + threadIdx.x;  // float4 index inside one matrix
  if (blockIdx.x == 0 && threadIdx.x == 0) n2_seg0[bh] = hnorm2 ? hnorm2[bh] : 0.0f;
  if (e4 * 4 >= DD) return;
  f32x4 sh = {0.f, 0.f, 0.f, 0.f}, su = {0.f, 0.f, 0.f, 0.f};
  if (h) {
    sh = reinterpret_cast<const f32x4*>(h + (size_t)bh * DD)[e4];
    su = reinterpret_cast<const f32x4*>(u + (size_t)bh * DD)[e4];
  }
  for (int s = 0; s < S; ++s) {
    f32x4* ph = reinterpret_cast<f32x4*>(st + ((size_t)bh * S + s) * 2 * DD) + e4;
    f32x4* pu = reinterpret_cast<f32x4*>(st + ((size_t)bh * S + s) * 2 * DD + DD) + e4;
    const f32x4 dh = *ph, du = *pu;
    *ph = sh;
    *pu = su;
    const float g = exp2f(log2g[(size_t)bh * S + s]);
    sh = g * sh + dh;
    su = g * su + du;
  }
  if (h) {
    reinterpret_cast<f32x4*>(h + (size_t)bh * DD)[e4] = sh;
    reinterpret_cast<f32x4*>(u + (size_t)bh * DD)[e4] = su;
  }
}

template <typename T, int D, int C>
static hipError_t launch_walk_t(const FwdPlan& pl, bool summary, const WalkArgs& a,
                                const ChebConsts& cc, hipStream_t stream) {
  using Cfg = WalkCfg<T, D, C>;
  const dim3 grid(pl.S, pl.B * pl.H);
  if (summary) {
    auto kern = walk_kernel<T, D, C, true>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)Cfg::bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, dim3(Cfg::NT), Cfg::bytes, stream, a, pl.B, pl.T,
                       pl.H, pl.N, pl.S, pl.J, cc);
  } else {
    auto kern = walk_kernel<T, D, C, false>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)Cfg::bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, dim3(Cfg::NT), Cfg::bytes, stream, a, pl.B, pl.T, pl.H,
                       pl.N, pl.S, pl.J, cc);
  }
  return hipGetLastError();
}

hipError_t launch_walk(const FwdPlan& pl, bool summary, const WalkArgs& a, const ChebConsts& cc,
                       hipStream_t stream) {
  if (pl.dtype == 0) {
    if (pl.C == 64) {
      switch (pl.D) {
        case 32: return launch_walk_t<bf16, 32, 64>(pl, summary, a, cc, stream);
        case 64: return launch_walk_t<bf16, 64, 64>(pl, summary, a, cc, stream);
        case 128: return launch_walk_t<bf16, 128, 64>(pl, summary, a, cc, stream);
      }
    } else if (pl.C == 32) {
      switch (pl.D) {
        case 32: return launch_walk_t<bf16, 32, 32>(pl, summary, a, cc, stream);
        case 64: return launch_walk_t<bf16, 64, 32>(pl, summary, a, cc, stream);
        case 128: return launch_walk_t<bf16, 128, 32>(pl, summary, a, cc, stream);
      }
    }
  } else {
    if (pl.C == 16) {
      switch (pl.D) {
        case 16: return launch_walk_t<float, 16, 16>(pl, summary, a, cc, stream);
        case 32: return launch_walk_t<float, 32, 16>(pl, summary, a, cc, stream);
        case 64: return launch_walk_t<float, 64, 16>(pl, summary, a, cc, stream);
      }
    } else if (pl.C == 32) {
      switch (pl.D) {
        case 16: return launch_walk_t<float, 16, 32>(pl, summary, a, cc, stream);
        case 32: return launch_walk_t<float, 32, 32>(pl, summary, a, cc, stream);
        case 64: return launch_walk_t<float, 64, 32>(pl, summary, a, cc, stream);
      }
    } else if (pl.C == 64) {
      switch (pl.D) {
        case 16: return launch_walk_t<float, 16, 64>(pl, summary, a, cc, stream);
        case 32: return launch_walk_t<float, 32, 64>(pl, summary, a, cc, stream);
        case 64: return launch_walk_t<float, 64, 64>(pl, summary, a, cc, stream);
      }
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_scan(const FwdPlan& pl, float* ws_states, const float* ws_log2g, float* h,
                       float* u, const float* hnorm2, float* n2_seg0, hipStream_t stream) {
  const int DD = pl.D * pl.D;
  const dim3 grid((DD / 4 + 255) / 256, pl.B * pl.H);
  hipLaunchKernelGGL(scan_kernel, grid, dim3(256), 0, stream, ws_states, ws_log2g, h, u, hnorm2,
                     n2_seg0, pl.S, DD);
  return hipGetLastError();
}

}  // namespace gka
