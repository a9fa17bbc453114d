// gka_fwd_chunked: chunk-wise forward of the Gated KalmaNet layer (prefill / training forward).
//
// The chunk-wise form follows "Methodology in Plain English" on the ai.info summary of
// arXiv 2511.21016: the sequence is cut into chunks of C tokens, only the chunk-initial states
// are carried from chunk to chunk, everything inside a chunk is parallel, and ||H_t||_F comes
// from a closed form over the chunk's key Gram matrix G = K K^T ("Key Contributions" 3). For a
// chunk starting from (H0, U0, n0^2 = ||H0||^2), with in-chunk log2-gate prefix cl_t,
// Gam_t = 2^cl_t and the causal decay mask M_ts = 2^(cl_t - cl_s) [s <= t]:
//
//   H_t x   = Gam_t H0 x + sum_{s<=t} M_ts (k_s . x) k_s
//   U_t x   = Gam_t U0 x + sum_{s<=t} M_ts (k_s . x) v_s
//   n_t^2   = gamma_t^2 n_{t-1}^2 + 2 gamma_t k_t^T H_{t-1} k_t + G_tt^2,  where
//             k_t^T H_{t-1} k_t = Gam_{t-1} k_t^T H0 k_t + sum_{s<t} M_{t-1,s} G_st^2
//             (the Frobenius-norm recurrence with H_{t-1} in chunk form; an affine scan over t)
//   carry     H0 <- Gam_C H0 + K^T diag(w) K,  U0 <- Gam_C U0 + V^T diag(w) K,  w_s = 2^(cl_C - cl_s)
//
// With the optional write gate beta_t (the variant of "Main Findings" on the ai.info summary,
// H_t = gamma_t H_{t-1} + beta_t k_t k_t^T and likewise U_t) all of the above holds with k_s and
// v_s replaced by sqrt(beta_s) k_s and sqrt(beta_s) v_s: the walk scales the rows where they are
// converted to operands, the segment summary multiplies beta_s into the weight w_s.
//
// The Chebyshev iteration runs on the system divided by ||H_t||_F (spectrum in [a, 1 + a]), so
// its step and weights are launch constants, and on the residuals R_i = Q - A X_i:
//   R_0 = Q, R_1 = R_0 - c A R_0, R_{i+1} = R_{i-1} + omega_i (R_i - R_{i-1} - c A R_i),
//   X_r = sum_i beta_i R_i,  A(R) = diag(s) R H0hat + ((R K^T) o Mhat) K + a R
// with H0hat = H0 / n0, s_t = Gam_t n0 / n_t, Mhat_ts = M_ts / n_t (same iterates as the
// three-term recurrence on X in exact arithmetic). The output is
//   O = diag(s) X U0hat^T + ((X K^T) o Mhat) V,  U0hat = U0 / n0.
// Matrix-core operands are fp16 for bf16 inputs (float32 for float32 inputs) with float32
// accumulation; the products act on the shrinking residual, and the two output products take
// the iterate split into hi + lo fp16 parts, because X has components of size |q| / a in the null
// space of H_t whose rounding error would otherwise reach the key directions.
// All products are computed transposed (feature x token outputs): the accumulator layout
// (4 consecutive rows per lane) then maps to 4 consecutive features of one token.
//
// Work split of a workgroup (8 waves, one walk over the chunks of one (segment, head)):
// wave w = (fg = w % FG, tg = w / FG) owns feature tiles fg*FPW.. of the feature x token blocks,
// token tiles tg*TPW.., the s-blocks sb = fg, fg+FG, .. of the C x C products, and the state
// tiles (rows of its feature tiles) x (column tiles tg*CBW..). H0hat, K^T and K operand
// fragments of the wave's rows stay in registers for the whole chunk; the iterate and the masked
// product are exchanged through LDS once per iteration. The float32 state (H, and U transposed)
// lives in matrix-core accumulators for the whole walk.
//
// Kernels of one call:
//   1. summary walk (only with S > 1 segments): per (segment, head), the state reached from a zero
//      state over the segment's chunks, and the segment's total gate (log2);
//   2. segment scan: elementwise affine scan over segments -> segment-start states, final state;
//   3. fused walk: per (segment, head), from the segment-start state, chunk by chunk.
#include <type_traits>

#include "gka_internal.hpp"

namespace gka {

// Tiling of one workgroup of NWaves waves: 8 for the fused walk (two waves per SIMD, each with
// the register room for its share of the state, the iterate and the resident fragments); 16 for
// the summary walk, which holds only the state and so spreads it over four waves per SIMD.
template <typename T, int D, int C, int NWaves = 8>
struct WalkCfg {
  // matrix-core operand type: fp16 for bf16 inputs, whose products take blocks of 32 features
  // and 32 tokens; float32 for float32 inputs, and for bf16 inputs with D = 16 or C = 16 (exact
  // for bf16 values)
  typedef typename std::conditional<(D < 32 || C < 32), float, typename OperandOf<T>::type>::type O;
  static constexpr int NW = NWaves;
  static constexpr int NT = NW * kWave;
  static constexpr int FT = D / 16;  // feature tiles
  static constexpr int CT = C / 16;  // token tiles
  static constexpr int cmin(int a, int b) { return a < b ? a : b; }
  static constexpr int FG = cmin(4, FT);          // feature groups
  static constexpr int TG = cmin(NW / FG, CT);    // token groups (waves with tg >= TG idle there)
  static constexpr int SG = cmin(NW / FG, FT);    // state column groups
  static constexpr int FPW = FT / FG;             // feature tiles per wave
  static constexpr int TPW = CT / TG;             // token tiles per wave
  static constexpr int SBW = (CT + FG - 1) / FG;  // s-blocks per wave (guarded by sb < CT)
  static constexpr int CBW = FT / SG;             // state column tiles per wave
  static constexpr int PAD = 16 / (int)sizeof(O);
  static constexpr int LDD = D + PAD;  // row stride of [*][D] operand tiles (elements)
  static constexpr int LDC = C + PAD;  // row stride of [*][C] operand tiles (elements)
  static constexpr int K = Mma<O>::K;
  static constexpr int E = Mma<O>::E;
  static constexpr bool SPLIT = sizeof(O) == 2;  // hi/lo operands for the output products
  static_assert(D % K == 0 && C % K == 0 && C <= kWave, "unsupported D / C");
  static_assert(NT <= 1024, "workgroup size");

  // LDS layout (bytes)
  static constexpr size_t szRD = (size_t)C * LDD * sizeof(O);  // [C][LDD]
  static constexpr size_t szRC = (size_t)C * LDC * sizeof(O);  // [C][LDC]
  static constexpr size_t szDC = (size_t)D * LDC * sizeof(O);  // [D][LDC]
  static constexpr size_t szDD = (size_t)D * LDD * sizeof(O);  // [D][LDD]
  static constexpr size_t szVec = (size_t)(8 * C + 2 * NW * C + 32) * sizeof(float);
  static constexpr size_t oRs = 0;            // operand (R or X hi), token-major
  static constexpr size_t oPs = oRs + szRD;   // masked product (hi), token-major
  static constexpr size_t oKs = oPs + szRC;   // K, token-major
  static constexpr size_t oKT = oKs + szRD;   // K^T
  static constexpr size_t oVT = oKT + szDC;   // V^T
  // the lo part of the output's iterate reuses the K buffer: by the time it is written K lives in
  // registers (resident fragments)
  static constexpr size_t oRl = oKs;
  static constexpr size_t oSt = oVT + szDC;                // H0hat, then U0hat (row-major)
  static constexpr size_t oVec = oSt + szDD;
  // next chunk's raw K, V (16-byte units, [unit column][token]) and gates, filled by
  // direct global-to-LDS loads while the current chunk computes
  static constexpr int VEC = 16 / (int)sizeof(T);         // elements per 16-byte unit
  static constexpr int UPR = D / VEC;                     // units per token row
  static constexpr int NU = C * UPR;                      // units per matrix
  // It is a static LDS object of its own, apart from the dynamic buffer above, so that the
  // compiler can tell reads of the other buffers from the in-flight direct loads and does not
  // make them wait for the whole prefetch.
  static constexpr size_t szPreM = (size_t)NU * 16;
  static constexpr size_t szPre = 2 * szPreM + (size_t)C * sizeof(float);
  static constexpr size_t bytes = oVec + szVec;  // dynamic part
  static_assert(NU % kWave == 0, "prefetch units must fill whole waves");
  static_assert(bytes + szPre <= 160 * 1024, "LDS budget of one CU exceeded");
};

// Direct global-to-LDS loads of chunk chn's K, V and gates into the prefetch buffer. Unit
// u = (column c, token t) with u = c*C + t holds K[t][c*VEC .. c*VEC+VEC-1]; tokens past the end
// of the sequence are not loaded. (A plain device function, whose body exists in the device
// compilation pass only.)
template <typename T, int D, int C, int NWaves, typename V>
__device__ inline void prefetch_chunk(V* PreK, V* PreV, float* PreG, const T* kg, const T* vg,
                                      const float* gamma, long long seq0, int h, int Hn, int Tlen, int chn,
                                      int wave, int lane) {
#if defined(__HIP_DEVICE_COMPILE__)  // device code only: the host pass has no LDS address space
  using Cfg = WalkCfg<T, D, C, NWaves>;
  typedef __attribute__((address_space(3))) void lds_void;
  constexpr int NI = Cfg::NU / kWave;  // wave instructions per matrix
  const long long tok_stride = (long long)Hn * D;
  const int t0n = chn * C;
  const int nvn = min(C, Tlen - t0n);
  for (int q = wave; q < 2 * NI; q += Cfg::NW) {
    const bool isv = q >= NI;
    const int qq = isv ? q - NI : q;
    const int u = qq * kWave + lane;
    const int t = u % C, c = u / C;
    const uint32_t base = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(lds_void*)((isv ? PreV : PreK) + qq * kWave));
    if (t < nvn) {
      const T* src = (isv ? vg : kg) + (seq0 + t0n + t) * tok_stride +
                     (long long)h * D + c * Cfg::VEC;
      dma_load16(src, base);
    }
  }
  if (wave == Cfg::NW - 1) {
    const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)PreG);
    if (lane < nvn) dma_load4(gamma + (seq0 + t0n + lane) * Hn + h, base);
  }
#endif
}

// RES: residual mode, which also writes ||q_t - A_t x_i|| for i = 0..iters to A.resid
template <typename T, int D, int C, bool RES>
__global__ __launch_bounds__(512) void walk_kernel(WalkArgs A, int B, int Tmax, int Hn, int N,
                                                   int S, int J, ChebConsts cc) {
  using Cfg = WalkCfg<T, D, C, 8>;
  using O = typename Cfg::O;
  using M = Mma<O>;
  using Frag = typename M::frag;
  constexpr int NW = Cfg::NW, LDD = Cfg::LDD, LDC = Cfg::LDC;
  constexpr int CT = Cfg::CT, FG = Cfg::FG, TG = Cfg::TG, SG = Cfg::SG;
  constexpr int FPW = Cfg::FPW, TPW = Cfg::TPW, SBW = Cfg::SBW, CBW = Cfg::CBW;
  constexpr int K = Cfg::K, E = Cfg::E, KD = D / K, KC = C / K;
  constexpr bool SPLIT = Cfg::SPLIT;

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  O* Rs = reinterpret_cast<O*>(smem + Cfg::oRs);
  O* Rl = reinterpret_cast<O*>(smem + Cfg::oRl);
  O* Ps = reinterpret_cast<O*>(smem + Cfg::oPs);
  O* Ks = reinterpret_cast<O*>(smem + Cfg::oKs);
  O* KT = reinterpret_cast<O*>(smem + Cfg::oKT);
  O* VT = reinterpret_cast<O*>(smem + Cfg::oVT);
  O* St = reinterpret_cast<O*>(smem + Cfg::oSt);
  float* vec = reinterpret_cast<float*>(smem + Cfg::oVec);
  float* v_cl = vec;            // [C] in-chunk log2 gate prefix
  float* v_gam = v_cl + C;      // [C] 2^cl
  float* v_w = v_gam + C;       // [C] carry weights 2^(cl_C - cl_s)
  float* v_g = v_w + C;         // [C] gate gamma_t (1 past the end of the sequence)
  float* v_ninv = v_g + C;      // [C] 1 / ||H_t|| (0 when ||H_t|| = 0)
  float* v_s = v_ninv + C;      // [C] Gam_t n0 / ||H_t||
  float* v_n2 = v_s + C;        // [C] ||H_t||^2
  float* v_kk = v_n2 + C;       // [C] ||k_t||^2
  float* p_u = v_kk + C;        // [NW][C] partials of k_t^T H0hat k_t
  float* p_v = p_u + NW * C;    // [NW][C] partials of sum_{s<t} M_{t-1,s} G_st^2
  float* v_sc = p_v + NW * C;   // [32] scalars
  typedef T vecT __attribute__((ext_vector_type(Cfg::VEC)));
  // the next chunk is loaded straight into this LDS buffer ([UPR][C] units of K, then of V,
  // then [C] gates) while the current one computes
  __shared__ __attribute__((aligned(16))) unsigned char pre_buf[Cfg::szPre];
  vecT* PreK = reinterpret_cast<vecT*>(pre_buf);
  vecT* PreV = PreK + Cfg::NU;
  float* PreG = reinterpret_cast<float*>(PreV + Cfg::NU);

  const int seg = blockIdx.x;
  int b, h;
  head_of(A, blockIdx.y, Hn, b, h);
  const int bh = b * Hn + h;
  const int wave = threadIdx.x / kWave;
  // Per-lane indices. They are passed through refresh() at the start of every phase of the chunk
  // walk, so that the many addresses derived from them are recomputed where they are used instead
  // of being computed once for the whole walk and kept live (which would spill them).
  int tid = threadIdx.x, lane = tid % kWave;
  int lr = lane % 16;  // row (operand A) / column (operand B, accumulator) inside a tile
  int lg = lane / 16;  // lane group: operand K offset E*lg, accumulator rows 4*lg..
  auto refresh = [&]() {
    asm volatile("" : "+v"(tid), "+v"(lane), "+v"(lr), "+v"(lg));
  };
  const int fg = wave % FG, tg = wave / FG;
  const bool tok_active = tg < TG;    // this wave owns feature x token tiles
  const bool state_active = tg < SG;  // this wave owns state tiles
  long long seq0;  // first row of sequence b
  int Tlen;        // its length
  seq_range(A, b, Tmax, seq0, Tlen);
  // segments past the sequence's last one have nothing to do (packed batches); the last one
  // writes the final state
  const int last = last_segment(Tlen, J, C);
  if (seg > last) return;
  const int c_begin = seg * J;
  const int c_end = min(min(N, c_begin + J), (Tlen + C - 1) / C);
  const long long tok_stride = (long long)Hn * D;
  const T* qg = static_cast<const T*>(A.q);
  const T* kg = static_cast<const T*>(A.k);
  const T* vg = static_cast<const T*>(A.v);
  T* og = static_cast<T*>(A.o);
  auto row_of = [&](int jf) { return 16 * (fg * FPW + jf); };  // first feature of own tile jf
  auto tok_of = [&](int jt) { return 16 * (tg * TPW + jt); };  // first token of own tile jt
  auto col_of = [&](int jc) { return 16 * (tg * CBW + jc); };  // first column of state tile jc
  auto sblk_of = [&](int js) { return fg + FG * js; };         // own s-block js

  // ---- float32 state in accumulator tiles: H[row][col] and U^T[row][col] = U[col][row] -------
  f32x4 Hst[FPW][CBW], Ust[FPW][CBW];
#pragma unroll
  for (int jf = 0; jf < FPW; ++jf)
#pragma unroll
    for (int jc = 0; jc < CBW; ++jc) {
      Hst[jf][jc] = f32x4{0.f, 0.f, 0.f, 0.f};
      Ust[jf][jc] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  float n0sq = 0.0f;
  {
    float sq = 0.0f;
    if (A.in_h && state_active) {
      const float* ih = A.in_h + bh * A.in_bh + seg * A.in_seg;
      const float* iu = A.in_u + bh * A.in_bh + seg * A.in_seg;
#pragma unroll
      for (int jf = 0; jf < FPW; ++jf)
#pragma unroll
        for (int jc = 0; jc < CBW; ++jc) {
          const int r = row_of(jf) + 4 * lg, c = col_of(jc) + lr;
          // H is symmetric: H[r..r+3][c] is read as H[c][r..r+3]
          Hst[jf][jc] = *reinterpret_cast<const f32x4*>(ih + (size_t)c * D + r);
          Ust[jf][jc] = *reinterpret_cast<const f32x4*>(iu + (size_t)c * D + r);
          sq += Hst[jf][jc][0] * Hst[jf][jc][0] + Hst[jf][jc][1] * Hst[jf][jc][1] +
                Hst[jf][jc][2] * Hst[jf][jc][2] + Hst[jf][jc][3] * Hst[jf][jc][3];
        }
    }
    sq = wave_sum(sq);
    if (lane == 0) v_sc[wave] = sq;
    __syncthreads();
    if (seg == 0 && A.n2_in) {
      n0sq = A.n2_in[bh];
    } else if (A.in_h) {
      for (int w = 0; w < NW; ++w) n0sq += v_sc[w];
    }
  }

  auto prefetch = [&](int chn) {
    if (chn < c_end)
      prefetch_chunk<T, D, C, NW, vecT>(PreK, PreV, PreG, kg, vg, A.gamma, seq0, h, Hn, Tlen, chn,
                                        wave, lane);
  };
  // The output tile of a chunk is staged token-major (in the operand buffer, idle by then) and
  // written out after the next workgroup barrier in 16-byte units, consecutive threads covering
  // a token's row (whole cache lines instead of 8-byte pieces spread over 16 rows)
  T* Ob = reinterpret_cast<T*>(smem + Cfg::oRs);  // [C][LDD] elements of T
  int pend_t0 = 0, pend_nv = 0;                   // the staged tile: first token, tokens
  auto flush_o = [&]() {
    if (pend_nv > 0) {
      for (int e = tid; e < Cfg::NU; e += Cfg::NT) {
        const int t = e / Cfg::UPR, c = e % Cfg::UPR;
        if (t < pend_nv) {
          const vecT v = *reinterpret_cast<const vecT*>(Ob + t * LDD + c * Cfg::VEC);
          *reinterpret_cast<vecT*>(og + (seq0 + pend_t0 + t) * tok_stride +
                                   (long long)h * D + c * Cfg::VEC) = v;
        }
      }
      pend_nv = 0;
    }
  };
  prefetch(c_begin);

  for (int ch = c_begin; ch < c_end; ++ch) {
    refresh();
    const int t0 = ch * C;
    const int nv = min(C, Tlen - t0);  // valid tokens of this chunk
    const float n0 = sqrtf(n0sq);
    const float n0inv = n0 > 0.0f ? 1.0f / n0 : 0.0f;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's direct loads of this chunk have landed
    __syncthreads();                // all waves' loads have landed; LDS of the previous chunk is free
    flush_o();                      // the previous chunk's output

    // ---- stage K (token-major), K^T, V^T as operands from the prefetch buffer -----------------
    // The token index runs fastest across lanes: unit reads are consecutive and the transposed
    // 2-byte writes of a wave cover consecutive addresses of one row of K^T / V^T.
    {
      constexpr int VEC = Cfg::VEC;
      typedef O vecO __attribute__((ext_vector_type(VEC)));
      for (int e = tid; e < Cfg::NU; e += Cfg::NT) {
        const int t = e % C, d0 = (e / C) * VEC;
        vecT kv, vv;
        float sb = 1.0f;  // sqrt(beta_t): the write gate on the token's key and value
        if (t < nv) {
          kv = PreK[e];
          vv = PreV[e];
          if (A.beta) sb = sqrtf(A.beta[(seq0 + t0 + t) * Hn + h]);
        } else {
#pragma unroll
          for (int i = 0; i < VEC; ++i) {
            kv[i] = (T)0.0f;
            vv[i] = (T)0.0f;
          }
        }
        vecO ko;
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          ko[i] = to_op<O>((float)kv[i] * sb);
          KT[(d0 + i) * LDC + t] = ko[i];
          VT[(d0 + i) * LDC + t] = to_op<O>((float)vv[i] * sb);
        }
        *reinterpret_cast<vecO*>(Ks + t * LDD + d0) = ko;
      }
    }
    // ---- queries of the own tiles (issued early; zeroed below where ||H_t|| = 0) ---------------
    typedef T raw4 __attribute__((ext_vector_type(4)));
    raw4 Qraw[FPW][TPW];
    {
#pragma unroll
      for (int jt = 0; jt < TPW; ++jt)
#pragma unroll
        for (int jf = 0; jf < FPW; ++jf) {
          const int t = tok_of(jt) + lr;
          raw4 qv = {(T)0.0f, (T)0.0f, (T)0.0f, (T)0.0f};
          if (tok_active && t < nv) {
            const long long off = (seq0 + t0 + t) * tok_stride + (long long)h * D + row_of(jf) + 4 * lg;
            qv = *reinterpret_cast<const raw4*>(qg + off);
          }
          Qraw[jf][jt] = qv;
        }
    }
    // ---- gate prologue (wave 0) -----------------------------------------------------------------
    if (wave == 0) {
      float g = 1.0f, l2 = 0.0f;  // tokens past the end: gamma = 1 with k = v = q = 0
      if (lane < nv) {
        g = PreG[lane];
        l2 = log2_gate(g);
      }
      const float cl = scan_add<kWave>(l2);
      const float clast = lane_value(cl, C - 1);
      if (lane < C) {
        v_cl[lane] = cl;
        v_gam[lane] = fast_exp2(cl);
        v_w[lane] = fast_exp2(fminf(clast - cl, 0.0f));
        v_g[lane] = g;
      }
    }
    // ---- H0hat = H0 / n0 into the staging buffer (row-major; H symmetric) ----------------------
    if (state_active) {
#pragma unroll
      for (int jf = 0; jf < FPW; ++jf)
#pragma unroll
        for (int jc = 0; jc < CBW; ++jc)
          store4<O>(St + (col_of(jc) + lr) * LDD + row_of(jf) + 4 * lg, Hst[jf][jc] * n0inv);
    }
    lds_barrier();
    // the prefetch buffer has been consumed. The next chunk's loads are issued once this chunk's
    // queries are in registers: the memory counter retires in order, so any wait for a load issued
    // after them (the queries, spill reloads) would also wait for the whole prefetch.

    // ---- operand fragments of the wave's rows, resident for the chunk --------------------------
    Frag fKT[FPW][KC];  // A operand K^T[f][s] (rows = own features)
#pragma unroll
    for (int jf = 0; jf < FPW; ++jf)
#pragma unroll
      for (int kk = 0; kk < KC; ++kk) fKT[jf][kk] = M::load(KT, LDC, row_of(jf) + lr, kk * K + E * lg);

    // ---- state carry: H <- Gam_C H + K^T diag(w) K, U^T <- Gam_C U^T + K^T diag(w) V ----------
    // (runs before the output products: the U0 copy for the output is staged already)
    auto carry = [&]() {
      if (!state_active) return;
      const float gC = v_gam[C - 1];
      // A operand K^T[f][s] w_s of the own rows; for fp16 operands split into hi + lo parts so
      // the float32 state gets the weighted keys to float32 accuracy
      Frag aw[FPW][KC], awl[FPW][KC];
#pragma unroll
      for (int kk = 0; kk < KC; ++kk) {
        float wv[E];  // weights of this lane's k-slots
#pragma unroll
        for (int e = 0; e < E; ++e) wv[e] = v_w[kk * K + E * lg + e];
#pragma unroll
        for (int jf = 0; jf < FPW; ++jf) {
          const Frag kf = fKT[jf][kk];
          if constexpr (E == 1) {
            aw[jf][kk] = kf * wv[0];
          } else {
#pragma unroll
            for (int e = 0; e < E; ++e) {
              const float x = (float)kf[e] * wv[e];
              aw[jf][kk][e] = (O)x;
              awl[jf][kk][e] = (O)(x - (float)aw[jf][kk][e]);
            }
          }
        }
      }
      // each B operand (columns of K^T and V^T) is loaded once and used for all own rows
#pragma unroll
      for (int jc = 0; jc < CBW; ++jc) {
        Frag bk[KC], bv[KC];
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) {
          bk[kk] = M::load(KT, LDC, col_of(jc) + lr, kk * K + E * lg);
          bv[kk] = M::load(VT, LDC, col_of(jc) + lr, kk * K + E * lg);
        }
#pragma unroll
        for (int jf = 0; jf < FPW; ++jf) {
          f32x4 hacc = Hst[jf][jc] * gC, uacc = Ust[jf][jc] * gC;
#pragma unroll
          for (int kk = 0; kk < KC; ++kk) {
            hacc = M::mma(aw[jf][kk], bk[kk], hacc);
            uacc = M::mma(aw[jf][kk], bv[kk], uacc);
            if constexpr (E != 1) {
              hacc = M::mma(awl[jf][kk], bk[kk], hacc);
              uacc = M::mma(awl[jf][kk], bv[kk], uacc);
            }
          }
          Hst[jf][jc] = hacc;
          Ust[jf][jc] = uacc;
        }
      }
    };

    {
      Frag fK[SBW][KD];  // A operand K[s][d] (rows = own s-blocks)
#pragma unroll
      for (int js = 0; js < SBW; ++js)
#pragma unroll
        for (int kk = 0; kk < KD; ++kk)
          fK[js][kk] = sblk_of(js) < CT ? M::load(Ks, LDD, 16 * sblk_of(js) + lr, kk * K + E * lg)
                                        : Frag{};

      refresh();
      // ---- norm phase ----------------------------------------------------------------------------
      // (a) G tiles (own s-blocks x own token tiles): partial sum_{s<t} 2^(cl_{t-1}-cl_s) G_st^2
      //     and ||k_t||^2 from the diagonal; (b) Y = H0hat K^T (own features x own tokens):
      //     partial k_t^T H0hat k_t over the own features.
      if (tok_active) {
        // all operand fragments first (one round of loads): K rows of the own tokens (B operand)
        // and H0hat rows of the own features (A operand)
        Frag fbt[TPW][KD], fh[FPW][KD];
#pragma unroll
        for (int jt = 0; jt < TPW; ++jt)
#pragma unroll
          for (int kk = 0; kk < KD; ++kk) fbt[jt][kk] = M::load(Ks, LDD, tok_of(jt) + lr, kk * K + E * lg);
#pragma unroll
        for (int jf = 0; jf < FPW; ++jf)
#pragma unroll
          for (int kk = 0; kk < KD; ++kk) fh[jf][kk] = M::load(St, LDD, row_of(jf) + lr, kk * K + E * lg);
        float pv[TPW], pu[TPW];
#pragma unroll
        for (int jt = 0; jt < TPW; ++jt) {
          const int t = tok_of(jt) + lr;
          pv[jt] = 0.0f;
          pu[jt] = 0.0f;
          const float clp = t > 0 ? v_cl[t - 1] : 0.0f;
#pragma unroll
          for (int js = 0; js < SBW; ++js) {
            const int sb = sblk_of(js);
            if (sb < CT) {
              f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int kk = 0; kk < KD; ++kk) acc = M::mma(fK[js][kk], fbt[jt][kk], acc);
              // accumulator rows s = 16 sb + 4 lg + i of column t
              const f32x4 cls = *reinterpret_cast<const f32x4*>(v_cl + 16 * sb + 4 * lg);
              float kd = 0.0f;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int s = 16 * sb + 4 * lg + i;
                const float e = fast_exp2(fminf(clp - cls[i], 0.0f)) * (acc[i] * acc[i]);
                pv[jt] += s < t ? e : 0.0f;
                kd = s == t ? acc[i] : kd;
              }
              if (sb == (t >> 4) && lg == ((t & 15) >> 2)) v_kk[t] = kd;  // the lane with G_tt
            }
          }
#pragma unroll
          for (int jf = 0; jf < FPW; ++jf) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KD; ++kk) acc = M::mma(fh[jf][kk], fbt[jt][kk], acc);
            const f32x4 kf = load4<O>(Ks + t * LDD + row_of(jf) + 4 * lg);
            pu[jt] += acc[0] * kf[0] + acc[1] * kf[1] + acc[2] * kf[2] + acc[3] * kf[3];
          }
        }
#pragma unroll
        for (int jt = 0; jt < TPW; ++jt) {
          float x = pv[jt], y = pu[jt];
          x += __shfl_xor(x, 16, kWave);
          x += __shfl_xor(x, 32, kWave);
          y += __shfl_xor(y, 16, kWave);
          y += __shfl_xor(y, 32, kWave);
          if (lg == 0) {
            p_v[fg * C + tok_of(jt) + lr] = x;
            p_u[fg * C + tok_of(jt) + lr] = y;
          }
        }
      }
      lds_barrier();
      // (c) n_t^2 by an affine scan over the chunk (wave 0, lane = token)
      if (wave == 0) {
        const int t = lane;
        float a = 1.0f, bb = 0.0f;
        if (t < C) {
          float u = 0.0f, vv = 0.0f;
          for (int f = 0; f < FG; ++f) {
            u += p_u[f * C + t];
            vv += p_v[f * C + t];
          }
          const float g = v_g[t];
          const float gprev = t > 0 ? v_gam[t - 1] : 1.0f;
          const float kk = v_kk[t];
          a = g * g;
          bb = 2.0f * g * (gprev * n0 * u + vv) + kk * kk;
        }
        scan_affine(a, bb);
        if (t < C) {
          const float n2 = a * n0sq + bb;
          const bool zero = !(n2 > 0.0f);
          const float ninv = zero ? 0.0f : 1.0f / sqrtf(n2);
          v_n2[t] = n2;
          v_ninv[t] = ninv;
          v_s[t] = v_gam[t] * n0 * ninv;
          if (A.hnorm_t && t < nv) A.hnorm_t[(seq0 + t0 + t) * Hn + h] = sqrtf(n2);
        }
      }
      lds_barrier();

      refresh();
      // ---- Chebyshev loop on the residuals -------------------------------------------------------
      f32x4 R[FPW][TPW], Rp[FPW][TPW], Xa[FPW][TPW], Y[FPW][TPW];
      float sv[TPW];
      f32x4 Mh[SBW][TPW];  // Mhat^T[s][t] of the own P^T tiles
#pragma unroll
      for (int jt = 0; jt < TPW; ++jt) {
        const int t = tok_of(jt) + lr;
        sv[jt] = tok_active ? v_s[t] : 0.0f;
#pragma unroll
        for (int js = 0; js < SBW; ++js) {
          f32x4 m4 = {0.f, 0.f, 0.f, 0.f};
          const int sb = sblk_of(js);
          if (tok_active && sb < CT) {
            const float ninv = v_ninv[t], clt = v_cl[t];
            const f32x4 cls = *reinterpret_cast<const f32x4*>(v_cl + 16 * sb + 4 * lg);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int s = 16 * sb + 4 * lg + i;
              const float m = fast_exp2(fminf(clt - cls[i], 0.0f)) * ninv;
              m4[i] = s <= t ? m : 0.0f;
            }
          }
          Mh[js][jt] = m4;
        }
#pragma unroll
        for (int jf = 0; jf < FPW; ++jf) {
          f32x4 qv = {0.f, 0.f, 0.f, 0.f};
          if (tok_active && v_ninv[t] > 0.0f) {  // ||H_t|| = 0: x_t = 0
#pragma unroll
            for (int i = 0; i < 4; ++i) qv[i] = to_f32(Qraw[jf][jt][i]);
          }
          R[jf][jt] = qv;
          Rp[jf][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
          Xa[jf][jt] = cc.beta[0] * qv;
        }
      }

      // operand V of the own tiles -> token-major LDS (hi in Rs, lo in Rl when split)
      auto write_operand = [&](f32x4(&V)[FPW][TPW], bool split) {
        if (tok_active) {
#pragma unroll
          for (int jf = 0; jf < FPW; ++jf)
#pragma unroll
            for (int jt = 0; jt < TPW; ++jt) {
              const int o = (tok_of(jt) + lr) * LDD + row_of(jf) + 4 * lg;
              if (SPLIT && split) store4_split<O>(Rs + o, Rl + o, V[jf][jt]);
              else store4<O>(Rs + o, V[jf][jt]);
            }
        }
      };
      // Y = Mat V^T (own tiles; Mat read from LDS, row-major) and P'^T = (K V^T) o Mhat^T -> Ps;
      // with split, V is taken as its hi + lo parts (P' itself is rounded once: its entries are
      // the key-direction components, which carry no cancellation); the k-step loop is outermost
      // so independent accumulators interleave
      auto products_1 = [&](const O* Mat, bool split) {
        if (tok_active) {
          f32x4 Pa[SBW][TPW];
#pragma unroll
          for (int jt = 0; jt < TPW; ++jt) {
#pragma unroll
            for (int jf = 0; jf < FPW; ++jf) Y[jf][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int js = 0; js < SBW; ++js) Pa[js][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
#pragma unroll
          for (int kk = 0; kk < KD; ++kk) {
            Frag fb[TPW], fl[TPW], fa[FPW];
#pragma unroll
            for (int jt = 0; jt < TPW; ++jt) {
              fb[jt] = M::load(Rs, LDD, tok_of(jt) + lr, kk * K + E * lg);
              if (SPLIT && split) fl[jt] = M::load(Rl, LDD, tok_of(jt) + lr, kk * K + E * lg);
            }
#pragma unroll
            for (int jf = 0; jf < FPW; ++jf) fa[jf] = M::load(Mat, LDD, row_of(jf) + lr, kk * K + E * lg);
#pragma unroll
            for (int jt = 0; jt < TPW; ++jt) {
#pragma unroll
              for (int jf = 0; jf < FPW; ++jf) {
                Y[jf][jt] = M::mma(fa[jf], fb[jt], Y[jf][jt]);
                if (SPLIT && split) Y[jf][jt] = M::mma(fa[jf], fl[jt], Y[jf][jt]);
              }
#pragma unroll
              for (int js = 0; js < SBW; ++js) {
                if (sblk_of(js) < CT) {
                  Pa[js][jt] = M::mma(fK[js][kk], fb[jt], Pa[js][jt]);
                  if (SPLIT && split) Pa[js][jt] = M::mma(fK[js][kk], fl[jt], Pa[js][jt]);
                }
              }
            }
          }
#pragma unroll
          for (int jt = 0; jt < TPW; ++jt)
#pragma unroll
            for (int js = 0; js < SBW; ++js) {
              const int sb = sblk_of(js);
              if (sb < CT) {
                const int o = (tok_of(jt) + lr) * LDC + 16 * sb + 4 * lg;
                store4<O>(Ps + o, Pa[js][jt] * Mh[js][jt]);
              }
            }
        }
      };
      // Y = diag(s) Y + Mat2 P'^T (Mat2 fragments fB: K^T in the loop, V^T for the output)
      auto products_2 = [&](Frag(&fB)[FPW][KC]) {
        if (tok_active) {
#pragma unroll
          for (int jt = 0; jt < TPW; ++jt) {
            Frag pb[KC];
#pragma unroll
            for (int kk = 0; kk < KC; ++kk) pb[kk] = M::load(Ps, LDC, tok_of(jt) + lr, kk * K + E * lg);
#pragma unroll
            for (int jf = 0; jf < FPW; ++jf) {
              f32x4 acc = Y[jf][jt] * sv[jt];
#pragma unroll
              for (int kk = 0; kk < KC; ++kk) acc = M::mma(fB[jf][kk], pb[kk], acc);
              Y[jf][jt] = acc;
            }
          }
        }
      };

      // residual update after the products of iteration it (Y = A R_i - a R_i):
      // R_{i+1} = R_{i-1} + omega_i (R_i - R_{i-1} - c A R_i) (R_1 = R_0 - c A R_0), applied as
      // kp_i R_{i-1} + kr_i R_i + ky_i Y with the coefficients expanded on the host; and
      // X += beta_{i+1} R_{i+1} (not for the residual mode's extra step, which gives R_iters)
      auto update = [&](int it, bool updx) {
        const float kp = cc.kp[it], kr = cc.kr[it], ky = cc.ky[it];
        const float bn = updx ? cc.beta[it + 1] : 0.0f;
#pragma unroll
        for (int jf = 0; jf < FPW; ++jf)
#pragma unroll
          for (int jt = 0; jt < TPW; ++jt) {
            const f32x4 rn = kp * Rp[jf][jt] + kr * R[jf][jt] + ky * Y[jf][jt];
            Rp[jf][jt] = R[jf][jt];
            R[jf][jt] = rn;
            if (updx) Xa[jf][jt] += bn * rn;
          }
      };
      // Residual mode: ||R_i|| per token, summed over the wave's features and lane groups, then
      // over the feature groups through LDS (p_u is free after the norm phase); every wave
      // takes part in the barriers, waves of feature group 0 write. A token with ||H_t|| = 0
      // has x_i = 0 for every i: its residuals are all ||q_t||.
      float res_q[TPW] = {};
      auto res_reduce = [&](float(&part)[TPW], float(&out)[TPW]) {
        if (tok_active) {
#pragma unroll
          for (int jt = 0; jt < TPW; ++jt) {
            float x = part[jt];
            x += __shfl_xor(x, 16, kWave);
            x += __shfl_xor(x, 32, kWave);
            if (lg == 0) p_u[fg * C + tok_of(jt) + lr] = x;
          }
        }
        lds_barrier();
        if (tok_active && fg == 0) {
#pragma unroll
          for (int jt = 0; jt < TPW; ++jt) {
            float x = 0.0f;
            for (int f = 0; f < FG; ++f) x += p_u[f * C + tok_of(jt) + lr];
            out[jt] = x;
          }
        }
        lds_barrier();
      };
      auto res_write = [&](int i, const float(&val)[TPW]) {
        if (tok_active && fg == 0 && lg == 0) {
#pragma unroll
          for (int jt = 0; jt < TPW; ++jt) {
            const int t = tok_of(jt) + lr;
            if (t < nv) {
              const float x = v_ninv[t] > 0.0f ? val[jt] : res_q[jt];
              A.resid[((seq0 + t0 + t) * Hn + h) * (cc.iters + 1) + i] = x;
            }
          }
        }
      };
      auto res_emit = [&](int i) {
        float part[TPW], out[TPW] = {};
#pragma unroll
        for (int jt = 0; jt < TPW; ++jt) {
          float x = 0.0f;
#pragma unroll
          for (int jf = 0; jf < FPW; ++jf) {
            const f32x4 r = R[jf][jt];
            x += r[0] * r[0] + r[1] * r[1] + r[2] * r[2] + r[3] * r[3];
          }
          part[jt] = x;
        }
        res_reduce(part, out);
#pragma unroll
        for (int jt = 0; jt < TPW; ++jt) out[jt] = sqrtf(out[jt]);
        res_write(i, out);
      };
      if constexpr (RES) {
        float part[TPW];
#pragma unroll
        for (int jt = 0; jt < TPW; ++jt) {
          float x = 0.0f;
#pragma unroll
          for (int jf = 0; jf < FPW; ++jf)
#pragma unroll
            for (int i = 0; i < 4; ++i) x += to_f32(Qraw[jf][jt][i]) * to_f32(Qraw[jf][jt][i]);
          part[jt] = x;
        }
        res_reduce(part, res_q);
#pragma unroll
        for (int jt = 0; jt < TPW; ++jt) res_q[jt] = sqrtf(res_q[jt]);
        res_write(0, res_q);  // x_0 = 0
      }

      prefetch(ch + 1);
      for (int it = 0; it + 1 < cc.iters; ++it) {
        write_operand(R, false);
        lds_barrier();
        products_1(St, false);
        lds_barrier();
        products_2(fKT);
        update(it, true);
        if constexpr (RES) res_emit(it + 1);
      }
      if constexpr (RES) {  // one more step on R_{r-1} gives R_r
        write_operand(R, false);
        lds_barrier();
        products_1(St, false);
        lds_barrier();
        products_2(fKT);
        update(cc.iters - 1, false);
        res_emit(cc.iters);
      }

      refresh();
      // U0hat = U0 / n0 into the staging buffer (every wave is past its last read of H0hat:
      // the loop ends with a barrier after the products that read it)
      if (state_active) {
#pragma unroll
        for (int jf = 0; jf < FPW; ++jf)
#pragma unroll
          for (int jc = 0; jc < CBW; ++jc)
            store4<O>(St + (col_of(jc) + lr) * LDD + row_of(jf) + 4 * lg, Ust[jf][jc] * n0inv);
      }
      carry();

      // ---- output O^T = diag(s) U0hat X^T + V^T P'^T (X split into hi + lo) --------------------
      // V^T fragments replace those of K^T; U0hat was staged into the H0hat buffer after the loop
      Frag fVT[FPW][KC];
#pragma unroll
      for (int jf = 0; jf < FPW; ++jf)
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) fVT[jf][kk] = M::load(VT, LDC, row_of(jf) + lr, kk * K + E * lg);
      write_operand(Xa, true);
      lds_barrier();
      products_1(St, true);
      lds_barrier();
      products_2(fVT);
      // every wave is past its reads of the operand buffer (the barrier before products_2)
      if (tok_active) {
#pragma unroll
        for (int jf = 0; jf < FPW; ++jf)
#pragma unroll
          for (int jt = 0; jt < TPW; ++jt)
            // (the iterate was formed times a power of two)
            store4<T>(Ob + (tok_of(jt) + lr) * LDD + row_of(jf) + 4 * lg, Y[jf][jt] * cc.inv_xsc);
      }
      pend_t0 = t0;
      pend_nv = nv;
    }

    n0sq = v_n2[C - 1];
  }

  lds_barrier();  // the last chunk's output tile is staged
  flush_o();
  // ---- results of the walk ------------------------------------------------------------------
  if (A.out_h && state_active && seg == last) {
    float* oh = A.out_h + (size_t)bh * D * D;
    float* ou = A.out_u + (size_t)bh * D * D;
#pragma unroll
    for (int jf = 0; jf < FPW; ++jf)
#pragma unroll
      for (int jc = 0; jc < CBW; ++jc) {
        const int r = row_of(jf) + 4 * lg, c = col_of(jc) + lr;
        *reinterpret_cast<f32x4*>(oh + (size_t)c * D + r) = Hst[jf][jc];
        *reinterpret_cast<f32x4*>(ou + (size_t)c * D + r) = Ust[jf][jc];
      }
  }
  if (A.n2_out && seg == last && tid == 0) A.n2_out[bh] = n0sq;
}

// Segment summaries (carry only): for each (segment, head), the state reached from a zero state
// over the segment's chunks,
//   H <- Gam_C H + K^T diag(w) K,  U^T <- Gam_C U^T + K^T diag(w) V  per chunk,
// and the segment's total log2 gate. One workgroup of 16 waves per (segment, head), four waves
// per SIMD, each holding its tiles of the float32 state. Per chunk every wave computes the gate
// prefix of the chunk itself (lane = token, a scan over groups of C lanes). Each thread loads one
// 16-byte unit of K and of V for the next chunk into registers (consecutive threads cover a
// token's row: whole cache lines); they are staged token-major into LDS together with the
// gate-weighted keys w K (split into hi + lo fp16 parts), one 16-byte write each, and the
// carry reads its operands K^T, V^T and (w K)^T with transposing LDS reads.
template <typename T, int D, int C>
__global__ __launch_bounds__(1024) void summary_kernel(WalkArgs A, int B, int Tmax, int Hn, int N,
                                                       int S, int J) {
  using Cfg = WalkCfg<T, D, C, 16>;
  using O = typename Cfg::O;
  using M = Mma<O>;
  using Frag = typename M::frag;
  constexpr int LDD = Cfg::LDD, FG = Cfg::FG, SG = Cfg::SG, FPW = Cfg::FPW, CBW = Cfg::CBW;
  constexpr int K = Cfg::K, E = Cfg::E, KC = C / K, VEC = Cfg::VEC, UPR = Cfg::UPR;
  constexpr bool SPLIT = Cfg::SPLIT;
  static_assert(Cfg::NU <= Cfg::NT, "one unit of K and V per thread");
  static_assert(kWave % C == 0, "a chunk's tokens fit a wave");

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  O* Kt = reinterpret_cast<O*>(smem);  // [C][LDD] K, token-major
  O* Vt = Kt + C * LDD;                // [C][LDD] V
  O* Wh = Vt + C * LDD;                // [C][LDD] w K, hi part
  O* Wl = Wh + C * LDD;                // [C][LDD] w K, lo part (fp16 operands only)
  typedef T vecT __attribute__((ext_vector_type(VEC)));
  typedef O vecO __attribute__((ext_vector_type(VEC)));

  const int seg = blockIdx.x;
  int b, h;
  head_of(A, blockIdx.y, Hn, b, h);
  const int bh = b * Hn + h;
  const int wave = threadIdx.x / kWave;
  int tid = threadIdx.x, lane = tid % kWave;
  int lr = lane % 16, lg = lane / 16;
  auto refresh = [&]() { asm volatile("" : "+v"(tid), "+v"(lane), "+v"(lr), "+v"(lg)); };
  const int fg = wave % FG, tg = wave / FG;
  const bool state_active = tg < SG;
  long long seq0;  // first row of sequence b
  int Tlen;        // its length
  seq_range(A, b, Tmax, seq0, Tlen);
  // the last segment of the sequence needs no summary (its walk writes the final state), nor
  // do the segments past it
  if (seg >= last_segment(Tlen, J, C)) return;
  const int c_begin = seg * J;
  const int c_end = min(N, c_begin + J);
  const long long tok_stride = (long long)Hn * D;
  const T* kg = static_cast<const T*>(A.k);
  const T* vg = static_cast<const T*>(A.v);
  auto row_of = [&](int jf) { return 16 * (fg * FPW + jf); };
  auto col_of = [&](int jc) { return 16 * (tg * CBW + jc); };

  f32x4 Hst[FPW][CBW], Ust[FPW][CBW];
#pragma unroll
  for (int jf = 0; jf < FPW; ++jf)
#pragma unroll
    for (int jc = 0; jc < CBW; ++jc) {
      Hst[jf][jc] = f32x4{0.f, 0.f, 0.f, 0.f};
      Ust[jf][jc] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  float log2g_seg = 0.0f;

  // registers of the next two chunks (slot 0: the next one, slot 1: the one after): unit
  // (token tid / UPR, column tid % UPR) of K and V, and the gate of token lane % C. Two chunks
  // in flight keep enough bytes outstanding per compute unit to cover the memory latency.
  vecT kreg[2] = {}, vreg[2] = {};
  float greg[2] = {1.0f, 1.0f}, breg[2] = {1.0f, 1.0f};  // gates and write gates
  auto prefetch = [&](int chn, int slot) {
    if (chn >= c_end) return;
    const int t0n = chn * C, nvn = min(C, Tlen - t0n);
    const int t = tid / UPR, c = tid % UPR;
    if (tid < Cfg::NU && t < nvn) {
      const long long off =
          (seq0 + t0n + t) * tok_stride + (long long)h * D + c * VEC;
      kreg[slot] = *reinterpret_cast<const vecT*>(kg + off);
      vreg[slot] = *reinterpret_cast<const vecT*>(vg + off);
    }
    if (lane % C < nvn) {
      const long long gi = (seq0 + t0n + lane % C) * Hn + h;
      greg[slot] = A.gamma[gi];
      if (A.beta) breg[slot] = A.beta[gi];
    }
  };
  prefetch(c_begin, 0);
  prefetch(c_begin + 1, 1);

  // one chunk; its data are in register slot SLOT (chunks alternate between the two slots, so
  // that no register of a load in flight is ever copied)
  auto chunk = [&](int ch, auto slot_tag) {
    constexpr int SLOT = decltype(slot_tag)::value;
    refresh();
    const int nv = min(C, Tlen - ch * C);
    const int tl = lane % C;  // this lane's token for the gate prefix
    // in-chunk log2 gate prefix over the lane's group of C lanes; tokens past the end of the
    // sequence have gamma = 1 (and zero keys and values)
    const float gcur = greg[SLOT];
    const float cl = scan_add<C>(tl < nv ? log2_gate(gcur) : 0.0f);
    float clast;  // prefix at the last token of the lane's group
    if constexpr (C == kWave) clast = lane_value(cl, C - 1);
    else clast = __shfl(cl, C - 1, C);
    // carry weight of token tl, times its write gate
    const float wl = fast_exp2(fminf(clast - cl, 0.0f)) * breg[SLOT];
    const float gC = fast_exp2(clast);
    log2g_seg += clast;
    const int t = tid / UPR, c = tid % UPR;  // this thread's unit
    const float w = __shfl(wl, t % kWave);   // carry weight of its token (lane t holds it)
    const vecT kv = kreg[SLOT], vv = vreg[SLOT];
    lds_barrier();           // every wave is past the previous chunk's carry
    prefetch(ch + 2, SLOT);  // in flight during this chunk and the next
    if (tid < Cfg::NU) {
      vecO ko, vo, xh, xl;
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        ko[i] = t < nv ? to_op<O>(kv[i]) : (O)0.0f;
        vo[i] = t < nv ? to_op<O>(vv[i]) : (O)0.0f;
        const float x = (float)ko[i] * w;
        xh[i] = (O)x;
        xl[i] = (O)(x - (float)xh[i]);
      }
      const int o = t * LDD + c * VEC;
      *reinterpret_cast<vecO*>(Kt + o) = ko;
      *reinterpret_cast<vecO*>(Vt + o) = vo;
      *reinterpret_cast<vecO*>(Wh + o) = xh;
      if (SPLIT) *reinterpret_cast<vecO*>(Wl + o) = xl;
    }
    lds_barrier();  // the operands of this chunk are staged
    if (state_active) {
#pragma unroll
      for (int jf = 0; jf < FPW; ++jf) {
        Frag aw[KC], awl[KC];
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) {
          aw[kk] = load_trans<O>(Wh, LDD, row_of(jf), kk * K, lr, lg);
          if (SPLIT) awl[kk] = load_trans<O>(Wl, LDD, row_of(jf), kk * K, lr, lg);
        }
#pragma unroll
        for (int jc = 0; jc < CBW; ++jc) {
          f32x4 hacc = Hst[jf][jc] * gC, uacc = Ust[jf][jc] * gC;
#pragma unroll
          for (int kk = 0; kk < KC; ++kk) {
            const Frag bk = load_trans<O>(Kt, LDD, col_of(jc), kk * K, lr, lg);
            const Frag bv = load_trans<O>(Vt, LDD, col_of(jc), kk * K, lr, lg);
            hacc = M::mma(aw[kk], bk, hacc);
            uacc = M::mma(aw[kk], bv, uacc);
            if (SPLIT) {
              hacc = M::mma(awl[kk], bk, hacc);
              uacc = M::mma(awl[kk], bv, uacc);
            }
          }
          Hst[jf][jc] = hacc;
          Ust[jf][jc] = uacc;
        }
      }
    }
  };
  for (int ch = c_begin; ch < c_end; ch += 2) {
    chunk(ch, std::integral_constant<int, 0>());
    if (ch + 1 < c_end) chunk(ch + 1, std::integral_constant<int, 1>());
  }

  if (state_active) {
    float* oh = A.sum_h + bh * A.sum_bh + seg * A.sum_seg;
    float* ou = A.sum_u + bh * A.sum_bh + seg * A.sum_seg;
#pragma unroll
    for (int jf = 0; jf < FPW; ++jf)
#pragma unroll
      for (int jc = 0; jc < CBW; ++jc) {
        const int r = row_of(jf) + 4 * lg, c = col_of(jc) + lr;
        *reinterpret_cast<f32x4*>(oh + (size_t)c * D + r) = Hst[jf][jc];
        *reinterpret_cast<f32x4*>(ou + (size_t)c * D + r) = Ust[jf][jc];
      }
  }
  if (tid == 0) A.log2g_out[(long long)bh * S + seg] = log2g_seg;
}

// Dispatch order of a packed batch: thread b counts the sequences that come before it (longer,
// or as long with a smaller index) over tiles of the lengths staged in LDS; that count is its
// rank. One thread per sequence, B <= kMaxOrdered.
__global__ __launch_bounds__(256) void order_kernel(const int* __restrict__ cu, int B, int Tmax,
                                                    int* __restrict__ order) {
  __shared__ int len_s[256];
  const int b = blockIdx.x * 256 + threadIdx.x;
  auto len_of = [&](int j) { return min(max(cu[j + 1] - cu[j], 0), Tmax); };
  const int mine = b < B ? len_of(b) : 0;
  int rank = 0;
  for (int j0 = 0; j0 < B; j0 += 256) {
    __syncthreads();  // the previous tile is read
    if (j0 + (int)threadIdx.x < B) len_s[threadIdx.x] = len_of(j0 + threadIdx.x);
    __syncthreads();
    const int n = min(256, B - j0);
    for (int i = 0; i < n; ++i) {
      const int l = len_s[i], j = j0 + i;
      rank += (l > mine) || (l == mine && j < b);
    }
  }
  if (b < B) order[rank] = b;
}

hipError_t launch_order(const int* cu, int B, int Tmax, int* order, hipStream_t stream) {
  hipLaunchKernelGGL(order_kernel, dim3((B + 255) / 256), dim3(256), 0, stream, cu, B, Tmax,
                     order);
  return hipGetLastError();
}

// Affine scan over segments, elementwise over the D x D entries of H and U.
__global__ __launch_bounds__(256) void scan_kernel(float* __restrict__ st,
                                                   const float* __restrict__ log2g,
                                                   float* __restrict__ h, float* __restrict__ u,
                                                   const float* __restrict__ hnorm2,
                                                   float* __restrict__ n2_seg0, int S, int DD,
                                                   const int* __restrict__ cu, int Tmax, int Hn,
                                                   int J, int C) {
  const int bh = blockIdx.y;
  const int e4 = blockIdx.x * blockDim.x + threadIdx.x;  // float4 index inside one matrix
  if (blockIdx.x == 0 && threadIdx.x == 0) n2_seg0[bh] = hnorm2 ? hnorm2[bh] : 0.0f;
  if (e4 * 4 >= DD) return;
  // packed batches: start states up to the sequence's last segment only (summaries exist
  // below it); a dense batch has last = S - 1
  int last = S - 1;
  if (cu) {
    const int b = bh / Hn;
    last = last_segment(min(max(cu[b + 1] - cu[b], 0), Tmax), J, C);
  }
  f32x4 sh = {0.f, 0.f, 0.f, 0.f}, su = {0.f, 0.f, 0.f, 0.f};
  if (h) {
    sh = reinterpret_cast<const f32x4*>(h + (size_t)bh * DD)[e4];
    su = reinterpret_cast<const f32x4*>(u + (size_t)bh * DD)[e4];
  }
  for (int s = 0; s <= last; ++s) {
    f32x4* ph = reinterpret_cast<f32x4*>(st + ((size_t)bh * S + s) * 2 * DD) + e4;
    f32x4* pu = reinterpret_cast<f32x4*>(st + ((size_t)bh * S + s) * 2 * DD + DD) + e4;
    f32x4 dh = {0.f, 0.f, 0.f, 0.f}, du = {0.f, 0.f, 0.f, 0.f};
    if (s < last) {  // the last segment has no summary
      dh = *ph;
      du = *pu;
    }
    *ph = sh;
    *pu = su;
    if (s < last) {
      const float g = exp2f(log2g[(size_t)bh * S + s]);
      sh = g * sh + dh;
      su = g * su + du;
    }
  }
}

template <typename T, int D, int C, bool RES>
static hipError_t launch_walk_rt(const FwdPlan& pl, const WalkArgs& a, const ChebConsts& cc,
                                 hipStream_t stream) {
  using Cfg = WalkCfg<T, D, C, 8>;
  auto kern = walk_kernel<T, D, C, RES>;
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(kern), (int)Cfg::bytes, lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(pl.S, pl.B * pl.H), dim3(Cfg::NT), Cfg::bytes, stream, a, pl.B,
                     pl.T, pl.H, pl.N, pl.S, pl.J, cc);
  return hipGetLastError();
}

template <typename T, int D, int C>
static hipError_t launch_walk_t(const FwdPlan& pl, bool summary, const WalkArgs& a,
                                const ChebConsts& cc, hipStream_t stream) {
  using Cfg = WalkCfg<T, D, C, 8>;
  using CfgS = WalkCfg<T, D, C, 16>;
  if (summary) {
    // segments 0 .. S-2: the last segment's walk produces the final state itself
    const dim3 sgrid(pl.S - 1, pl.B * pl.H);
    const size_t bytes = 4 * CfgS::szRD;  // K, V, w K hi and lo (token-major)
    auto kern = summary_kernel<T, D, C>;
    static std::atomic<uint64_t> lds_set{0};
    hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(kern), (int)bytes, lds_set);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, sgrid, dim3(CfgS::NT), bytes, stream, a, pl.B, pl.T, pl.H, pl.N,
                       pl.S, pl.J);
    return hipGetLastError();
  }
  if (a.resid) return launch_walk_rt<T, D, C, true>(pl, a, cc, stream);
  return launch_walk_rt<T, D, C, false>(pl, a, cc, stream);
}

hipError_t launch_walk(const FwdPlan& pl, bool summary, const WalkArgs& a, const ChebConsts& cc,
                       hipStream_t stream) {
  if (!summary && walk_tok_supported(pl)) return launch_walk_tok(pl, a, cc, stream);
  if (summary && summary_tok_supported(pl)) return launch_summary_tok(pl, a, stream);
  if (pl.dtype == 0) {
    if (pl.C == 16) {
      switch (pl.D) {
        case 32: return launch_walk_t<bf16, 32, 16>(pl, summary, a, cc, stream);
        case 64: return launch_walk_t<bf16, 64, 16>(pl, summary, a, cc, stream);
        case 128: return launch_walk_t<bf16, 128, 16>(pl, summary, a, cc, stream);
      }
    } else if (pl.C == 64) {
      switch (pl.D) {
        case 16: return launch_walk_t<bf16, 16, 64>(pl, summary, a, cc, stream);
        case 32: return launch_walk_t<bf16, 32, 64>(pl, summary, a, cc, stream);
        case 64: return launch_walk_t<bf16, 64, 64>(pl, summary, a, cc, stream);
        case 128: return launch_walk_t<bf16, 128, 64>(pl, summary, a, cc, stream);
      }
    } else if (pl.C == 32) {
      switch (pl.D) {
        case 16: return launch_walk_t<bf16, 16, 32>(pl, summary, a, cc, stream);
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
        case 128: return launch_walk_t<float, 128, 16>(pl, summary, a, cc, stream);
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
                       float* u, const float* hnorm2, float* n2_seg0, const int* cu,
                       hipStream_t stream) {
  const int DD = pl.D * pl.D;
  const dim3 grid((DD / 4 + 255) / 256, pl.B * pl.H);
  hipLaunchKernelGGL(scan_kernel, grid, dim3(256), 0, stream, ws_states, ws_log2g, h, u, hnorm2,
                     n2_seg0, pl.S, DD, cu, pl.T, pl.H, pl.J, pl.C);
  return hipGetLastError();
}

}  // namespace gka
