// Backward pass of the Gated KalmaNet layer on the matrix cores: bf16 inputs, chunks of 64
// tokens, D = 32, 64, 128.
//
// The gradients are those of gka_bwd_ref's definition (implicit differentiation of the solve,
// ai.info summary, "Methodology in Plain English" and "Main Findings": the backward re-runs the
// solver on the upstream gradient and uses a full interaction mask; Lemma 2 for the query):
//   x_t = A_t^-1 q_t, g_t = U_t^T do_t, y_t = A_t^-1 g_t, c_t = -a (y_t . x_t) / ||H_t||_F,
//   G_t = -y_t x_t^T + c_t H_t, W_t = do_t x_t^T, Gb_t = G_t + gamma_{t+1} Gb_{t+1} (Wb alike),
//   dq_t = y_t, dk_t = beta_t ((Gb_t + Gb_t^T) k_t + Wb_t^T v_t), dv_t = beta_t Wb_t k_t,
//   dbeta_t = k_t^T Gb_t k_t + v_t^T Wb_t k_t, dgamma_t = <Gb_t, H_{t-1}> + <Wb_t, U_{t-1}>.
//
// Chunk form. In a chunk with start state (H0, U0), log2 gate prefix l_t (token t's gate
// included, l_{-1} = 0), Gam_t = 2^l_t, and the gradients (Gn, Wn) that reach the chunk's last
// state from the later chunks:
//   Gb_t = sum_{u>=t} 2^(l_u - l_t) G_u + e_t Gn,  e_t = 2^(l_{C-1} - l_t)   (Wb alike)
// and with H_u = Gam_u H0 + sum_{s<=u} 2^(l_u - l_s) beta_s k_s k_s^T, every gradient is a sum
// over the chunk's token pairs. With E_m = sum_{u>=m} 2^(2 (l_u - l_m)) c_u (a suffix scan),
// the decay mask Dm[t][u] = 2^(l_u - l_t) [u >= t] and the interaction mask
// ME[t][s] = 2^(2 l_m - l_t - l_s) E_m, m = max(s, t) (the mask Dm diag(c Gam^2) Dm^T of the
// c_u H_u terms):
//   (Gb_t + Gb_t^T) k_t = -[(Dm o K X^T) Y + (Dm o K Y^T) X]_t + 2 Gam_t E_t H0 k_t
//                         + 2 [(ME o K K^T) diag(beta) K]_t + e_t (Gn + Gn^T) k_t
//   Wb_t^T v_t = [(Dm o V DO^T) X]_t + e_t Wn^T v_t,   Wb_t k_t = [(Dm o K X^T) DO]_t + e_t Wn k_t
//   dbeta_t = (k_t . dkraw_t + v_t . dvraw_t) / 2  (dkraw, dvraw: dk, dv before the beta_t factor)
//   dgamma_t = Gam_{t-1} <Sb_t, S0> + sum_{s<t} 2^(l_{t-1} - l_s) beta_s Z[s][t]
//     <Sb_t, S0> = sum_{u>=t} 2^(l_u - l_t) sigma_u + e_t (<Gn, H0> + <Wn, U0>),
//     sigma_u = -y_u^T H0 x_u + c_u <H_u, H0> + do_u^T U0 x_u,
//     Z[s][t] = sum_u Dm[t][u] P1[s][u] + sum_{s'} ME[t][s'] beta_s' (k_s . k_s')^2
//               + Gam_t E_t k_s^T H0 k_s + e_t (k_s^T Gn k_s + v_s^T Wn k_s),
//     P1[s][u] = (v_s . do_u - k_s . y_u) (k_s . x_u)
// and the chunk's own gradient at its start, carried to the earlier chunks by the segment scan
// run over the chunks in reverse order (dG_c + P_c Gn_c, P_c = Gam_{C-1}):
//   dG = -(Gam o X)^T Y + Gam_0^2 E_0 H0 + K^T diag(beta Gam E) K,   dW = (Gam o X)^T DO.
// Gn enters only as Gs = Gn + Gn^T ((Gn + Gn^T) k, k^T Gn k = k^T Gs k / 2, and <Gn, H0> =
// <Gs, H0> / 2 with H0 symmetric), and the scan is linear: the solve kernel writes dG + dG^T
// and the scan carries Gs itself.
//
// Two kernels, one workgroup per (chunk, head), four waves, wave w owning tokens 16w..16w+15:
//  * bwd_solve_kernel: the chunk's two Chebyshev solves on the forward walk's scheme (the
//    iterate in accumulators, H0hat, K and K^T fragments resident), x for q and y for g, then
//    dq, c, sigma, k^T H0 k, 2 Gam E H0 k (written for the second kernel) and dG, dW;
//  * bwd_grad_kernel: after the reverse scan, the token-pair products above (16-bit operands
//    with exact power-of-two scales, float32 accumulation), dk, dv, dbeta, dgamma.
// The chunks' start states come from the forward's segment summaries and scan with one chunk per
// segment.
#include "gka_internal.hpp"
#include "gka_tok.hpp"

namespace gka {
namespace {

template <int D>
struct BwdCfg {
  static constexpr int C = 64;         // tokens per chunk
  static constexpr int NW = 4;         // waves: one per SIMD
  static constexpr int NT = NW * kWave;
  static constexpr int FT = D / 16;    // feature tiles
  static constexpr int KD = D / 32;    // 32-deep blocks over the features
  static constexpr int KC = C / 32;    // 32-deep blocks over the tokens
  static constexpr int ST = C / 16;    // token tiles
  // Row stride of the [*][D] fp16 tiles. At D = 128 the rows are unpadded and the 16-byte
  // units of row r are permuted by XOR with (5 r) & 15 (tix), which halves the LDS bank
  // conflicts of the transposing fragment reads; at D <= 64 a 16-byte pad does better.
  static constexpr bool SWZ = D == 128;
  static constexpr int LDD = SWZ ? D : D + 8;
  static constexpr int LDP = C + 8;    // row stride of the [C][C] fp16 tiles
  static constexpr int UPR = D / 8;    // 16-byte units per bf16 token row
  static constexpr int NU = C * UPR;   // units per token-major chunk matrix
  static constexpr int NH4 = D * D / 4 / NT;  // float4 units of a D x D matrix per thread
  static constexpr int TPW = FT * FT / NW;    // D x D output tiles per wave
  static constexpr bool PIN = D >= 128;       // resident fragments in AGPRs
  static constexpr size_t szTok = (size_t)C * LDD * 2;
  static constexpr size_t szDD = (size_t)D * LDD * 2;
  static constexpr size_t szCC = (size_t)C * LDP * 2;
  static constexpr int NVEC = 8 * C + 64 + 4 * 64;
  // solve kernel: K, V, DO (token-major, permuted features), H0hat and U0 (D x D), x (float32,
  // accumulator layout per wave), vectors
  static constexpr size_t aK = 0, aV = aK + szTok, aDo = aV + szTok, aHs = aDo + szTok;
  static constexpr size_t aUs = aHs + szDD, aXs = aUs + szDD, aVec = aXs + (size_t)C * D * 4;
  static constexpr size_t aBytes = aVec + (size_t)NVEC * 4;
  // gradient kernel: K, V, DO, X, Y, Hs, P1, K2, vectors
  static constexpr size_t gK = 0, gV = gK + szTok, gDo = gV + szTok, gX = gDo + szTok;
  static constexpr size_t gY = gX + szTok, gHs = gY + szTok, gP1 = gHs + szDD, gK2 = gP1 + szCC;
  static constexpr size_t gVec = gK2 + szCC;
  static constexpr size_t gBytes = gVec + (size_t)NVEC * 4;
  static_assert(D % 32 == 0 && TPW >= 1 && NH4 >= 1, "unsupported D");
  static_assert(NU % NT == 0, "staging units must fill whole workgroups");
  static_assert(gBytes <= 160 * 1024 && aBytes <= 160 * 1024, "LDS budget of one CU exceeded");
};

__device__ inline float absmax4(f32x4 x) {
  return fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
}
__device__ inline float dot4(f32x4 a, f32x4 b) {
  return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
}
// sum / maximum over the four lane groups that hold one column of a 16-column tile
__device__ inline float group_sum(float x, int lane) {
  x += lane_read(x, lane ^ 16);
  return x + lane_read(x, lane ^ 32);
}
__device__ inline float group_max(float x, int lane) {
  x = fmaxf(x, lane_read(x, lane ^ 16));
  return fmaxf(x, lane_read(x, lane ^ 32));
}
__device__ inline void buffer_store16f(f32x4 x, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, off, 0, 0);
}
// 2^e for any integer e (exp2_int needs -126 <= e <= 127)
__device__ inline float pow2f(int e) { return ldexpf(1.0f, e); }
// element offset of column position e (permuted features) in row `row` of a [*][D] tile
template <int D>
__device__ inline int tix(int row, int e) {
  return row * BwdCfg<D>::LDD + (BwdCfg<D>::SWZ ? e ^ (8 * ((5 * row) & 15)) : e);
}
// the XOR of the element offsets of a transposing read of rows s + (lr >> 2), s = 4 lg modulo
// 16 (the same for both reads of frag_trans, whose rows differ by 16)
template <int D>
__device__ inline int tix_trans(int lg, int lr) {
  return BwdCfg<D>::SWZ ? 8 * ((5 * (4 * lg + (lr >> 2))) & 15) : 0;
}
// the four fp16 values of a token-major permuted row at logical features d..d+3 (d % 4 == 0)
template <int D>
__device__ inline f32x4 row4(const f16* tile, int row, int d) {
  const f16x4 h = *reinterpret_cast<const f16x4*>(tile + tix<D>(row, pcol(d)));
  return f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
}
template <int D>
__device__ inline void put_row4(f16* tile, int row, int d, f32x4 x) {
  *reinterpret_cast<f16x4*>(tile + tix<D>(row, pcol(d))) = f16x4{(f16)x[0], (f16)x[1], (f16)x[2], (f16)x[3]};
}

// A thread's groups of four elements of a row-major D x D fp16 matrix: group j is element
// 4 e4(j). At D >= 64 they come in pairs, one 16-byte load of eight elements per pair (the
// loads of these matrices are latency-bound: fewer, wider loads are faster).
template <int D>
struct DDGroups {
  static constexpr int NT = 256;
  static constexpr int N4 = D * D / 4 / NT;  // groups per thread
  static constexpr bool PAIRS = N4 % 2 == 0;
  __device__ static int e4(int tid, int j) {
    return PAIRS ? 2 * (tid + (j >> 1) * NT) + (j & 1) : tid + j * NT;
  }
};
__device__ inline void widen8(const f16* p, float sc, f32x4& lo, f32x4& hi) {
  const f16x8 h = *reinterpret_cast<const f16x8*>(p);
  lo = f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]} * sc;
  hi = f32x4{(float)h[4], (float)h[5], (float)h[6], (float)h[7]} * sc;
}
__device__ inline f32x4 widen4(const f16* p, float sc) {
  const f16x4 h = *reinterpret_cast<const f16x4*>(p);
  return f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]} * sc;
}

// bf16 16-byte units of a chunk's token rows (bounds-checked: rows past the end read as 0;
// nv <= 0, a chunk past the sequence, is an empty range)
template <int D>
struct ChunkRows {
  __amdgpu_buffer_rsrc_t r;
  uint32_t tok_bytes;
  __device__ ChunkRows(const void* base, long long row0, int nv, int Hn) {
    tok_bytes = (uint32_t)Hn * D * 2u;
    r = buffer_rsrc(static_cast<const bf16*>(base) + row0,
                    nv > 0 ? (uint32_t)(nv - 1) * tok_bytes + D * 2u : 0u);
  }
  __device__ bf16x8 unit(int u) const {
    const int tt = (uint32_t)u / (D / 8), cu = (uint32_t)u % (D / 8);
    return buffer_load16<bf16x8>(r, (uint32_t)tt * tok_bytes + (uint32_t)cu * 16u);
  }
};

// stage 16-byte bf16 units into a token-major permuted fp16 tile, times sc
template <int D>
__device__ inline void stage_unit(f16* dst, int u, bf16x8 x, float sc) {
  const int tt = (uint32_t)u / (D / 8), cu = (uint32_t)u % (D / 8);
  f16x4 a, b;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = (f16)((float)x[i] * sc);
    b[i] = (f16)((float)x[4 + i] * sc);
  }
  *reinterpret_cast<f16x4*>(dst + tix<D>(tt, pcol(8 * cu))) = a;
  *reinterpret_cast<f16x4*>(dst + tix<D>(tt, pcol(8 * cu + 4))) = b;
}

// ============================================================================================
// Solves of a chunk: x, y, and what the gradient kernel and the reverse scan need.
// ============================================================================================
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, D >= 128 ? 1 : 2)))
void bwd_solve_kernel(BwdArgs A, int Tlen, int Hn, int N, ChebConsts cc) {
  using Cfg = BwdCfg<D>;
  using M = Mma<f16>;
  typedef f16x8 Frag;
  constexpr int C = Cfg::C, NW = Cfg::NW, NT = Cfg::NT, FT = Cfg::FT, KD = Cfg::KD;
  constexpr int KC = Cfg::KC, ST = Cfg::ST, LDD = Cfg::LDD, NU = Cfg::NU, NH4 = Cfg::NH4;

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  f16* Kp = reinterpret_cast<f16*>(smem + Cfg::aK);
  f16* Vp = reinterpret_cast<f16*>(smem + Cfg::aV);
  f16* Dp = reinterpret_cast<f16*>(smem + Cfg::aDo);
  f16* Hs = reinterpret_cast<f16*>(smem + Cfg::aHs);
  f16* Us = reinterpret_cast<f16*>(smem + Cfg::aUs);  // U0 times 2^-ue, row-major (d, e)
  // x_t of the own tokens between the two solves: f32x4 slot (ft, lane) of wave w
  f32x4* Xs = reinterpret_cast<f32x4*>(smem + Cfg::aXs);
  float* v_cl = reinterpret_cast<float*>(smem + Cfg::aVec);  // [C] log2 gate prefix l_t
  float* v_bt = v_cl + C;   // [C] write gates (1 without them and past the end)
  float* v_g = v_bt + C;    // [C] gates (1 past the end)
  float* v_a = v_g + C;     // [C] n^2 scan: gamma_t^2
  float* v_b = v_a + C;     // [C] n^2 scan: the rest
  float* v_c = v_b + C;     // [C] c_t
  float* v_kh = v_c + C;    // [C] k_t^T H0 k_t
  float* v_w = v_kh + C;    // [C] weights of K^T diag(w) K in dG, times 2^-we
  float* v_sc = v_w + C;    // [64] block reductions
  float* v_coef = v_sc + 64;  // [iters][4] krs, kys, bts

  const int ch = blockIdx.x, bh = blockIdx.y;
  const int b = bh / Hn, h = bh % Hn;
  // Per-lane indices, passed through refresh() at the start of every phase so that addresses
  // derived from them are recomputed where they are used instead of being kept live through the
  // solves (which would spill them)
  int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  int lr = lane % 16, lg = lane / 16;
  int t = 16 * wave + lr;  // own token: column lr of the wave's accumulator tiles
  auto refresh = [&]() {
    asm volatile("" : "+v"(tid), "+v"(lane), "+v"(lr), "+v"(lg), "+v"(t), "+v"(wave));
  };
  const int t0 = ch * C, nv = min(C, Tlen - t0);
  const long long row0 = ((long long)b * Tlen + t0) * Hn * D + (long long)h * D;
  const ChunkRows<D> rk(A.k, row0, nv, Hn), rv(A.v, row0, nv, Hn), rd(A.dout, row0, nv, Hn);
  const uint32_t tok_bytes = rk.tok_bytes;

  // ---- loads: K, V, DO rows, gates (lane = token), the chunk's start state -----------------
  bf16x8 kin[NU / NT], vin[NU / NT], din[NU / NT];
#pragma unroll
  for (int j = 0; j < NU / NT; ++j) {
    kin[j] = rk.unit(tid + j * NT);
    vin[j] = rv.unit(tid + j * NT);
    din[j] = rd.unit(tid + j * NT);
  }
  const long long gb = ((long long)b * Tlen + t0) * Hn + h;
  const uint32_t gvalid = (uint32_t)(nv - 1) * Hn * 4u + 4u;
  const auto rg = buffer_rsrc(A.gamma + gb, gvalid);
  const auto rb = buffer_rsrc((A.beta ? A.beta : A.gamma) + gb, gvalid);
  float g_l = buffer_load4f(rg, (uint32_t)lane * Hn * 4u);
  float bt_l = buffer_load4f(rb, (uint32_t)lane * Hn * 4u);
  if (lane >= nv) g_l = 1.0f;
  if (lane >= nv || !A.beta) bt_l = 1.0f;
  // the own token's query, accumulator layout: Qraw[ft] = q_t[16 ft + 4 lg .. + 3]
  bf16x4 Qraw[FT];
  {
    const auto rq = buffer_rsrc(static_cast<const bf16*>(A.q) + row0,
                                (uint32_t)(nv - 1) * tok_bytes + D * 2u);
    const uint32_t qoff = (uint32_t)t * tok_bytes + (uint32_t)lg * 8u;
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) Qraw[ft] = buffer_load8<bf16x4>(rq, qoff + 32u * ft);
  }
  // the chunk's start state (fp16, each matrix times a power of two)
  const size_t fslot = (size_t)bh * N + ch;
  const f16* H0g = static_cast<const f16*>(A.fs16) + fslot * 2 * D * D;
  const f16* U0g = H0g + D * D;
  const float h0sc = pow2f((int)A.fexp[2 * fslot]), u0sc = pow2f((int)A.fexp[2 * fslot + 1]);
  using DG = DDGroups<D>;
  f32x4 hreg[NH4], ureg[NH4];
  float sq = 0.0f, um = 0.0f;
#pragma unroll
  for (int j = 0; j < NH4; j += DG::PAIRS ? 2 : 1) {
    const int e4 = DG::e4(tid, j);
    if constexpr (DG::PAIRS) {
      widen8(H0g + 4 * e4, h0sc, hreg[j], hreg[j + 1]);
      widen8(U0g + 4 * e4, u0sc, ureg[j], ureg[j + 1]);
    } else {
      hreg[j] = widen4(H0g + 4 * e4, h0sc);
      ureg[j] = widen4(U0g + 4 * e4, u0sc);
    }
  }
#pragma unroll
  for (int j = 0; j < NH4; ++j) {
    sq += dot4(hreg[j], hreg[j]);
    um = fmaxf(um, absmax4(ureg[j]));
  }
  {
    float mk = 0.0f, mv = 0.0f, md = 0.0f;
#pragma unroll
    for (int j = 0; j < NU / NT; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        mk = fmaxf(mk, fabsf((float)kin[j][i]));
        mv = fmaxf(mv, fabsf((float)vin[j][i]));
        md = fmaxf(md, fabsf((float)din[j][i]));
      }
    mk = wave_max(mk);
    mv = wave_max(mv);
    md = wave_max(md);
    sq = wave_sum(sq);
    um = wave_max(um);
    if (lane == 0) {
      v_sc[wave] = mk;
      v_sc[4 + wave] = mv;
      v_sc[8 + wave] = md;
      v_sc[12 + wave] = sq;
      v_sc[16 + wave] = um;
    }
  }
  // gate prefix (every wave; lane = token)
  const float cl = scan_add<kWave>(log2_gate(g_l));
  const float gam = fast_exp2(cl);
  const float cl_first = lane_value(cl, 0), cl_last = lane_value(cl, C - 1);
  if (wave == 0) {
    v_cl[lane] = cl;
    v_bt[lane] = bt_l;
    v_g[lane] = g_l;
  }
  if (tid < cc.iters_rs) {
    v_coef[4 * tid] = cc.krs[tid];
    v_coef[4 * tid + 1] = cc.kys[tid];
    v_coef[4 * tid + 2] = cc.bts[tid];
    v_coef[4 * tid + 3] = 0.0f;
  }
  __syncthreads();
  float km = v_sc[0], vm = v_sc[4], dm = v_sc[8], n0sq = v_sc[12], umx = v_sc[16];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    km = fmaxf(km, v_sc[w]);
    vm = fmaxf(vm, v_sc[4 + w]);
    dm = fmaxf(dm, v_sc[8 + w]);
    n0sq += v_sc[12 + w];
    umx = fmaxf(umx, v_sc[16 + w]);
  }
  const int ke = pow2_exponent(km, 30), ve = pow2_exponent(vm, 60), de = pow2_exponent(dm, 60);
  const int ue = pow2_exponent(umx, 100);
  const float ks2 = exp2_int(2 * ke);
  const float n0 = sqrtf(n0sq), n0inv = n0 > 0.0f ? 1.0f / n0 : 0.0f;

  // ---- stage K, V, DO (fp16, times 2^-ke, 2^-ve, 2^-de, permuted features), H0hat and U0
  // (times 2^-ue), the D x D matrices row-major with permuted columns ------------------------
#pragma unroll
  for (int j = 0; j < NU / NT; ++j) {
    const int u = tid + j * NT;
    stage_unit<D>(Kp, u, kin[j], exp2_int(-ke));
    stage_unit<D>(Vp, u, vin[j], exp2_int(-ve));
    stage_unit<D>(Dp, u, din[j], exp2_int(-de));
  }
  {
    const float usc = pow2f(-ue);
#pragma unroll
    for (int j = 0; j < NH4; ++j) {
      const int e4 = DG::e4(tid, j), r = e4 / (D / 4), c4 = e4 % (D / 4);
      put_row4<D>(Hs, r, 4 * c4, hreg[j] * n0inv);
      put_row4<D>(Us, r, 4 * c4, ureg[j] * usc);
    }
  }
  lds_barrier();

  // ---- resident fragments: H0hat (rows = features), K (rows = tokens), K^T (permuted tokens)
  Frag Hres[FT][KD];
#pragma unroll
  for (int ft = 0; ft < FT; ++ft)
#pragma unroll
    for (int kk = 0; kk < KD; ++kk)
      Hres[ft][kk] = *reinterpret_cast<const Frag*>(Hs + tix<D>(16 * ft + lr, 32 * kk + 8 * lg));
  // K fragments (rows = tokens) are read from LDS where they are used (K stays staged until
  // both solves are done): resident, they would push the solves past the register file
  auto kfrag = [&](int kk, int sb) {
    return *reinterpret_cast<const Frag*>(Kp + tix<D>(16 * sb + lr, 32 * kk + 8 * lg));
  };
  Frag ktr[KC][FT];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc)
#pragma unroll
    for (int ft = 0; ft < FT; ++ft)
      ktr[kc][ft] = frag_trans<LDD>(Kp, 32 * kc + 4 * lg, 32 * kc + 16 + 4 * lg,
                                    pcol(16 * ft + 4 * (lr & 3)), lr, tix_trans<D>(lg, lr));
  if constexpr (Cfg::PIN) {
#pragma unroll
    for (int ft = 0; ft < FT; ++ft)
#pragma unroll
      for (int kk = 0; kk < KD; ++kk) keep_in_agpr(Hres[ft][kk]);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) keep_in_agpr(ktr[kc][ft]);
  }

  // ---- norm phase: k_t^T H0hat k_t, sum_{s<t} 2^(l_{t-1} - l_s) beta_s (k_s . k_t)^2 -------
  Frag kb[KD];  // B fragments of the own token's key
#pragma unroll
  for (int kk = 0; kk < KD; ++kk)
    kb[kk] = *reinterpret_cast<const Frag*>(Kp + tix<D>(t, 32 * kk + 8 * lg));
  {
    f32x4 z[FT];
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) z[ft] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KD; ++kk)
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) z[ft] = M::mma(Hres[ft][kk], kb[kk], z[ft]);
    float pu = 0.0f;
#pragma unroll
    for (int ft = 0; ft < FT; ++ft)
#pragma unroll
      for (int i = 0; i < 4; ++i) pu += z[ft][i] * (float)kb[ft / 2][4 * (ft % 2) + i];
    f32x4 gram[ST];
#pragma unroll
    for (int sb = 0; sb < ST; ++sb) gram[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KD; ++kk)
#pragma unroll
      for (int sb = 0; sb < ST; ++sb) gram[sb] = M::mma(kfrag(kk, sb), kb[kk], gram[sb]);
    const float clp = t > 0 ? v_cl[t - 1] : 0.0f;
    float pv = 0.0f, kd = 0.0f;
#pragma unroll
    for (int sb = 0; sb < ST; ++sb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = 16 * sb + 4 * lg + i;
        const float gs = gram[sb][i];
        const float e = fast_exp2(fminf(clp - v_cl[s], 0.0f)) * v_bt[s] * (gs * gs);
        pv += s < t ? e : 0.0f;
        kd = s == t ? gs : kd;
      }
    pu = group_sum(pu, lane);
    pv = group_sum(pv, lane);
    kd = group_sum(kd, lane);
    const float gt = v_g[t], btt = v_bt[t];
    const float gprev = t > 0 ? fast_exp2(v_cl[t - 1]) : 1.0f;
    const float kh_t = n0 * (pu * ks2);  // k_t^T H0 k_t
    if (lg == 0) {
      const float kdt = btt * (kd * ks2);  // beta_t ||k_t||^2
      v_a[t] = gt * gt;
      v_b[t] = 2.0f * gt * btt * (gprev * kh_t + (pv * ks2) * ks2) + kdt * kdt;
      v_kh[t] = kh_t;
    }
  }
  lds_barrier();

  // ---- n_t by an affine scan over the chunk; the own token's scalars and mask --------------
  float sa = v_a[lane], sb_ = v_b[lane];
  scan_affine(sa, sb_);
  const float n2 = sa * n0sq + sb_;
  const float ninv = n2 > 0.0f ? 1.0f / sqrtf(n2) : 0.0f;
  const float ninv_t = lane_read(ninv, t);
  const float gam_t = lane_read(gam, t);
  const float s_t = gam_t * n0 * ninv_t;
  const float cl_t = lane_read(cl, t);
  const bool live = ninv_t > 0.0f;  // ||H_t|| = 0: x_t = y_t = 0
  f32x4 Mh[ST];  // Mhat_{t, s} for the staged keys (times 2^2ke)
#pragma unroll
  for (int sb = 0; sb < ST; ++sb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = 16 * sb + 4 * lg + i;
      const float e = fast_exp2(fminf(cl_t - v_cl[s], 0.0f)) * v_bt[s] * (ninv_t * ks2);
      Mh[sb][i] = s <= t ? e : 0.0f;
    }

  // ---- Chebyshev iteration on the rescaled residuals of the own token (as the forward walk):
  //   Ro <- Ro + krs Rc + H0hat (kys s_t Rc) + K^T ((K Rc) o kys Mhat),  X += bts Rc
  auto step = [&](auto first, f32x4(&Ro)[FT], f32x4(&Rc)[FT], f32x4(&X)[FT], int it) {
    constexpr bool FIRST = decltype(first)::value;
    const f32x4 cf = *reinterpret_cast<const f32x4*>(v_coef + 4 * it);
    Frag rf[KD], rs[KD], pf[KC];
    f32x4 pa[ST];
#pragma unroll
    for (int kk = 0; kk < KD; ++kk) rf[kk] = pack8(Rc[2 * kk], Rc[2 * kk + 1]);
#pragma unroll
    for (int sb = 0; sb < ST; ++sb) pa[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KD; ++kk)
#pragma unroll
      for (int sb = 0; sb < ST; ++sb) pa[sb] = M::mma(kfrag(kk, sb), rf[kk], pa[sb]);
    const float kys = cf[1] * s_t;
#pragma unroll
    for (int kk = 0; kk < KD; ++kk) rs[kk] = pack8(Rc[2 * kk] * kys, Rc[2 * kk + 1] * kys);
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) Ro[ft] = FIRST ? cf[0] * Rc[ft] : Ro[ft] + cf[0] * Rc[ft];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < KD; ++kk)
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) Ro[ft] = M::mma(Hres[ft][kk], rs[kk], Ro[ft]);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
      pf[kc] = pack8(pa[2 * kc] * Mh[2 * kc] * cf[1], pa[2 * kc + 1] * Mh[2 * kc + 1] * cf[1]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) Ro[ft] = M::mma(ktr[kc][ft], pf[kc], Ro[ft]);
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) X[ft] = FIRST ? cf[2] * Rc[ft] : X[ft] + cf[2] * Rc[ft];
    __builtin_amdgcn_sched_barrier(0);
  };
  // X = sum_{i < iters} bts_i Rt_i from Rt_0 = Ra (Ra and Rb are overwritten)
  auto solve = [&](f32x4(&Ra)[FT], f32x4(&Rb)[FT], f32x4(&X)[FT]) {
    using T1 = std::integral_constant<bool, true>;
    using T0 = std::integral_constant<bool, false>;
    const int iters = cc.iters_rs;
    const float bl = v_coef[4 * (iters - 1) + 2];
    if (iters == 1) {
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) X[ft] = bl * Ra[ft];
      return;
    }
    step(T1{}, Rb, Ra, X, 0);
    int it = 1;
    for (; it + 2 < iters; it += 2) {
      step(T0{}, Ra, Rb, X, it);
      step(T0{}, Rb, Ra, X, it + 1);
    }
    if (it + 1 < iters) {
      step(T0{}, Ra, Rb, X, it);
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) X[ft] += bl * Ra[ft];
    } else {
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) X[ft] += bl * Rb[ft];
    }
  };

  const uint32_t xrow = (uint32_t)D * 4u;  // bytes per token row of the float32 workspaces
  const size_t wrow0 = ((size_t)bh * Tlen + t0) * D;  // first workspace row of the chunk
  const uint32_t wvalid = (uint32_t)(nv - 1) * xrow + xrow;
  // byte offset of the own token's row and lane group in the float32 workspaces
  auto woff = [&]() { return (uint32_t)t * xrow + (uint32_t)lg * 16u; };

  // ---- x: the solve for q_t (the query times 2^-qe: its largest element lies in [1, 2)) ---
  refresh();
  f32x4 xv[FT];  // x_t, accumulator layout: x_t[16 ft + 4 lg + i]
  {
    float qm = 0.0f;
#pragma unroll
    for (int ft = 0; ft < FT; ++ft)
#pragma unroll
      for (int j = 0; j < 4; ++j) qm = fmaxf(qm, fabsf((float)Qraw[ft][j]));
    const int qe = pow2_exponent(group_max(qm, lane), 60);
    const float qsc = live ? cc.inv_s0 * exp2_int(-qe) : 0.0f;
    f32x4 Ra[FT], Rb[FT], X[FT];
#pragma unroll
    for (int ft = 0; ft < FT; ++ft)
      Ra[ft] = f32x4{(float)Qraw[ft][0], (float)Qraw[ft][1], (float)Qraw[ft][2], (float)Qraw[ft][3]} * qsc;
    solve(Ra, Rb, X);
    const float xs = cc.inv_xsc * exp2_int(qe) * ninv_t;
    const auto rx = buffer_rsrc(A.xs + wrow0, wvalid);
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) {
      xv[ft] = X[ft] * xs;
      buffer_store16f(xv[ft], rx, woff() + 64u * ft);
      Xs[(ft * NW + wave) * kWave + lane] = xv[ft];
    }
  }


  // ---- g_t = U_t^T do_t = Gam_t U0^T do_t + sum_{s<=t} 2^(l_t - l_s) beta_s (v_s . do_t) k_s
  // (U0'^T do'_t into accumulators -- U0^T fragments by transposing reads of the row-major U0
  // -- then the in-chunk term added by K^T products on the masked V DO^T column; g_t = 2^(ke + ve
  // + de) times the accumulators)
  float sigU;  // do_t^T U0 x_t
  f32x4 gacc[FT];
  {
    Frag db[KD];
#pragma unroll
    for (int kk = 0; kk < KD; ++kk)
      db[kk] = *reinterpret_cast<const Frag*>(Dp + tix<D>(t, 32 * kk + 8 * lg));
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) gacc[ft] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KD; ++kk)
#pragma unroll
      for (int ft = 0; ft < FT; ++ft)
        gacc[ft] = M::mma(frag_trans<LDD>(Us, 32 * kk + 4 * lg, 32 * kk + 16 + 4 * lg,
                                          pcol(16 * ft + 4 * (lr & 3)), lr, tix_trans<D>(lg, lr)),
                          db[kk], gacc[ft]);
    f32x4 pa[ST];
#pragma unroll
    for (int sb = 0; sb < ST; ++sb) pa[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KD; ++kk)
#pragma unroll
      for (int sb = 0; sb < ST; ++sb)
        pa[sb] = M::mma(*reinterpret_cast<const Frag*>(Vp + tix<D>(16 * sb + lr, 32 * kk + 8 * lg)),
                        db[kk], pa[sb]);
    float su = 0.0f;
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) su += dot4(gacc[ft], xv[ft]);
    sigU = group_sum(su, lane) * pow2f(ue + de);
    Frag pf[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      f32x4 m0, m1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s0 = 32 * kc + 4 * lg + i, s1 = s0 + 16;
        const float e0 = fast_exp2(fminf(cl_t - v_cl[s0], 0.0f)) * v_bt[s0];
        const float e1 = fast_exp2(fminf(cl_t - v_cl[s1], 0.0f)) * v_bt[s1];
        m0[i] = s0 <= t ? e0 : 0.0f;
        m1[i] = s1 <= t ? e1 : 0.0f;
      }
      pf[kc] = pack8(pa[2 * kc] * m0, pa[2 * kc + 1] * m1);
    }
    const float gsc = gam_t * pow2f(ue - ke - ve);
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) gacc[ft] = gacc[ft] * gsc;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) gacc[ft] = M::mma(ktr[kc][ft], pf[kc], gacc[ft]);
  }

  // ---- y: the solve for g_t (times 2^-ge, its largest element in [1, 2)) --------------------
  refresh();
  f32x4 yv[FT];
  {
    float gm = 0.0f;
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) gm = fmaxf(gm, absmax4(gacc[ft]));
    const int ge = pow2_exponent(group_max(gm, lane), 100);
    const float gsc = live ? cc.inv_s0 * pow2f(-ge) : 0.0f;
    f32x4 Rb[FT], Y[FT];
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) gacc[ft] = gacc[ft] * gsc;
    solve(gacc, Rb, Y);
    const float ys = cc.inv_xsc * pow2f(ge + ke + ve + de) * ninv_t;
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) yv[ft] = Y[ft] * ys;
  }

  // ---- per token: c_t, y_t^T H0 x_t, H0 k_t (products on the resident H0hat) ---------------
  // (x_t is read back from the lane's own LDS slots: not held through the y solve)
  refresh();
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) xv[ft] = Xs[(ft * NW + wave) * kWave + lane];
  float xy = 0.0f, ymax = 0.0f, gxmax = 0.0f;
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) {
    xy += dot4(xv[ft], yv[ft]);
    ymax = fmaxf(ymax, absmax4(yv[ft]));
    gxmax = fmaxf(gxmax, absmax4(xv[ft]));
  }
  xy = group_sum(xy, lane);
  ymax = group_max(ymax, lane);
  gxmax = group_max(gxmax, lane) * gam_t;
  const float c_t = live ? -cc.a * xy * ninv_t : 0.0f;
  float yHx;  // y_t^T H0 x_t
  f32x4 hk[FT];  // H0hat k'_t
  {
#pragma unroll
    for (int kk = 0; kk < KD; ++kk)
      kb[kk] = *reinterpret_cast<const Frag*>(Kp + tix<D>(t, 32 * kk + 8 * lg));
    const int ye = pow2_exponent(ymax, 126);
    const float yi = pow2f(-ye);
    Frag yf[KD];
#pragma unroll
    for (int kk = 0; kk < KD; ++kk) yf[kk] = pack8(yv[2 * kk] * yi, yv[2 * kk + 1] * yi);
    f32x4 hy[FT];
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) {
      hy[ft] = f32x4{0.f, 0.f, 0.f, 0.f};
      hk[ft] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int kk = 0; kk < KD; ++kk)
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) {
        hy[ft] = M::mma(Hres[ft][kk], yf[kk], hy[ft]);
        hk[ft] = M::mma(Hres[ft][kk], kb[kk], hk[ft]);
      }
    float s = 0.0f;
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) s += dot4(hy[ft], xv[ft]);
    yHx = group_sum(s, lane) * n0 * pow2f(ye);
  }
  if (lg == 0) v_c[t] = c_t;
  {
    const float a = wave_max(gxmax), bm = wave_max(ymax);
    if (lane == 0) {
      v_sc[24 + wave] = a;
      v_sc[28 + wave] = bm;
    }
  }
  lds_barrier();  // c of every token; no wave reads K, V from LDS after this point

  // ---- E_t = c_t + gamma_{t+1}^2 E_{t+1} (lane l: token C - 1 - l); <H_u, H0> by a prefix
  // scan hh_u = gamma_u hh_{u-1} + beta_u k_u^T H0 k_u, hh_{-1} = ||H0||^2 ---------------------
  const int tr = C - 1 - lane;
  float ea = tr + 1 < C ? v_g[tr + 1] * v_g[tr + 1] : 0.0f, eb = v_c[tr];
  scan_affine(ea, eb);  // eb = E_tr
  const float E_t = lane_read(eb, C - 1 - t);
  const float E_0 = lane_value(eb, C - 1);
  float wsum = v_bt[tr] * fast_exp2(v_cl[tr]) * eb;  // weight beta_s Gam_s E_s of token s = tr
  const int we = pow2_exponent(wave_max(fabsf(wsum)), 126);
  if (wave == 0) v_w[tr] = wsum * pow2f(-we);
  float ha = v_g[lane], hb = v_bt[lane] * v_kh[lane];
  scan_affine(ha, hb);
  const float hh_t = lane_read(ha * n0sq + hb, t);
  const float sig_t = -yHx + c_t * hh_t + sigU;

  // the start state's values at the wave's dG tiles (read here, used at the end)
  const int wave_u = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  f32x4 h0t[Cfg::TPW];
#pragma unroll
  for (int q = 0; q < Cfg::TPW; ++q) {
    const int tile = wave_u * Cfg::TPW + q, a = tile / FT, bq = tile % FT;
    h0t[q] = load4(H0g + (size_t)(16 * bq + lr) * D + 16 * a + 4 * lg) * h0sc;
  }

  // ---- outputs of the token: dq = y, the workspaces x (written above), y, 2 Gam E H0 k, and
  // (c, sigma, k^T H0 k) ------------------------------------------------------------------------
  {
    const auto ry = buffer_rsrc(A.ys + wrow0, wvalid);
    const auto rh = buffer_rsrc(A.dkh + wrow0, wvalid);
    const auto rq = buffer_rsrc(static_cast<bf16*>(A.dq) + row0,
                                (uint32_t)(nv - 1) * tok_bytes + D * 2u);
    const uint32_t qoff = (uint32_t)t * tok_bytes + (uint32_t)lg * 8u;
    const float hsc = 2.0f * gam_t * E_t * n0 * exp2_int(ke);
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) {
      buffer_store16f(yv[ft], ry, woff() + 64u * ft);
      buffer_store16f(hk[ft] * hsc, rh, woff() + 64u * ft);
      const bf16x4 o = {(bf16)yv[ft][0], (bf16)yv[ft][1], (bf16)yv[ft][2], (bf16)yv[ft][3]};
      buffer_store8(o, rq, qoff + 32u * ft);
    }
    if (lg == 0 && t < nv) {
      float* tv = A.tokv + ((size_t)bh * Tlen + t0 + t) * 4;
      *reinterpret_cast<f32x4*>(tv) = f32x4{c_t, sig_t, v_kh[t], 0.0f};
    }
  }

  // ---- the chunk's gradient at its start, into reverse-scan slot N - 1 - ch (slot N - 1, of
  // chunk 0, is never read by the scan):
  //   dG + dG^T = -(Gam o X)^T Y - Y^T (Gam o X) + 2 Gam_0^2 E_0 H0 + 2 K^T diag(w) K,
  //   dW^T = (Gam o X)^T DO
  // (Gam o X and Y staged token-major, fp16 times 2^-xe2, 2^-ye2, over K and V) --------------
  if (ch == 0) return;
  float gxm = v_sc[24], ym = v_sc[28];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    gxm = fmaxf(gxm, v_sc[24 + w]);
    ym = fmaxf(ym, v_sc[28 + w]);
  }
  const int xe2 = pow2_exponent(gxm, 126), ye2 = pow2_exponent(ym, 126);
  {
    const float xi = gam_t * pow2f(-xe2), yi = pow2f(-ye2);
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) {
      put_row4<D>(Vp, t, 16 * ft + 4 * lg, xv[ft] * xi);
      put_row4<D>(Kp, t, 16 * ft + 4 * lg, yv[ft] * yi);
    }
  }
  lds_barrier();
  const size_t rslot = (size_t)bh * N + (N - 1 - ch);
  f16* rs = static_cast<f16*>(A.rd16) + rslot * 2 * D * D;
  signed char* rx = A.rdx + rslot * 2 * D * (D / 16);
  if (tid == 0) A.rlog2[rslot] = cl_last;
  // a lane's four values (a row segment) to slot matrix `mat`, fp16, the 16 columns of the row
  // segment's tile times the power of two of their largest magnitude (the lane groups of the
  // column share it; lane group 0 stores it)
  auto put16 = [&](f32x4 x, size_t o, int row, int blk, int mat) {
    const int e = pow2_exponent(group_max(absmax4(x), lane), 126);
    const f32x4 y = x * pow2f(-e);
    *reinterpret_cast<f16x4*>(rs + (size_t)mat * D * D + o) = f16x4{(f16)y[0], (f16)y[1], (f16)y[2], (f16)y[3]};
    if (lg == 0) rx[(size_t)mat * D * (D / 16) + row * (D / 16) + blk] = (signed char)e;
  };
  const float hsc0 = fast_exp2(2.0f * cl_first) * E_0;
  const float sxy = -pow2f(xe2 + ye2), sw = pow2f(2 * ke + we), sxd = pow2f(xe2 + de);
  // (one instance per wave: the tile indices, and with them the resident K^T fragments of the
  // tile's rows and columns, are compile-time constants)
  auto dg_tiles = [&](auto W) {
    constexpr int w = decltype(W)::value;
    static_for<0, Cfg::TPW>([&](auto Q) {
      constexpr int q = decltype(Q)::value, tile = w * Cfg::TPW + q;
      constexpr int a = tile / FT, bq = tile % FT;
      f32x4 acc1 = {0.f, 0.f, 0.f, 0.f}, acc2 = acc1, acc3 = acc1;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const int s0 = 32 * kc + 4 * lg, s1 = s0 + 16;
        const int ca = pcol(16 * a + 4 * (lr & 3)), cb = pcol(16 * bq + 4 * (lr & 3));
        const Frag xa = frag_trans<LDD>(Vp, s0, s1, ca, lr, tix_trans<D>(lg, lr));
        const Frag yb = frag_trans<LDD>(Kp, s0, s1, cb, lr, tix_trans<D>(lg, lr));
        const Frag ya = frag_trans<LDD>(Kp, s0, s1, ca, lr, tix_trans<D>(lg, lr));
        const Frag xb = frag_trans<LDD>(Vp, s0, s1, cb, lr, tix_trans<D>(lg, lr));
        const Frag dbf = frag_trans<LDD>(Dp, s0, s1, cb, lr, tix_trans<D>(lg, lr));
        // (w K)^T over the permuted tokens of ktr, and K as B
        const f32x4 w0 = *reinterpret_cast<const f32x4*>(v_w + s0);
        const f32x4 w1 = *reinterpret_cast<const f32x4*>(v_w + s1);
        const Frag ka = ktr[kc][a];
        Frag wa;
#pragma unroll
        for (int j = 0; j < 8; ++j) wa[j] = (f16)((float)ka[j] * (j < 4 ? w0[j] : w1[j - 4]));
        acc1 = M::mma(xa, yb, acc1);
        acc1 = M::mma(ya, xb, acc1);
        acc2 = M::mma(wa, ktr[kc][bq], acc2);
        acc3 = M::mma(xa, dbf, acc3);
      }
      // lane: element [16a + 4lg + i][16bq + lr] of the products, stored at [16bq + lr][16a +
      // 4lg + i]: the transpose for dW, the same matrix for the symmetric dG + dG^T (H0
      // symmetric)
      const size_t o = (size_t)(16 * bq + lr) * D + 16 * a + 4 * lg;
      put16(acc1 * sxy + acc2 * (2.0f * sw) + h0t[q] * (2.0f * hsc0), o, 16 * bq + lr, a, 0);
      put16(acc3 * sxd, o, 16 * bq + lr, a, 1);
    });
  };
  switch (wave_u) {
    case 0: dg_tiles(IC<0>{}); break;
    case 1: dg_tiles(IC<1>{}); break;
    case 2: dg_tiles(IC<2>{}); break;
    default: dg_tiles(IC<3>{}); break;
  }
}


// ============================================================================================
// Gradients of a chunk's tokens from its solves and the gradients (Gn, Wn) of the later chunks.
// ============================================================================================
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, D >= 128 ? 1 : 2)))
void bwd_grad_kernel(BwdArgs A, int Tlen, int Hn, int N) {
  using Cfg = BwdCfg<D>;
  using M = Mma<f16>;
  typedef f16x8 Frag;
  constexpr int C = Cfg::C, NW = Cfg::NW, NT = Cfg::NT, FT = Cfg::FT, KD = Cfg::KD;
  constexpr int KC = Cfg::KC, ST = Cfg::ST, LDD = Cfg::LDD, LDP = Cfg::LDP, NU = Cfg::NU;
  constexpr int NH4 = Cfg::NH4, NX4 = C * D / 4 / NT;

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  f16* Kp = reinterpret_cast<f16*>(smem + Cfg::gK);
  f16* Vp = reinterpret_cast<f16*>(smem + Cfg::gV);
  f16* Dp = reinterpret_cast<f16*>(smem + Cfg::gDo);
  f16* Xp = reinterpret_cast<f16*>(smem + Cfg::gX);
  f16* Yp = reinterpret_cast<f16*>(smem + Cfg::gY);
  f16* Hs = reinterpret_cast<f16*>(smem + Cfg::gHs);
  f16* P1s = reinterpret_cast<f16*>(smem + Cfg::gP1);  // [s][u] P1, times 2^-p1e
  f16* K2s = reinterpret_cast<f16*>(smem + Cfg::gK2);  // [s][s'] (k's . k's')^2 / (4D)^2
  float* v_cl = reinterpret_cast<float*>(smem + Cfg::gVec);  // [C] log2 gate prefix
  float* v_bt = v_cl + C;  // [C] write gates
  float* v_E = v_bt + C;   // [C] E_t
  float* v_kh = v_E + C;   // [C] k_t^T H0 k_t
  float* v_nx = v_kh + C;  // [C] k_t^T Gn k_t + v_t^T Wn k_t
  float* v_sc = v_nx + C;  // [64] block reductions

  const int ch = blockIdx.x, bh = blockIdx.y;
  const int b = bh / Hn, h = bh % Hn;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int lr = lane % 16, lg = lane / 16;
  const int t = 16 * wave + lr;
  const int t0 = ch * C, nv = min(C, Tlen - t0);
  const long long row0 = ((long long)b * Tlen + t0) * Hn * D + (long long)h * D;
  const ChunkRows<D> rk(A.k, row0, nv, Hn), rv(A.v, row0, nv, Hn), rd(A.dout, row0, nv, Hn);
  const uint32_t tok_bytes = rk.tok_bytes;
  const uint32_t xrow = (uint32_t)D * 4u;
  const size_t wrow0 = ((size_t)bh * Tlen + t0) * D;
  const uint32_t wvalid = (uint32_t)nv * xrow;
  const auto rx = buffer_rsrc(A.xs + wrow0, wvalid);
  const auto ry = buffer_rsrc(A.ys + wrow0, wvalid);

  // ---- loads ---------------------------------------------------------------------------------
  bf16x8 kin[NU / NT], vin[NU / NT], din[NU / NT];
#pragma unroll
  for (int j = 0; j < NU / NT; ++j) {
    kin[j] = rk.unit(tid + j * NT);
    vin[j] = rv.unit(tid + j * NT);
    din[j] = rd.unit(tid + j * NT);
  }
  f32x4 xin[NX4], yin[NX4];  // float4 units u: token u / (D/4), features 4 (u % (D/4)) ..
#pragma unroll
  for (int j = 0; j < NX4; ++j) {
    const uint32_t off = (uint32_t)(tid + j * NT) * 16u;
    xin[j] = buffer_load16<f32x4>(rx, off);
    yin[j] = buffer_load16<f32x4>(ry, off);
  }
  const long long gb = ((long long)b * Tlen + t0) * Hn + h;
  const uint32_t gvalid = (uint32_t)(nv - 1) * Hn * 4u + 4u;
  const auto rg = buffer_rsrc(A.gamma + gb, gvalid);
  const auto rb = buffer_rsrc((A.beta ? A.beta : A.gamma) + gb, gvalid);
  float g_l = buffer_load4f(rg, (uint32_t)lane * Hn * 4u);
  float bt_l = buffer_load4f(rb, (uint32_t)lane * Hn * 4u);
  if (lane >= nv) g_l = 1.0f;
  if (lane >= nv || !A.beta) bt_l = 1.0f;
  // 2 Gam_t E_t H0 k_t of the own token from the solve kernel, accumulator layout
  f32x4 dkh[FT];
  {
    const auto rh = buffer_rsrc(A.dkh + wrow0, wvalid);
    const uint32_t woff = (uint32_t)t * xrow + (uint32_t)lg * 16u;
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) dkh[ft] = buffer_load16<f32x4>(rh, woff + 64u * ft);
  }
  // (c, sigma, k^T H0 k) of token `lane` (zero past the end)
  const auto rt = buffer_rsrc(A.tokv + ((size_t)bh * Tlen + t0) * 4, (uint32_t)nv * 16u);
  const f32x4 tv = buffer_load16<f32x4>(rt, (uint32_t)lane * 16u);
  // the later chunks' gradients (Gs = Gn + Gn^T and Wn: reverse-scan slot N - 1 - ch, fp16 rows
  // with an exponent each) and the start state
  const size_t rslot = (size_t)bh * N + (N - 1 - ch);
  const f16* Gs16 = static_cast<const f16*>(A.rs16) + rslot * 2 * D * D;
  const f16* Wn16 = Gs16 + D * D;
  const float* Gsx = A.rexp + rslot * 2 * D;
  const float* Wnx = Gsx + D;
  const size_t fslot = (size_t)bh * N + ch;
  const f16* H0g = static_cast<const f16*>(A.fs16) + fslot * 2 * D * D;
  const f16* U0g = H0g + D * D;
  const float h0sc = pow2f((int)A.fexp[2 * fslot]), u0sc = pow2f((int)A.fexp[2 * fslot + 1]);
  f32x4 gs[NH4], wn[NH4];
  float sdot = 0.0f, wmx = 0.0f, gmx = 0.0f;  // sdot: <Gn, H0> + <Wn, U0>
  using DG = DDGroups<D>;
#pragma unroll
  for (int j = 0; j < NH4; j += DG::PAIRS ? 2 : 1) {
    const int e4 = DG::e4(tid, j), r = e4 / (D / 4);  // (a pair shares its row)
    const float gsc = pow2f((int)Gsx[r]), wsc = pow2f((int)Wnx[r]);
    f32x4 h0[2], u0[2];
    if constexpr (DG::PAIRS) {
      widen8(Gs16 + 4 * e4, gsc, gs[j], gs[j + 1]);
      widen8(Wn16 + 4 * e4, wsc, wn[j], wn[j + 1]);
      widen8(H0g + 4 * e4, 1.0f, h0[0], h0[1]);
      widen8(U0g + 4 * e4, 1.0f, u0[0], u0[1]);
    } else {
      gs[j] = widen4(Gs16 + 4 * e4, gsc);
      wn[j] = widen4(Wn16 + 4 * e4, wsc);
      h0[0] = widen4(H0g + 4 * e4, 1.0f);
      u0[0] = widen4(U0g + 4 * e4, 1.0f);
    }
#pragma unroll
    for (int h = 0; h < (DG::PAIRS ? 2 : 1); ++h) {
      sdot += 0.5f * h0sc * dot4(gs[j + h], h0[h]) + u0sc * dot4(wn[j + h], u0[h]);
      wmx = fmaxf(wmx, absmax4(wn[j + h]));
      gmx = fmaxf(gmx, absmax4(gs[j + h]));
    }
  }
  {
    float mk = 0.0f, mv = 0.0f, md = 0.0f, mx = 0.0f, my = 0.0f;
#pragma unroll
    for (int j = 0; j < NU / NT; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        mk = fmaxf(mk, fabsf((float)kin[j][i]));
        mv = fmaxf(mv, fabsf((float)vin[j][i]));
        md = fmaxf(md, fabsf((float)din[j][i]));
      }
#pragma unroll
    for (int j = 0; j < NX4; ++j) {
      mx = fmaxf(mx, absmax4(xin[j]));
      my = fmaxf(my, absmax4(yin[j]));
    }
    const float r0 = wave_max(mk), r1 = wave_max(mv), r2 = wave_max(md), r3 = wave_max(mx);
    const float r4 = wave_max(my), r5 = wave_max(gmx), r6 = wave_max(wmx), r7 = wave_sum(sdot);
    if (lane == 0) {
      v_sc[wave] = r0;
      v_sc[4 + wave] = r1;
      v_sc[8 + wave] = r2;
      v_sc[12 + wave] = r3;
      v_sc[16 + wave] = r4;
      v_sc[20 + wave] = r5;
      v_sc[24 + wave] = r6;
      v_sc[28 + wave] = r7;
    }
  }
  // gate prefix, E_t = c_t + gamma_{t+1}^2 E_{t+1} and vs_t = sigma_t + gamma_{t+1} vs_{t+1}
  // (suffix scans: lane l holds token C - 1 - l), every wave
  const float cl = scan_add<kWave>(log2_gate(g_l));
  const float clast = lane_value(cl, C - 1);
  const int tr = C - 1 - lane;
  const float gnext = lane_read(g_l, tr + 1 < C ? tr + 1 : 0);
  float ea = tr + 1 < C ? gnext * gnext : 0.0f, eb = lane_read(tv[0], tr);
  scan_affine(ea, eb);
  float va = tr + 1 < C ? gnext : 0.0f, vb_ = lane_read(tv[1], tr);
  scan_affine(va, vb_);
  if (wave == 0) {
    v_cl[lane] = cl;
    v_bt[lane] = bt_l;
    v_E[tr] = eb;
    v_kh[lane] = tv[2];
  }
  const float vs_t = lane_read(vb_, C - 1 - t);
  __syncthreads();
  float km = v_sc[0], vm = v_sc[4], dm = v_sc[8], xm = v_sc[12], ym = v_sc[16];
  float gsm = v_sc[20], wnm = v_sc[24], Sdot = v_sc[28];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    km = fmaxf(km, v_sc[w]);
    vm = fmaxf(vm, v_sc[4 + w]);
    dm = fmaxf(dm, v_sc[8 + w]);
    xm = fmaxf(xm, v_sc[12 + w]);
    ym = fmaxf(ym, v_sc[16 + w]);
    gsm = fmaxf(gsm, v_sc[20 + w]);
    wnm = fmaxf(wnm, v_sc[24 + w]);
    Sdot += v_sc[28 + w];
  }
  const int ke = pow2_exponent(km, 30), ve = pow2_exponent(vm, 60), de = pow2_exponent(dm, 60);
  const int xe = pow2_exponent(xm, 126), ye = pow2_exponent(ym, 126);
  const int gse = pow2_exponent(gsm, 126), wne = pow2_exponent(wnm, 126);

  // ---- stage K, V, DO, X, Y (fp16, scaled, permuted features) and Gn + Gn^T ----------------
#pragma unroll
  for (int j = 0; j < NU / NT; ++j) {
    const int u = tid + j * NT;
    stage_unit<D>(Kp, u, kin[j], exp2_int(-ke));
    stage_unit<D>(Vp, u, vin[j], exp2_int(-ve));
    stage_unit<D>(Dp, u, din[j], exp2_int(-de));
  }
  {
    const float xi = pow2f(-xe), yi = pow2f(-ye);
#pragma unroll
    for (int j = 0; j < NX4; ++j) {
      const int u = tid + j * NT, tt = u / (D / 4), c4 = u % (D / 4);
      put_row4<D>(Xp, tt, 4 * c4, xin[j] * xi);
      put_row4<D>(Yp, tt, 4 * c4, yin[j] * yi);
    }
    const float gi = pow2f(-gse);
#pragma unroll
    for (int j = 0; j < NH4; ++j) {
      const int e4 = DG::e4(tid, j), r = e4 / (D / 4), c4 = e4 % (D / 4);
      put_row4<D>(Hs, r, 4 * c4, gs[j] * gi);
    }
  }
  lds_barrier();

  // ---- the own token: B fragments, values in the accumulator layout, scalars ---------------
  Frag kb[KD], vbf[KD];
#pragma unroll
  for (int kk = 0; kk < KD; ++kk) {
    kb[kk] = *reinterpret_cast<const Frag*>(Kp + tix<D>(t, 32 * kk + 8 * lg));
    vbf[kk] = *reinterpret_cast<const Frag*>(Vp + tix<D>(t, 32 * kk + 8 * lg));
  }
  f32x4 kv[FT], vv[FT];  // k_t, v_t [16 ft + 4 lg + i]
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) {
    kv[ft] = row4<D>(Kp, t, 16 * ft + 4 * lg) * exp2_int(ke);
    vv[ft] = row4<D>(Vp, t, 16 * ft + 4 * lg) * exp2_int(ve);
  }
  const float cl_t = v_cl[t], clp = t > 0 ? v_cl[t - 1] : 0.0f;
  const float e_t = fast_exp2(fminf(clast - cl_t, 0.0f));
  const float gE_t = fast_exp2(cl_t) * v_E[t];  // Gam_t E_t
  const float bt_t = v_bt[t];

  // ---- products with the later chunks' gradients, one D x D operand at a time --------------
  f32x4 dk[FT], dv[FT];  // dk, dv of the own token before the beta_t factor
  float nx = 0.0f;
  auto dd_product = [&](const Frag(&bf)[KD], f32x4(&acc)[FT]) {
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) acc[ft] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KD; ++kk)
#pragma unroll
      for (int ft = 0; ft < FT; ++ft)
        acc[ft] = M::mma(*reinterpret_cast<const Frag*>(Hs + tix<D>(16 * ft + lr, 32 * kk + 8 * lg)),
                         bf[kk], acc[ft]);
  };
  {
    f32x4 p[FT];
    dd_product(kb, p);  // Gs k_t
    const float sc = pow2f(gse + ke);
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) {
      dk[ft] = p[ft] * (e_t * sc);
      nx += 0.5f * sc * dot4(p[ft], kv[ft]);
    }
  }
  lds_barrier();
  {
    const float wi = pow2f(-wne);
#pragma unroll
    for (int j = 0; j < NH4; ++j) {  // Wn, row-major (from the registers of the first load)
      const int e4 = DG::e4(tid, j), r = e4 / (D / 4), c4 = e4 % (D / 4);
      put_row4<D>(Hs, r, 4 * c4, wn[j] * wi);
    }
  }
  lds_barrier();
  {
    // Wn k_t from row fragments, Wn^T v_t from transposing reads of the same rows
    f32x4 p[FT], pt[FT];
    dd_product(kb, p);
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) pt[ft] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KD; ++kk)
#pragma unroll
      for (int ft = 0; ft < FT; ++ft)
        pt[ft] = M::mma(frag_trans<LDD>(Hs, 32 * kk + 4 * lg, 32 * kk + 16 + 4 * lg,
                                        pcol(16 * ft + 4 * (lr & 3)), lr, tix_trans<D>(lg, lr)),
                        vbf[kk], pt[ft]);
    const float sc = pow2f(wne + ke), sct = pow2f(wne + ve);
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) {
      dv[ft] = p[ft] * (e_t * sc);
      nx += sc * dot4(p[ft], vv[ft]);
      dk[ft] += pt[ft] * (e_t * sct) + dkh[ft];
    }
  }
  nx = group_sum(nx, lane);
  if (lg == 0) v_nx[t] = nx;

  // ---- token-pair products of the own column t ---------------------------------------------
  //   pKX[u] = x_u . k_t, pKY[u] = y_u . k_t, pVD[u] = do_u . v_t, pKK[s] = k_s . k_t
  // (rows u, s = 16 sb + 4 lg + i of the accumulator tiles; staged operands)
  Frag pf1[KC], pf2[KC], pf3[KC], pf4[KC];
  int fk, fv;
  {
    f32x4 pKX[ST], pKY[ST], pVD[ST], pKK[ST];
#pragma unroll
    for (int sb = 0; sb < ST; ++sb) {
      pKX[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
      pKY[sb] = pKX[sb];
      pVD[sb] = pKX[sb];
      pKK[sb] = pKX[sb];
    }
#pragma unroll
    for (int kk = 0; kk < KD; ++kk)
#pragma unroll
      for (int sb = 0; sb < ST; ++sb) {
        const int ro = tix<D>(16 * sb + lr, 32 * kk + 8 * lg);
        pKX[sb] = M::mma(*reinterpret_cast<const Frag*>(Xp + ro), kb[kk], pKX[sb]);
        pKY[sb] = M::mma(*reinterpret_cast<const Frag*>(Yp + ro), kb[kk], pKY[sb]);
        pVD[sb] = M::mma(*reinterpret_cast<const Frag*>(Dp + ro), vbf[kk], pVD[sb]);
        pKK[sb] = M::mma(*reinterpret_cast<const Frag*>(Kp + ro), kb[kk], pKK[sb]);
      }
    // B operands in true units times the A operand's scale:
    //   b1 = -Dm KX 2^ye (A = Y^T), b2 = Dm (VD - KY) 2^xe (A = X^T), b3 = 2 ME beta KK 2^ke
    //   (A = K^T), b4 = Dm KX 2^de (A = DO^T, for dv)
    const float sKX = pow2f(xe + ke), sKY = pow2f(ye + ke), sVD = pow2f(de + ve);
    const float sKK = exp2_int(2 * ke);
    const float f1 = -pow2f(ye), f2 = pow2f(xe), f3 = 2.0f * exp2_int(ke), f4 = pow2f(de);
    float mk4 = 0.0f, mv4 = 0.0f;
#pragma unroll
    for (int sb = 0; sb < ST; ++sb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int u = 16 * sb + 4 * lg + i;
        const float clu = v_cl[u];
        const float dmk = u >= t ? fast_exp2(fminf(clu - cl_t, 0.0f)) : 0.0f;
        const int m = u > t ? u : t;
        const float me = fast_exp2(fminf(2.0f * v_cl[m] - cl_t - clu, 0.0f)) * v_E[m];
        const float kx = pKX[sb][i] * sKX, ky = pKY[sb][i] * sKY, vd = pVD[sb][i] * sVD;
        const float kk2 = pKK[sb][i];
        // (k's . k't)^2 / (4D)^2 < 1 for the interaction sums of dgamma
        const float kn = kk2 * (1.0f / (4.0f * D));
        K2s[u * LDP + t] = (f16)(kn * kn);
        pKX[sb][i] = dmk * kx * f1;
        pKY[sb][i] = dmk * (vd - ky) * f2;
        pKK[sb][i] = me * v_bt[u] * (kk2 * sKK) * f3;
        pVD[sb][i] = dmk * kx * f4;
        mk4 = fmaxf(mk4, fmaxf(fabsf(pKX[sb][i]), fmaxf(fabsf(pKY[sb][i]), fabsf(pKK[sb][i]))));
        mv4 = fmaxf(mv4, fabsf(pVD[sb][i]));
      }
    fk = pow2_exponent(group_max(mk4, lane), 126);
    fv = pow2_exponent(group_max(mv4, lane), 126);
    const float ik = pow2f(-fk), iv = pow2f(-fv);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      pf1[kc] = pack8(pKX[2 * kc] * ik, pKX[2 * kc + 1] * ik);
      pf2[kc] = pack8(pKY[2 * kc] * ik, pKY[2 * kc + 1] * ik);
      pf3[kc] = pack8(pKK[2 * kc] * ik, pKK[2 * kc + 1] * ik);
      pf4[kc] = pack8(pVD[2 * kc] * iv, pVD[2 * kc + 1] * iv);
    }
  }
  // ---- dk, dv: Y^T b1 + X^T b2 + K^T b3 and DO^T b4 over the permuted tokens -----------------
  {
    f32x4 ak[FT], av[FT];
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) {
      ak[ft] = f32x4{0.f, 0.f, 0.f, 0.f};
      av[ft] = ak[ft];
    }
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int s0 = 32 * kc + 4 * lg, s1 = s0 + 16;
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) {
        const int co = pcol(16 * ft + 4 * (lr & 3));
        ak[ft] = M::mma(frag_trans<LDD>(Yp, s0, s1, co, lr, tix_trans<D>(lg, lr)), pf1[kc], ak[ft]);
        ak[ft] = M::mma(frag_trans<LDD>(Xp, s0, s1, co, lr, tix_trans<D>(lg, lr)), pf2[kc], ak[ft]);
        ak[ft] = M::mma(frag_trans<LDD>(Kp, s0, s1, co, lr, tix_trans<D>(lg, lr)), pf3[kc], ak[ft]);
        av[ft] = M::mma(frag_trans<LDD>(Dp, s0, s1, co, lr, tix_trans<D>(lg, lr)), pf4[kc], av[ft]);
      }
    }
    const float sk = pow2f(fk), sv = pow2f(fv);
    float db = 0.0f;
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) {
      dk[ft] += ak[ft] * sk;
      dv[ft] += av[ft] * sv;
      db += dot4(kv[ft], dk[ft]) + dot4(vv[ft], dv[ft]);
    }
    db = 0.5f * group_sum(db, lane);
    const auto rdk = buffer_rsrc(static_cast<bf16*>(A.dk) + row0,
                                 (uint32_t)(nv - 1) * tok_bytes + D * 2u);
    const auto rdv = buffer_rsrc(static_cast<bf16*>(A.dv) + row0,
                                 (uint32_t)(nv - 1) * tok_bytes + D * 2u);
    const uint32_t ooff = (uint32_t)t * tok_bytes + (uint32_t)lg * 8u;
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) {
      const f32x4 a = dk[ft] * bt_t, c = dv[ft] * bt_t;
      buffer_store8(bf16x4{(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3]}, rdk, ooff + 32u * ft);
      buffer_store8(bf16x4{(bf16)c[0], (bf16)c[1], (bf16)c[2], (bf16)c[3]}, rdv, ooff + 32u * ft);
    }
    if (lg == 0 && t < nv && A.dbeta) A.dbeta[((long long)b * Tlen + t0 + t) * Hn + h] = db;
  }

  // ---- P1[s][u] = (v_s . do_u - k_s . y_u) (k_s . x_u) of the own column u = t -------------
  f32x4 p1[ST];
  {
    Frag dbf[KD], xbf[KD], ybf[KD];
#pragma unroll
    for (int kk = 0; kk < KD; ++kk) {
      dbf[kk] = *reinterpret_cast<const Frag*>(Dp + tix<D>(t, 32 * kk + 8 * lg));
      xbf[kk] = *reinterpret_cast<const Frag*>(Xp + tix<D>(t, 32 * kk + 8 * lg));
      ybf[kk] = *reinterpret_cast<const Frag*>(Yp + tix<D>(t, 32 * kk + 8 * lg));
    }
    f32x4 a1[ST], a2[ST];
#pragma unroll
    for (int sb = 0; sb < ST; ++sb) {
      p1[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
      a1[sb] = p1[sb];
      a2[sb] = p1[sb];
    }
#pragma unroll
    for (int kk = 0; kk < KD; ++kk)
#pragma unroll
      for (int sb = 0; sb < ST; ++sb) {
        const int ro = tix<D>(16 * sb + lr, 32 * kk + 8 * lg);
        const Frag kf = *reinterpret_cast<const Frag*>(Kp + ro);
        a1[sb] = M::mma(*reinterpret_cast<const Frag*>(Vp + ro), dbf[kk], a1[sb]);
        a2[sb] = M::mma(kf, ybf[kk], a2[sb]);
        p1[sb] = M::mma(kf, xbf[kk], p1[sb]);
      }
    const float sVD = pow2f(ve + de), sKY = pow2f(ke + ye), sKX = pow2f(ke + xe);
    float mp = 0.0f;
#pragma unroll
    for (int sb = 0; sb < ST; ++sb) {
      p1[sb] = (a1[sb] * sVD - a2[sb] * sKY) * (p1[sb] * sKX);
      mp = fmaxf(mp, absmax4(p1[sb]));
    }
    mp = wave_max(mp);
    if (lane == 0) v_sc[32 + wave] = mp;
  }
  lds_barrier();  // P1 maxima, v_nx and K2s of every column
  const int p1e = pow2_exponent(fmaxf(fmaxf(v_sc[32], v_sc[33]), fmaxf(v_sc[34], v_sc[35])), 126);
  {
    const float pi = pow2f(-p1e);
#pragma unroll
    for (int sb = 0; sb < ST; ++sb)
#pragma unroll
      for (int i = 0; i < 4; ++i) P1s[(16 * sb + 4 * lg + i) * LDP + t] = (f16)(p1[sb][i] * pi);
  }
  lds_barrier();

  // ---- Z[s][t] and dgamma_t --------------------------------------------------------------------
  //   Z1 = sum_u P1[s][u] Dm[t][u], Z2 = sum_s' K2[s][s'] beta_s' ME[t][s'] (k-slots j of lane
  //   group lg: token 32 kc + 8 lg + j, the order of the staged rows)
  {
    Frag bz1[KC], bz2[KC];
    float b2v[KC][8];
    float mz = 0.0f;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int u = 32 * kc + 8 * lg + j;
        const float clu = v_cl[u];
        bz1[kc][j] = (f16)(u >= t ? fast_exp2(fminf(clu - cl_t, 0.0f)) : 0.0f);
        const int m = u > t ? u : t;
        const float me = fast_exp2(fminf(2.0f * v_cl[m] - cl_t - clu, 0.0f)) * v_E[m];
        b2v[kc][j] = me * v_bt[u];
        mz = fmaxf(mz, fabsf(b2v[kc][j]));
      }
    const int fe = pow2_exponent(group_max(mz, lane), 126);
    const float fi = pow2f(-fe);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
      for (int j = 0; j < 8; ++j) bz2[kc][j] = (f16)(b2v[kc][j] * fi);
    f32x4 z1[ST], z2[ST];
#pragma unroll
    for (int sb = 0; sb < ST; ++sb) {
      z1[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
      z2[sb] = z1[sb];
    }
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
      for (int sb = 0; sb < ST; ++sb) {
        const int ro = (16 * sb + lr) * LDP + 32 * kc + 8 * lg;
        z1[sb] = M::mma(*reinterpret_cast<const Frag*>(P1s + ro), bz1[kc], z1[sb]);
        z2[sb] = M::mma(*reinterpret_cast<const Frag*>(K2s + ro), bz2[kc], z2[sb]);
      }
    const float s1 = pow2f(p1e);
    const float s2 = pow2f(fe + 4 * ke) * (16.0f * D * D);
    float dg = 0.0f;
#pragma unroll
    for (int sb = 0; sb < ST; ++sb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = 16 * sb + 4 * lg + i;
        const float z = z1[sb][i] * s1 + z2[sb][i] * s2 + gE_t * v_kh[s] + e_t * v_nx[s];
        const float w = fast_exp2(fminf(clp - v_cl[s], 0.0f)) * v_bt[s];
        dg += s < t ? w * z : 0.0f;
      }
    dg = group_sum(dg, lane) + fast_exp2(clp) * (vs_t + e_t * Sdot);
    if (lg == 0 && t < nv) A.dgamma[((long long)b * Tlen + t0 + t) * Hn + h] = dg;
  }
}

// ============================================================================================
// The chunks' incoming gradients: the segment scan over the chunks in reverse order (slot N - 1 -
// c holds chunk c's dG + dG^T and dW, float32; log2g its gate product), the running sum in
// float32 per thread, each start state written as fp16 rows, row r times 2^-e_r (e_r from the
// row's largest element, in oexp). Thread e4 holds elements 4 e4 .. 4 e4 + 3 of both matrices;
// the D / 4 lanes of a row share its exponent.
// ============================================================================================
template <int D>
__global__ __launch_bounds__(256) void bwd_rscan_kernel(const f16* __restrict__ st,
                                                        const signed char* __restrict__ stx,
                                                        const float* __restrict__ log2g,
                                                        f16* __restrict__ out,
                                                        float* __restrict__ oexp, int N) {
  constexpr int DD = D * D, G = D / 4, NB = D / 16;
  static_assert((DD / 4) % 256 == 0 && kWave % G == 0, "rows within waves");
  const int bh = blockIdx.y;
  const int e4 = blockIdx.x * 256 + threadIdx.x;
  const int lane = threadIdx.x % kWave, r = e4 / G, blk = (e4 % G) / 4;
  f32x4 sh = {0.f, 0.f, 0.f, 0.f}, su = sh;
  auto put = [&](f32x4 x, size_t slot, int mat) {
    float m = absmax4(x);
#pragma unroll
    for (int k = 1; k < G; k <<= 1) m = fmaxf(m, lane_read(m, lane ^ k));
    const int e = pow2_exponent(m, 126);
    const f32x4 y = x * pow2f(-e);
    *reinterpret_cast<f16x4*>(out + slot * 2 * DD + (size_t)mat * DD + 4 * e4) =
        f16x4{(f16)y[0], (f16)y[1], (f16)y[2], (f16)y[3]};
    if (lane % G == 0) oexp[slot * 2 * D + (size_t)mat * D + r] = (float)e;
  };
  // a slot's two chunk gradients (fp16 with a power of two per 16 columns of a row) and gate;
  // loaded one slot ahead of their use. The last slot has none (chunk 0): its index is clamped
  // to the one before (to slot 0 with a single chunk), whose values are loaded and not used.
  struct Src {
    f16x4 h, u;
    signed char xh, xu;
    float lg2;
  };
  auto load = [&](int s) {
    const size_t slot = (size_t)bh * N + max(min(s, N - 2), 0);
    Src v;
    v.h = reinterpret_cast<const f16x4*>(st + slot * 2 * DD)[e4];
    v.u = reinterpret_cast<const f16x4*>(st + slot * 2 * DD + DD)[e4];
    v.xh = stx[slot * 2 * D * NB + r * NB + blk];
    v.xu = stx[slot * 2 * D * NB + D * NB + r * NB + blk];
    v.lg2 = log2g[slot];
    return v;
  };
  auto widen = [](f16x4 x, signed char e) {
    const float sc = pow2f((int)e);
    return f32x4{(float)x[0] * sc, (float)x[1] * sc, (float)x[2] * sc, (float)x[3] * sc};
  };
  Src cur = load(0);
  for (int s = 0; s < N; ++s) {
    const size_t slot = (size_t)bh * N + s;
    const Src nxt = load(s + 1);
    put(sh, slot, 0);
    put(su, slot, 1);
    if (s + 1 < N) {  // the last slot has no summary
      const float g = exp2f(cur.lg2);
      sh = g * sh + widen(cur.h, cur.xh);
      su = g * su + widen(cur.u, cur.xu);
    }
    cur = nxt;
  }
}

// ============================================================================================
// Every chunk's start state: a walk over the chunks of each (segment, head) of the forward's
// segment plan, from the segment's start state, writing the state at every chunk start. Per
// chunk H <- Gam_C H + K^T diag(w) K and U^T <- Gam_C U^T + K^T diag(w) V, w_s = 2^(l_{C-1} -
// l_s) beta_s, with (w K)^T split into fp16 hi + lo (float32-accurate products). Wave w holds
// the float32 tiles q = w TPW .. of H and U^T in registers (tile (a, b): H[16a + 4lg + i][16b +
// lr] in a lane; U^T likewise, so that the lane's four values are a row segment of U).
// ============================================================================================
template <int D>
__global__ __launch_bounds__(256) void bwd_states_kernel(BwdArgs A, int Tlen, int Hn, int N,
                                                         int J, const float* seg_states, int S) {
  using Cfg = BwdCfg<D>;
  using M = Mma<f16>;
  typedef f16x8 Frag;
  constexpr int C = Cfg::C, NW = Cfg::NW, NT = Cfg::NT, FT = Cfg::FT, KC = Cfg::KC;
  constexpr int LDD = Cfg::LDD, NU = Cfg::NU, TPW = Cfg::TPW;
  __shared__ __attribute__((aligned(16))) f16 Kp[C * LDD];
  __shared__ __attribute__((aligned(16))) f16 Vp[C * LDD];
  __shared__ __attribute__((aligned(16))) float v_w[C];
  __shared__ float v_sc[2 * NW];
  __shared__ float v_sm[2 * NW];  // the state's maxima per wave

  const int seg = blockIdx.x, bh = blockIdx.y;
  const int b = bh / Hn, h = bh % Hn;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int lr = lane % 16, lg = lane / 16;
  const int c_begin = seg * J, c_end = min(N, c_begin + J);
  if (c_begin >= c_end) return;

  f32x4 Ht[TPW], Ut[TPW];
  {
    const float* st = seg_states + ((size_t)bh * S + seg) * 2 * D * D;
#pragma unroll
    for (int q = 0; q < TPW; ++q) {
      const int tile = wave * TPW + q, a = tile / FT, bq = tile % FT;
      const size_t o = (size_t)(16 * bq + lr) * D + 16 * a + 4 * lg;
      Ht[q] = *reinterpret_cast<const f32x4*>(st + o);          // H symmetric
      Ut[q] = *reinterpret_cast<const f32x4*>(st + D * D + o);  // U[16bq + lr][16a + 4lg ..]
    }
  }
  // Rows and gates of two chunks in flight: set q holds chunk c_begin + q + 2 i. A chunk's loads
  // are issued right after the chunk two before it is staged, so that a whole chunk's work
  // covers their latency. Chunks past the segment's last one load empty ranges.
  bf16x8 kin[2][NU / NT], vin[2][NU / NT];
  float g_l[2] = {1.0f, 1.0f}, bt_l[2] = {1.0f, 1.0f};  // past the end of the sequence: 0 as loaded
  int nv_l[2] = {0, 0};                                   // valid rows of the loaded chunk
  auto load = [&](int c, auto Q) __attribute__((always_inline)) {
    constexpr int q = decltype(Q)::value;
    const int t0 = c * C, nv = c < c_end ? min(C, Tlen - t0) : 0;
    const long long row0 = ((long long)b * Tlen + t0) * Hn * D + (long long)h * D;
    const ChunkRows<D> rk(A.k, row0, nv, Hn), rv(A.v, row0, nv, Hn);
#pragma unroll
    for (int j = 0; j < NU / NT; ++j) {
      kin[q][j] = rk.unit(tid + j * NT);
      vin[q][j] = rv.unit(tid + j * NT);
    }
    const long long gb = ((long long)b * Tlen + t0) * Hn + h;
    const uint32_t gvalid = nv > 0 ? (uint32_t)(nv - 1) * Hn * 4u + 4u : 0u;
    // (the write gates are read from the gates when there are none: an unconditional load, so
    // that the compiler counts the loads in flight exactly; rows past the end get gate 1 where
    // the values are used, so that nothing waits for these loads here)
    g_l[q] = buffer_load4f(buffer_rsrc(A.gamma + gb, gvalid), (uint32_t)lane * Hn * 4u);
    bt_l[q] = buffer_load4f(buffer_rsrc((A.beta ? A.beta : A.gamma) + gb, gvalid),
                            (uint32_t)lane * Hn * 4u);
    nv_l[q] = nv;
  };
  // the start state of chunk c, from the tiles: fp16, each matrix times 2^-e (e from its
  // largest element, over the four waves)
  auto store_state = [&](int c) __attribute__((always_inline)) {
    float mh = 0.0f, mu = 0.0f;
#pragma unroll
    for (int q = 0; q < TPW; ++q) {
      mh = fmaxf(mh, absmax4(Ht[q]));
      mu = fmaxf(mu, absmax4(Ut[q]));
    }
    mh = wave_max(mh);
    mu = wave_max(mu);
    if (lane == 0) {
      v_sm[wave] = mh;
      v_sm[NW + wave] = mu;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      mh = fmaxf(mh, v_sm[w]);
      mu = fmaxf(mu, v_sm[NW + w]);
    }
    __syncthreads();  // v_sm is read before the next state's maxima are written
    const int eh = pow2_exponent(mh, 126), eu = pow2_exponent(mu, 126);
    const float ih = pow2f(-eh), iu = pow2f(-eu);
    const size_t slot = (size_t)bh * N + c;
    f16* out = static_cast<f16*>(A.fs16) + slot * 2 * D * D;
#pragma unroll
    for (int q = 0; q < TPW; ++q) {
      const int tile = wave * TPW + q, a = tile / FT, bq = tile % FT;
      const size_t o = (size_t)(16 * bq + lr) * D + 16 * a + 4 * lg;
      const f32x4 x = Ht[q] * ih, y = Ut[q] * iu;
      *reinterpret_cast<f16x4*>(out + o) = f16x4{(f16)x[0], (f16)x[1], (f16)x[2], (f16)x[3]};
      *reinterpret_cast<f16x4*>(out + D * D + o) = f16x4{(f16)y[0], (f16)y[1], (f16)y[2], (f16)y[3]};
    }
    if (tid == 0) {
      A.fexp[2 * slot] = (float)eh;
      A.fexp[2 * slot + 1] = (float)eu;
    }
  };
  // Per chunk with a successor in the segment: stage the rows loaded before, issue the loads of
  // the chunk two ahead into the freed register set, then the state stores (after the loads, so
  // that waiting for the loads does not wait for the stores), then the products. The segment's
  // last chunk only stores its start state (the next segment starts from the scan).
  auto step = [&](int c, auto Q) __attribute__((always_inline)) {
    constexpr int set = decltype(Q)::value;
    // scales of the chunk, gate prefix and carry weights
    float mk = 0.0f, mv = 0.0f;
#pragma unroll
    for (int j = 0; j < NU / NT; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        mk = fmaxf(mk, fabsf((float)kin[set][j][i]));
        mv = fmaxf(mv, fabsf((float)vin[set][j][i]));
      }
    mk = wave_max(mk);
    mv = wave_max(mv);
    const bool valid = lane < nv_l[set];
    const float gv = valid ? g_l[set] : 1.0f, bv = valid && A.beta ? bt_l[set] : 1.0f;
    const float cl = scan_add<kWave>(log2_gate(gv));
    const float clast = lane_value(cl, C - 1);
    __syncthreads();  // the previous chunk's products have read Kp, Vp, v_w
    if (lane == 0) {
      v_sc[wave] = mk;
      v_sc[NW + wave] = mv;
    }
    if (wave == 0) v_w[lane] = fast_exp2(fminf(clast - cl, 0.0f)) * bv;
    __syncthreads();
    float km = v_sc[0], vm = v_sc[NW];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      km = fmaxf(km, v_sc[w]);
      vm = fmaxf(vm, v_sc[NW + w]);
    }
    const int ke = pow2_exponent(km, 30), ve = pow2_exponent(vm, 60);
#pragma unroll
    for (int j = 0; j < NU / NT; ++j) {
      stage_unit<D>(Kp, tid + j * NT, kin[set][j], exp2_int(-ke));
      stage_unit<D>(Vp, tid + j * NT, vin[set][j], exp2_int(-ve));
    }
    lds_barrier();
    load(c + 2, Q);  // the rows of the chunk two ahead, in flight during the next two chunks
    store_state(c);
    const float gC = fast_exp2(clast);
    const float sh = exp2_int(2 * ke), su = exp2_int(ke + ve);
    // The wave's tiles q = r NC + c: NR row tiles (the A operands (w K)^T, split hi + lo once
    // per chunk) by NC column tiles (the K and V fragments of a column read once for its rows)
    constexpr int NR = TPW >= FT ? TPW / FT : 1, NC = TPW / NR;
    const int xt = tix_trans<D>(lg, lr);
    Frag awh[NR][KC], awl[NR][KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int s0 = 32 * kc + 4 * lg, s1 = s0 + 16;
      const f32x4 w0 = *reinterpret_cast<const f32x4*>(v_w + s0);
      const f32x4 w1 = *reinterpret_cast<const f32x4*>(v_w + s1);
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const int a = (wave * TPW + r * NC) / FT;
        const Frag ka = frag_trans<LDD>(Kp, s0, s1, pcol(16 * a + 4 * (lr & 3)), lr, xt);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float x = (float)ka[j] * (j < 4 ? w0[j] : w1[j - 4]);
          awh[r][kc][j] = (f16)x;
          awl[r][kc][j] = (f16)(x - (float)awh[r][kc][j]);
        }
      }
    }
#pragma unroll
    for (int cq = 0; cq < NC; ++cq) {
      const int bq = (wave * TPW + cq) % FT;
      f32x4 ah[NR], au[NR];
#pragma unroll
      for (int r = 0; r < NR; ++r) ah[r] = au[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const int s0 = 32 * kc + 4 * lg, s1 = s0 + 16;
        const Frag kbf = frag_trans<LDD>(Kp, s0, s1, pcol(16 * bq + 4 * (lr & 3)), lr, xt);
        const Frag vbf = frag_trans<LDD>(Vp, s0, s1, pcol(16 * bq + 4 * (lr & 3)), lr, xt);
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          ah[r] = M::mma(awh[r][kc], kbf, ah[r]);
          ah[r] = M::mma(awl[r][kc], kbf, ah[r]);
          au[r] = M::mma(awh[r][kc], vbf, au[r]);
          au[r] = M::mma(awl[r][kc], vbf, au[r]);
        }
      }
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const int q = r * NC + cq;
        Ht[q] = Ht[q] * gC + ah[r] * sh;
        Ut[q] = Ut[q] * gC + au[r] * su;
      }
    }
  };
  load(c_begin, IC<0>{});
  load(c_begin + 1, IC<1>{});
  int c = c_begin;
  for (; c + 2 < c_end; c += 2) {
    step(c, IC<0>{});
    step(c + 1, IC<1>{});
  }
  if (c + 1 < c_end) {
    step(c, IC<0>{});
    ++c;
  }
  store_state(c_end - 1);
}

template <int D>
hipError_t launch_bwd_tok_t(const FwdPlan& pl, const BwdArgs& a, const ChebConsts& cc,
                            hipStream_t stream) {
  using Cfg = BwdCfg<D>;
  const dim3 grid(pl.N, pl.B * pl.H);
  auto ks = bwd_solve_kernel<D>;
  static std::atomic<uint64_t> lds_a{0};
  hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(ks), (int)Cfg::aBytes, lds_a);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ks, grid, dim3(Cfg::NT), Cfg::aBytes, stream, a, pl.T, pl.H, pl.N, cc);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // every chunk's incoming gradients: the segment scan over the chunks in reverse order
  hipLaunchKernelGGL(bwd_rscan_kernel<D>, dim3(D * D / 4 / 256, pl.B * pl.H), dim3(256), 0,
                     stream, static_cast<const f16*>(a.rd16), a.rdx, a.rlog2,
                     static_cast<f16*>(a.rs16), a.rexp, pl.N);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  auto kg = bwd_grad_kernel<D>;
  static std::atomic<uint64_t> lds_g{0};
  if ((e = ensure_dynamic_lds(reinterpret_cast<const void*>(kg), (int)Cfg::gBytes, lds_g)) !=
      hipSuccess)
    return e;
  hipLaunchKernelGGL(kg, grid, dim3(Cfg::NT), Cfg::gBytes, stream, a, pl.T, pl.H, pl.N);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_states(const FwdPlan& ps, const BwdArgs& a, const float* seg_states,
                             hipStream_t stream) {
  const dim3 grid(ps.S, ps.B * ps.H);
  const int N = ps.N;
  switch (ps.D) {
    case 32:
      hipLaunchKernelGGL(bwd_states_kernel<32>, grid, dim3(256), 0, stream, a, ps.T, ps.H, N,
                         ps.J, seg_states, ps.S);
      return hipGetLastError();
    case 64:
      hipLaunchKernelGGL(bwd_states_kernel<64>, grid, dim3(256), 0, stream, a, ps.T, ps.H, N,
                         ps.J, seg_states, ps.S);
      return hipGetLastError();
    case 128:
      hipLaunchKernelGGL(bwd_states_kernel<128>, grid, dim3(256), 0, stream, a, ps.T, ps.H, N,
                         ps.J, seg_states, ps.S);
      return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

bool bwd_tok_supported(const FwdPlan& pl) {
  const long long chunk_bytes = 64LL * pl.H * pl.D * 2;
  const long long ws_rows = (long long)pl.T * pl.D * 4;  // float32 workspace rows of one head
  return pl.dtype == 0 && pl.C == 64 && (pl.D == 32 || pl.D == 64 || pl.D == 128) &&
         chunk_bytes < (1LL << 31) && ws_rows < (1LL << 31);
}

hipError_t launch_bwd_tok(const FwdPlan& pl, const BwdArgs& a, const ChebConsts& cc,
                          hipStream_t stream) {
  switch (pl.D) {
    case 32: return launch_bwd_tok_t<32>(pl, a, cc, stream);
    case 64: return launch_bwd_tok_t<64>(pl, a, cc, stream);
    case 128: return launch_bwd_tok_t<128>(pl, a, cc, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace gka
