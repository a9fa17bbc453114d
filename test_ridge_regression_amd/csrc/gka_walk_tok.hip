// Chunk walk of gka_fwd_chunked with token-owning waves (bf16 inputs, chunks of 64 tokens): the
// key-side recurrence and the Chebyshev solves. The value side (o_t = U_t x_t and the carry of U)
// is the output pass of gka_out.hip, which reads the solves this walk leaves in o's rows.
//
// The chunk algebra follows "Methodology in Plain English" and "Key Contributions" 3 on the
// ai.info summary of arXiv 2511.21016: per chunk,
//   Y_t   = s_t H0hat R_t + sum_{s<=t} Mhat_ts (k_s . R_t) k_s    (the system minus a I, on R_t)
//   n_t^2 = gamma_t^2 n_{t-1}^2 + 2 gamma_t beta_t k_t^T H_{t-1} k_t + beta_t^2 ||k_t||^4
//           (an affine scan over t)
//   carry H <- Gam_C H + K^T diag(w) K
// with H0hat = H0 / n0, s_t = Gam_t n0 / n_t, Mhat_ts = 2^(cl_t - cl_s) beta_s / n_t and carry
// weights w_s = 2^(cl_C - cl_s) beta_s. beta_t is the optional write gate ("Main Findings" on the
// ai.info summary: H_t = gamma_t H_{t-1} + beta_t k_t k_t^T; 1 without it); it enters only
// through these weights, so the key rows stay exact operands.
//
// Every token's Chebyshev iteration is a system of its own: Y_t needs R_t and the chunk's
// shared matrices (H0hat, K), nothing of the other tokens' iterates. Wave w (one per SIMD)
// therefore owns the 16 tokens 16w..16w+15 and all D features of them, and runs the whole
// Chebyshev loop without exchanging anything with the other waves: the iterate stays in
// matrix-core accumulators and is fed back as the B operand of the next products directly.
//
// For that the reduction index of a product over features (or tokens) is taken in a permuted
// order within each block of 32: k-slot j of lane group g (slots 8g..8g+7 of the block) stands
// for index 16 (j / 4) + 4 g + j % 4. The accumulator of a 16x16 output tile holds, in lane
// (column c, group g), rows 4g..4g+3; with this order the B fragment of block kk of a
// feature x token matrix is the accumulator rows of tiles 2kk and 2kk+1 of the same lane.
// The A operands are laid out to match: K and H0hat are staged in LDS with their feature columns
// permuted the same way (a fragment is one 16-byte read), and K^T fragments in the permuted token
// order come from transposing LDS reads.
//
// Range of the 16-bit operands: the keys of a chunk are staged times 2^-e (e from the chunk's
// largest |k|, so the staged rows lie below 2) and the queries of a token times 2^-e_t; both are
// exact powers of two, undone in float32 where the products are used (norm terms, mask, carry
// weights) or carried into the solve's own scale. Any bf16 input whose squares stay in float32's
// range is therefore an fp16 operand of full precision.
//
// Per chunk: stage K (fp16), gates and H0hat; the norm phase (k_t^T H0hat k_t from the resident
// H0hat fragments, the Gram tiles of the own tokens) and a scan over the 64 tokens; the carry
// advances the float32 H state (held as accumulator tiles, a quarter per wave); the next chunk's
// keys and gates are loaded into registers; the Chebyshev loop; the solve of every token is
// written, scaled to lie below 2 in magnitude, as fp16 to its row of o, with its scale over
// ||H_t||_F in a per-token float.
#include "gka_internal.hpp"

#include <type_traits>

namespace gka {
namespace {

template <int D>
struct TokCfg {
  static constexpr int C = 64;               // tokens per chunk
  static constexpr int NW = 4;               // waves: one per SIMD
  static constexpr int NT = NW * kWave;
  static constexpr int FT = D / 16;          // feature tiles
  static constexpr int KD = D / 32;          // 32-deep blocks over the features
  static constexpr int KC = C / 32;          // 32-deep blocks over the tokens
  static constexpr int ST = C / 16;          // token (s) tiles
  static constexpr int NST = FT * FT / NW;   // state tiles per wave
  static constexpr int NRT = NST >= FT ? NST / FT : 1;  // state row tiles per wave
  static constexpr int NCT = NST >= FT ? FT : NST;      // state column tiles per wave
  static constexpr int LDD = D + 8;          // row stride of the [*][D] fp16 tiles
  static constexpr bool PIN = D >= 128;      // resident fragments and state in AGPRs
  static constexpr int VEC = 8;              // bf16 elements per 16-byte unit
  static constexpr int UPR = D / VEC;        // units per token row
  static constexpr int NU = C * UPR;         // units per matrix
  static constexpr size_t szTok = (size_t)C * LDD * 2;
  static constexpr size_t szHs = (size_t)D * LDD * 2;
  static constexpr size_t oKp = 0;               // K, token-major, permuted features (fp16)
  static constexpr size_t oHs = oKp + szTok;     // H0hat: row-major, permuted columns (fp16)
  static constexpr size_t oKraw = oHs + szHs;    // the next chunk's key rows as loaded (bf16)
  static constexpr size_t oGraw = oKraw + (size_t)C * D * 2;  // its gates, write gates [C]
  static constexpr size_t oVec = oGraw + (size_t)2 * C * sizeof(float);
  static constexpr size_t szVec = (size_t)(5 * C + 16 + 4 * 64) * sizeof(float);
  static constexpr size_t bytes = oVec + szVec;  // dynamic LDS
  static_assert(D % 32 == 0 && NST >= 1, "unsupported D");
  static_assert(NU % NT == 0, "staging units must fill whole workgroups");
  static_assert(bytes <= 160 * 1024, "LDS budget of one CU exceeded");
};

// column of logical feature d in a permuted row: within each block of 32, the four-element
// group 4g + 16h (g = 0..3, h = 0, 1) sits at 8g + 4h
__device__ constexpr int pcol(int d) {
  return (d & ~31) + 8 * ((d >> 2) & 3) + 4 * ((d >> 4) & 1) + (d & 3);
}

// Operand fragment of M^T for a token-major matrix M[s][*] in LDS (row stride LDD): rows
// (output index) col0 + lr, where the four columns col0 + 4q .. + 3 of a row start at element
// off(q) of that row; the eight k-slots of lane group lg are tokens s0 + m (first read) and
// s1 + m (second read), m = 0..3. Two transposing 8-byte reads (ds_read_b64_tr_b16): within a
// group of 16 lanes, lane i receives element i % 4 of the chunks addressed by lanes i / 4 + 4m,
// so lane q addresses row s + q / 4 at the four columns of lane group q % 4.
template <int LDD>
__device__ inline f16x8 frag_trans(const f16* base, int s0, int s1, int coff, int lr) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(3))) fp16x4_t lds_fp16x4;
  const int r = lr >> 2;
  const fp16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4*)(base + (s0 + r) * LDD + coff));
  const fp16x4_t y = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4*)(base + (s1 + r) * LDD + coff));
  return f16x8{(f16)x[0], (f16)x[1], (f16)x[2], (f16)x[3],
               (f16)y[0], (f16)y[1], (f16)y[2], (f16)y[3]};
#else
  return f16x8{};
#endif
}

// Register-class hints for values that only matrix-core instructions read between chunk
// boundaries: the resident operand fragments and the float32 state live in the accumulator
// registers (AGPRs), leaving the vector registers to the iterate and the products. An empty
// asm statement with an AGPR operand makes the allocator keep the value there.
template <typename V>
__device__ inline void keep_in_agpr(V& x) {
  asm volatile("" : "+a"(x));
}

__device__ inline f16x8 pack8(f32x4 a, f32x4 b) {
  return f16x8{(f16)a[0], (f16)a[1], (f16)a[2], (f16)a[3], (f16)b[0], (f16)b[1], (f16)b[2],
               (f16)b[3]};
}

// RES: residual mode, which also writes ||q_t - A_t x_i|| for i = 0..iters to A.resid
template <int D, bool RES>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void walk_tok_kernel(WalkArgs A, int B, int Tmax, int Hn, int N, int S, int J, ChebConsts cc) {
  using Cfg = TokCfg<D>;
  using M = Mma<f16>;
  typedef f16x8 Frag;
  constexpr int C = Cfg::C, NW = Cfg::NW, NT = Cfg::NT, FT = Cfg::FT, KD = Cfg::KD;
  constexpr int KC = Cfg::KC, ST = Cfg::ST, LDD = Cfg::LDD, UPR = Cfg::UPR, NU = Cfg::NU;
  constexpr int NRT = Cfg::NRT, NCT = Cfg::NCT;

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  f16* Kp = reinterpret_cast<f16*>(smem + Cfg::oKp);
  f16* Hs = reinterpret_cast<f16*>(smem + Cfg::oHs);
  const bf16x8* Kraw = reinterpret_cast<const bf16x8*>(smem + Cfg::oKraw);  // unit u at [u]
  const float* Graw = reinterpret_cast<const float*>(smem + Cfg::oGraw);    // [C] gates
  const float* Braw = Graw + C;                                               // [C] write gates
  float* v_cl = reinterpret_cast<float*>(smem + Cfg::oVec);  // [C] in-chunk log2 gate prefix
  float* v_w = v_cl + C;    // [C] carry weights 2^(cl_C - cl_s) beta_s
  float* v_a = v_w + C;     // [C] n^2 scan: a_t = gamma_t^2
  float* v_b = v_a + C;     // [C] n^2 scan: b_t
  float* v_bt = v_b + C;    // [C] write gates beta_s (1 without them)
  float* v_sc = v_bt + C;   // [16] scratch: [0, NW) state norms, [4, 4 + NW) largest |k| per wave
  float* v_coef = v_sc + 16;  // [iters][4] krs, kys, bts of each iteration (rescaled form)

  const int seg = blockIdx.x;
  int b, h;
  head_of(A, blockIdx.y, Hn, b, h);
  const int bh = b * Hn + h;
  int wave = threadIdx.x / kWave;
  // Per-lane indices, passed through refresh() at the start of every phase so that the
  // addresses derived from them are recomputed where they are used instead of being hoisted
  // out of the chunk loop and kept live for the whole walk (which would spill them)
  int tid = threadIdx.x, lane = tid % kWave;
  int lr = lane % 16, lg = lane / 16;
  int t = 16 * wave + lr;  // own token (column of the wave's accumulator tiles)
  // (the wave's state tiles a0, b0 likewise)
  int a0 = (wave * Cfg::NST) / FT, b0 = (wave * Cfg::NST) % FT;
  auto refresh = [&]() {
    asm volatile("" : "+v"(tid), "+v"(lane), "+v"(lr), "+v"(lg), "+v"(t), "+v"(wave));
    asm volatile("" : "+v"(a0), "+v"(b0));
  };
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
  const uint32_t tok_bytes = (uint32_t)Hn * D * 2u;  // 64 rows span < 2^31 bytes (host check)
  const bf16* qg = static_cast<const bf16*>(A.q);
  const bf16* kg = static_cast<const bf16*>(A.k);
  f16* yg = static_cast<f16*>(A.o);  // the solves (fp16) go to o's rows; the output pass reads
                                     // them back and writes o over them

  // ---- float32 state: tiles (a0 + jr, b0 + jc) of H, held in registers ----------------------
  f32x4 Hst[NRT][NCT];
#pragma unroll
  for (int jr = 0; jr < NRT; ++jr)
#pragma unroll
    for (int jc = 0; jc < NCT; ++jc) Hst[jr][jc] = f32x4{0.f, 0.f, 0.f, 0.f};
  float n0sq = 0.0f;
  {
    float sq = 0.0f;
    if (A.in_h) {
      const float* ih = A.in_h + bh * A.in_bh + seg * A.in_seg;
#pragma unroll
      for (int jr = 0; jr < NRT; ++jr)
#pragma unroll
        for (int jc = 0; jc < NCT; ++jc) {
          // H[r..r+3][c] is read as H[c][r..r+3] (symmetric)
          const size_t o = (size_t)(16 * (b0 + jc) + lr) * D + 16 * (a0 + jr) + 4 * lg;
          Hst[jr][jc] = *reinterpret_cast<const f32x4*>(ih + o);
          const f32x4 x = Hst[jr][jc];
          sq += x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
        }
    }
    sq = wave_sum(sq);
    if (lane == 0) v_sc[wave] = sq;
    // Chebyshev coefficients, read from LDS in the loop (scalar loads in flight would make
    // every wait for an LDS fragment a wait for all of them)
    if (tid < cc.iters_rs) {
      v_coef[4 * tid] = cc.krs[tid];
      v_coef[4 * tid + 1] = cc.kys[tid];
      v_coef[4 * tid + 2] = cc.bts[tid];
      v_coef[4 * tid + 3] = 0.0f;
    }
    __syncthreads();
    if (seg == 0 && A.n2_in) {
      n0sq = A.n2_in[bh];
    } else if (A.in_h) {
      for (int w = 0; w < NW; ++w) n0sq += v_sc[w];
    }
  }

  // The next chunk's key rows (16-byte units, consecutive threads along a token row) and gates
  // (lane = token) are prefetched straight into LDS by direct loads, issued after the chunk's
  // staging and in flight through its loop, so that no registers are held for them. A wave
  // waits for its own loads (vmcnt) before it reads them (the largest |k| below); the barrier
  // at the top of the next chunk orders them for the other waves. Lanes of rows past the end of
  // the sequence load nothing: those rows are zeroed where they are read.
  // (the write gates are read from the gates when there are none, and then not used)
  const float* bsrc = A.beta ? A.beta : A.gamma;
  typedef __attribute__((address_space(3))) void lds_void;
  auto prefetch_k = [&](int chn) {
    refresh();
    const int t0n = chn * C;
    const int nvn = min(C, Tlen - t0n);
    const bf16* src = kg + (seq0 + t0n) * tok_stride + (long long)h * D;
#pragma unroll
    for (int k = 0; k < NU / NT; ++k) {
      const int u = tid + k * NT;
      const int tt = (uint32_t)u / UPR, cu = (uint32_t)u % UPR;  // u >= 0
      const uint32_t base = __builtin_amdgcn_readfirstlane(
          (uint32_t)(uintptr_t)(lds_void*)(Kraw + (u - lane)));
      if (tt < nvn) dma_load16_so(src, (uint32_t)tt * tok_bytes + (uint32_t)cu * 16u, base);
    }
    if (wave < 2) {
      const float* gs = (wave == 0 ? A.gamma : bsrc) + (seq0 + t0n) * Hn + h;
      const uint32_t base = __builtin_amdgcn_readfirstlane(
          (uint32_t)(uintptr_t)(lds_void*)(wave == 0 ? Graw : Braw));
      if (lane < nvn) dma_load4_so(gs, (uint32_t)lane * Hn * 4u, base);
    }
  };
  // the largest |k| of the prefetched rows of chunk chn (this wave's units), to v_sc[4 + wave]
  auto kmax_put = [&](int chn) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's direct loads have landed
    refresh();
    const int nvn = min(C, Tlen - chn * C);
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < NU / NT; ++k) {
      const int u = tid + k * NT;
      const bf16x8 kv = Kraw[u];
      float um = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) um = fmaxf(um, fabsf((float)kv[i]));
      if ((int)((uint32_t)u / UPR) < nvn) m = fmaxf(m, um);  // rows past the end hold stale data
    }
    m = wave_max(m);
    if (lane == 0) v_sc[4 + wave] = m;
  };
  // state tiles (times sc) -> Hs as fp16 rows e = column index of the tile, permuted columns
  auto stage_tile = [&](int jr, int jc, f32x4 x) {
    f16x4 y = {(f16)x[0], (f16)x[1], (f16)x[2], (f16)x[3]};
    *reinterpret_cast<f16x4*>(Hs + (16 * (b0 + jc) + lr) * LDD + pcol(16 * (a0 + jr) + 4 * lg)) = y;
  };
  auto stage_h = [&](float sc) {
#pragma unroll
    for (int jr = 0; jr < NRT; ++jr)
#pragma unroll
      for (int jc = 0; jc < NCT; ++jc) stage_tile(jr, jc, Hst[jr][jc] * sc);
  };
  // A fragment of K (rows = tokens 16 sb + lr) over feature block kk
  auto frag_k = [&](int sb, int kk) {
    return *reinterpret_cast<const Frag*>(Kp + (16 * sb + lr) * LDD + 32 * kk + 8 * lg);
  };
  // A fragment of K^T (rows = features 16 ft + lr) over token block kc, permuted token order
  // (k-slot j of lane group lg: token 32 kc + 16 (j / 4) + 4 lg + j % 4), by two transposing
  // reads of K
  auto frag_kt = [&](int ft, int kc) {
    return frag_trans<LDD>(Kp, 32 * kc + 4 * lg, 32 * kc + 16 + 4 * lg, pcol(16 * ft + 4 * (lr & 3)), lr);
  };

  prefetch_k(c_begin);
  kmax_put(c_begin);

  for (int ch = c_begin; ch < c_end; ++ch) {
    refresh();
    const int t0 = ch * C;
    const int nv = min(C, Tlen - t0);
    const float n0 = sqrtf(n0sq);
    const float n0inv = n0 > 0.0f ? 1.0f / n0 : 0.0f;
    lds_barrier();  // the last chunk's LDS reads are done; v_sc holds this chunk's |k| maxima

    // ---- key scale 2^-ke of the chunk: the staged rows lie below 2 in magnitude -------------
    float km = v_sc[4];
#pragma unroll
    for (int w = 1; w < NW; ++w) km = fmaxf(km, v_sc[4 + w]);
    const int ke = pow2_exponent(km, 30);
    const float kinv = exp2_int(-ke), ks2 = exp2_int(2 * ke);

    // ---- gate prefix (every wave; lane = token) ---------------------------------------------
    float g_l = 1.0f, l2 = 0.0f, bt_l = 1.0f;  // tokens past the end: gamma = 1, k = q = 0
    if (lane < nv) {
      g_l = Graw[lane];
      l2 = log2_gate(g_l);
      if (A.beta) bt_l = Braw[lane];
    }
    const float cl = scan_add<kWave>(l2);
    const float clast = lane_value(cl, C - 1);
    const float gam = fast_exp2(cl);
    const float gC = lane_value(gam, C - 1);
    if (wave == 0) {
      v_cl[lane] = cl;
      v_w[lane] = fast_exp2(fminf(clast - cl, 0.0f)) * bt_l;
      v_bt[lane] = bt_l;
    }
    // ---- stage K (fp16, times 2^-ke, permuted features) ------------------------------------
#pragma unroll
    for (int k = 0; k < NU / NT; ++k) {
      const int u = tid + k * NT;
      const int tt = (uint32_t)u / UPR, cu = (uint32_t)u % UPR;  // u >= 0
      const bf16x8 kv = Kraw[u];
      f16x8 ko;
#pragma unroll
      for (int i = 0; i < 8; ++i) ko[i] = (f16)((float)kv[i] * kinv);
      if (tt >= nv) ko = f16x8{};  // rows past the end hold stale data (never loaded): zero them
      *reinterpret_cast<f16x4*>(Kp + tt * LDD + pcol(8 * cu)) = f16x4{ko[0], ko[1], ko[2], ko[3]};
      *reinterpret_cast<f16x4*>(Kp + tt * LDD + pcol(8 * cu + 4)) = f16x4{ko[4], ko[5], ko[6], ko[7]};
    }
    stage_h(n0inv);  // H0hat
    lds_barrier();
    // the next chunk's keys and gates: in flight through this chunk
    if (ch + 1 < c_end) prefetch_k(ch + 1);

    refresh();

    // ---- resident H0hat fragments ------------------------------------------------------------
    Frag Hres[FT][KD];
#pragma unroll
    for (int ft = 0; ft < FT; ++ft)
#pragma unroll
      for (int kk = 0; kk < KD; ++kk)
        Hres[ft][kk] = *reinterpret_cast<const Frag*>(Hs + (16 * ft + lr) * LDD + 32 * kk + 8 * lg);
    if constexpr (Cfg::PIN) {
#pragma unroll
      for (int ft = 0; ft < FT; ++ft)
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) keep_in_agpr(Hres[ft][kk]);
    }

    // ---- every K fragment of the chunk (rows = tokens), resident in vector registers through
    // the loop ----------------------------------------------------------------------------------
    refresh();
    Frag kres[KD][ST];
#pragma unroll
    for (int kk = 0; kk < KD; ++kk)
#pragma unroll
      for (int sb = 0; sb < ST; ++sb) kres[kk][sb] = frag_k(sb, kk);

    // ---- norm phase: k_t^T H0hat k_t and sum_{s<t} 2^(cl_{t-1} - cl_s) beta_s G_st^2 --------
    // (on the staged keys k' = 2^-ke k: the terms are multiplied back by 2^2ke and 2^4ke)
    {
      Frag kb[KD];  // B fragments of the own token's key
#pragma unroll
      for (int kk = 0; kk < KD; ++kk)
        kb[kk] = *reinterpret_cast<const Frag*>(Kp + t * LDD + 32 * kk + 8 * lg);
      float pu = 0.0f;
      f32x4 z[FT];  // H0hat k of the own token, the FT accumulators taking turns
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) z[ft] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KD; ++kk)
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) z[ft] = M::mma(Hres[ft][kk], kb[kk], z[ft]);
#pragma unroll
      for (int ft = 0; ft < FT; ++ft)
#pragma unroll
        for (int i = 0; i < 4; ++i) pu += z[ft][i] * (float)kb[ft / 2][4 * (ft % 2) + i];
      const float clp = t > 0 ? v_cl[t - 1] : 0.0f;
      float pv = 0.0f, kd = 0.0f;
      f32x4 gram[ST];  // Gram tiles G[s][t] of the own token, accumulators taking turns
#pragma unroll
      for (int sb = 0; sb < ST; ++sb) gram[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KD; ++kk)
#pragma unroll
        for (int sb = 0; sb < ST; ++sb) gram[sb] = M::mma(kres[kk][sb], kb[kk], gram[sb]);
#pragma unroll
      for (int sb = 0; sb < ST; ++sb) {
        const f32x4 gacc = gram[sb];
        const f32x4 cls = *reinterpret_cast<const f32x4*>(v_cl + 16 * sb + 4 * lg);
        const f32x4 bts = *reinterpret_cast<const f32x4*>(v_bt + 16 * sb + 4 * lg);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s = 16 * sb + 4 * lg + i;
          const float e = fast_exp2(fminf(clp - cls[i], 0.0f)) * bts[i] * (gacc[i] * gacc[i]);
          pv += s < t ? e : 0.0f;
          kd = s == t ? gacc[i] : kd;
        }
      }
      pu += lane_read(pu, lane ^ 16);
      pu += lane_read(pu, lane ^ 32);
      pv += lane_read(pv, lane ^ 16);
      pv += lane_read(pv, lane ^ 32);
      kd += lane_read(kd, lane ^ 16);
      kd += lane_read(kd, lane ^ 32);
      const float gt = lane_read(g_l, t);
      const float gprev = lane_read(gam, t > 0 ? t - 1 : 0);
      const float btt = lane_read(bt_l, t);
      if (lg == 0) {
        const float kdt = btt * (kd * ks2);  // beta_t ||k_t||^2
        v_a[t] = gt * gt;
        v_b[t] = 2.0f * gt * btt * ((t > 0 ? gprev : 1.0f) * n0 * (pu * ks2) + (pv * ks2) * ks2) +
                 kdt * kdt;
      }
    }
    // ---- every K^T fragment of the chunk, resident in registers until the loop ends (after the
    // norm phase's products, which do not need them) ------------------------------------------
    refresh();
    Frag ktr[KC][FT];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) {
        ktr[kc][ft] = frag_kt(ft, kc);
        if constexpr (Cfg::PIN) keep_in_agpr(ktr[kc][ft]);
      }
    lds_barrier();

    // ---- n_t^2 by an affine scan over the chunk (every wave; lane = token) -------------------
    refresh();
    float sa = v_a[lane], sb_ = v_b[lane];
    scan_affine(sa, sb_);
    const float n2 = sa * n0sq + sb_;
    const float ninv = n2 > 0.0f ? 1.0f / sqrtf(n2) : 0.0f;
    if (wave == 0 && A.hnorm_t && lane < nv)
      A.hnorm_t[(seq0 + t0 + lane) * Hn + h] = sqrtf(n2);
    const float n2last = lane_value(n2, C - 1);
    const float ninv_t = lane_read(ninv, t);
    const float s_t = lane_read(gam, t) * n0 * ninv_t;
    const float cl_t = lane_read(cl, t);
    // Mhat^T tiles of the own token: Mh[sb][i] = Mhat_{t, 16 sb + 4 lg + i}, for the staged keys
    // (times 2^2ke)
    f32x4 Mh[ST];
    {
      const float mt = ninv_t * ks2;
#pragma unroll
      for (int sb = 0; sb < ST; ++sb) {
        const f32x4 cls = *reinterpret_cast<const f32x4*>(v_cl + 16 * sb + 4 * lg);
        const f32x4 bts = *reinterpret_cast<const f32x4*>(v_bt + 16 * sb + 4 * lg);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s = 16 * sb + 4 * lg + i;
          Mh[sb][i] = s <= t ? fast_exp2(fminf(cl_t - cls[i], 0.0f)) * bts[i] * mt : 0.0f;
        }
      }
    }

    // ---- queries of the own token, accumulator layout: Q[t][16 ft + 4 lg .. + 3], loaded
    // during the carry's products and consumed at the start of the loop ----------------------
    bf16x4 Qraw[FT];
    {
      // bounds-checked: tokens past the end read as 0
      const auto rq = buffer_rsrc(qg + (seq0 + t0) * tok_stride + (long long)h * D,
                                  (uint32_t)(nv - 1) * tok_bytes + D * 2u);
      const uint32_t qoff = (uint32_t)t * tok_bytes + (uint32_t)lg * 8u;
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) Qraw[ft] = buffer_load8<bf16x4>(rq, qoff + 32u * ft);
    }
    // ---- state carry: H <- Gam_C H + K^T diag(w) K ------------------------------------------
    // (on the staged keys: the product is accumulated onto Gam_C H / 2^2ke, and the sum is
    // multiplied by 2^2ke)
    {
      // A operands (w K)^T of the own row tiles, split hi + lo; tokens in the permuted order
      // of the K^T tile (k-slot j of lane group lg: token 32 kc + 16 (j / 4) + 4 lg + j % 4)
      Frag awh[NRT][KC], awl[NRT][KC];
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const f32x4 w0 = *reinterpret_cast<const f32x4*>(v_w + 32 * kc + 4 * lg);
        const f32x4 w1 = *reinterpret_cast<const f32x4*>(v_w + 32 * kc + 16 + 4 * lg);
#pragma unroll
        for (int jr = 0; jr < NRT; ++jr) {
          const Frag kf = frag_kt(a0 + jr, kc);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float x = (float)kf[j] * (j < 4 ? w0[j] : w1[j - 4]);
            awh[jr][kc][j] = (f16)x;
            awl[jr][kc][j] = (f16)(x - (float)awh[jr][kc][j]);
          }
        }
      }
      // The K operands of column tile bc are the resident K^T fragments of feature tile bc
      // (K[s][16 bc + lr], the same token slots) when the wave's column tiles are all of them
      // (b0 = 0), else read again.
      const float gsc = gC * exp2_int(-2 * ke);
#pragma unroll
      for (int jc = 0; jc < NCT; ++jc) {
        Frag bk[KC];
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          if constexpr (NCT == FT) {
            bk[kc] = ktr[kc][jc];
          } else {
            bk[kc] = frag_kt(b0 + jc, kc);
          }
        }
        f32x4 hacc[NRT];
#pragma unroll
        for (int jr = 0; jr < NRT; ++jr) hacc[jr] = Hst[jr][jc] * gsc;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
#pragma unroll
          for (int hl = 0; hl < 2; ++hl)
#pragma unroll
            for (int jr = 0; jr < NRT; ++jr)
              hacc[jr] = M::mma(hl == 0 ? awh[jr][kc] : awl[jr][kc], bk[kc], hacc[jr]);
#pragma unroll
        for (int jr = 0; jr < NRT; ++jr) {
          Hst[jr][jc] = hacc[jr] * ks2;
          if constexpr (Cfg::PIN) keep_in_agpr(Hst[jr][jc]);
        }
      }
    }

    // ---- Chebyshev loop on the residuals of the own token ----------------------------------
    // (the query is taken times 2^-qe, so that its largest element lies in [1, 2): the solve
    // is linear in q, and the scale is carried to the stored solve)
    refresh();
    const bool live = ninv_t > 0.0f;  // ||H_t|| = 0: x_t = 0
    int qe;
    f32x4 Ra[FT], Rb[FT], X[FT];  // (Rb and X are first written by the first step)
    {
      float qm = 0.0f;
#pragma unroll
      for (int ft = 0; ft < FT; ++ft)
#pragma unroll
        for (int j = 0; j < 4; ++j) qm = fmaxf(qm, fabsf((float)Qraw[ft][j]));
      qm = fmaxf(qm, lane_read(qm, lane ^ 16));
      qm = fmaxf(qm, lane_read(qm, lane ^ 32));
      qe = pow2_exponent(qm, 60);
      const float qsc = live ? cc.inv_s0 * exp2_int(-qe) : 0.0f;
#pragma unroll
      for (int ft = 0; ft < FT; ++ft)
        Ra[ft] = f32x4{(float)Qraw[ft][0], (float)Qraw[ft][1], (float)Qraw[ft][2], (float)Qraw[ft][3]} * qsc;
    }
    // One iteration it on the current rescaled residual Rc = Rt_it (the residuals divided by
    // host scalars that absorb the R_{it-1} coefficient of the recurrence):
    //   Ro <- Ro + krs Rc + H0hat (kys s_t Rc) + K^T ((K Rc) o kys Mhat)
    // (Ro held Rt_{it-1} and now holds Rt_{it+1}), and X += bts_it Rt_it.
    // The work forms three instruction groups (sched_barrier boundaries), each pairing
    // matrix-core products with independent vector work and with the LDS reads of a later
    // group: (A) the K products P = K Rc^T and the recurrence start; (B) the H0hat products on
    // the scaled operands and the P' operands; (C) the K^T products, the X update and the
    // next step's first K fragments. With one wave per SIMD nothing else hides latency.
    // (the first step, FIRST = true, has Rt_{-1} = 0 and X = 0: it writes Ro and X outright)
    auto step = [&](auto first, f32x4(&Ro)[FT], f32x4(&Rc)[FT], int it, auto... no_x) {
      constexpr bool FIRST = decltype(first)::value;
      constexpr bool UPDX = sizeof...(no_x) == 0;  // the residual mode's last step leaves X
      const f32x4 cf = *reinterpret_cast<const f32x4*>(v_coef + 4 * it);  // krs, kys, bts
      Frag rf[KD], rs[KD], pf[KC];
      f32x4 pa[ST];
      // (A)
#pragma unroll
      for (int kk = 0; kk < KD; ++kk) rf[kk] = pack8(Rc[2 * kk], Rc[2 * kk + 1]);
#pragma unroll
      for (int sb = 0; sb < ST; ++sb) pa[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KD; ++kk)
#pragma unroll
        for (int sb = 0; sb < ST; ++sb) pa[sb] = M::mma(kres[kk][sb], rf[kk], pa[sb]);
      const float kys = cf[1] * s_t;
      rs[0] = pack8(Rc[0] * kys, Rc[1] * kys);
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) Ro[ft] = FIRST ? cf[0] * Rc[ft] : Ro[ft] + cf[0] * Rc[ft];
      __builtin_amdgcn_sched_barrier(0);
      // (B)
#pragma unroll
      for (int kk = 1; kk < KD; ++kk) rs[kk] = pack8(Rc[2 * kk] * kys, Rc[2 * kk + 1] * kys);
#pragma unroll
      for (int kk = 0; kk < KD; ++kk)
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) Ro[ft] = M::mma(Hres[ft][kk], rs[kk], Ro[ft]);
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
        pf[kc] = pack8(pa[2 * kc] * Mh[2 * kc] * cf[1], pa[2 * kc + 1] * Mh[2 * kc + 1] * cf[1]);
      __builtin_amdgcn_sched_barrier(0);
      // (C)
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) Ro[ft] = M::mma(ktr[kc][ft], pf[kc], Ro[ft]);
      if constexpr (UPDX) {
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) X[ft] = FIRST ? cf[2] * Rc[ft] : X[ft] + cf[2] * Rc[ft];
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    // Residual mode: ||R_i|| = |s_i| ||Rt_i|| of the own token (a sum over the lane's features,
    // then over the four lane groups), written by lane group 0; a token with ||H_t|| = 0 has
    // x_i = 0 for every i, so its residuals are all ||q_t||. Rows past the end of the sequence
    // (and the other lane groups) store out of the buffer's range, which drops the store.
    // (The residual is formed on the query times 2^-qe: its norm is multiplied back.)
    float res_qn = 0.0f;
    const int res_i1 = cc.iters + 1;
    const uint32_t res_row = (uint32_t)Hn * (uint32_t)res_i1 * 4u;  // bytes per token
    const auto res_rsrc =
        buffer_rsrc(RES ? A.resid + ((seq0 + t0) * Hn + h) * res_i1 : nullptr,
                    RES ? (uint32_t)(nv - 1) * res_row + (uint32_t)res_i1 * 4u : 0u);
    const uint32_t res_off = lg == 0 ? (uint32_t)t * res_row : 0x80000000u;
    auto lane_sum = [&](float x) {
      x += lane_read(x, lane ^ 16);
      return x + lane_read(x, lane ^ 32);
    };
    auto res_put = [&](int i, float val) { buffer_store4f(val, res_rsrc, res_off + 4u * (uint32_t)i); };
    const float res_sc = exp2_int(qe);
    auto res_step = [&](int i, const f32x4(&R)[FT]) {
      float x = 0.0f;
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) x += R[ft][0] * R[ft][0] + R[ft][1] * R[ft][1] + R[ft][2] * R[ft][2] + R[ft][3] * R[ft][3];
      x = lane_sum(x);
      res_put(i, live ? fabsf(cc.sres[i]) * sqrtf(x) * res_sc : res_qn);
    };
    if constexpr (RES) {
      float x = 0.0f;
#pragma unroll
      for (int ft = 0; ft < FT; ++ft)
#pragma unroll
        for (int j = 0; j < 4; ++j) x += (float)Qraw[ft][j] * (float)Qraw[ft][j];
      res_qn = sqrtf(lane_sum(x));
      res_put(0, res_qn);  // x_0 = 0
    }
    {
      using T1 = std::integral_constant<bool, true>;
      using T0 = std::integral_constant<bool, false>;
      const int iters = cc.iters_rs;
      const float bl = v_coef[4 * (iters - 1) + 2];  // X += bts_{r-1} Rt_{r-1}
      // residual mode: one more step on Rt_{r-1} without the X update gives Rt_r
      const bool extra = RES && cc.res_extra;
      if (iters == 1) {
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) X[ft] = bl * Ra[ft];
        if constexpr (RES) {
          if (extra) {
            step(T1{}, Rb, Ra, 0, 0);
            res_step(1, Rb);
          }
        }
      } else {
        step(T1{}, Rb, Ra, 0);  // Rb = Rt_1
        if constexpr (RES) res_step(1, Rb);
        int it = 1;
        for (; it + 2 < iters; it += 2) {
          step(T0{}, Ra, Rb, it);      // Ra = Rt_{it+1}
          if constexpr (RES) res_step(it + 1, Ra);
          step(T0{}, Rb, Ra, it + 1);  // Rb = Rt_{it+2}
          if constexpr (RES) res_step(it + 2, Rb);
        }
        if (it + 1 < iters) {
          step(T0{}, Ra, Rb, it);
          if constexpr (RES) res_step(it + 1, Ra);
#pragma unroll
          for (int ft = 0; ft < FT; ++ft) X[ft] += bl * Ra[ft];
          if constexpr (RES) {
            if (extra) {
              step(T0{}, Rb, Ra, iters - 1, 0);
              res_step(iters, Rb);
            }
          }
        } else {
#pragma unroll
          for (int ft = 0; ft < FT; ++ft) X[ft] += bl * Rb[ft];
          if constexpr (RES) {
            if (extra) {
              step(T0{}, Ra, Rb, iters - 1, 0);
              res_step(iters, Ra);
            }
          }
        }
      }
      // residuals past a truncated recurrence are below 2^-64 of ||q_t||: written as 0
      if constexpr (RES) {
        for (int i = extra ? cc.iters + 1 : iters; i <= cc.iters; ++i) res_put(i, live ? 0.0f : res_qn);
      }
    }

    // ---- the solve of the own token to o's row (fp16), scaled by 2^-xe so that its largest
    // element lies in [1, 2); phi_t = 2^xe / ||H_t||_F (times the iterate's own scales) to the
    // per-token array: o_t = phi_t U_t y_t ---------------------------------------------------
    refresh();
    if (ch + 1 < c_end) kmax_put(ch + 1);
    {
      float xm = 0.0f;
#pragma unroll
      for (int ft = 0; ft < FT; ++ft)
#pragma unroll
        for (int j = 0; j < 4; ++j) xm = fmaxf(xm, fabsf(X[ft][j]));
      xm = fmaxf(xm, lane_read(xm, lane ^ 16));
      xm = fmaxf(xm, lane_read(xm, lane ^ 32));
      const int xe = pow2_exponent(xm, 100);
      const float xinv = exp2_int(-xe);
      // (bounds-checked: the stores of tokens past the end are dropped)
      const auto ry = buffer_rsrc(yg + (seq0 + t0) * tok_stride + (long long)h * D,
                                  (uint32_t)(nv - 1) * tok_bytes + D * 2u);
      const uint32_t yoff = (uint32_t)t * tok_bytes + (uint32_t)lg * 8u;
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) {
        const f32x4 yv = X[ft] * xinv;
        const f16x4 y4 = {(f16)yv[0], (f16)yv[1], (f16)yv[2], (f16)yv[3]};
        buffer_store8(y4, ry, yoff + 32u * ft);
      }
      // phi_t: 2^xe undoes the solve's scale, inv_xsc the iterate's power of two, 2^qe the
      // query's, and 1 / ||H_t||_F turns the solve of the normalised system into x_t
      const float phi = exp2_int(xe) * cc.inv_xsc * exp2_int(qe) * ninv_t;
      const auto rp = buffer_rsrc(A.phi + (seq0 + t0) * Hn + h, (uint32_t)(nv - 1) * Hn * 4u + 4u);
      buffer_store4f(phi, rp, lg == 0 ? (uint32_t)t * Hn * 4u : 0x80000000u);
    }
    n0sq = n2last;
  }
  if (A.out_h && seg == last) {
    float* oh = A.out_h + (size_t)bh * D * D;
#pragma unroll
    for (int jr = 0; jr < NRT; ++jr)
#pragma unroll
      for (int jc = 0; jc < NCT; ++jc) {
        const size_t o = (size_t)(16 * (b0 + jc) + lr) * D + 16 * (a0 + jr) + 4 * lg;
        *reinterpret_cast<f32x4*>(oh + o) = Hst[jr][jc];
      }
  }
  if (A.n2_out && seg == last && tid == 0) A.n2_out[bh] = n0sq;
}

// ---- segment summaries -------------------------------------------------------------------
// For each (segment, head): the state reached from a zero state over the segment's tokens and
// the segment's total log2 gate. Unrolling the carry H <- Gam_C H + K^T diag(w) K over the
// segment gives one weighted sum over its tokens,
//   dH = sum_s w_s k_s k_s^T,  dU = sum_s w_s v_s k_s^T,  w_s = 2^(log2 of the gates after s)
// (times beta_s with the write gate),
// so the tokens are taken in blocks of 64 from the last block to the first, with the gate sum
// of the blocks already taken as the suffix of every weight, and no rescaling of the state.
// Matrix-core operands are bf16: K and V exactly, the weighted keys w k as a hi + lo pair
// (about 2^-17 relative). Eight waves, two per SIMD; wave w holds the float32 tiles (row tiles
// RT*(w % 2).., column tiles CT*(w / 2)..) of dH and of dU (rows = value features), computed as
// dH = K^T diag(w) K and dU = V^T diag(w) K, so that both take the weighted keys of the wave's
// column tiles as their second operand (weighted by the two waves that share those tiles).
// Per block every wave reads its own operand fragments with transposing reads of the block's
// K and V rows in LDS (bf16, padded rows), in the walk's permuted token order; the block's
// weights were computed one block earlier, from its gates in registers. The rows of
// the next block go to the other of two LDS slots, from registers loaded two blocks ahead with
// bounds-checked buffer loads (rows past the end read as 0): one barrier per block.
template <int D>
struct SumCfg {
  static constexpr int CB = 64;                // tokens per block (a chunk)
  static constexpr int KB = CB / 32;           // 32-deep token blocks per block
  static constexpr int NW = 8;                 // waves, two per SIMD
  static constexpr int NT = NW * kWave;
  static constexpr int FT = D / 16;
  static constexpr int RT = FT / 2;            // state row tiles per wave (more rows than
  static constexpr int CT = FT / 4;            // columns: fewer operand fragments per product)
  static constexpr int LDR = D + 8;            // row stride of a block's K or V rows (bf16)
  static constexpr int VEC = 8, UPR = D / VEC, NU = CB * UPR;
  static constexpr int NUT = (NU + NT - 1) / NT;  // 16-byte units per thread and matrix
  static constexpr size_t szRows = (size_t)CB * LDR * 2;
  static constexpr size_t szSlot = 2 * szRows;  // K rows, V rows
  static constexpr size_t bytes = 2 * szSlot + 2 * (size_t)NW * CB * sizeof(float);  // + weights
  static_assert(D == 64 || D == 128, "summary tiling");
  static_assert(bytes <= 160 * 1024, "LDS budget of one CU exceeded");
};

// fragment of M^T for rows M[s][*] (bf16, row stride LDR) in the permuted token order: two
// transposing 8-byte reads (lane layout as in frag_trans)
template <int LDR>
__device__ inline bf16x8 frag_trans_bf16(const bf16* base, int s0, int s1, int coff, int lr) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(3))) fp16x4_t lds_fp16x4;
  const int r = lr >> 2;
  const fp16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4*)(base + (s0 + r) * LDR + coff));
  const fp16x4_t y = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4*)(base + (s1 + r) * LDR + coff));
  const bf16x4 bx = __builtin_bit_cast(bf16x4, x), by = __builtin_bit_cast(bf16x4, y);
  return bf16x8{bx[0], bx[1], bx[2], bx[3], by[0], by[1], by[2], by[3]};
#else
  return bf16x8{};
#endif
}

template <int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void summary_tok_kernel(WalkArgs A, int B, int Tmax, int Hn, int N, int S, int J) {
  using Cfg = SumCfg<D>;
  using M = Mma<bf16>;
  typedef bf16x8 Frag;
  constexpr int CB = Cfg::CB, NT = Cfg::NT, RT = Cfg::RT, CT = Cfg::CT, LDR = Cfg::LDR;
  constexpr int UPR = Cfg::UPR, NU = Cfg::NU, NUT = Cfg::NUT;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  auto krows = [&](int slot) { return reinterpret_cast<bf16*>(smem + slot * Cfg::szSlot); };
  auto vrows = [&](int slot) { return krows(slot) + CB * LDR; };

  const int seg = blockIdx.x;
  int b, h;
  head_of(A, blockIdx.y, Hn, b, h);
  const int bh = b * Hn + h;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  int tid = threadIdx.x, lane = tid % kWave;
  int lr = lane % 16, lg = lane / 16;
  auto refresh = [&]() { asm volatile("" : "+v"(tid), "+v"(lane), "+v"(lr), "+v"(lg)); };
  // the wave's weights of two blocks (block p in half p % 2)
  float* v_wl = reinterpret_cast<float*>(smem + 2 * Cfg::szSlot) + wave * 2 * CB;
  const int a0 = RT * (wave % 2), b0 = CT * (wave / 2);
  // the segment's tokens [t_begin, t_end) in blocks of CB (= the chunk), block 0 the last one
  const int t_begin = seg * J * CB;
  long long seq0;  // first row of sequence b
  int Tlen;        // its length
  seq_range(A, b, Tmax, seq0, Tlen);
  // the last segment of the sequence needs no summary (its walk writes the final state), nor
  // do the segments past it
  if (seg >= last_segment(Tlen, J, CB)) return;
  const int t_end = min(Tlen, t_begin + J * CB);
  const int NB = (t_end - t_begin + CB - 1) / CB;
  const long long tok_stride = (long long)Hn * D;
  const uint32_t tok_bytes = (uint32_t)Hn * D * 2u;
  auto block_t0 = [&](int p) { return t_begin + (NB - 1 - p) * CB; };

  // rows of two blocks in registers (register set q holds block p with p % 2 == q)
  bf16x8 kr[2][NUT], vr[2][NUT];
  float gr[2], br[2];  // gates and write gates (lane = token)
  // the write gates are read from the gates when there are none (and then not used)
  const float* bsrc = A.beta ? A.beta : A.gamma;
  auto load_block = [&](int p, int q) {
    refresh();
    const int pv = p < NB ? p : NB - 1;
    const int t0n = block_t0(pv);
    const int nvn = p < NB ? min(CB, t_end - t0n) : 0;
    const long long row0 = (seq0 + t0n) * tok_stride + (long long)h * D;
    const uint32_t valid = nvn > 0 ? (uint32_t)(nvn - 1) * tok_bytes + D * 2u : 0u;
    const auto rk = buffer_rsrc(static_cast<const bf16*>(A.k) + row0, valid);
    const auto rv = buffer_rsrc(static_cast<const bf16*>(A.v) + row0, valid);
#pragma unroll
    for (int k = 0; k < NUT; ++k) {
      const int u = (tid + k * NT) % NU;  // (threads past NU repeat a unit; never written)
      const int tt = (uint32_t)u / UPR, cu = (uint32_t)u % UPR;  // u >= 0
      const uint32_t off = (uint32_t)tt * tok_bytes + (uint32_t)cu * 16u;
      kr[q][k] = buffer_load16<bf16x8>(rk, off);
      vr[q][k] = buffer_load16<bf16x8>(rv, off);
    }
    const uint32_t gvalid = nvn > 0 ? (uint32_t)(nvn - 1) * Hn * 4u + 4u : 0u;
    const auto rg = buffer_rsrc(A.gamma + (seq0 + t0n) * Hn + h, gvalid);
    const auto rb = buffer_rsrc(bsrc + (seq0 + t0n) * Hn + h, gvalid);
    gr[q] = buffer_load4f(rg, (uint32_t)lane * Hn * 4u);
    br[q] = buffer_load4f(rb, (uint32_t)lane * Hn * 4u);
  };
  auto write_block = [&](int slot, int q) {
    refresh();
#pragma unroll
    for (int k = 0; k < NUT; ++k) {
      const int u = tid + k * NT;
      if (NU % NT == 0 || u < NU) {
        const int tt = (uint32_t)u / UPR, cu = (uint32_t)u % UPR;  // u >= 0
        *reinterpret_cast<bf16x8*>(krows(slot) + tt * LDR + cu * 8) = kr[q][k];
        *reinterpret_cast<bf16x8*>(vrows(slot) + tt * LDR + cu * 8) = vr[q][k];
      }
    }
  };

  f32x4 Hst[RT][CT], Ust[RT][CT];
#pragma unroll
  for (int jr = 0; jr < RT; ++jr)
#pragma unroll
    for (int jc = 0; jc < CT; ++jc) {
      Hst[jr][jc] = f32x4{0.f, 0.f, 0.f, 0.f};
      Ust[jr][jc] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  float suffix = 0.0f;  // log2 gate sum of the blocks already weighted (the later ones)

  // weights of block p (lane = token), from its gates in register set q, one phase before
  // its products: 2^(log2 of the gates after the token), times the token's write gate
  auto weigh = [&](int p, int q) {
    const int nv = p < NB ? min(CB, t_end - block_t0(p)) : 0;
    const float l2 = lane < nv ? log2_gate(gr[q]) : 0.0f;
    const float cl = scan_add<kWave>(l2);
    const float clast = lane_value(cl, CB - 1);
    const float bw = A.beta ? br[q] : 1.0f;
    v_wl[(p & 1) * CB + lane] = fast_exp2(fminf(clast - cl + suffix, 0.0f)) * bw;
    suffix += clast;
  };
  // block p from slot p % 2 into the state
  auto accumulate = [&](int p) {
    refresh();
    const int slot = p & 1;
    const float* wl = v_wl + (p & 1) * CB;
    const bf16* kb = krows(slot);
    const bf16* vb = vrows(slot);
    const int cq = 4 * (lr & 3);
#pragma unroll
    for (int kc = 0; kc < Cfg::KB; ++kc) {
      const int s0 = 32 * kc + 4 * lg, s1 = s0 + 16;
      // A operands: K^T and V^T row fragments; B operands: the weighted keys of the column
      // tiles, hi + lo (shared by the two products: dH = K^T diag(w) K, dU = V^T diag(w) K)
      Frag ak[RT], av[RT], bh[CT], bl[CT];
#pragma unroll
      for (int jr = 0; jr < RT; ++jr) {
        ak[jr] = frag_trans_bf16<LDR>(kb, s0, s1, 16 * (a0 + jr) + cq, lr);
        av[jr] = frag_trans_bf16<LDR>(vb, s0, s1, 16 * (a0 + jr) + cq, lr);
      }
      const f32x4 w0 = *reinterpret_cast<const f32x4*>(wl + s0);
      const f32x4 w1 = *reinterpret_cast<const f32x4*>(wl + s1);
#pragma unroll
      for (int jc = 0; jc < CT; ++jc) {
        const Frag f = frag_trans_bf16<LDR>(kb, s0, s1, 16 * (b0 + jc) + cq, lr);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float x = (float)f[j] * (j < 4 ? w0[j] : w1[j - 4]);
          bh[jc][j] = (bf16)x;
          bl[jc][j] = (bf16)(x - (float)bh[jc][j]);
        }
      }
#pragma unroll
      for (int jc = 0; jc < CT; ++jc)
#pragma unroll
        for (int jr = 0; jr < RT; ++jr) {
          Hst[jr][jc] = M::mma(ak[jr], bh[jc], Hst[jr][jc]);
          Ust[jr][jc] = M::mma(av[jr], bh[jc], Ust[jr][jc]);
          Hst[jr][jc] = M::mma(ak[jr], bl[jc], Hst[jr][jc]);
          Ust[jr][jc] = M::mma(av[jr], bl[jc], Ust[jr][jc]);
        }
    }
  };
  // phase p: the rows of block p + 1 (register set (p + 1) % 2) go to slot (p + 1) % 2, that set
  // is reloaded with block p + 3, and block p is accumulated from slot p % 2
  auto phase = [&](int p, int q) {
    if (p + 1 < NB) {
      write_block(q, q);
      weigh(p + 1, q);
      load_block(p + 3, q);
    }
    accumulate(p);
    lds_barrier();  // slot (p + 1) % 2 is written; slot p % 2 is read
  };
  load_block(0, 0);
  load_block(1, 1);
  write_block(0, 0);
  weigh(0, 0);
  load_block(2, 0);
  lds_barrier();
  for (int p = 0; p < NB; p += 2) {
    phase(p, 1);
    if (p + 1 < NB) phase(p + 1, 0);
  }

  if (wave == 0 && lane == 0) A.log2g_out[(long long)bh * S + seg] = suffix;
  float* oh = A.sum_h + bh * A.sum_bh + seg * A.sum_seg;
  float* ou = A.sum_u + bh * A.sum_bh + seg * A.sum_seg;
#pragma unroll
  for (int jr = 0; jr < RT; ++jr)
#pragma unroll
    for (int jc = 0; jc < CT; ++jc) {
      // H[r..r+3][c] is written as H[c][r..r+3] (symmetric); the tile of U holds
      // U[r..r+3][c] (rows = value features), four scattered stores
      const size_t o = (size_t)(16 * (b0 + jc) + lr) * D + 16 * (a0 + jr) + 4 * lg;
      *reinterpret_cast<f32x4*>(oh + o) = Hst[jr][jc];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ou[(size_t)(16 * (a0 + jr) + 4 * lg + i) * D + 16 * (b0 + jc) + lr] = Ust[jr][jc][i];
    }
}

template <int D>
hipError_t launch_sum(const FwdPlan& pl, const WalkArgs& a, hipStream_t stream) {
  using Cfg = SumCfg<D>;
  auto kern = summary_tok_kernel<D>;
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(kern), (int)Cfg::bytes, lds_set);
  if (e != hipSuccess) return e;
  // the last segment needs no summary: the walk of that segment produces the final state
  hipLaunchKernelGGL(kern, dim3(pl.S - 1, pl.B * pl.H), dim3(Cfg::NT), Cfg::bytes, stream, a,
                     pl.B, pl.T, pl.H, pl.N, pl.S, pl.J);
  return hipGetLastError();
}

template <int D, bool RES>
hipError_t launch_tok(const FwdPlan& pl, const WalkArgs& a, const ChebConsts& cc,
                      hipStream_t stream) {
  using Cfg = TokCfg<D>;
  auto kern = walk_tok_kernel<D, RES>;
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(kern), (int)Cfg::bytes, lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(pl.S, pl.B * pl.H), dim3(Cfg::NT), Cfg::bytes, stream, a, pl.B,
                     pl.T, pl.H, pl.N, pl.S, pl.J, cc);
  return hipGetLastError();
}

}  // namespace

bool walk_tok_supported(const FwdPlan& pl) {
  // per-lane byte offsets within a chunk of 64 token rows are 32-bit
  const long long chunk_bytes = 64LL * pl.H * pl.D * 2;
  return pl.dtype == 0 && pl.C == 64 && (pl.D == 32 || pl.D == 64 || pl.D == 128) &&
         chunk_bytes < (1LL << 31);
}

bool summary_tok_supported(const FwdPlan& pl) {
  // the buffer loads address a block of 64 tokens with 32-bit byte offsets per lane
  const long long block_bytes = 64LL * pl.H * pl.D * 2;
  return pl.dtype == 0 && pl.C == 64 && (pl.D == 64 || pl.D == 128) && block_bytes < (1LL << 31);
}

hipError_t launch_summary_tok(const FwdPlan& pl, const WalkArgs& a, hipStream_t stream) {
  switch (pl.D) {
    case 64: return launch_sum<64>(pl, a, stream);
    case 128: return launch_sum<128>(pl, a, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_walk_tok(const FwdPlan& pl, const WalkArgs& a, const ChebConsts& cc,
                           hipStream_t stream) {
  if (a.resid) {
    // 32-bit byte offsets of a chunk's residual rows
    if (64LL * pl.H * (cc.iters + 1) * 4 >= (1LL << 31)) return hipErrorInvalidValue;
    switch (pl.D) {
      case 32: return launch_tok<32, true>(pl, a, cc, stream);
      case 64: return launch_tok<64, true>(pl, a, cc, stream);
      case 128: return launch_tok<128, true>(pl, a, cc, stream);
    }
    return hipErrorInvalidValue;
  }
  switch (pl.D) {
    case 32: return launch_tok<32, false>(pl, a, cc, stream);
    case 64: return launch_tok<64, false>(pl, a, cc, stream);
    case 128: return launch_tok<128, false>(pl, a, cc, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace gka
