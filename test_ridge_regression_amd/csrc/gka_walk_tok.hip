// Chunk walk of gka_fwd_chunked with token-owning waves (bf16 inputs, chunks of 64 tokens).
//
// The chunk algebra follows "Methodology in Plain English" and "Key Contributions" 3 on the
// ai.info summary of arXiv 2511.21016: per chunk,
//   Y_t   = s_t H0hat R_t + sum_{s<=t} Mhat_ts (k_s . R_t) k_s    (the system minus a I, on R_t)
//   n_t^2 = gamma_t^2 n_{t-1}^2 + 2 gamma_t beta_t k_t^T H_{t-1} k_t + beta_t^2 ||k_t||^4
//           (an affine scan over t)
//   o_t   = s_t U0hat X_t + sum_{s<=t} Mhat_ts (k_s . X_t) v_s
//   carry H <- Gam_C H + K^T diag(w) K,  U^T <- Gam_C U^T + K^T diag(w) V
// with H0hat = H0 / n0, U0hat = U0 / n0, s_t = Gam_t n0 / n_t, Mhat_ts = 2^(cl_t - cl_s) beta_s /
// n_t and carry weights w_s = 2^(cl_C - cl_s) beta_s. beta_t is the optional write gate ("Main
// Findings" on the ai.info summary: H_t = gamma_t H_{t-1} + beta_t k_t k_t^T, likewise U_t; 1
// without it); it enters only through these weights, so the key and value rows stay exact
// operands.
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
// The A operands are laid out to match: K and H0hat (U0hat) are staged in LDS with their
// feature columns permuted the same way (a fragment is one 16-byte read), and K^T / V^T
// fragments in the permuted token order come from transposing LDS reads.
//
// Range of the 16-bit operands: the keys and the values of a chunk are staged times 2^-e (e from
// the chunk's largest |k|, |v|, so the staged rows lie below 2), U0hat times 2^-e from the
// largest |U0| entry, the queries and the iterate of a token times 2^-e_t; all are exact powers
// of two, undone in float32 where the products are used (norm terms, mask, carry, output).
// Any bf16 input whose products stay in float32's range is therefore an fp16 operand of full
// precision.
//
// Per chunk: stage K, V (fp16), gates and H0hat; the norm phase (k_t^T H0hat k_t from the
// resident H0hat fragments, the Gram tiles of the own tokens) and a scan over the 64 tokens;
// the carry advances the float32 state (H as accumulator tiles in registers, U^T in LDS) and
// stages U0hat from the U^T tiles it reads; the Chebyshev loop; the output products. The next chunk's K, V and gates are
// loaded into registers during the output phase and staged at the top of the next chunk.
#include "gka_internal.hpp"
#include "gka_tok.hpp"

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
  // Row stride of the [*][D] fp16 tiles (K, V, H0hat / U0hat). At D = 128 the rows are
  // unpadded and the 16-byte units of row r are permuted by XOR with (5 r) & 15 (swz): the
  // transposing reads (eight rows by four column groups per 32 lanes) then meet each LDS bank
  // at most twice, against four times with a 16-byte pad, while the 16-byte row reads stay
  // conflict-free. At D <= 64 a 16-byte pad does better.
  static constexpr bool SWZ = D == 128;
  static constexpr int LDD = SWZ ? D : D + 8;
  static constexpr bool PIN = D >= 128;      // resident fragments and state in AGPRs
  static constexpr int VEC = 8;              // bf16 elements per 16-byte unit
  static constexpr int UPR = D / VEC;        // units per token row
  static constexpr int NU = C * UPR;         // units per matrix
  static constexpr size_t szTok = (size_t)C * LDD * 2;
  static constexpr size_t szHs = (size_t)D * LDD * 2;
  static constexpr size_t oKp = 0;               // K, token-major, permuted features (fp16)
  static constexpr size_t oVp = oKp + szTok;     // V, token-major (fp16)
  static constexpr size_t oHs = oVp + szTok;     // H0hat, then U0hat: row-major, permuted columns
  static constexpr int LDC = C + 8;              // row stride of the [D][C] fp16 tile
  static constexpr size_t oVT = oHs + szHs;      // V^T: row-major, tokens permuted (fp16)
  static constexpr size_t oUs = oVT + (size_t)D * LDC * 2;  // float32 U^T state, tile-major
  static constexpr size_t oVec = oUs + (size_t)D * D * sizeof(float);
  static constexpr size_t szVec = (size_t)(5 * C + 16 + 4 * 64) * sizeof(float);
  static constexpr size_t bytes = oVec + szVec;  // dynamic LDS
  static_assert(D % 32 == 0 && NST >= 1, "unsupported D");
  static_assert(NU % NT == 0, "staging units must fill whole workgroups");
  static_assert(bytes <= 160 * 1024, "LDS budget of one CU exceeded");
};

// RES: residual mode, which also writes ||q_t - A_t x_i|| for i = 0..iters to A.resid.
// D = 128 takes a whole SIMD per wave (its resident operands fill the register file); D <= 64
// fits in half of it, so two workgroups share a CU (their LDS fits too) and hide each other's
// latencies.
template <int D, bool RES>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, D >= 128 ? 1 : 2)))
void walk_tok_kernel(WalkArgs A, int B, int Tmax, int Hn, int N, int S, int J, ChebConsts cc) {
  using Cfg = TokCfg<D>;
  using M = Mma<f16>;
  typedef f16x8 Frag;
  constexpr int C = Cfg::C, NW = Cfg::NW, NT = Cfg::NT, FT = Cfg::FT, KD = Cfg::KD;
  constexpr int KC = Cfg::KC, ST = Cfg::ST, LDD = Cfg::LDD, UPR = Cfg::UPR, NU = Cfg::NU;
  // element offset of column position e in row `row` of a [*][D] tile (the units permuted)
  auto sw = [](int row, int e) { return Cfg::SWZ ? e ^ (8 * ((5 * row) & 15)) : e; };
  // the XOR of a transposing read's rows s + (lr >> 2), s a multiple of 4: the same for every
  // s that differs by a multiple of 16
  auto swt = [](int s, int lr_) { return Cfg::SWZ ? 8 * ((5 * (s + (lr_ >> 2))) & 15) : 0; };
  constexpr int NRT = Cfg::NRT, NCT = Cfg::NCT, LDC = Cfg::LDC;

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  f16* Kp = reinterpret_cast<f16*>(smem + Cfg::oKp);
  f16* Vp = reinterpret_cast<f16*>(smem + Cfg::oVp);
  f16* Hs = reinterpret_cast<f16*>(smem + Cfg::oHs);
  f16* VT = reinterpret_cast<f16*>(smem + Cfg::oVT);
  float* Us = reinterpret_cast<float*>(smem + Cfg::oUs);
  float* v_cl = reinterpret_cast<float*>(smem + Cfg::oVec);  // [C] in-chunk log2 gate prefix
  float* v_w = v_cl + C;    // [C] carry weights 2^(cl_C - cl_s) beta_s
  float* v_a = v_w + C;     // [C] n^2 scan: a_t = gamma_t^2
  float* v_b = v_a + C;     // [C] n^2 scan: b_t
  float* v_bt = v_b + C;    // [C] write gates beta_s (1 without them)
  // [16] scratch: [0, NW) state norms; per wave the largest |k| [4 + w], |U| [8 + w] and
  // |v| [12 + w]
  float* v_sc = v_bt + C;
  float* v_coef = v_sc + 16;  // [iters][4] krs, kys, bts, |s| of each iteration (rescaled form)

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
  // sum and max over the four lanes of a token (lane % 16 + 16 j): at D = 128, with one wave per
  // SIMD, by the row swaps (no LDS round trip to wait for); at D <= 64 the other wave on the
  // SIMD hides the round trip of the crossbar reads, which take fewer instructions. The two
  // give the same sums (the same pairs are added in the same order).
  auto gsum = [&](float x) {
    if constexpr (D >= 128) {
      return group_sum(x);
    } else {
      x += lane_read(x, lane ^ 16);
      return x + lane_read(x, lane ^ 32);
    }
  };
  auto gmax = [&](float x) {
    if constexpr (D >= 128) {
      return group_max(x);
    } else {
      x = fmaxf(x, lane_read(x, lane ^ 16));
      return fmaxf(x, lane_read(x, lane ^ 32));
    }
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
  const bf16* vg = static_cast<const bf16*>(A.v);
  bf16* og = static_cast<bf16*>(A.o);

  // ---- float32 state: the wave's tiles of H, held in registers. H is symmetric: at D = 128
  // (TRI) the waves hold only the 36 tiles on and above the diagonal, wave w the nine of row
  // tiles w and 7 - w (from the diagonal to the last column); the mirror tiles are written from
  // them where H is staged or stored. Otherwise the wave holds the block (a0 + jr, b0 + jc),
  // jr < NRT, jc < NCT, of the full grid. The tiles are kept times 2^-2E (E: the key scale of
  // the last carry), so that the carry needs no second rescaling ------------------------------
  constexpr bool TRI = D == 128;
  constexpr int NTL = TRI ? 9 : NRT * NCT;  // tiles per wave
  const int wave_u = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  // f(j, a, b, r) for the wave's tiles j = 0 .. NTL - 1: tile (a, b) holds H[16a + 4lg + i]
  // [16b + lr] (i = 0..3) in a lane; r selects the A operand of its row tile in the carry. With
  // TRI, j, a, b and r are compile-time constants (one instantiation per wave).
  auto for_tiles = [&](auto f) {
    if constexpr (TRI) {
      auto run = [&](auto W) {
        constexpr int w = decltype(W)::value, n0 = FT - w;
        static_for<0, NTL>([&](auto J) {
          constexpr int j = decltype(J)::value;
          f(J, IC<(j < n0 ? w : FT - 1 - w)>{}, IC<(j < n0 ? w + j : FT - 1 - w + (j - n0))>{},
            IC<(j < n0 ? 0 : 1)>{});
        });
      };
      switch (wave_u) {
        case 0: run(IC<0>{}); break;
        case 1: run(IC<1>{}); break;
        case 2: run(IC<2>{}); break;
        default: run(IC<3>{}); break;
      }
    } else {
      static_for<0, NTL>([&](auto J) {
        constexpr int j = decltype(J)::value;
        f(J, a0 + j / NCT, b0 + j % NCT, IC<j / NCT>{});
      });
    }
  };
  f32x4 Hst[NTL];
#pragma unroll
  for (int j = 0; j < NTL; ++j) Hst[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  int Ek = 0;  // H = Hst 2^2Ek
  // ---- U^T (rows = key features) in LDS, the wave's tiles only: the row tiles of its H tiles
  // (w and 7 - w with TRI, else a0 + jr) across every column, one f32x4 per lane and tile,
  // tile-major. Kept times 2^-Eu (Eu: key plus value scale of the last carry) -----------------
  constexpr int NUTL = TRI ? 2 * FT : NRT * NCT;  // U tiles per wave
  auto urow = [&](int r) { return TRI ? (r == 0 ? wave_u : FT - 1 - wave_u) : a0 + r; };
  // f(j, a, b, r) for the wave's U tiles j = 0 .. NUTL - 1 (row tile a = urow(r), column b)
  auto for_utiles = [&](auto f) {
    static_for<0, NUTL>([&](auto J) {
      constexpr int j = decltype(J)::value;
      constexpr int r = TRI ? j / FT : j / NCT;
      f(J, urow(r), TRI ? j % FT : b0 + j % NCT, IC<r>{});
    });
  };
  auto us_tile = [&](int j) {
    return reinterpret_cast<f32x4*>(Us) + ((j * NW + wave_u) * kWave + lane);
  };
  int Eu = 0;  // U = Us 2^Eu
  float n0sq = 0.0f;
  {
    // The segment-start state: slot seg of in_h / in_u, or, with in_log2g (a call from the
    // zero state), composed here from the summaries d_j of the segments before this one --
    // the affine scan over segments: start = sum_{j < seg} 2^(log2 gates of segments
    // j+1 .. seg-1) d_j, taken from j = seg - 1 down (the first source has weight 1 exactly)
    const int nsrc = A.in_log2g ? seg : (A.in_h ? 1 : 0);
    float lam = 0.0f;
    for (int i = 0; i < nsrc; ++i) {
      const int sl = A.in_log2g ? seg - 1 - i : seg;
      const float wj = exp2f(lam);
      const float* ih = A.in_h + bh * A.in_bh + sl * A.in_seg;
      const float* iu = A.in_u + bh * A.in_bh + sl * A.in_seg;
      for_tiles([&](auto J, auto a, auto b, auto) {
        constexpr int j = decltype(J)::value;
        // H[r..r+3][c] is read as H[c][r..r+3] (symmetric)
        const size_t o = (size_t)(16 * (int)b + lr) * D + 16 * (int)a + 4 * lg;
        const f32x4 x = *reinterpret_cast<const f32x4*>(ih + o);
#pragma unroll
        for (int e = 0; e < 4; ++e) Hst[j][e] = fmaf(wj, x[e], Hst[j][e]);
      });
      // U^T[r..r+3][c] = U[c][r..r+3], accumulated in the lane's own LDS slots
      for_utiles([&](auto J, int a, int b, auto) {
        constexpr int j = decltype(J)::value;
        const f32x4 x =
            *reinterpret_cast<const f32x4*>(iu + (size_t)(16 * b + lr) * D + 16 * a + 4 * lg);
        f32x4 y = i == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : *us_tile(j);
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = fmaf(wj, x[e], y[e]);
        *us_tile(j) = y;
      });
      if (A.in_log2g) lam += A.in_log2g[(long long)bh * S + sl];
    }
    float sq = 0.0f;
    for_tiles([&](auto J, auto a, auto b, auto) {
      const f32x4 x = Hst[decltype(J)::value];
      const float m = TRI && (int)a != (int)b ? 2.0f : 1.0f;  // an upper tile stands for two
      sq += m * (x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3]);
    });
    sq = wave_sum(sq);
    if (lane == 0) v_sc[wave] = sq;
    float um = 0.0f;
    for_utiles([&](auto J, int, int, auto) {
      constexpr int j = decltype(J)::value;
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
      if (nsrc > 0) x = *us_tile(j);
      else *us_tile(j) = x;
      um = fmaxf(um, fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3]))));
    });
    um = wave_max(um);
    if (lane == 0) v_sc[8 + wave_u] = um;
    // Chebyshev coefficients, read from LDS in the loop (scalar loads in flight would make
    // every wait for an LDS fragment a wait for all of them)
    if (tid < cc.iters_rs) {
      v_coef[4 * tid] = cc.krs[tid];
      v_coef[4 * tid + 1] = cc.kys[tid];
      v_coef[4 * tid + 2] = cc.bts[tid];
      v_coef[4 * tid + 3] = RES ? fabsf(cc.sres[tid]) : 0.0f;  // residual mode: |s_i|
    }
    __syncthreads();
    if (seg == 0 && A.n2_in) {
      n0sq = A.n2_in[bh];
    } else if (A.in_h) {
      for (int w = 0; w < NW; ++w) n0sq += v_sc[w];
    }
  }

  // The next chunk's K and V (16-byte units, consecutive threads along a token row) and gates
  // (lane = token) are loaded into registers at the start of the output phase, where few
  // registers are live, and staged at the top of the next chunk. Rows past the end of the
  // sequence are zero, with gate 1.
  bf16x8 kin[NU / NT], vin[NU / NT];
  float gin = 1.0f, bin = 1.0f;  // gate and write gate of token `lane`
  // the write gates are read from the gates when there are none (and then not used)
  const float* bsrc = A.beta ? A.beta : A.gamma;
  auto load_kv = [&](int chn) {
    refresh();  // keeps the per-lane addresses from being hoisted out of the chunk loop
    // Bounds-checked buffer loads: rows past the end of the sequence (or of the segment) read
    // as 0, with no branch, so the compiler counts these loads and waits for exactly them
    // where they are used. The values are defined on every path.
    const int chv = chn < c_end ? chn : c_end - 1;
    const int t0n = chv * C;
    const int nvn = chn < c_end ? min(C, Tlen - t0n) : 0;
    const long long row0 = (seq0 + t0n) * tok_stride + (long long)h * D;
    const uint32_t valid = nvn > 0 ? (uint32_t)(nvn - 1) * tok_bytes + D * 2u : 0u;
    const auto rk = buffer_rsrc(kg + row0, valid);
    const auto rv = buffer_rsrc(vg + row0, valid);
#pragma unroll
    for (int k = 0; k < NU / NT; ++k) {
      const int u = tid + k * NT;
      const int tt = (uint32_t)u / UPR, cu = (uint32_t)u % UPR;  // u >= 0
      const uint32_t off = (uint32_t)tt * tok_bytes + (uint32_t)cu * 16u;
      kin[k] = buffer_load16<bf16x8>(rk, off);
      vin[k] = buffer_load16<bf16x8>(rv, off);
    }
    const uint32_t gvalid = nvn > 0 ? (uint32_t)(nvn - 1) * Hn * 4u + 4u : 0u;
    const auto rg = buffer_rsrc(A.gamma + (seq0 + t0n) * Hn + h, gvalid);
    const auto rb = buffer_rsrc(bsrc + (seq0 + t0n) * Hn + h, gvalid);
    gin = buffer_load4f(rg, (uint32_t)lane * Hn * 4u);
    bin = buffer_load4f(rb, (uint32_t)lane * Hn * 4u);
  };
  // the largest |k| and |v| of the loaded rows (this wave's units), to v_sc[4 + wave] and
  // v_sc[12 + wave]: read by every wave after the barrier at the top of the chunk
  auto kvmax_put = [&]() {
    float mk = absmax_bf16<NU / NT>(kin), mv = absmax_bf16<NU / NT>(vin);
    mk = wave_max(mk);
    mv = wave_max(mv);
    if (lane == 0) {
      v_sc[4 + wave_u] = mk;
      v_sc[12 + wave_u] = mv;
    }
  };
  // state tiles (times sc) -> Hs as fp16: row e of Hs holds H[e][*] (permuted columns); tile
  // (a, b) gives rows 16b + lr (H[16b + lr][16a + 4lg ..] = H[16a + 4lg ..][16b + lr]). In the
  // symmetric scheme (b >= a) these are the blocks on and below the diagonal of Hs only: the
  // fragments of the blocks above it are read transposed from their mirrors (h0_frag).
  auto stage_h = [&](float sc) {
    for_tiles([&](auto J, auto a, auto b, auto) {
      constexpr int j = decltype(J)::value;
      const f32x4 x = Hst[j] * sc;
      const f16x4 y = {(f16)x[0], (f16)x[1], (f16)x[2], (f16)x[3]};
      *reinterpret_cast<f16x4*>(Hs + (16 * (int)b + lr) * LDD + sw(16 * (int)b + lr, pcol(16 * (int)a + 4 * lg))) = y;
    });
  };
  // A fragment of H0hat (rows 16 ft + lr) over feature block kk, i.e. the column tiles 2 kk and
  // 2 kk + 1. With the symmetric scheme only the blocks of Hs on and below the diagonal are
  // staged: a column tile right of the diagonal (c > ft) is read as the transpose of block
  // (c, ft) (H0hat[16 ft + lr][16 c + m] = Hs[16 c + m][16 ft + lr]), by a transposing read of the
  // rows of that block, in the permuted k order of the direct read.
  auto h0_frag = [&](auto FTc, auto KKc) -> Frag {
    constexpr int ft = decltype(FTc)::value, kk = decltype(KKc)::value;
    const f16* row = Hs + (16 * ft + lr) * LDD + sw(16 * ft + lr, 32 * kk + 8 * lg);
    const int coff = pcol(16 * ft + 4 * (lr & 3));
    if constexpr (!TRI || ft > 2 * kk) {
      return *reinterpret_cast<const Frag*>(row);
    } else if constexpr (ft < 2 * kk) {
      return frag_trans<LDD>(Hs, 32 * kk + 4 * lg, 32 * kk + 16 + 4 * lg, coff, lr, swt(4 * lg, lr));
    } else {  // ft == 2 kk: the diagonal block, then the block right of it
      const f16x4 lo = *reinterpret_cast<const f16x4*>(row);
      const f16x4 hi = frag_trans_half<LDD>(Hs, 32 * kk + 16 + 4 * lg, coff, lr, swt(4 * lg, lr));
      return Frag{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  };
  // A fragment of K (rows = tokens 16 sb + lr) over feature block kk
  auto frag_k = [&](int sb, int kk) {
    return *reinterpret_cast<const Frag*>(Kp + (16 * sb + lr) * LDD + sw(16 * sb + lr, 32 * kk + 8 * lg));
  };
  // A fragment of K^T (V^T) (rows = features 16 ft + lr) over token block kc, permuted token
  // order (k-slot j of lane group lg: token 32 kc + 16 (j / 4) + 4 lg + j % 4); K^T by two
  // transposing reads of K, V^T from its tile
  auto frag_kt = [&](int ft, int kc) {
    return frag_trans<LDD>(Kp, 32 * kc + 4 * lg, 32 * kc + 16 + 4 * lg, pcol(16 * ft + 4 * (lr & 3)), lr,
                           swt(4 * lg, lr));
  };
  auto frag_vt = [&](int ft, int kc) {
    return *reinterpret_cast<const Frag*>(VT + (16 * ft + lr) * LDC + 32 * kc + 8 * lg);
  };

  load_kv(c_begin);
  kvmax_put();
  // nothing in flight on entry to the chunk loop, so that the compiler's wait at its top counts
  // only the loads issued in the output phase of the previous chunk (and not its stores)
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0)

  for (int ch = c_begin; ch < c_end; ++ch) {
    refresh();
    const int t0 = ch * C;
    const int nv = min(C, Tlen - t0);
    const float n0 = sqrtf(n0sq);
    const float n0inv = n0 > 0.0f ? 1.0f / n0 : 0.0f;
    lds_barrier();  // the last chunk's LDS reads are done; v_sc holds this chunk's maxima

    // ---- scales of the chunk: keys 2^-ke and values 2^-ve (the staged rows lie below 2 in
    // magnitude), U0hat 2^-ue (its largest element lies below 2) -----------------------------
    float km = v_sc[4], vm = v_sc[12], umx = v_sc[8];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      km = fmaxf(km, v_sc[4 + w]);
      vm = fmaxf(vm, v_sc[12 + w]);
      umx = fmaxf(umx, v_sc[8 + w]);
    }
    const int ke = pow2_exponent(km, 30), ve = pow2_exponent(vm, 60);
    const float kinv = exp2_int(-ke), ks2 = exp2_int(2 * ke), vinv = exp2_int(-ve);
    // U0 / n0 = Us 2^Eu / n0: its largest element is umx 2^Eu n0inv
    const int ue = pow2_exponent(umx * exp2_int(Eu) * n0inv, 100);

    // ---- gate prefix (every wave; lane = token) ---------------------------------------------
    float g_l = 1.0f, l2 = 0.0f, bt_l = 1.0f;  // tokens past the end: gamma = 1, k = q = 0
    if (lane < nv) {
      g_l = gin;
      l2 = log2_gate(g_l);
      if (A.beta) bt_l = bin;
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
    // ---- stage K (fp16, times 2^-ke, permuted features) and V (fp16, times 2^-ve) --------
#pragma unroll
    for (int k = 0; k < NU / NT; ++k) {
      const int u = tid + k * NT;
      const int tt = (uint32_t)u / UPR, cu = (uint32_t)u % UPR;  // u >= 0
      const bf16x8 kv = kin[k], vv = vin[k];  // rows past the end were read as 0
      f16x8 ko, vo;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ko[i] = (f16)((float)kv[i] * kinv);
        vo[i] = (f16)((float)vv[i] * vinv);
      }
      *reinterpret_cast<f16x8*>(Vp + tt * LDD + sw(tt, 8 * cu)) = vo;
      *reinterpret_cast<f16x4*>(Kp + tt * LDD + sw(tt, pcol(8 * cu))) = f16x4{ko[0], ko[1], ko[2], ko[3]};
      *reinterpret_cast<f16x4*>(Kp + tt * LDD + sw(tt, pcol(8 * cu + 4))) = f16x4{ko[4], ko[5], ko[6], ko[7]};
    }
    stage_h(n0inv * exp2_int(2 * Ek));  // H0hat
    lds_barrier();

    refresh();

    // ---- resident H0hat fragments ------------------------------------------------------------
    Frag Hres[FT][KD];
    static_for<0, FT>([&](auto F) {
      static_for<0, KD>([&](auto K) { Hres[decltype(F)::value][decltype(K)::value] = h0_frag(F, K); });
    });
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
        kb[kk] = *reinterpret_cast<const Frag*>(Kp + t * LDD + sw(t, 32 * kk + 8 * lg));
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
      pu = gsum(pu);
      pv = gsum(pv);
      kd = gsum(kd);
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
    // ---- V^T with the tokens in the permuted order (fragments from transposing reads of V,
    // written back as rows: every later operand of it is one 16-byte read), and every K^T
    // fragment of the chunk, resident in registers until the loop ends (after the norm
    // phase's products, which do not need them) ----------------------------------------------
    // (every read is issued before the first write and before the register-class hints, so
    // that one wait covers them: a write between reads orders the later reads behind it)
    refresh();
    {
      constexpr int NVT = (FT * KC + NW - 1) / NW;
      Frag g[NVT];
#pragma unroll
      for (int k = 0; k < NVT; ++k) {
        const int phi = wave + k * NW;
        if (FT * KC % NW == 0 || phi < FT * KC) {
          const int ft = phi / KC, kc = phi % KC;
          g[k] = frag_trans<LDD>(Vp, 32 * kc + 4 * lg, 32 * kc + 16 + 4 * lg,
                                 16 * ft + 4 * (lr & 3), lr, swt(4 * lg, lr));
        }
      }
#pragma unroll
      for (int k = 0; k < NVT; ++k) {
        const int phi = wave + k * NW;
        if (FT * KC % NW == 0 || phi < FT * KC) {
          const int ft = phi / KC, kc = phi % KC;
          *reinterpret_cast<Frag*>(VT + (16 * ft + lr) * LDC + 32 * kc + 8 * lg) = g[k];
        }
      }
    }
    Frag ktr[KC][FT];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) ktr[kc][ft] = frag_kt(ft, kc);
    if constexpr (Cfg::PIN) {
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) keep_in_agpr(ktr[kc][ft]);
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
          // (computed for every s and then selected: a conditional exp2 becomes a branch)
          const float e = fast_exp2(fminf(cl_t - cls[i], 0.0f)) * bts[i] * mt;
          Mh[sb][i] = s <= t ? e : 0.0f;
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
    // (on the staged keys k' = 2^-ke k: the tiles, kept times 2^-2E, are rescaled to 2^-2ke and
    // the product on k' added; E becomes ke)
    {
      // A operands (w K)^T of the wave's row tiles, split hi + lo; tokens in the permuted order
      // of the K^T tile (k-slot j of lane group lg: token 32 kc + 16 (j / 4) + 4 lg + j % 4)
      constexpr int NR = TRI ? 2 : NRT;
      Frag awh[NR][KC], awl[NR][KC];
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const f32x4 w0 = *reinterpret_cast<const f32x4*>(v_w + 32 * kc + 4 * lg);
        const f32x4 w1 = *reinterpret_cast<const f32x4*>(v_w + 32 * kc + 16 + 4 * lg);
#pragma unroll
        for (int jr = 0; jr < NR; ++jr) {
          const int ar = TRI ? (jr == 0 ? wave_u : FT - 1 - wave_u) : a0 + jr;
          const Frag kf = frag_kt(ar, kc);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float x = (float)kf[j] * (j < 4 ? w0[j] : w1[j - 4]);
            awh[jr][kc][j] = (f16)x;
            awl[jr][kc][j] = (f16)(x - (float)awh[jr][kc][j]);
          }
        }
      }
      // The K operands of column tile b are the resident K^T fragments of feature tile b
      // (K[s][16 b + lr], the same token slots) where b is a compile-time constant, else read
      // again.
      const float gsc = gC * exp2_int(2 * (Ek - ke));
      for_tiles([&](auto J, auto a, auto b, auto R) {
        constexpr int j = decltype(J)::value, r = decltype(R)::value;
        Frag bk[KC];
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          if constexpr (TRI) {
            bk[kc] = ktr[kc][decltype(b)::value];
          } else if constexpr (NCT == FT) {
            bk[kc] = ktr[kc][j % NCT];
          } else {
            bk[kc] = frag_kt((int)b, kc);
          }
        }
        f32x4 hacc = Hst[j] * gsc;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          hacc = M::mma(awh[r][kc], bk[kc], hacc);
          hacc = M::mma(awl[r][kc], bk[kc], hacc);
        }
        Hst[j] = hacc;
        if constexpr (Cfg::PIN) keep_in_agpr(Hst[j]);
      });
      Ek = ke;
      // U^T tiles: the same A operands against the V^T fragments of their column tiles, on
      // Gam_C U^T rescaled to the frame 2^(ke + ve) of the product; the largest |U| of the
      // wave's tiles to v_sc[8 + wave] for the next chunk's U0hat. Column by column: the V^T
      // fragments and U^T tiles of the next two columns are read while the current one's
      // products run, and the rows of a column share them. The tiles as read are
      // this chunk's U0: each is also staged to Hs as U0hat times 2^-ue (fp16; row v of Hs
      // holds U[v][*], permuted columns), which the output reads after its barrier (every wave
      // has read its H0hat fragments from Hs before the barrier ahead of the norm scan).
      const float u0sc = exp2_int(Eu - ue) * n0inv;
      const float usc = gC * exp2_int(Eu - ke - ve);
      constexpr int NUR = TRI ? 2 : NRT, NUC = TRI ? FT : NCT;  // U row, column tiles per wave
      float um = 0.0f;
      constexpr int NB = NUC > 2 ? 3 : 2;  // column buffers: the reads run two columns ahead
      Frag bv[NB][KC];
      f32x4 ub[NB][NUR];
      auto load_col = [&](int c, int buf) {
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) bv[buf][kc] = frag_vt(TRI ? c : b0 + c, kc);
#pragma unroll
        for (int r = 0; r < NUR; ++r) ub[buf][r] = *us_tile(r * NUC + c);
      };
#pragma unroll
      for (int c = 0; c < NB - 1 && c < NUC; ++c) load_col(c, c);
#pragma unroll
      for (int c = 0; c < NUC; ++c) {
        if (c + NB - 1 < NUC) load_col(c + NB - 1, (c + NB - 1) % NB);
        f32x4 uacc[NUR];
#pragma unroll
        for (int r = 0; r < NUR; ++r) {
          // U^T tile (urow(r), column b) holds U[16 b + lr][16 urow(r) + 4 lg ..]
          const f32x4 y = ub[c % NB][r] * u0sc;
          const int hrow = 16 * (TRI ? c : b0 + c) + lr;
          *reinterpret_cast<f16x4*>(Hs + hrow * LDD + sw(hrow, pcol(16 * urow(r) + 4 * lg))) =
              f16x4{(f16)y[0], (f16)y[1], (f16)y[2], (f16)y[3]};
          uacc[r] = ub[c % NB][r] * usc;
        }
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
#pragma unroll
          for (int hl = 0; hl < 2; ++hl)
#pragma unroll
            for (int r = 0; r < NUR; ++r)
              uacc[r] = M::mma(hl == 0 ? awh[r][kc] : awl[r][kc], bv[c % NB][kc], uacc[r]);
#pragma unroll
        for (int r = 0; r < NUR; ++r) {
          *us_tile(r * NUC + c) = uacc[r];
          const f32x4 x = uacc[r];
          um = fmaxf(um, fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3]))));
        }
      }
      Eu = ke + ve;
      um = wave_max(um);
      if (lane == 0) v_sc[8 + wave_u] = um;
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
      qm = gmax(qm);
      qe = pow2_exponent(qm, 60);
      const float qsc = live ? cc.inv_s0 * exp2_int(-qe) : 0.0f;
#pragma unroll
      for (int ft = 0; ft < FT; ++ft)
        Ra[ft] = f32x4{(float)Qraw[ft][0], (float)Qraw[ft][1], (float)Qraw[ft][2], (float)Qraw[ft][3]} * qsc;
    }
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
    // a lane's sum of squares of a residual, taken on its fp16 operand copy (the values the
    // products use): two elements per dot-product instruction, float32 accumulation
    auto sumsq = [&](const Frag(&rf)[KD]) {
      float x = 0.0f;
#pragma unroll
      for (int kk = 0; kk < KD; ++kk) {
        x = __builtin_amdgcn_fdot2(__builtin_shufflevector(rf[kk], rf[kk], 0, 1), __builtin_shufflevector(rf[kk], rf[kk], 0, 1), x, false);
        x = __builtin_amdgcn_fdot2(__builtin_shufflevector(rf[kk], rf[kk], 2, 3), __builtin_shufflevector(rf[kk], rf[kk], 2, 3), x, false);
        x = __builtin_amdgcn_fdot2(__builtin_shufflevector(rf[kk], rf[kk], 4, 5), __builtin_shufflevector(rf[kk], rf[kk], 4, 5), x, false);
        x = __builtin_amdgcn_fdot2(__builtin_shufflevector(rf[kk], rf[kk], 6, 7), __builtin_shufflevector(rf[kk], rf[kk], 6, 7), x, false);
      }
      return x;
    };
    auto res_put = [&](int i, float val) { buffer_store4f(val, res_rsrc, res_off + 4u * (uint32_t)i); };
    const float res_sc = exp2_int(qe);
    // the residual from a lane's sum of squares x summed over the lane groups, and |s_i|
    auto res_val = [&](float x, float s_abs) {
      return live ? s_abs * __builtin_amdgcn_sqrtf(x) * res_sc : res_qn;
    };
    auto res_step = [&](int i, const f32x4(&R)[FT]) {
      Frag rf[KD];
#pragma unroll
      for (int kk = 0; kk < KD; ++kk) rf[kk] = pack8(R[2 * kk], R[2 * kk + 1]);
      float x = sumsq(rf);
      x = gsum(x);
      res_put(i, res_val(x, fabsf(cc.sres[i])));
    };
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
    // In the residual mode a step with RESC = true also writes ||R_it|| of its operand: the
    // lane's sum of squares in (A), the sums over the lane groups (two cross-lane reads, whose
    // LDS round trips pass under the products) in (B) and (C), the store in (C).
    auto step = [&](auto first, auto resc, f32x4(&Ro)[FT], f32x4(&Rc)[FT], int it, auto... no_x) {
      constexpr bool FIRST = decltype(first)::value;
      constexpr bool RESC = RES && decltype(resc)::value;
      constexpr bool UPDX = sizeof...(no_x) == 0;  // the residual mode's last step leaves X
      const f32x4 cf = *reinterpret_cast<const f32x4*>(v_coef + 4 * it);  // krs, kys, bts, |s|
      Frag rf[KD], rs[KD], pf[KC];
      f32x4 pa[ST];
      float rsq = 0.0f, rsx = 0.0f;
      // (A)
#pragma unroll
      for (int kk = 0; kk < KD; ++kk) rf[kk] = pack8(Rc[2 * kk], Rc[2 * kk + 1]);
      if constexpr (RESC) {
        rsq = sumsq(rf);
        rsx = lane_read(rsq, lane ^ 16);
      }
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
      if constexpr (RESC) {
        rsq += rsx;
        rsx = lane_read(rsq, lane ^ 32);
      }
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
      if constexpr (RESC) res_put(it, res_val(rsq + rsx, cf[3]));
      __builtin_amdgcn_sched_barrier(0);
    };
    if constexpr (RES) {
      float x = 0.0f;
#pragma unroll
      for (int ft = 0; ft < FT; ++ft)
#pragma unroll
        for (int j = 0; j < 4; ++j) x += (float)Qraw[ft][j] * (float)Qraw[ft][j];
      x = gsum(x);
      res_qn = sqrtf(x);
      res_put(0, res_qn);  // x_0 = 0
    }
    {
      using T1 = std::integral_constant<bool, true>;
      using T0 = std::integral_constant<bool, false>;
      const int iters = cc.iters_rs;
      const float bl = v_coef[4 * (iters - 1) + 2];  // X += bts_{r-1} Rt_{r-1}
      // residual mode: one more step on Rt_{r-1} without the X update gives Rt_r
      const bool extra = RES && cc.res_extra;
      // (residual mode: step it also writes ||R_it|| for it >= 1; the last one or two residuals
      // come from res_step)
      if (iters == 1) {
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) X[ft] = bl * Ra[ft];
        if constexpr (RES) {
          if (extra) {
            step(T1{}, T0{}, Rb, Ra, 0, 0);
            res_step(1, Rb);
          }
        }
      } else {
        step(T1{}, T0{}, Rb, Ra, 0);  // Rb = Rt_1
        int it = 1;
        for (; it + 2 < iters; it += 2) {
          step(T0{}, T1{}, Ra, Rb, it);      // Ra = Rt_{it+1}
          step(T0{}, T1{}, Rb, Ra, it + 1);  // Rb = Rt_{it+2}
        }
        if (it + 1 < iters) {
          step(T0{}, T1{}, Ra, Rb, it);  // Ra = Rt_{iters-1}
#pragma unroll
          for (int ft = 0; ft < FT; ++ft) X[ft] += bl * Ra[ft];
          if constexpr (RES) {
            if (extra) {
              step(T0{}, T1{}, Rb, Ra, iters - 1, 0);
              res_step(iters, Rb);
            } else {
              res_step(iters - 1, Ra);
            }
          }
        } else {  // Rb = Rt_{iters-1}
#pragma unroll
          for (int ft = 0; ft < FT; ++ft) X[ft] += bl * Rb[ft];
          if constexpr (RES) {
            if (extra) {
              step(T0{}, T1{}, Ra, Rb, iters - 1, 0);
              res_step(iters, Ra);
            } else {
              res_step(iters - 1, Rb);
            }
          }
        }
      }
      // residuals past a truncated recurrence are below 2^-64 of ||q_t||: written as 0
      if constexpr (RES) {
        for (int i = extra ? cc.iters + 1 : iters; i <= cc.iters; ++i) res_put(i, live ? 0.0f : res_qn);
      }
    }

    // ---- output O^T = diag(s) U0hat X^T + V^T ((K X^T) o Mhat) ------------------------------
    // (X is taken times 2^-xe, so that its largest element lies in [1, 2), and U0hat, K and V
    // are the staged, scaled operands: their powers of two are undone at the store)
    // Instruction groups: (1) U0hat and K fragment reads, X as fp16; (2) the K products
    // and the V^T fragment reads; (3) the U0hat products; (4) the V^T products and the stores.
    lds_barrier();  // U0hat is staged
    load_kv(ch + 1);
    refresh();
    {
#pragma unroll
      for (int ft = 0; ft < FT; ++ft)
#pragma unroll
        for (int kk = 0; kk < KD; ++kk)
          Hres[ft][kk] = *reinterpret_cast<const Frag*>(Hs + (16 * ft + lr) * LDD + sw(16 * ft + lr, 32 * kk + 8 * lg));
      if constexpr (Cfg::PIN) {
#pragma unroll
        for (int ft = 0; ft < FT; ++ft)
#pragma unroll
          for (int kk = 0; kk < KD; ++kk) keep_in_agpr(Hres[ft][kk]);
      }
      float xm = 0.0f;
#pragma unroll
      for (int ft = 0; ft < FT; ++ft)
#pragma unroll
        for (int j = 0; j < 4; ++j) xm = fmaxf(xm, fabsf(X[ft][j]));
      xm = gmax(xm);
      const int xe = pow2_exponent(xm, 100);
      const float xinv = exp2_int(-xe);
      // (one fp16 rounding of X: o is stored in bf16, whose rounding is 4x coarser; a lo part of
      // X measured 1.8e-3 against 1.9e-3 relative error of o at B8 T2048 H8 D128 and cost 3.5%
      // of the call)
      Frag vq[KC][FT], xh[KD], pf[KC];
#pragma unroll
      for (int kk = 0; kk < KD; ++kk) xh[kk] = pack8(X[2 * kk] * xinv, X[2 * kk + 1] * xinv);
      __builtin_amdgcn_sched_barrier(0);
      f32x4 pa[ST];
#pragma unroll
      for (int sb = 0; sb < ST; ++sb) pa[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KD; ++kk)
#pragma unroll
        for (int sb = 0; sb < ST; ++sb) pa[sb] = M::mma(kres[kk][sb], xh[kk], pa[sb]);
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) vq[kc][ft] = frag_vt(ft, kc);
      __builtin_amdgcn_sched_barrier(0);
      f32x4 y[FT];
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) y[ft] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KD; ++kk)
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) y[ft] = M::mma(Hres[ft][kk], xh[kk], y[ft]);
      // (the loop's mask Mh carries 2^2ke, the K product 2^-ke: their product is the masked
      // K X^T times 2^ke)
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) pf[kc] = pack8(pa[2 * kc] * Mh[2 * kc], pa[2 * kc + 1] * Mh[2 * kc + 1]);
      __builtin_amdgcn_sched_barrier(0);
      // o = inv_xsc 2^(qe + xe + ve - ke) (s_t 2^(ue - ve + ke) U0hat' X'' + V'^T pf)
      const float ysc = s_t * exp2_int(ue - ve + ke);
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) y[ft] = y[ft] * ysc;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) y[ft] = M::mma(vq[kc][ft], pf[kc], y[ft]);
      // o of the own token straight from the accumulators: 8 bytes per lane, 32 per token row
      // and tile (bounds-checked: the stores of tokens past the end are dropped)
      const float osc = cc.inv_xsc * exp2_int(qe + xe) * exp2_int(ve - ke);
      const auto ro = buffer_rsrc(og + (seq0 + t0) * tok_stride + (long long)h * D,
                                  (uint32_t)(nv - 1) * tok_bytes + D * 2u);
      const uint32_t ooff = (uint32_t)t * tok_bytes + (uint32_t)lg * 8u;
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) {
        const f32x4 yo = y[ft] * osc;
        const bf16x4 ov = {(bf16)yo[0], (bf16)yo[1], (bf16)yo[2], (bf16)yo[3]};
        buffer_store8(ov, ro, ooff + 32u * ft);
      }
    }
    kvmax_put();  // the next chunk's rows: their largest |k|, |v| for its scales
    n0sq = n2last;
  }
  if (A.out_h && seg == last) {
    float* oh = A.out_h + (size_t)bh * D * D;
    const float sc = exp2_int(2 * Ek);
    for_tiles([&](auto J, auto a, auto b, auto) {
      constexpr int j = decltype(J)::value;
      const f32x4 x = Hst[j] * sc;
      *reinterpret_cast<f32x4*>(oh + (size_t)(16 * (int)b + lr) * D + 16 * (int)a + 4 * lg) = x;
      if constexpr (TRI) {
        if constexpr (decltype(a)::value != decltype(b)::value) {
#pragma unroll
          for (int i = 0; i < 4; ++i) oh[(size_t)(16 * (int)a + 4 * lg + i) * D + 16 * (int)b + lr] = x[i];
        }
      }
    });
  }
  if (A.out_u && seg == last) {
    float* ou = A.out_u + (size_t)bh * D * D;
    const float sc = exp2_int(Eu);
    for_utiles([&](auto J, int a, int b, auto) {
      constexpr int j = decltype(J)::value;
      // U^T[r..r+3][c] is written as U[c][r..r+3]
      *reinterpret_cast<f32x4*>(ou + (size_t)(16 * b + lr) * D + 16 * a + 4 * lg) = *us_tile(j) * sc;
    });
  }
  if (A.n2_out && seg == last && tid == 0) A.n2_out[bh] = n0sq;
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
