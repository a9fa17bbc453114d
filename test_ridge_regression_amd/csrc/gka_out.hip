// Output pass of gka_fwd_chunked for the token walk's configurations (bf16 inputs, chunks of 64):
// o_t = U_t x_t chunk by chunk, with the value-side recurrence U_t = gamma_t U_{t-1} +
// beta_t v_t k_t^T carried from the segment's start ("Methodology in Plain English" on the
// ai.info summary of arXiv 2511.21016: the output of the closed form is U_t x_t, and only the
// chunk-initial states are carried). The walk has left every token's solve as y_t (fp16, in
// o's row) with x_t = phi_t y_t (phi in a per-token float array). Per chunk of C tokens, with
// U0 the chunk-start state, Gam_t and cl_t the in-chunk gate product and its log2:
//   o_t = phi_t ( Gam_t U0 y_t + sum_{s<=t} 2^(cl_t - cl_s) beta_s (k_s . y_t) v_s )
//   U   <- Gam_C U + V^T diag(w) K,   w_s = 2^(cl_C - cl_s) beta_s
// computed transposed (value feature x token), so that a lane's accumulator holds four
// consecutive features of one token.
//
// One wave per 16 value features: it holds the float32 state tiles U^T[k][v] of its features
// (all key rows), and forms its rows of o^T and of the carry. Operands:
//   - U0 y^T: fp16, U0 times a power of two from the wave's largest |U| entry (so it lies below
//     2) and y as the walk left it; the accumulator rows of two U^T tiles are the operand
//     fragment directly (the key index taken in the walk's permuted order, see pcol);
//   - the in-chunk products P = K y^T and V^T P': bf16, K and V exactly, y as a hi + lo pair
//     (exact: y has 11 significant bits), P' = P o mask as a hi + lo pair (2^-17);
//   - the carry K^T diag(w) V: bf16, K exactly, w V as a hi + lo pair.
// bf16 operands keep float32's range; every scale is an exact power of two.
#include "gka_internal.hpp"

namespace gka {
namespace {

template <int D>
struct OutCfg {
  static constexpr int C = 64;              // tokens per chunk
  static constexpr int NW = D / 16;         // waves: one per 16 value features
  static constexpr int NT = NW * kWave;
  static constexpr int FT = D / 16;         // feature tiles
  static constexpr int KD = D / 32;         // 32-deep feature blocks
  static constexpr int ST = C / 16;         // token tiles
  static constexpr int SB = C / 32;         // 32-deep token blocks
  static constexpr int LDR = D + 8;         // row stride of the [C][D] tiles (16-bit elements)
  static constexpr int LDP = C + 8;         // row stride of the [C][C] P'^T tiles
  static constexpr int UPR = D / 8;         // 16-byte units per token row
  static constexpr int NU = C * UPR;        // units per [C][D] matrix
  static constexpr int NUT = NU / NT;       // units per thread
  static constexpr size_t szRow = (size_t)C * LDR * 2;
  static constexpr size_t szP = (size_t)C * LDP * 2;
  static constexpr size_t oK = 0;                  // K rows, permuted features (bf16)
  static constexpr size_t oV = oK + szRow;         // V rows (bf16)
  static constexpr size_t oY = oV + szRow;         // y rows, permuted features (fp16)
  static constexpr size_t oYh = oY + szRow;        // y as bf16 hi, permuted
  static constexpr size_t oYl = oYh + szRow;       // y as bf16 lo, permuted
  static constexpr size_t oPh = oYl + szRow;       // P'^T [t][s] bf16 hi
  static constexpr size_t oPl = oPh + szP;         // P'^T [t][s] bf16 lo
  static constexpr size_t oVec = oPl + szP;
  static constexpr size_t bytes = oVec + (size_t)5 * C * sizeof(float);
  static_assert(NU % NT == 0, "staging units must fill whole workgroups");
  static_assert(bytes <= 160 * 1024, "LDS budget of one CU exceeded");
};

// column of logical feature d in a permuted row (the token walk's order): within each block of
// 32, the four-element group 4g + 16h (g = 0..3, h = 0, 1) sits at 8g + 4h
__device__ constexpr int pcol(int d) {
  return (d & ~31) + 8 * ((d >> 2) & 3) + 4 * ((d >> 4) & 1) + (d & 3);
}

typedef __attribute__((address_space(3))) fp16x4_t lds_x4;

// Transposing fragment of a token-major bf16 matrix M[s][*] (row stride ld): fragment rows are
// the columns whose four-element groups start at coff (per lane, see below), k-slots the tokens
// s0 + 8 lg + m (m = 0..7) in natural order. Two 8-byte transposing reads: lane j of a group of
// 16 addresses row s0 + 8 lg + 4 h + j / 4 at its column group, lane i receives element i % 4
// of lanes i / 4 + 4 m, i.e. M[s0 + 8 lg + 4 h + m][column i].
__device__ inline bf16x8 frag_tr(const bf16* base, int ld, int s0, int coff, int lr, int lg) {
#if defined(__HIP_DEVICE_COMPILE__)
  const int s = s0 + 8 * lg + (lr >> 2);
  const fp16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_x4*)(base + s * ld + coff));
  const fp16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_x4*)(base + (s + 4) * ld + coff));
  const bf16x4 x = __builtin_bit_cast(bf16x4, a), y = __builtin_bit_cast(bf16x4, b);
  return bf16x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
#else
  return bf16x8{};
#endif
}

// x as hi + lo bf16 parts (hi = round(x), lo = round(x - hi))
__device__ inline bf16 hi_bf16(float x) { return (bf16)x; }
__device__ inline bf16 lo_bf16(float x, bf16 hi) { return (bf16)(x - (float)hi); }

template <int D>
__global__ __launch_bounds__(OutCfg<D>::NT) void output_kernel(WalkArgs A, int B, int Tmax,
                                                               int Hn, int N, int S, int J) {
  using Cfg = OutCfg<D>;
  using MB = Mma<bf16>;
  using MH = Mma<f16>;
  constexpr int C = Cfg::C, NT = Cfg::NT, FT = Cfg::FT, KD = Cfg::KD, ST = Cfg::ST;
  constexpr int SB = Cfg::SB, LDR = Cfg::LDR, LDP = Cfg::LDP, UPR = Cfg::UPR, NUT = Cfg::NUT;

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  bf16* Kr = reinterpret_cast<bf16*>(smem + Cfg::oK);
  bf16* Vr = reinterpret_cast<bf16*>(smem + Cfg::oV);
  f16* Yf = reinterpret_cast<f16*>(smem + Cfg::oY);
  bf16* Yh = reinterpret_cast<bf16*>(smem + Cfg::oYh);
  bf16* Yl = reinterpret_cast<bf16*>(smem + Cfg::oYl);
  bf16* Ph = reinterpret_cast<bf16*>(smem + Cfg::oPh);
  bf16* Pl = reinterpret_cast<bf16*>(smem + Cfg::oPl);
  float* v_cl = reinterpret_cast<float*>(smem + Cfg::oVec);  // [C] in-chunk log2 gate prefix
  float* v_w = v_cl + C;     // [C] carry weights 2^(cl_C - cl_s) beta_s
  float* v_bt = v_w + C;     // [C] write gates beta_s
  float* v_phi = v_bt + C;   // [C] phi_t
  float* v_gph = v_phi + C;  // [C] Gam_t phi_t

  const int seg = blockIdx.x;
  int b, h;
  head_of(A, blockIdx.y, Hn, b, h);
  const int bh = b * Hn + h;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  int tid = threadIdx.x, lane = tid % kWave;
  int lr = lane % 16, lg = lane / 16;
  auto refresh = [&]() { asm volatile("" : "+v"(tid), "+v"(lane), "+v"(lr), "+v"(lg)); };
  long long seq0;
  int Tlen;
  seq_range(A, b, Tmax, seq0, Tlen);
  const int last = last_segment(Tlen, J, C);
  if (seg > last) return;
  const int c_begin = seg * J;
  const int c_end = min(min(N, c_begin + J), (Tlen + C - 1) / C);
  const long long tok_stride = (long long)Hn * D;
  const uint32_t tok_bytes = (uint32_t)Hn * D * 2u;  // 64 rows span < 2^31 bytes (host check)
  const bf16* kg = static_cast<const bf16*>(A.k);
  const bf16* vg = static_cast<const bf16*>(A.v);
  bf16* og = static_cast<bf16*>(A.o);  // holds the walk's y (fp16) until overwritten with o
  const int vf = 16 * wave;            // the wave's value features vf .. vf + 15

  // ---- float32 state: U^T tiles (rows = key features 16 kt + 4 lg + i, column = value
  // feature vf + lr), i.e. U[vf + lr][16 kt + 4 lg .. + 3] in a lane -------------------------
  f32x4 Ust[FT];
#pragma unroll
  for (int kt = 0; kt < FT; ++kt) Ust[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (A.in_u) {
    const float* iu = A.in_u + bh * A.in_bh + seg * A.in_seg;
#pragma unroll
    for (int kt = 0; kt < FT; ++kt)
      Ust[kt] = *reinterpret_cast<const f32x4*>(iu + (size_t)(vf + lr) * D + 16 * kt + 4 * lg);
  }

  // the next chunk's K, V and y rows (16-byte units along a token row) and gates, phi (lane =
  // token), loaded into registers one chunk ahead; rows past the end read as 0
  bf16x8 kin[NUT], vin[NUT];
  f16x8 yin[NUT];
  float gin = 1.0f, bin = 1.0f, pin = 0.0f;
  const float* bsrc = A.beta ? A.beta : A.gamma;
  auto load_rows = [&](int chn) {
    refresh();
    const int chv = chn < c_end ? chn : c_end - 1;
    const int t0n = chv * C;
    const int nvn = chn < c_end ? min(C, Tlen - t0n) : 0;
    const long long row0 = (seq0 + t0n) * tok_stride + (long long)h * D;
    const uint32_t valid = nvn > 0 ? (uint32_t)(nvn - 1) * tok_bytes + D * 2u : 0u;
    const auto rk = buffer_rsrc(kg + row0, valid);
    const auto rv = buffer_rsrc(vg + row0, valid);
    const auto ry = buffer_rsrc(og + row0, valid);
#pragma unroll
    for (int k = 0; k < NUT; ++k) {
      const int u = tid + k * NT;
      const int tt = (uint32_t)u / UPR, cu = (uint32_t)u % UPR;
      const uint32_t off = (uint32_t)tt * tok_bytes + (uint32_t)cu * 16u;
      kin[k] = buffer_load16<bf16x8>(rk, off);
      vin[k] = buffer_load16<bf16x8>(rv, off);
      yin[k] = buffer_load16<f16x8>(ry, off);
    }
    const uint32_t gvalid = nvn > 0 ? (uint32_t)(nvn - 1) * Hn * 4u + 4u : 0u;
    const long long grow = (seq0 + t0n) * Hn + h;
    gin = buffer_load4f(buffer_rsrc(A.gamma + grow, gvalid), (uint32_t)lane * Hn * 4u);
    bin = buffer_load4f(buffer_rsrc(bsrc + grow, gvalid), (uint32_t)lane * Hn * 4u);
    pin = buffer_load4f(buffer_rsrc(A.phi + grow, gvalid), (uint32_t)lane * Hn * 4u);
  };

  // P' tiles (s tile, t tile): the ten with s tile <= t tile, then the two zero tiles that
  // complete the 32-deep token blocks of t tiles 0 and 2 (s = 16..31 of t tile 0, s = 48..63 of
  // t tile 2)
  constexpr int kTiles = 12;
  auto tile_s = [](int i) { return i < 10 ? (i >= 6 ? i - 6 : i >= 3 ? i - 3 : i >= 1 ? i - 1 : 0) : (i == 10 ? 1 : 3); };
  auto tile_t = [](int i) { return i < 10 ? (i >= 6 ? 3 : i >= 3 ? 2 : i >= 1 ? 1 : 0) : (i == 10 ? 0 : 2); };

  load_rows(c_begin);
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0)

  for (int ch = c_begin; ch < c_end; ++ch) {
    refresh();
    const int t0 = ch * C;
    const int nv = min(C, Tlen - t0);
    lds_barrier();  // the last chunk's LDS reads are done

    // ---- gates (every wave; lane = token) ---------------------------------------------------
    float l2 = 0.0f, bt_l = 1.0f, ph_l = 0.0f;  // tokens past the end: gamma = 1, phi = 0
    if (lane < nv) {
      l2 = log2_gate(gin);
      if (A.beta) bt_l = bin;
      ph_l = pin;
    }
    const float cl = scan_add<kWave>(l2);
    const float clast = lane_value(cl, C - 1);
    const float gam = fast_exp2(cl);
    const float gC = lane_value(gam, C - 1);
    if (wave == 0) {
      v_cl[lane] = cl;
      v_w[lane] = fast_exp2(fminf(clast - cl, 0.0f)) * bt_l;
      v_bt[lane] = bt_l;
      v_phi[lane] = ph_l;
      v_gph[lane] = gam * ph_l;
    }
    // ---- stage K, V, y (and y as bf16 hi + lo) ----------------------------------------------
#pragma unroll
    for (int k = 0; k < NUT; ++k) {
      const int u = tid + k * NT;
      const int tt = (uint32_t)u / UPR, cu = (uint32_t)u % UPR;
      const bf16x8 kv = kin[k];
      const f16x8 yv = yin[k];
      *reinterpret_cast<bf16x4*>(Kr + tt * LDR + pcol(8 * cu)) = bf16x4{kv[0], kv[1], kv[2], kv[3]};
      *reinterpret_cast<bf16x4*>(Kr + tt * LDR + pcol(8 * cu + 4)) = bf16x4{kv[4], kv[5], kv[6], kv[7]};
      *reinterpret_cast<bf16x8*>(Vr + tt * LDR + 8 * cu) = vin[k];
      *reinterpret_cast<f16x4*>(Yf + tt * LDR + pcol(8 * cu)) = f16x4{yv[0], yv[1], yv[2], yv[3]};
      *reinterpret_cast<f16x4*>(Yf + tt * LDR + pcol(8 * cu + 4)) = f16x4{yv[4], yv[5], yv[6], yv[7]};
      bf16x8 hi, lo;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bf16 x = hi_bf16((float)yv[i]);
        hi[i] = x;
        lo[i] = lo_bf16((float)yv[i], x);
      }
      *reinterpret_cast<bf16x4*>(Yh + tt * LDR + pcol(8 * cu)) = bf16x4{hi[0], hi[1], hi[2], hi[3]};
      *reinterpret_cast<bf16x4*>(Yh + tt * LDR + pcol(8 * cu + 4)) = bf16x4{hi[4], hi[5], hi[6], hi[7]};
      *reinterpret_cast<bf16x4*>(Yl + tt * LDR + pcol(8 * cu)) = bf16x4{lo[0], lo[1], lo[2], lo[3]};
      *reinterpret_cast<bf16x4*>(Yl + tt * LDR + pcol(8 * cu + 4)) = bf16x4{lo[4], lo[5], lo[6], lo[7]};
    }
    load_rows(ch + 1);
    lds_barrier();

    // ---- P' = (K y^T) o mask, written transposed ([t][s]) as bf16 hi + lo -------------------
    refresh();
    for (int i = wave; i < kTiles; i += Cfg::NW) {
      const int st = tile_s(i), tt = tile_t(i);
      const int t = 16 * tt + lr;
      const int s0 = 16 * st + 4 * lg;
      bf16x4 hi4 = {}, lo4 = {};
      if (i < 10) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(Kr + (16 * st + lr) * LDR + 32 * kk + 8 * lg);
          const bf16x8 yh = *reinterpret_cast<const bf16x8*>(Yh + t * LDR + 32 * kk + 8 * lg);
          const bf16x8 yl = *reinterpret_cast<const bf16x8*>(Yl + t * LDR + 32 * kk + 8 * lg);
          acc = MB::mma(a, yh, acc);
          acc = MB::mma(a, yl, acc);
        }
        const float cl_t = v_cl[t], ph_t = v_phi[t];
        const f32x4 cls = *reinterpret_cast<const f32x4*>(v_cl + s0);
        const f32x4 bts = *reinterpret_cast<const f32x4*>(v_bt + s0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p = s0 + j <= t ? acc[j] * fast_exp2(fminf(cl_t - cls[j], 0.0f)) * bts[j] * ph_t : 0.0f;
          const bf16 x = hi_bf16(p);
          hi4[j] = x;
          lo4[j] = lo_bf16(p, x);
        }
      }
      *reinterpret_cast<bf16x4*>(Ph + t * LDP + s0) = hi4;
      *reinterpret_cast<bf16x4*>(Pl + t * LDP + s0) = lo4;
    }

    // ---- o^T = U0 (y^T diag(Gam phi)) for the wave's features (fp16, U0 times 2^-fe) ---------
    f32x4 o[ST];
    {
      float um = 0.0f;
#pragma unroll
      for (int kt = 0; kt < FT; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) um = fmaxf(um, fabsf(Ust[kt][j]));
      const int fe = pow2_exponent(wave_max(um), 100);
      const float usc = exp2_int(-fe), uback = exp2_int(fe);
      f16x8 ua[KD];
#pragma unroll
      for (int kk = 0; kk < KD; ++kk) {
        const f32x4 x0 = Ust[2 * kk] * usc, x1 = Ust[2 * kk + 1] * usc;
        ua[kk] = f16x8{(f16)x0[0], (f16)x0[1], (f16)x0[2], (f16)x0[3],
                       (f16)x1[0], (f16)x1[1], (f16)x1[2], (f16)x1[3]};
      }
#pragma unroll
      for (int tt = 0; tt < ST; ++tt) {
        o[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) {
          const f16x8 yb = *reinterpret_cast<const f16x8*>(Yf + (16 * tt + lr) * LDR + 32 * kk + 8 * lg);
          o[tt] = MH::mma(ua[kk], yb, o[tt]);
        }
        o[tt] = o[tt] * (v_gph[16 * tt + lr] * uback);
      }
    }
    // V^T fragments of the wave's features (rows vf + lr, token slots 8 lg.. of block sb): the
    // A operands of V^T P' and, weighted, the B operands of the carry
    bf16x8 vt[SB];
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) vt[sb] = frag_tr(Vr, LDR, 32 * sb, vf + 4 * (lr & 3), lr, lg);
    lds_barrier();  // P'^T is complete

    // ---- o^T += V^T P' (token blocks at or before the t tile), stored --------------------------
    refresh();
    {
      const auto ro = buffer_rsrc(og + (seq0 + t0) * tok_stride + (long long)h * D,
                                  (uint32_t)(nv - 1) * tok_bytes + D * 2u);
#pragma unroll
      for (int tt = 0; tt < ST; ++tt) {
        const int t = 16 * tt + lr;
#pragma unroll
        for (int sb = 0; sb < SB; ++sb) {
          if (32 * sb <= 16 * tt + 15) {
            const bf16x8 ph = *reinterpret_cast<const bf16x8*>(Ph + t * LDP + 32 * sb + 8 * lg);
            const bf16x8 pl = *reinterpret_cast<const bf16x8*>(Pl + t * LDP + 32 * sb + 8 * lg);
            o[tt] = MB::mma(vt[sb], ph, o[tt]);
            o[tt] = MB::mma(vt[sb], pl, o[tt]);
          }
        }
        // lane (token t, group lg) holds o[t][vf + 4 lg .. + 3]; tokens past the end are dropped
        const bf16x4 ov = {(bf16)o[tt][0], (bf16)o[tt][1], (bf16)o[tt][2], (bf16)o[tt][3]};
        buffer_store8(ov, ro, (uint32_t)t * tok_bytes + (uint32_t)(vf + 4 * lg) * 2u);
      }
    }

    // ---- carry: U^T <- Gam_C U^T + K^T (diag(w) V) ------------------------------------------
    {
      bf16x8 wvh[SB], wvl[SB];
#pragma unroll
      for (int sb = 0; sb < SB; ++sb) {
        const f32x4 w0 = *reinterpret_cast<const f32x4*>(v_w + 32 * sb + 8 * lg);
        const f32x4 w1 = *reinterpret_cast<const f32x4*>(v_w + 32 * sb + 8 * lg + 4);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float x = (float)vt[sb][j] * (j < 4 ? w0[j] : w1[j - 4]);
          const bf16 hx = hi_bf16(x);
          wvh[sb][j] = hx;
          wvl[sb][j] = lo_bf16(x, hx);
        }
      }
#pragma unroll
      for (int kt = 0; kt < FT; ++kt) {
        f32x4 acc = Ust[kt] * gC;
#pragma unroll
        for (int sb = 0; sb < SB; ++sb) {
          const bf16x8 ka = frag_tr(Kr, LDR, 32 * sb, pcol(16 * kt + 4 * (lr & 3)), lr, lg);
          acc = MB::mma(ka, wvh[sb], acc);
          acc = MB::mma(ka, wvl[sb], acc);
        }
        Ust[kt] = acc;
      }
    }
  }
  if (A.out_u && seg == last) {
    float* ou = A.out_u + (size_t)bh * D * D;
#pragma unroll
    for (int kt = 0; kt < FT; ++kt)
      *reinterpret_cast<f32x4*>(ou + (size_t)(vf + lr) * D + 16 * kt + 4 * lg) = Ust[kt];
  }
}

template <int D>
hipError_t launch_out(const FwdPlan& pl, const WalkArgs& a, hipStream_t stream) {
  using Cfg = OutCfg<D>;
  auto kern = output_kernel<D>;
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(kern), (int)Cfg::bytes, lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(pl.S, pl.B * pl.H), dim3(Cfg::NT), Cfg::bytes, stream, a, pl.B,
                     pl.T, pl.H, pl.N, pl.S, pl.J);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_output(const FwdPlan& pl, const WalkArgs& a, hipStream_t stream) {
  switch (pl.D) {
    case 32: return launch_out<32>(pl, a, stream);
    case 64: return launch_out<64>(pl, a, stream);
    case 128: return launch_out<128>(pl, a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace gka
