// Segment summaries of gka_fwd_chunked for the token-owning walk's configurations (bf16 inputs,
// chunks of 64 tokens, D = 64 and 128): for every segment but the last, the state its tokens
// reach from the zero state and the log2 of its gate product (the affine-scan elements of the
// segment scan; "Methodology in Plain English" on the ai.info summary of arXiv 2511.21016: only
// the chunk-initial states are carried sequentially).
#include "gka_internal.hpp"

namespace gka {
namespace {

// ---- segment summaries -------------------------------------------------------------------
// For each (segment, head): the state reached from a zero state over the segment's tokens and
// the segment's total log2 gate. Unrolling the carry H <- Gam_C H + K^T diag(w) K over the
// segment gives one weighted sum over its tokens,
//   dH = sum_s w_s k_s k_s^T,  dU = sum_s w_s v_s k_s^T,  w_s = 2^(log2 of the gates after s)
// (times beta_s with the write gate),
// so the tokens are taken in blocks of 64 from the last block to the first, with the gate sum
// of the blocks already taken as the suffix of every weight, and no rescaling of the state.
// Matrix-core operands are bf16: K and V exactly, the weighted keys w k as a hi + lo pair
// (about 2^-17 relative), formed once per block when its rows are staged to LDS. Eight waves,
// two per SIMD; wave w holds the float32 tiles (row tiles RT*(w % 2).., column tiles
// CT*(w / 2)..) of dH and of dU (rows = value features), computed as dH = K^T diag(w) K and
// dU = V^T diag(w) K, so that both take the weighted keys of the wave's column tiles as their
// second operand. Per block every wave reads its operand fragments with transposing reads of
// the block's K, V and weighted-key rows in LDS (bf16, padded rows), in the walk's permuted
// token order; the block's weights are computed from its gates in registers just before its
// rows are staged. The rows of the next block go to the other of two LDS slots, from registers
// loaded two blocks ahead with bounds-checked buffer loads (rows past the end read as 0): one
// barrier per block.
template <int D>
struct SumCfg {
  static constexpr int CB = 64;                // tokens per block (a chunk)
  static constexpr int KB = CB / 32;           // 32-deep token blocks per block
  static constexpr int NW = 8;                 // waves, two per SIMD
  static constexpr int NT = NW * kWave;
  static constexpr int FT = D / 16;
  static constexpr int RT = FT / 2;            // state row tiles per wave (more rows than
  static constexpr int CT = FT / 4;            // columns: fewer operand fragments per product)
  static constexpr int LDR = D + 16;  // row stride of the rows (bf16): 8 banks apart, so the
                                      // 16 rows of a transposing read share no bank
  static constexpr int VEC = 8, UPR = D / VEC, NU = CB * UPR;
  static constexpr int NUT = (NU + NT - 1) / NT;  // 16-byte units per thread and matrix
  static constexpr size_t szRows = (size_t)CB * LDR * 2;
  static constexpr size_t szSlot = 4 * szRows;  // rows of K, V, (w k) hi and (w k) lo
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
  auto hirows = [&](int slot) { return krows(slot) + 2 * CB * LDR; };  // (w k) hi
  auto lorows = [&](int slot) { return krows(slot) + 3 * CB * LDR; };  // (w k) lo

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
  auto load_block = [&](int p, int q) __attribute__((always_inline)) {
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
  // rows of register set q to slot `slot`, with the weighted keys (weights wl, token-indexed)
  auto write_block = [&](int slot, int q, const float* wl) __attribute__((always_inline)) {
    refresh();
#pragma unroll
    for (int k = 0; k < NUT; ++k) {
      const int u = tid + k * NT;
      if (NU % NT == 0 || u < NU) {
        const int tt = (uint32_t)u / UPR, cu = (uint32_t)u % UPR;  // u >= 0
        const int o = tt * LDR + cu * 8;
        *reinterpret_cast<bf16x8*>(krows(slot) + o) = kr[q][k];
        *reinterpret_cast<bf16x8*>(vrows(slot) + o) = vr[q][k];
        const float w = wl[tt];
        bf16x8 hi, lo;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float x = (float)kr[q][k][j] * w;
          hi[j] = (bf16)x;
          lo[j] = (bf16)(x - (float)hi[j]);
        }
        *reinterpret_cast<bf16x8*>(hirows(slot) + o) = hi;
        *reinterpret_cast<bf16x8*>(lorows(slot) + o) = lo;
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
  auto weigh = [&](int p, int q) __attribute__((always_inline)) {
    const int nv = p < NB ? min(CB, t_end - block_t0(p)) : 0;
    const float l2 = lane < nv ? log2_gate(gr[q]) : 0.0f;
    const float cl = scan_add<kWave>(l2);
    const float clast = lane_value(cl, CB - 1);
    const float bw = A.beta ? br[q] : 1.0f;
    v_wl[(p & 1) * CB + lane] = fast_exp2(fminf(clast - cl + suffix, 0.0f)) * bw;
    suffix += clast;
  };
  // block p from slot p % 2 into the state: every fragment of the block first, then the
  // products, the hi halves of all tiles before the lo halves (dependent products far apart)
  auto accumulate = [&](int p) __attribute__((always_inline)) {
    refresh();
    const int slot = p & 1;
    const bf16* kb = krows(slot);
    const bf16* vb = vrows(slot);
    const bf16* hb = hirows(slot);
    const bf16* lb = lorows(slot);
    const int cq = 4 * (lr & 3);
    constexpr int KB = Cfg::KB;
    // A operands: K^T and V^T row fragments; B operands: the weighted keys of the column tiles,
    // hi and lo (shared by the two products: dH = K^T diag(w) K, dU = V^T diag(w) K)
    Frag ak[KB][RT], av[KB][RT], bh[KB][CT], bl[KB][CT];
#pragma unroll
    for (int kc = 0; kc < KB; ++kc) {
      const int s0 = 32 * kc + 4 * lg, s1 = s0 + 16;
#pragma unroll
      for (int jr = 0; jr < RT; ++jr) {
        ak[kc][jr] = frag_trans_bf16<LDR>(kb, s0, s1, 16 * (a0 + jr) + cq, lr);
        av[kc][jr] = frag_trans_bf16<LDR>(vb, s0, s1, 16 * (a0 + jr) + cq, lr);
      }
#pragma unroll
      for (int jc = 0; jc < CT; ++jc) {
        bh[kc][jc] = frag_trans_bf16<LDR>(hb, s0, s1, 16 * (b0 + jc) + cq, lr);
        bl[kc][jc] = frag_trans_bf16<LDR>(lb, s0, s1, 16 * (b0 + jc) + cq, lr);
      }
    }
#pragma unroll
    for (int kc = 0; kc < KB; ++kc) {
#pragma unroll
      for (int jc = 0; jc < CT; ++jc)
#pragma unroll
        for (int jr = 0; jr < RT; ++jr) {
          Hst[jr][jc] = M::mma(ak[kc][jr], bh[kc][jc], Hst[jr][jc]);
          Ust[jr][jc] = M::mma(av[kc][jr], bh[kc][jc], Ust[jr][jc]);
        }
#pragma unroll
      for (int jc = 0; jc < CT; ++jc)
#pragma unroll
        for (int jr = 0; jr < RT; ++jr) {
          Hst[jr][jc] = M::mma(ak[kc][jr], bl[kc][jc], Hst[jr][jc]);
          Ust[jr][jc] = M::mma(av[kc][jr], bl[kc][jc], Ust[jr][jc]);
        }
    }
  };
  // phase p: the rows of block p + 1 (register set (p + 1) % 2) go to slot (p + 1) % 2, that set
  // is reloaded with block p + 3, and block p is accumulated from slot p % 2. The two waves of a
  // SIMD (w and w + 4) take the two halves in opposite orders: while one issues its products,
  // the other stages, so the matrix pipe stays busy through the staging.
  const bool stage_first = wave >= Cfg::NW / 2;
  // (every phase stages and loads, also past the last block -- zero rows from loads with an
  // empty range -- so that every path through the loop has the same loads in flight)
  auto stage = [&](int p, int q) __attribute__((always_inline)) {
    weigh(p + 1, q);
    write_block(q, q, v_wl + ((p + 1) & 1) * CB);
    load_block(p + 3, q);
  };
  load_block(0, 0);
  load_block(1, 1);
  weigh(0, 0);
  write_block(0, 0, v_wl);
  load_block(2, 0);
  lds_barrier();
  // (one loop per order: with the order fixed inside a loop the compiler tracks which loads
  // are still in flight, and waits for the older register set only)
  if (stage_first) {
    for (int p = 0; p < NB; p += 2) {
      stage(p, 1);
      accumulate(p);
      lds_barrier();  // slot (p + 1) % 2 is written; slot p % 2 is read
      stage(p + 1, 0);
      if (p + 1 < NB) accumulate(p + 1);
      lds_barrier();
    }
  } else {
    for (int p = 0; p < NB; p += 2) {
      accumulate(p);
      stage(p, 1);
      lds_barrier();
      if (p + 1 < NB) accumulate(p + 1);
      stage(p + 1, 0);
      lds_barrier();
    }
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

}  // namespace

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

}  // namespace gka
