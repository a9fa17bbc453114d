// Segment summaries of gka_fwd_chunked for the token-owning walk's configurations (bf16 inputs,
// chunks of 64 tokens, D = 64 and 128): for every segment but the last, the state its tokens
// reach from the zero state and the log2 of its gate product (the affine-scan elements of the
// segment scan; "Methodology in Plain English" on the ai.info summary of arXiv 2511.21016: only
// the chunk-initial states are carried sequentially).
#include "gka_internal.hpp"

#include <type_traits>

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
// (about 2^-17 relative), formed once per block when its rows are staged to LDS.
//
// Two kinds of wave share each SIMD. A product wave (waves 0..3, one per SIMD) holds the float32
// tiles of dH = K^T diag(w) K and dU = V^T diag(w) K for its row tiles (two at D = 128, w and
// 7 - w, which pair the longer and the shorter row of dH's upper triangle, so that each wave
// has 9 tiles of dH and 16 of dU; one at D = 64, all columns) and only issues products, with
// operands from transposing LDS reads of the block's rows (the walk's permuted token order).
// A staging wave (waves 4..7) only moves data: it loads the rows of the block after next into
// registers (bounds-checked buffer loads: rows past the end read as 0), computes the next
// block's weights from its gates, and writes the next block's K, V and weighted-key rows to the
// other of two LDS slots. One barrier per block separates the slots' uses, so the matrix pipe of
// a SIMD runs its product wave while its staging wave works.
template <int D>
struct SumCfg {
  static constexpr int CB = 64;                // tokens per block (a chunk)
  static constexpr int KB = CB / 32;           // 32-deep token blocks per block
  static constexpr int NWC = 4;                // product waves, one per SIMD
  static constexpr int NWS = 4;                // staging waves, one per SIMD
  static constexpr int NW = NWC + NWS;
  static constexpr int NT = NW * kWave;
  static constexpr int NTS = NWS * kWave;      // staging threads
  static constexpr int FT = D / 16;            // feature tiles
  static constexpr bool TRI = D == 128;        // dH from its upper-triangle tiles
  // tiles of a product wave: NR row tiles by NC column tiles (D = 128: rows w and 7 - w, all
  // columns; D = 64: row w, all columns; D = 32: row w / 2, column w % 2)
  static constexpr int NR = FT >= NWC ? FT / NWC : 1;
  static constexpr int NC = FT >= NWC ? FT : FT * FT / NWC;
  static constexpr int LDR = D + 16;  // row stride of the rows (bf16): 8 banks apart, so the
                                      // 16 rows of a transposing read share no bank
  static constexpr int VEC = 8, UPR = D / VEC, NU = CB * UPR;
  static constexpr int NUS = NU / NTS;         // 16-byte units per staging thread and matrix
  static constexpr size_t szRows = (size_t)CB * LDR * 2;
  static constexpr size_t szSlot = 4 * szRows;  // rows of K, V, (w k) hi and (w k) lo
  static constexpr size_t bytes = 2 * szSlot + (size_t)NWS * CB * sizeof(float);  // + weights
  static_assert(D == 32 || D == 64 || D == 128, "summary tiling");
  static_assert(NU % NTS == 0 && NR * NC * NWC == FT * FT, "summary work split");
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

template <int V>
using IC = std::integral_constant<int, V>;

template <int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void summary_tok_kernel(WalkArgs A, int B, int Tmax, int Hn, int N, int S, int J) {
  using Cfg = SumCfg<D>;
  using M = Mma<bf16>;
  typedef bf16x8 Frag;
  constexpr int CB = Cfg::CB, LDR = Cfg::LDR, FT = Cfg::FT, NR = Cfg::NR, NC = Cfg::NC;
  constexpr int UPR = Cfg::UPR, NUS = Cfg::NUS, NTS = Cfg::NTS, NWC = Cfg::NWC;
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
  auto block_t0 = [&](int p) { return t_begin + (NB - 1 - p) * CB; };

  if (wave >= NWC) {
    // ======== staging wave ========
    const int ts = tid - NWC * kWave;  // 0 .. NTS - 1
    float* v_wl = reinterpret_cast<float*>(smem + 2 * Cfg::szSlot) + (wave - NWC) * CB;
    const long long tok_stride = (long long)Hn * D;
    const uint32_t tok_bytes = (uint32_t)Hn * D * 2u;
    // rows of two blocks in registers (register set q holds block p with p % 2 == q)
    bf16x8 kr[2][NUS], vr[2][NUS];
    float gr[2], br[2];  // gates and write gates (lane = token)
    // the write gates are read from the gates when there are none (and then not used)
    const float* bsrc = A.beta ? A.beta : A.gamma;
    float suffix = 0.0f;  // log2 gate sum of the blocks already weighted (the later ones)
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
      for (int k = 0; k < NUS; ++k) {
        const int u = ts + k * NTS;
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
    // weights of block p (lane = token) from its gates in register set q, into this wave's
    // v_wl: 2^(log2 of the gates after the token), times the token's write gate
    // (the asm statements below tie the register sets to the phase that consumes them: without
    // them the compiler hoists their arithmetic above the previous barrier, and with it the wait
    // for loads issued one phase ago instead of two)
    auto weigh = [&](int p, int q) __attribute__((always_inline)) {
      asm volatile("" : "+v"(gr[q]), "+v"(br[q]));
      const int nv = p < NB ? min(CB, t_end - block_t0(p)) : 0;
      const float l2 = lane < nv ? log2_gate(gr[q]) : 0.0f;
      const float cl = scan_add<kWave>(l2);
      const float clast = lane_value(cl, CB - 1);
      const float bw = A.beta ? br[q] : 1.0f;
      v_wl[lane] = fast_exp2(fminf(clast - cl + suffix, 0.0f)) * bw;
      suffix += clast;
    };
    // rows of register set q to slot `slot`, with the weighted keys (weights from v_wl)
    // (the weights of the thread's tokens are read before any row is written: a read after a
    // write would wait for the write)
    auto write_block = [&](int slot, int q) __attribute__((always_inline)) {
      refresh();
#pragma unroll
      for (int k = 0; k < NUS; ++k) asm volatile("" : "+v"(kr[q][k]), "+v"(vr[q][k]));
      float w[NUS];
#pragma unroll
      for (int k = 0; k < NUS; ++k) w[k] = v_wl[(uint32_t)(ts + k * NTS) / UPR];
#pragma unroll
      for (int k = 0; k < NUS; ++k) {
        const int u = ts + k * NTS;
        const int tt = (uint32_t)u / UPR, cu = (uint32_t)u % UPR;  // u >= 0
        const int o = tt * LDR + cu * 8;
        bf16x8 hi, lo;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float x = (float)kr[q][k][j] * w[k];
          hi[j] = (bf16)x;
          lo[j] = (bf16)(x - (float)hi[j]);
        }
        *reinterpret_cast<bf16x8*>(krows(slot) + o) = kr[q][k];
        *reinterpret_cast<bf16x8*>(vrows(slot) + o) = vr[q][k];
        *reinterpret_cast<bf16x8*>(hirows(slot) + o) = hi;
        *reinterpret_cast<bf16x8*>(lorows(slot) + o) = lo;
      }
    };
    // block p + 1 (register set q) to slot q, and set q reloaded with block p + 3 (every phase
    // stages and loads, also past the last block -- zero rows from loads with an empty range --
    // so that every path through the loop has the same loads in flight)
    auto stage = [&](int p, int q) __attribute__((always_inline)) {
      weigh(p + 1, q);
      write_block(q, q);
      load_block(p + 3, q);
    };
    load_block(0, 0);
    load_block(1, 1);
    weigh(0, 0);
    write_block(0, 0);
    load_block(2, 0);
    lds_barrier();
    for (int p = 0; p < NB; p += 2) {
      stage(p, 1);
      lds_barrier();  // slot (p + 1) % 2 is written; slot p % 2 has been read
      stage(p + 1, 0);
      lds_barrier();
    }
    if (wave == NWC && lane == 0) A.log2g_out[(long long)bh * S + seg] = suffix;
    return;
  }

  // ======== product wave ========
  // (one instantiation per wave: its row tiles, and with TRI which tiles of dH it holds, are
  // compile-time constants)
  auto run = [&](auto W) __attribute__((always_inline)) {
    constexpr int w = decltype(W)::value;
    auto row = [](int r) {
      return Cfg::TRI ? (r == 0 ? w : FT - 1 - w) : NC == FT ? w * NR + r : w / (FT / NC);
    };
    auto col = [](int c) { return NC == FT ? c : (w % (FT / NC)) * NC + c; };
    // tile (r, c) of dH is held when it lies on or above the diagonal (with TRI; at D = 32 the
    // wave below it holds dU only)
    auto held = [&](int r, int c) { return Cfg::TRI || NC < FT ? col(c) >= row(r) : true; };
    f32x4 Hacc[NR][NC], Uacc[NR][NC];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        Hacc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
        Uacc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    // block p from slot p % 2: per 32-token block the A operands (K^T and V^T of the own row
    // tiles), then column by column the B operands (weighted keys hi and lo) and the products,
    // the hi halves of a column's tiles before its lo halves
    auto accumulate = [&](int p) __attribute__((always_inline)) {
      refresh();
      const int slot = p & 1;
      const bf16* kb = krows(slot);
      const bf16* vb = vrows(slot);
      const bf16* hb = hirows(slot);
      const bf16* lb = lorows(slot);
      const int cq = 4 * (lr & 3);
#pragma unroll
      for (int kc = 0; kc < Cfg::KB; ++kc) {
        const int s0 = 32 * kc + 4 * lg, s1 = s0 + 16;
        Frag ak[NR], av[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          ak[r] = frag_trans_bf16<LDR>(kb, s0, s1, 16 * row(r) + cq, lr);
          av[r] = frag_trans_bf16<LDR>(vb, s0, s1, 16 * row(r) + cq, lr);
        }
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const Frag bhf = frag_trans_bf16<LDR>(hb, s0, s1, 16 * col(c) + cq, lr);
          const Frag blf = frag_trans_bf16<LDR>(lb, s0, s1, 16 * col(c) + cq, lr);
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            if (held(r, c)) Hacc[r][c] = M::mma(ak[r], bhf, Hacc[r][c]);
            Uacc[r][c] = M::mma(av[r], bhf, Uacc[r][c]);
          }
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            if (held(r, c)) Hacc[r][c] = M::mma(ak[r], blf, Hacc[r][c]);
            Uacc[r][c] = M::mma(av[r], blf, Uacc[r][c]);
          }
        }
      }
    };
    lds_barrier();  // block 0 is staged
    for (int p = 0; p < NB; p += 2) {
      accumulate(p);
      lds_barrier();
      if (p + 1 < NB) accumulate(p + 1);
      lds_barrier();
    }
    float* oh = A.sum_h + bh * A.sum_bh + seg * A.sum_seg;
    float* ou = A.sum_u + bh * A.sum_bh + seg * A.sum_seg;
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        // a tile (a, b) holds X[16 a + 4 lg + i][16 b + lr], i = 0..3. dH (symmetric) is written
        // transposed as the rows 16 b + lr (one 16-byte store), and for an upper tile also as
        // the mirror rows 16 a + 4 lg + i; dU (rows = value features) as four scattered stores
        const int a = row(r), bc = col(c);
        if (held(r, c)) {
          const f32x4 x = Hacc[r][c];
          *reinterpret_cast<f32x4*>(oh + (size_t)(16 * bc + lr) * D + 16 * a + 4 * lg) = x;
          if ((Cfg::TRI || NC < FT) && bc != a) {  // (with every tile held, no mirrors)
#pragma unroll
            for (int i = 0; i < 4; ++i) oh[(size_t)(16 * a + 4 * lg + i) * D + 16 * bc + lr] = x[i];
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
          ou[(size_t)(16 * a + 4 * lg + i) * D + 16 * bc + lr] = Uacc[r][c][i];
      }
  };
  switch (wave) {
    case 0: run(IC<0>{}); break;
    case 1: run(IC<1>{}); break;
    case 2: run(IC<2>{}); break;
    default: run(IC<3>{}); break;
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
  return pl.dtype == 0 && pl.C == 64 && (pl.D == 32 || pl.D == 64 || pl.D == 128) &&
         block_bytes < (1LL << 31);
}

hipError_t launch_summary_tok(const FwdPlan& pl, const WalkArgs& a, hipStream_t stream) {
  switch (pl.D) {
    case 32: return launch_sum<32>(pl, a, stream);
    case 64: return launch_sum<64>(pl, a, stream);
    case 128: return launch_sum<128>(pl, a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace gka
