// Layout helpers of the token-owning kernels (the fused chunk walk and the backward pass):
// permuted feature columns, transposing fragment reads, register-class hints, compile-time
// loops. The reduction index of a product is taken in a permuted order within each block of
// 32: k-slot j of lane group g stands for index 16 (j / 4) + 4 g + j % 4, so that the
// accumulator rows of two 16x16 output tiles, as a lane holds them, are the B operand fragment
// of the next product.
#pragma once

#include <type_traits>

#include "gka_common.hpp"

namespace gka {

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
// so lane q addresses row s + q / 4 at the four columns of lane group q % 4. x: the lane's XOR
// of the element offset in the rows it addresses (a row-dependent unit permutation of the
// layout, the same for both reads; 0 for plain rows).
template <int LDD>
__device__ inline f16x8 frag_trans(const f16* base, int s0, int s1, int coff, int lr, int x = 0) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(3))) fp16x4_t lds_fp16x4;
  const int r = lr >> 2;
  const fp16x4_t x0 = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4*)(base + (s0 + r) * LDD + (coff ^ x)));
  const fp16x4_t y0 = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4*)(base + (s1 + r) * LDD + (coff ^ x)));
  return f16x8{(f16)x0[0], (f16)x0[1], (f16)x0[2], (f16)x0[3],
               (f16)y0[0], (f16)y0[1], (f16)y0[2], (f16)y0[3]};
#else
  return f16x8{};
#endif
}

// The first half of frag_trans: the k-slots of tokens s + m, m = 0..3, only (one transposing
// read)
template <int LDD>
__device__ inline f16x4 frag_trans_half(const f16* base, int s, int coff, int lr, int xo = 0) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(3))) fp16x4_t lds_fp16x4;
  const fp16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4*)(base + (s + (lr >> 2)) * LDD + (coff ^ xo)));
  return f16x4{(f16)x[0], (f16)x[1], (f16)x[2], (f16)x[3]};
#else
  return f16x4{};
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

// The largest |x| over N units of eight bf16 values, as a float. The bit pattern of a bf16
// without its sign orders like its magnitude, so the maxima are taken on the integers, two
// halves to a register (v_pk_max_u16), and the result is the bf16 pattern widened to float.
template <int N>
__device__ inline float absmax_bf16(const bf16x8* x) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  u16x2 acc = {0, 0};
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const u32x4 w = __builtin_bit_cast(u32x4, x[k]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc = __builtin_elementwise_max(acc, __builtin_bit_cast(u16x2, w[j] & 0x7fff7fffu));
  }
  const uint32_t m = acc[0] > acc[1] ? acc[0] : acc[1];
  return __uint_as_float(m << 16);
}

template <int I>
using IC = std::integral_constant<int, I>;

// f(IC<I>), ..., f(IC<N - 1>): a loop whose index is a compile-time constant in the body
template <int I, int N, typename F>
__device__ inline void static_for(F&& f) {
  if constexpr (I < N) {
    f(IC<I>{});
    static_for<I + 1, N>(f);
  }
}

}  // namespace gka
