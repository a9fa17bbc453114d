// Device-side building blocks shared by the GKA kernels (gfx950 / CDNA4 only).
//
// Matrix-core tiles are 16x16 outputs with float32 accumulation:
//   fp16 operands: v_mfma_f32_16x16x32_f16  (K step 32, 8 elements per lane)
//   bf16 operands: v_mfma_f32_16x16x32_bf16 (K step 32, 8 elements per lane)
//   fp32 operands: v_mfma_f32_16x16x4_f32   (K step 4, 1 element per lane)
// Lane l of a wave holds, for an A operand (16 x K, row-major in LDS), row l%16 and the
// E consecutive columns starting at E*(l/16); for a B operand (K x 16) column l%16 and rows
// E*(l/16)..+E-1. The 16x16 accumulator of lane l holds rows 4*(l/16)+i (i = 0..3) of
// column l%16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gka {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

template <typename T>
struct Mma;

template <>
struct Mma<bf16> {
  static constexpr int K = 32;  // reduction depth of one instruction
  static constexpr int E = 8;   // operand elements per lane
  typedef bf16x8 frag;
  __device__ static inline f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // operand fragment: E consecutive elements of row `row` starting at column `col`
  __device__ static inline frag load(const bf16* base, int ld, int row, int col) {
    return *reinterpret_cast<const bf16x8*>(base + row * ld + col);
  }
};

typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

template <>
struct Mma<f16> {
  static constexpr int K = 32;
  static constexpr int E = 8;
  typedef f16x8 frag;
  __device__ static inline f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  __device__ static inline frag load(const f16* base, int ld, int row, int col) {
    return *reinterpret_cast<const f16x8*>(base + row * ld + col);
  }
};

template <>
struct Mma<float> {
  static constexpr int K = 4;
  static constexpr int E = 1;
  typedef float frag;
  __device__ static inline f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  __device__ static inline frag load(const float* base, int ld, int row, int col) {
    return base[row * ld + col];
  }
};

// ---- operand fragments of a transposed matrix ---------------------------------------------
// Fragment of M^T (rows r0 + lr of a 16-row tile, k-slots k0 + E lg .. + E - 1) for a matrix
// stored row-major as M[k][r] with ld elements per row, i.e. the rows of M are the k index.
// fp16: two transposing 8-byte LDS reads (ds_read_b64_tr_b16). Within each group of 16 lanes,
// lane i of such a read receives element i % 4 of the 8-byte chunks addressed by lanes
// i / 4 + 4 m (m = 0..3) of its group; lane j therefore addresses row k0 + 8 lg + 4 h + j / 4,
// columns r0 + 4 (j % 4) .. + 3 (read h = 0, 1), and lane i receives M[k0 + 8 lg + 4 h + m][r0 + i].
// Requires r0 and ld to be multiples of 4 (8-byte aligned chunks).
template <typename O>
__device__ inline typename Mma<O>::frag load_trans(const O* base, int ld, int r0, int k0, int lr,
                                                  int lg);
typedef __fp16 fp16x4_t __attribute__((__vector_size__(4 * sizeof(__fp16))));
template <>
__device__ inline f16x8 load_trans<f16>(const f16* base, int ld, int r0, int k0, int lr, int lg) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(3))) fp16x4_t lds_fp16x4;
  const int s = k0 + 8 * lg + (lr >> 2), c = r0 + 4 * (lr & 3);
  const fp16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4*)(base + s * ld + c));
  const fp16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4*)(base + (s + 4) * ld + c));
  return f16x8{(f16)a[0], (f16)a[1], (f16)a[2], (f16)a[3], (f16)b[0], (f16)b[1], (f16)b[2],
               (f16)b[3]};
#else
  return f16x8{};
#endif
}
// fp32 operands hold one k-slot per lane: a plain read of M[k0 + lg][r0 + lr]
template <>
__device__ inline float load_trans<float>(const float* base, int ld, int r0, int k0, int lr,
                                          int lg) {
  return base[(k0 + lg) * ld + r0 + lr];
}

// ---- element conversions ----------------------------------------------------------------
__device__ inline float to_f32(bf16 x) { return (float)x; }
__device__ inline float to_f32(float x) { return x; }
template <typename T>
__device__ inline T from_f32(float x);
template <>
__device__ inline bf16 from_f32<bf16>(float x) { return (bf16)x; }  // round to nearest even
template <>
__device__ inline float from_f32<float>(float x) { return x; }

// four consecutive elements <-> float4
template <typename T>
__device__ inline void store4(T* p, f32x4 v);
template <>
__device__ inline void store4<bf16>(bf16* p, f32x4 v) {
  bf16x4 h;
  h[0] = (bf16)v[0]; h[1] = (bf16)v[1]; h[2] = (bf16)v[2]; h[3] = (bf16)v[3];
  *reinterpret_cast<bf16x4*>(p) = h;
}
template <>
__device__ inline void store4<float>(float* p, f32x4 v) {
  *reinterpret_cast<f32x4*>(p) = v;
}
template <>
__device__ inline void store4<f16>(f16* p, f32x4 v) {
  f16x4 h;
  h[0] = (f16)v[0]; h[1] = (f16)v[1]; h[2] = (f16)v[2]; h[3] = (f16)v[3];
  *reinterpret_cast<f16x4*>(p) = h;
}

// four consecutive elements as hi + lo parts: hi = round(v), lo = round(v - hi); for float the
// value is exact and only hi is written
template <typename T>
__device__ inline void store4_split(T* hi, T* lo, f32x4 v);
template <>
__device__ inline void store4_split<f16>(f16* hi, f16* lo, f32x4 v) {
  f16x4 h, l;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = (f16)v[i];
    l[i] = (f16)(v[i] - (float)h[i]);
  }
  *reinterpret_cast<f16x4*>(hi) = h;
  *reinterpret_cast<f16x4*>(lo) = l;
}
template <>
__device__ inline void store4_split<float>(float* hi, float*, f32x4 v) {
  *reinterpret_cast<f32x4*>(hi) = v;
}

template <typename T>
__device__ inline f32x4 load4(const T* p);
template <>
__device__ inline f32x4 load4<bf16>(const bf16* p) {
  bf16x4 h = *reinterpret_cast<const bf16x4*>(p);
  return f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
}
template <>
__device__ inline f32x4 load4<float>(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}
template <>
__device__ inline f32x4 load4<f16>(const f16* p) {
  f16x4 h = *reinterpret_cast<const f16x4*>(p);
  return f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
}

// matrix-core operand type for an input element type: bf16 inputs are converted to fp16
// (exact for every bf16 value in fp16's normal range; 3 more mantissa bits for the rounded
// operands), fp32 inputs stay fp32
template <typename T>
struct OperandOf;
template <>
struct OperandOf<bf16> {
  typedef f16 type;
};
template <>
struct OperandOf<float> {
  typedef float type;
};
template <typename O>
__device__ inline O to_op(bf16 x) {
  return (O)(float)x;
}
template <typename O>
__device__ inline O to_op(float x) {
  return (O)x;
}

// ---- workgroup barrier for LDS exchange --------------------------------------------------
// Completes this wave's LDS instructions (lgkmcnt) and meets the other waves; global loads,
// stores and direct global-to-LDS loads stay in flight. __syncthreads() (and an LDS-scoped
// fence, which counts direct loads as LDS writes) would wait for all of them, stalling the
// barrier behind a prefetch issued for later use. Direct loads are never covered by this
// barrier: they are waited for explicitly (vmcnt) before their buffer is read. The memory
// clobber keeps the compiler from moving memory accesses across it.
__device__ inline void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// One direct global-to-LDS load per active lane: lane l copies 16 (or 4) bytes from src to
// LDS address lds_base + 16 l (+ 4 l); lds_base is wave-uniform. Issued from inline assembly so
// that the compiler does not track these loads as pending LDS writes: it would otherwise make
// every later LDS read wait for them (it cannot tell the prefetch buffer from the others). Their
// one consumer, the staging of the next chunk, waits for them explicitly (vmcnt(0) followed by
// a workgroup barrier). They have no register results.
__device__ inline void dma_load16(const void* src, uint32_t lds_base) {
  uint32_t m0_saved;  // m0 is reserved by the compiler: restore it
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
      : "=&s"(m0_saved)
      : "v"(src), "s"(lds_base)
      : "memory");
}
// The same with a wave-uniform 64-bit base in scalar registers and a 32-bit byte offset per
// lane (no 64-bit address arithmetic per lane). The base is read from the first lane.
__device__ inline void dma_load16_so(const void* base, uint32_t voff, uint32_t lds_base) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  // (readfirstlane returns a signed int: widen through uint32_t, never by sign extension)
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  const uint64_t sbase = lo | (hi << 32);
  uint32_t m0_saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
      : "=&s"(m0_saved)
      : "v"(voff), "s"(sbase), "s"(lds_base)
      : "memory");
}
// Buffer resource over `bytes` bytes from `base` (wave-uniform): raw buffer loads at byte
// offsets at or past the end return 0 and stores there are dropped, so ragged tails need no
// branches. Descriptor word 3 = 0x00020000 is the raw 32-bit-element layout of the gfx9 family.
// The base and size are read from the first lane: the compiler then keeps the descriptor in
// scalar registers even where it cannot prove the arguments uniform (otherwise every access
// becomes a loop over the distinct descriptors of the wave).
__device__ inline __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  const int n = __builtin_amdgcn_readfirstlane((int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>((uintptr_t)(lo | (hi << 32))),
                                           (short)0, n, 0x00020000);
}
template <typename V>
__device__ inline V buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  static_assert(sizeof(V) == 16, "16-byte element");
  return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
template <typename V>
__device__ inline V buffer_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  static_assert(sizeof(V) == 8, "8-byte element");
  return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ inline void buffer_store4f(float x, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, x), r, off, 0, 0);
}
__device__ inline float buffer_load4f(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
template <typename V>
__device__ inline void buffer_store8(V x, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  static_assert(sizeof(V) == 8, "8-byte element");
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, x), r, off, 0, 0);
}

// 4-byte form of dma_load16_so
__device__ inline void dma_load4_so(const void* base, uint32_t voff, uint32_t lds_base) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  const uint64_t sbase = lo | (hi << 32);
  uint32_t m0_saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
      "global_load_lds_dword %1, %2\n\ts_mov_b32 m0, %0"
      : "=&s"(m0_saved)
      : "v"(voff), "s"(sbase), "s"(lds_base)
      : "memory");
}
__device__ inline void dma_load4(const void* src, uint32_t lds_base) {
  uint32_t m0_saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
      "global_load_lds_dword %1, off\n\ts_mov_b32 m0, %0"
      : "=&s"(m0_saved)
      : "v"(src), "s"(lds_base)
      : "memory");
}

// ---- wave scans (DPP: register-to-register lane moves, no LDS round trip) -----------------
// dpp_ctrl encodings: row_shr:n = 0x110 + n (within rows of 16 lanes), row_bcast:15 = 0x142
// (lane 15 of a row to the whole next row), row_bcast:31 = 0x143 (lane 31 to rows 2 and 3).
// A lane whose source is outside its row, or whose row is masked off, keeps `old`.
template <int CTRL, int ROW_MASK>
__device__ inline float dpp_move(float old, float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old), __builtin_bit_cast(int, x),
                                         CTRL, ROW_MASK, 0xf, false));
}
// inclusive prefix sum over groups of W lanes (W = 16, 32 or 64)
template <int W>
__device__ inline float scan_add(float x) {
  static_assert(W == 16 || W == 32 || W == 64, "segment width");
  x += dpp_move<0x111, 0xf>(0.0f, x);
  x += dpp_move<0x112, 0xf>(0.0f, x);
  x += dpp_move<0x114, 0xf>(0.0f, x);
  x += dpp_move<0x118, 0xf>(0.0f, x);
  if constexpr (W >= 32) x += dpp_move<0x142, 0xa>(0.0f, x);
  if constexpr (W == 64) x += dpp_move<0x143, 0xc>(0.0f, x);
  return x;
}
// inclusive scan of affine maps y -> a y + b over the wave (lane order = application order):
// (a, b) of lane l becomes the composition of the maps of lanes 0..l
__device__ inline void scan_affine(float& a, float& b) {
  float ta, tb;
#define GKA_AFFINE_STEP(CTRL, MASK)        \
  ta = dpp_move<CTRL, MASK>(1.0f, a);      \
  tb = dpp_move<CTRL, MASK>(0.0f, b);      \
  b = a * tb + b;                          \
  a = a * ta;
  GKA_AFFINE_STEP(0x111, 0xf)
  GKA_AFFINE_STEP(0x112, 0xf)
  GKA_AFFINE_STEP(0x114, 0xf)
  GKA_AFFINE_STEP(0x118, 0xf)
  GKA_AFFINE_STEP(0x142, 0xa)
  GKA_AFFINE_STEP(0x143, 0xc)
#undef GKA_AFFINE_STEP
}

// value of x in lane l (wave-uniform l), read through a scalar register
__device__ inline float lane_value(float x, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

// value of x in lane src (0 <= src < 64, per lane), through the LDS crossbar (ds_bpermute)
__device__ inline float lane_read(float x, int src) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, x)));
}

// x combined with x of lane ^ 16 and lane ^ 32 (the four lanes l % 16 + 16 j) by the CDNA4 row
// swaps, without an LDS round trip. With both registers holding x, v_permlane16_swap exchanges
// the odd 16-lane rows of the first with the even rows of the second, so in every lane one of
// them holds x of the lane and the other x of lane ^ 16; v_permlane32_swap does the same for
// the two 32-lane halves. (Written as asm with two read-write operands: the matching compiler
// builtin's second result came out as a copy of its first in this toolchain's code.) The nop
// gives the swap the wait states it needs after a vector write of its operands.
__device__ inline void swap_rows16(float& a, float& b) {
  asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ inline void swap_rows32(float& a, float& b) {
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ inline float group_sum(float x) {
  float a = x, b = x;
  swap_rows16(a, b);
  x = a + b;
  a = x;
  b = x;
  swap_rows32(a, b);
  return a + b;
}
__device__ inline float group_max(float x) {
  float a = x, b = x;
  swap_rows16(a, b);
  x = fmaxf(a, b);
  a = x;
  b = x;
  swap_rows32(a, b);
  return fmaxf(a, b);
}

// ---- wave reductions (wave64) -------------------------------------------------------------
__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, kWave);
  return x;
}

// maximum over the wave, in every lane: a running maximum along the rows of 16 lanes (DPP row
// shifts; lanes without a source keep their own value), carried across rows by the row
// broadcasts of lanes 15 and 31 (as in scan_add), then lane 63's value
__device__ inline float wave_max(float x) {
  x = fmaxf(x, dpp_move<0x111, 0xf>(x, x));
  x = fmaxf(x, dpp_move<0x112, 0xf>(x, x));
  x = fmaxf(x, dpp_move<0x114, 0xf>(x, x));
  x = fmaxf(x, dpp_move<0x118, 0xf>(x, x));
  x = fmaxf(x, dpp_move<0x142, 0xa>(x, x));
  x = fmaxf(x, dpp_move<0x143, 0xc>(x, x));
  return lane_value(x, kWave - 1);
}

// ---- exact power-of-two scales (range of the 16-bit matrix operands) ----------------------
// floor(log2 x) for x > 0, clamped to [-lim, lim] (subnormal x gives -lim, infinity lim); 0 for
// x = 0 or NaN, where any scale serves
__device__ inline int pow2_exponent(float x, int lim) {
  const int e = (int)((__float_as_uint(x) >> 23) & 0xffu) - 127;
  return x > 0.0f ? min(max(e, -lim), lim) : 0;
}
// 2^e as a float, for -126 <= e <= 127
__device__ inline float exp2_int(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

// log2 of a gate with a finite floor for gamma = 0, so that differences of prefix sums stay
// finite; 2^x for x at or below the floor underflows to exactly 0 in float32.
constexpr float kLog2GateFloor = -160.0f;
// hardware 2^x and log2(x) (v_exp_f32 / v_log_f32, about 1 ulp); arguments of exp2 here are
// <= 0 and results below the normal range only ever act as vanishing decay weights
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline float log2_gate(float g) {
  return g >= 1.17549435e-38f ? __builtin_amdgcn_logf(g) : kLog2GateFloor;
}

// Chebyshev constants of the normalised system  (H_t / ||H_t||_F + a I) xh = q, whose spectrum
// lies in [a, 1 + a]: step c = 2 / (1 + 2a), weights omega_i (omega_0 = 2), and the weights
// beta_i of the iterate x_r = sum_i beta_i r_i as a combination of the residuals r_i of the
// same iteration. Filled on the host.
// The residual recurrence is applied as R_{i+1} = kp_i R_{i-1} + kr_i R_i + ky_i (A - a I) R_i.
// Rescaled form (no multiply by kp): with scalars s_0 = s_1 = s0 and s_{i+1} = kp_i s_{i-1},
// the residuals Rt_i = R_i / s_i obey Rt_{i+1} = Rt_{i-1} + krs_i Rt_i + kys_i (A - a I) Rt_i
// and x_r = sum_i bts_i Rt_i, with krs_i = kr_i s_i / s_{i+1}, kys_i = ky_i s_i / s_{i+1} and
// bts_i = beta_i s_i; Rt_0 = q * inv_s0. iters_rs <= iters is the count for that form: it stops
// before the first step whose |kp_i| is below 2^-64, where every later residual is below 2^-64
// of the first. s0 is a constant far from short binary fractions: with s0 = 1, the rescaled
// residuals of a system whose spectrum sits at both interval ends reproduce q exactly every
// second step, and the fp16 rounding of those (q on the bf16 grid plus a multiple of k) adds up
// along k; in a float64 model of the rounding that costs about 1.5x the error of the plain form
// when gates are 0, against about 1.15x with this s0.
struct ChebConsts {
  float a;
  float c;
  int iters;
  int iters_rs;
  float inv_s0;
  float omega[64];
  float beta[64];
  float kp[64];
  float kr[64];
  float ky[64];
  float krs[64];
  float kys[64];
  float bts[64];
  // residual mode: s_i of the rescaled residuals (R_i = s_i Rt_i) for i = 0..iters, and whether
  // the coefficients of one more step (it = iters - 1, giving R_iters) are set
  float sres[65];
  int res_extra;
  // the iterate is formed times xsc = 2^floor(log2 a) (1 for a < 2), a power of two that keeps
  // it (about |q| / a) in the normal range of the 16-bit operands of the output products; the
  // output accumulators are multiplied by inv_xsc = 1 / xsc before they are stored
  float inv_xsc;
};

}  // namespace gka
