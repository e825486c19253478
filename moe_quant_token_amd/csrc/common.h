// Internal helpers shared by the gfx950 kernels of libw8a8.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8a8 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// fp32 -> bf16 bit pattern, round to nearest even (finite values).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Symmetric int8 code: round-half-even of an IEEE quotient, clamped to +-127.
__device__ __forceinline__ int quant_code(float x, float s) {
  float t = x / s;  // correctly rounded fp32 division
  float r = __builtin_rintf(t);
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return (int)r;
}

// Fast quotient for bf16 rows: with r = 1/s (IEEE), q0 = x*r,
// e = fma(-q0, s, x) (exact), q = fma(e, r, q0).  For bf16 x with
// |x| <= amax and s = amax/127 >= 2^-100, rint(q) equals rint of the IEEE
// quotient x/s: checked exhaustively over every such (x, amax) pair.  fp32
// rows, and rows with a smaller scale, use the IEEE division.  That quotient
// is at most 127 + 2^-16 here, so the clamp never acts; adding 1.5 * 2^23
// rounds q to an integer, ties to even (the sum's ulp is 1), and leaves it,
// two's complement, in the low bits of the sum (the same check covers this).
__device__ __forceinline__ int quant_code_recip(float x, float s, float r) {
  const float q0 = x * r;
  const float e = __builtin_fmaf(-q0, s, x);
  const float q = __builtin_fmaf(e, r, q0);
  return (int)(__float_as_uint(q + 0x1.8p23f) - 0x4B400000u);
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Running maximum of |x| over two bf16 values a word, kept as bit patterns:
// for finite bf16 the magnitude orders as the unsigned integer of the low 15
// bits, so one packed u16 maximum covers two values.
__device__ __forceinline__ uint32_t bf16x2_absmax(uint32_t m, uint32_t w) {
  const u16x2 a = __builtin_bit_cast(u16x2, m);
  const u16x2 b = __builtin_bit_cast(u16x2, w & 0x7fff7fffu);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(a, b));
}
__device__ __forceinline__ float bf16x2_absmax_value(uint32_t m) {
  const uint32_t lo = m & 0xffffu, hi = m >> 16;
  return bf16_bits_to_f32(lo > hi ? lo : hi);
}

// Wave-wide maximum through DPP row shifts and row broadcasts (no LDS
// traffic); every lane gets the result.  A lane whose DPP source lies outside
// the row keeps its own value (bound_ctrl off, old = v), so any sign works.
__device__ __forceinline__ float wave_max(float v) {
#define W8A8_DPP_FMAX(ctrl, rmask)                                                          \
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), \
                                                          ctrl, rmask, 0xf, false)))
  W8A8_DPP_FMAX(0x111, 0xf);  // row_shr:1
  W8A8_DPP_FMAX(0x112, 0xf);  // row_shr:2
  W8A8_DPP_FMAX(0x114, 0xf);  // row_shr:4
  W8A8_DPP_FMAX(0x118, 0xf);  // row_shr:8
  W8A8_DPP_FMAX(0x142, 0xa);  // row_bcast:15
  W8A8_DPP_FMAX(0x143, 0xc);  // row_bcast:31
#undef W8A8_DPP_FMAX
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Weight bytes are read once per call: a non-temporal load keeps them from
// displacing what is read again soon (activations, the MoE intermediates).
__device__ __forceinline__ v4i ld_stream(const int8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p));
}

__device__ __forceinline__ v4i mfma_16x16x64_i8(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// 32x32x32 int8 MFMA.  On gfx950 it issues at twice the rate of the 16x16x64
// form for the same work.  Operands: lane l supplies 16 bytes of A row (l % 32)
// and of B column (l % 32) for k-slice (l / 32) of the 32-wide k step.
// Result lane l holds column l % 32, rows 8*(r/4) + 4*(l/32) + r%4, r < 16.
__device__ __forceinline__ v16i mfma_32x32x32_i8(v4i a, v4i b, v16i c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

// s_waitcnt immediate that waits for vmcnt <= v and leaves the other counters
// unconstrained (gfx9 encoding: vmcnt[3:0] at bits 3:0 and vmcnt[5:4] at bits
// 15:14, expcnt at 6:4, lgkmcnt at 11:8).
constexpr int vmcnt_imm(int v) { return (v & 15) | ((v >> 4) << 14) | (7 << 4) | (15 << 8); }

// s_waitcnt immediate that waits for lgkmcnt == 0 only (LDS, scalar memory).
constexpr int lgkmcnt0_imm() { return 15 | (3 << 14) | (7 << 4); }

// Wait until at most n (wave-uniform, 0..15) vector memory operations of this
// wave are outstanding.
__device__ __forceinline__ void wait_vmcnt_le(int n) {
  switch (n) {
#define W8A8_VMCNT_CASE(v) \
  case v:                  \
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(v)); \
    break;
    W8A8_VMCNT_CASE(1) W8A8_VMCNT_CASE(2) W8A8_VMCNT_CASE(3) W8A8_VMCNT_CASE(4)
    W8A8_VMCNT_CASE(5) W8A8_VMCNT_CASE(6) W8A8_VMCNT_CASE(7) W8A8_VMCNT_CASE(8)
    W8A8_VMCNT_CASE(9) W8A8_VMCNT_CASE(10) W8A8_VMCNT_CASE(11) W8A8_VMCNT_CASE(12)
    W8A8_VMCNT_CASE(13) W8A8_VMCNT_CASE(14) W8A8_VMCNT_CASE(15)
#undef W8A8_VMCNT_CASE
    default:
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  }
}

// Workgroup barrier that orders LDS accesses only: unlike __syncthreads() it
// does not wait for outstanding global loads, so register prefetches stay in
// flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Orders one wave's LDS stores before the same wave's later LDS loads of
// another lane's data (and its earlier loads before later stores): a release
// and an acquire fence at wavefront scope around a wave barrier.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// ---- fwht128: the unnormalised Sylvester Walsh-Hadamard transform of a
// 128-block, fp32 butterflies in natural order, stages h = 1, 2, ..., 64,
// pair (i, i+h) -> (a + b, a - b).  Register layout: 16 lanes hold one
// 128-block, 8 consecutive elements per lane; stages 1, 2, 4 stay inside a
// lane, stages 8..64 exchange with lane ^ (h/8).

struct Block8 {
  float v[8];
};

// The value of lane (lane ^ m), m in {1, 2, 4, 8}: DPP quad permutations for
// 1 and 2, a swizzle (xor mode, no LDS access) for 4 and 8.
__device__ __forceinline__ float lane_xor(float v, int m) {
  const int i = __float_as_int(v);
  int r;
  if (m == 1)
    r = __builtin_amdgcn_mov_dpp(i, 0xb1, 0xf, 0xf, false);  // quad_perm [1,0,3,2]
  else if (m == 2)
    r = __builtin_amdgcn_mov_dpp(i, 0x4e, 0xf, 0xf, false);  // quad_perm [2,3,0,1]
  else if (m == 4)
    r = __builtin_amdgcn_ds_swizzle(i, 0x1f | (4 << 10));  // and 0x1f, xor 4
  else
    r = __builtin_amdgcn_ds_swizzle(i, 0x1f | (8 << 10));  // and 0x1f, xor 8
  return __int_as_float(r);
}

// In-place butterfly of a 128-block spread over 16 lanes (l16 = lane % 16).
__device__ __forceinline__ void fwht128_lanes(Block8& b, int l16) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1)
#pragma unroll
    for (int c = 0; c < 8; c++)
      if ((c & h) == 0) {
        const float lo = b.v[c], hi = b.v[c + h];
        b.v[c] = lo + hi;
        b.v[c + h] = lo - hi;
      }
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) {
    const bool upper = (l16 & m) != 0;
#pragma unroll
    for (int c = 0; c < 8; c++) {
      const float mine = b.v[c];
      const float other = lane_xor(mine, m);
      b.v[c] = upper ? (other - mine) : (mine + other);
    }
  }
}

// Marks v as needed here: the compiler can neither sink the load that
// produces it below this point nor defer the wait for that load past it.
__device__ __forceinline__ void keep_live(float v) { asm volatile("" ::"v"(v)); }

// Pack four int8 codes (values in [-127, 127]) into one 32-bit word.
__device__ __forceinline__ uint32_t pack4_i8(int a, int b, int c, int d) {
  return (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) | ((uint32_t)(c & 0xff) << 16) |
         ((uint32_t)(d & 0xff) << 24);
}

}  // namespace w8a8
