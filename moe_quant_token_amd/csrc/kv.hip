// int8 KV-cache quantisation with an f16 scale per token and head.
//
// Source: "Qwen3.6-35B-A3B IQ8R - radiance container", Serve: kv-cache-dtype
// i8 stores the attention cache as int8 with an f16 scale per token and head.
// Per (token, head) row of D values: s = f16(amax / 127) (fp32 quotient,
// rounded to nearest even f16 by v_cvt_f16_f32), codes = round-half-even of
// x / float(s) (IEEE division), clamped to +-127; a zero scale gives zero
// codes.  The codes are formed against the stored f16 scale, so code * s is
// what the cache holds.
//
// One wave per row: lane l holds 16-byte chunks l, l + 64, ... (8 bf16 values
// each) in registers, the maximum comes from a DPP wave reduction, and each
// lane stores its codes as 8-byte pieces.  A workgroup of 4 waves takes 4
// consecutive rows (token-major, heads inner).  Rows of 64, 128 or 256
// values share a wave instead (k_kv_quant_i8_rows).  HBM-bound for prefill
// batches, latency-bound for a decode step.
#include <hip/hip_fp16.h>

#include "kernels.h"

namespace w8a8 {

template <int NCH>  // 8-value chunks a lane holds: D <= 512 * NCH
__global__ __launch_bounds__(256) void k_kv_quant_i8(const uint16_t* __restrict__ x, int64_t rows,
                                                     int Hk, int D, int64_t ldx,
                                                     const int32_t* __restrict__ slots,
                                                     int64_t cache_rows, int8_t* __restrict__ q,
                                                     int64_t ldq, uint16_t* __restrict__ s,
                                                     int64_t lds) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int64_t t = r / Hk;
  const int h = (int)(r - t * Hk);
  const int64_t dst = slots ? (int64_t)slots[t] : t;
  if (dst < 0 || dst >= cache_rows) return;  // a skipped token (wave-uniform)
  const uint16_t* xr = x + t * ldx + (int64_t)h * D;
  const int nc = D >> 3;
  v4u raw[NCH];
  float amax = 0.0f;
#pragma unroll
  for (int u = 0; u < NCH; u++) {
    const int c = lane + 64 * u;
    raw[u] = c < nc ? *reinterpret_cast<const v4u*>(xr + c * 8) : v4u{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      amax = fmaxf(amax, fabsf(bf16_bits_to_f32(raw[u][i] & 0xffffu)));
      amax = fmaxf(amax, fabsf(bf16_bits_to_f32(raw[u][i] >> 16)));
    }
  }
  amax = wave_max(amax);
  const __half sh = __float2half_rn(amax / 127.0f);
  const float sf = __half2float(sh);
  int8_t* qr = q + dst * ldq + (int64_t)h * D;
#pragma unroll
  for (int u = 0; u < NCH; u++) {
    const int c = lane + 64 * u;
    if (c >= nc) break;
    uint32_t w[2] = {0u, 0u};
    if (sf != 0.0f) {
#pragma unroll
      for (int i = 0; i < 2; i++)
        w[i] = pack4_i8(quant_code(bf16_bits_to_f32(raw[u][2 * i] & 0xffffu), sf),
                        quant_code(bf16_bits_to_f32(raw[u][2 * i] >> 16), sf),
                        quant_code(bf16_bits_to_f32(raw[u][2 * i + 1] & 0xffffu), sf),
                        quant_code(bf16_bits_to_f32(raw[u][2 * i + 1] >> 16), sf));
    }
    *reinterpret_cast<uint2*>(qr + c * 8) = make_uint2(w[0], w[1]);
  }
  if (lane == 0) s[dst * lds + h] = __half_as_ushort(sh);
}

// Rows of D = 8 LPR values (LPR = 8, 16 or 32 lanes a row): 64 / LPR rows a
// wave, one 8-value chunk a lane, the maximum by a shuffle reduction inside
// each row's lanes, so no lane idles (with one row a wave, a 256-value row
// occupies 32 of the 64 lanes).  Same arithmetic as k_kv_quant_i8.
template <int LPR>
__global__ __launch_bounds__(256) void k_kv_quant_i8_rows(
    const uint16_t* __restrict__ x, int64_t rows, int Hk, int64_t ldx,
    const int32_t* __restrict__ slots, int64_t cache_rows, int8_t* __restrict__ q, int64_t ldq,
    uint16_t* __restrict__ s, int64_t lds) {
  constexpr int D = 8 * LPR, RPW = 64 / LPR;
  const int lane = threadIdx.x & 63;
  const int c = lane % LPR;
  const int64_t r = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW + lane / LPR;
  const bool in = r < rows;
  const int64_t t = in ? r / Hk : 0;
  const int h = in ? (int)(r - t * Hk) : 0;
  const int64_t dst = !in ? -1 : slots ? (int64_t)slots[t] : t;
  const bool live = dst >= 0 && dst < cache_rows;  // a skipped token's row does nothing
  const v4u raw = live ? *reinterpret_cast<const v4u*>(x + t * ldx + (int64_t)h * D + c * 8)
                       : v4u{0u, 0u, 0u, 0u};
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    amax = fmaxf(amax, fabsf(bf16_bits_to_f32(raw[i] & 0xffffu)));
    amax = fmaxf(amax, fabsf(bf16_bits_to_f32(raw[i] >> 16)));
  }
#pragma unroll
  for (int off = 1; off < LPR; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  const __half sh = __float2half_rn(amax / 127.0f);
  const float sf = __half2float(sh);
  if (!live) return;
  uint32_t w[2] = {0u, 0u};
  if (sf != 0.0f) {
#pragma unroll
    for (int i = 0; i < 2; i++)
      w[i] = pack4_i8(quant_code(bf16_bits_to_f32(raw[2 * i] & 0xffffu), sf),
                      quant_code(bf16_bits_to_f32(raw[2 * i] >> 16), sf),
                      quant_code(bf16_bits_to_f32(raw[2 * i + 1] & 0xffffu), sf),
                      quant_code(bf16_bits_to_f32(raw[2 * i + 1] >> 16), sf));
  }
  *reinterpret_cast<uint2*>(q + dst * ldq + (int64_t)h * D + c * 8) = make_uint2(w[0], w[1]);
  if (c == 0) s[dst * lds + h] = __half_as_ushort(sh);
}

hipError_t launch_kv_quant_i8(const uint16_t* x, int64_t T, int64_t Hk, int64_t D, int64_t ldx,
                              const int32_t* slots, int64_t cache_rows, int8_t* q, int64_t ldq,
                              uint16_t* s, int64_t lds, hipStream_t stream) {
  const int64_t rows = T * Hk;
  // several rows a wave for bandwidth (4096 tokens x 4 heads x 256: 8.4 ->
  // 5.8 us); a decode step's few rows keep one row a wave (2.7 against 2.9 us
  // at one token), measured on MI355X
  if ((D == 64 || D == 128 || D == 256) && rows >= 256) {
    const int64_t rpb = 4 * (512 / D);  // rows a workgroup
    const dim3 g((unsigned)((rows + rpb - 1) / rpb)), b(256);
#define W8A8_KVR(lpr)                                                                       \
  hipLaunchKernelGGL((k_kv_quant_i8_rows<lpr>), g, b, 0, stream, x, rows, (int)Hk, ldx, slots, \
                     cache_rows, q, ldq, s, lds)
    if (D == 64) W8A8_KVR(8);
    else if (D == 128) W8A8_KVR(16);
    else W8A8_KVR(32);
#undef W8A8_KVR
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  const int64_t need = (D / 8 + 63) / 64;
#define W8A8_KV(n)                                                                              \
  hipLaunchKernelGGL((k_kv_quant_i8<n>), grid, block, 0, stream, x, rows, (int)Hk, (int)D, ldx, \
                     slots, cache_rows, q, ldq, s, lds)
  if (need <= 1) W8A8_KV(1);
  else if (need <= 2) W8A8_KV(2);
  else if (need <= 4) W8A8_KV(4);
  else W8A8_KV(8);
#undef W8A8_KV
  return hipGetLastError();
}

}  // namespace w8a8
