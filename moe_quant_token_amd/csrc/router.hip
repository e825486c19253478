// The MoE router gate in bf16: logits[t, e] = sum_h x[t, h] wg[e, h], bf16
// operands, fp32 accumulation, fp32 logits (the input of routing).
//
// Source: "Online INT8 W8A8 for Qwen3.6 27B / 35B-A3B" (ATOM pull request),
// intro: the precision split keeps the router gate in BF16 while the experts
// and dense GEMMs run A8W8.
//
// Two forms, both with a fixed summation order (bit-reproducible):
//   - up to 16 tokens: one wave per expert row; each lane walks its 8-value
//     chunks of the row (h = 512 c + 8 lane + 0..7) with fp32 FMAs (a bf16
//     product is exact in fp32) for every token, then a butterfly reduction
//     over the wave.  The weight row is read once for all tokens;
//   - more tokens: bf16 MFMA (v_mfma_f32_16x16x32_bf16) tiles of 16 tokens x
//     16 experts per wave, H split over 8 waves (up to 256 tokens); beyond,
//     16 tokens x 64 experts per wave with H split over 4 waves (or the
//     16 x 16 tiles over 2 waves where E or H do not divide), the slices'
//     partial sums added in slice order.
// Layouts: x bf16 [T, H] with row stride ldx; wg bf16 [E, H] contiguous;
// logits fp32 [T, E] with row stride ldl.
#include "kernels.h"

namespace w8a8 {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kRouterWaveTokens = 16;

__device__ __forceinline__ void unpack_bf16x8(const v4u raw, float* v) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    v[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
    v[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
  }
}

__global__ __launch_bounds__(256) void k_router_wave(const uint16_t* __restrict__ x, int T, int H,
                                                     int64_t ldx, const uint16_t* __restrict__ wg,
                                                     int E, float* __restrict__ logits,
                                                     int64_t ldl) {
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (e >= E) return;  // wave-uniform
  float acc[kRouterWaveTokens];
#pragma unroll
  for (int t = 0; t < kRouterWaveTokens; t++) acc[t] = 0.0f;
  const uint16_t* wr = wg + (int64_t)e * H;
  for (int h0 = lane * 8; h0 < H; h0 += 512) {
    float wv[8];
    unpack_bf16x8(*reinterpret_cast<const v4u*>(wr + h0), wv);
#pragma unroll
    for (int t = 0; t < kRouterWaveTokens; t++) {
      if (t < T) {
        float xv[8];
        unpack_bf16x8(*reinterpret_cast<const v4u*>(x + t * ldx + h0), xv);
#pragma unroll
        for (int c = 0; c < 8; c++) acc[t] = fmaf(xv[c], wv[c], acc[t]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kRouterWaveTokens; t++) {
    if (t < T) {
      float v = acc[t];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) v = v + __shfl_xor(v, off, 64);
      if (lane == 0) logits[t * ldl + e] = v;
    }
  }
}

// Workgroup = TB 16-token blocks x one 16-expert block; wave (tb, ks) takes
// token block tb and the ks-th of KS equal slices of H (H / KS a multiple of
// 32).  The KS partial sums are added in slice order by the first slice's
// wave (fixed order).
template <int TB, int KS>
__global__ __launch_bounds__(TB * KS * 64) void k_router_mfma(
    const uint16_t* __restrict__ x, int T, int H, int64_t ldx, const uint16_t* __restrict__ wg,
    float* __restrict__ logits, int64_t ldl) {
  __shared__ v4f red[TB][KS][64];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int tb = wv / KS, ks = wv - (wv / KS) * KS;
  const int j = lane & 15;
  const int g = lane >> 4;
  const int e0 = blockIdx.x * 16;
  const int t0 = (blockIdx.y * TB + tb) * 16;
  const int ta = min(t0 + j, T - 1);  // rows past T read a valid row; not stored
  const int hs = H / KS;
  const uint16_t* ap = x + (int64_t)ta * ldx + ks * hs + g * 8;
  const uint16_t* bp = wg + (int64_t)(e0 + j) * H + ks * hs + g * 8;
  v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
  if (t0 < T) {
    constexpr int U = 4;
    int k0 = 0;
    for (; k0 + 32 * U <= hs; k0 += 32 * U) {
      v4u a[U], b[U];
#pragma unroll
      for (int u = 0; u < U; u++) {
        a[u] = *reinterpret_cast<const v4u*>(ap + k0 + 32 * u);
        b[u] = *reinterpret_cast<const v4u*>(bp + k0 + 32 * u);
      }
#pragma unroll
      for (int u = 0; u < U; u++)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a[u]),
                                                      __builtin_bit_cast(v8bf, b[u]), acc, 0, 0,
                                                      0);
    }
    for (; k0 < hs; k0 += 32) {
      const v4u a = *reinterpret_cast<const v4u*>(ap + k0);
      const v4u b = *reinterpret_cast<const v4u*>(bp + k0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a),
                                                    __builtin_bit_cast(v8bf, b), acc, 0, 0, 0);
    }
  }
  red[tb][ks][lane] = acc;
  __syncthreads();
  if (ks != 0 || t0 >= T) return;
  v4f sum = red[tb][0][lane];
  for (int i = 1; i < KS; i++) {
    const v4f p = red[tb][i][lane];
    sum.x = sum.x + p.x;
    sum.y = sum.y + p.y;
    sum.z = sum.z + p.z;
    sum.w = sum.w + p.w;
  }
#pragma unroll
  for (int v = 0; v < 4; v++) {
    const int t = t0 + 4 * g + v;
    if (t < T) logits[(int64_t)t * ldl + e0 + j] = sum[v];
  }
}

// Larger batches: workgroup = 16 TB tokens x 16 EB experts x KS slices of H,
// the slices' partial sums added in slice order.  Wave (eh, ks) takes all TB
// token blocks and the EB / EH expert blocks of half eh (each weight fragment
// of a k step feeds TB MFMAs, each token fragment EB / EH), so the
// workgroup loads every weight fragment once and every token fragment EH
// times; each logit's sum (MFMA chain over its slice in k order, then the
// slices in order) is the same whatever the split over waves.  Each weight
// fragment is read by T / (16 TB) workgroups and each token fragment by
// E / (16 EB), against E / 16 for the one-expert-block form.
template <int TB, int KS, int EB, int EH>
__global__ __launch_bounds__(EH * KS * 64) void k_router_mfma_wide(
    const uint16_t* __restrict__ x, int T, int H, int64_t ldx, const uint16_t* __restrict__ wg,
    float* __restrict__ logits, int64_t ldl) {
  constexpr int EW = EB / EH;  // expert blocks a wave
  static_assert(EB % EH == 0, "expert blocks must split over the waves");
  __shared__ v4f red[TB][KS][EB][64];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int eh = wv / KS, ks = wv - (wv / KS) * KS;
  const int j = lane & 15;
  const int g = lane >> 4;
  const int e0 = blockIdx.x * 16 * EB;
  const int tw0 = blockIdx.y * TB * 16;
  const int hs = H / KS;
  const uint16_t* ap[TB];
#pragma unroll
  for (int tb = 0; tb < TB; tb++) {
    const int ta = min(tw0 + 16 * tb + j, T - 1);  // rows past T read a valid row; not stored
    ap[tb] = x + (int64_t)ta * ldx + ks * hs + g * 8;
  }
  const uint16_t* bp = wg + (int64_t)(e0 + 16 * EW * eh + j) * H + ks * hs + g * 8;
  v4f acc[TB][EW];
#pragma unroll
  for (int tb = 0; tb < TB; tb++)
#pragma unroll
    for (int e = 0; e < EW; e++) acc[tb][e] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  constexpr int U = 4;
  for (int k0 = 0; k0 < hs; k0 += 32 * U) {  // hs is a multiple of 32 U (launcher)
    v4u a[U][TB], b[U][EW];
#pragma unroll
    for (int u = 0; u < U; u++) {
#pragma unroll
      for (int tb = 0; tb < TB; tb++)
        a[u][tb] = *reinterpret_cast<const v4u*>(ap[tb] + k0 + 32 * u);
#pragma unroll
      for (int e = 0; e < EW; e++)
        b[u][e] = *reinterpret_cast<const v4u*>(bp + (int64_t)e * 16 * H + k0 + 32 * u);
    }
#pragma unroll
    for (int u = 0; u < U; u++)
#pragma unroll
      for (int tb = 0; tb < TB; tb++)
#pragma unroll
        for (int e = 0; e < EW; e++)
          acc[tb][e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(v8bf, a[u][tb]), __builtin_bit_cast(v8bf, b[u][e]), acc[tb][e],
              0, 0, 0);
  }
#pragma unroll
  for (int tb = 0; tb < TB; tb++)
#pragma unroll
    for (int e = 0; e < EW; e++) red[tb][ks][EW * eh + e][lane] = acc[tb][e];
  __syncthreads();
  if (ks != 0) return;
#pragma unroll
  for (int tb = 0; tb < TB; tb++) {
    const int t0 = tw0 + 16 * tb;
#pragma unroll
    for (int e = 0; e < EW; e++) {
      const int eb = EW * eh + e;
      v4f sum = red[tb][0][eb][lane];
      for (int i = 1; i < KS; i++) {
        const v4f p = red[tb][i][eb][lane];
        sum.x = sum.x + p.x;
        sum.y = sum.y + p.y;
        sum.z = sum.z + p.z;
        sum.w = sum.w + p.w;
      }
#pragma unroll
      for (int v = 0; v < 4; v++) {
        const int t = t0 + 4 * g + v;
        if (t < T) logits[(int64_t)t * ldl + e0 + 16 * eb + j] = sum[v];
      }
    }
  }
}

hipError_t launch_router_gate_bf16(const uint16_t* x, int64_t T, int64_t H, int64_t ldx,
                                   const uint16_t* wg, int64_t E, float* logits, int64_t ldl,
                                   hipStream_t stream) {
  if (T <= kRouterWaveTokens) {
    hipLaunchKernelGGL(k_router_wave, dim3((unsigned)((E + 3) / 4)), dim3(256), 0, stream, x,
                       (int)T, (int)H, ldx, wg, (int)E, logits, ldl);
  } else if (T <= 256 && H % 256 == 0) {
    hipLaunchKernelGGL((k_router_mfma<1, 8>), dim3((unsigned)(E / 16), (unsigned)((T + 15) / 16)),
                       dim3(512), 0, stream, x, (int)T, (int)H, ldx, wg, logits, ldl);
  } else if (E % 64 == 0 && H % 512 == 0) {
    // the widest expert block that still gives every CU a workgroup (a
    // workgroup's time is set by the bytes it reads: 32 tokens x 64 experts
    // read 512 KiB at H = 2048, 32 x 16 read 192 KiB); the logits do not
    // depend on the choice
    const unsigned ty = (unsigned)((T + 31) / 32);
    if ((E / 64) * ty >= 256)
      hipLaunchKernelGGL((k_router_mfma_wide<2, 4, 4, 2>), dim3((unsigned)(E / 64), ty),
                         dim3(512), 0, stream, x, (int)T, (int)H, ldx, wg, logits, ldl);
    else if ((E / 32) * ty >= 256)
      hipLaunchKernelGGL((k_router_mfma_wide<2, 4, 2, 2>), dim3((unsigned)(E / 32), ty),
                         dim3(512), 0, stream, x, (int)T, (int)H, ldx, wg, logits, ldl);
    else
      hipLaunchKernelGGL((k_router_mfma_wide<2, 4, 1, 1>), dim3((unsigned)(E / 16), ty),
                         dim3(256), 0, stream, x, (int)T, (int)H, ldx, wg, logits, ldl);
  } else if (H % 64 == 0) {
    hipLaunchKernelGGL((k_router_mfma<4, 2>), dim3((unsigned)(E / 16), (unsigned)((T + 63) / 64)),
                       dim3(512), 0, stream, x, (int)T, (int)H, ldx, wg, logits, ldl);
  } else {
    hipLaunchKernelGGL((k_router_mfma<4, 1>), dim3((unsigned)(E / 16), (unsigned)((T + 63) / 64)),
                       dim3(256), 0, stream, x, (int)T, (int)H, ldx, wg, logits, ldl);
  }
  return hipGetLastError();
}

}  // namespace w8a8
