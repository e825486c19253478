// Per-row dynamic int8 quantisation (per token for activations, per output
// channel for weights).  Source: "Qwen3.6-27B-Quark-W8A8-INT8" model card,
// Quantization Scheme table (symmetric INT8, per token / per channel);
// "Qwen3.6-35B-A3B IQ8R - radiance container", Trunk row (codes -127..127,
// round to nearest).  scale = amax/127 in fp32, code = rint(x / scale).
//
// One 256-thread workgroup per row.  Pass 1 reduces |x| to the row maximum
// (wave shuffles, then 4 partials through LDS); pass 2 re-reads the row (an
// L2 hit) and writes 16 codes per thread-iteration as one 16-byte store.
// HBM-bound: 2 (bf16) or 4 (fp32) bytes in and 1 byte out per element.
#include "kernels.h"

namespace w8a8 {

template <typename T>
struct Chunk16;  // 16 consecutive elements of a row, loaded with 16-byte loads

template <>
struct Chunk16<uint16_t> {
  float v[16];
  __device__ __forceinline__ void load(const uint16_t* p) {
    const v4u* q = reinterpret_cast<const v4u*>(p);
    v4u a = q[0], b = q[1];
    uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; i++) {
      v[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
      v[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
    }
  }
};

template <>
struct Chunk16<float> {
  float v[16];
  __device__ __forceinline__ void load(const float* p) {
    const v4f* q = reinterpret_cast<const v4f*>(p);
#pragma unroll
    for (int i = 0; i < 4; i++) {
      v4f a = q[i];
      v[4 * i] = a.x;
      v[4 * i + 1] = a.y;
      v[4 * i + 2] = a.z;
      v[4 * i + 3] = a.w;
    }
  }
};

// PACKED_OUT: write the codes in the 16-row x 64-byte MFMA tile layout of
// pack.hip (row m, bytes 16c..16c+15 of k chunk kc go to tile m/16, block kc,
// slot (m % 16) + 16 * (c % 4)) instead of row-major; ldq is then unused.
template <typename T, bool PACKED_OUT = false>
__global__ __launch_bounds__(256) void k_quant_rows(const T* __restrict__ x, int64_t ldx, int K,
                                                    int8_t* __restrict__ q, int64_t ldq,
                                                    float* __restrict__ s) {
  __shared__ float part[4];
  const int64_t row = blockIdx.x;
  const T* xr = x + row * ldx;
  int8_t* qr = PACKED_OUT ? nullptr : q + row * ldq;
  const int nchunk = K >> 4;

  float amax = 0.0f;
  for (int c = threadIdx.x; c < nchunk; c += 256) {
    Chunk16<T> ch;
    ch.load(xr + c * 16);
#pragma unroll
    for (int i = 0; i < 16; i++) amax = fmaxf(amax, fabsf(ch.v[i]));
  }
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
  const float sc = amax / 127.0f;

  for (int c = threadIdx.x; c < nchunk; c += 256) {
    Chunk16<T> ch;
    ch.load(xr + c * 16);
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      int c0 = 0, c1 = 0, c2 = 0, c3 = 0;
      if (amax != 0.0f) {
        c0 = quant_code(ch.v[4 * i], sc);
        c1 = quant_code(ch.v[4 * i + 1], sc);
        c2 = quant_code(ch.v[4 * i + 2], sc);
        c3 = quant_code(ch.v[4 * i + 3], sc);
      }
      w[i] = pack4_i8(c0, c1, c2, c3);
    }
    v4u out = {w[0], w[1], w[2], w[3]};
    if (PACKED_OUT) {
      const int64_t off = ((row >> 4) * (int64_t)(K >> 6) + (c >> 2)) * 1024 +
                          ((row & 15) + 16 * (c & 3)) * 16;
      *reinterpret_cast<v4u*>(q + off) = out;
    } else {
      *reinterpret_cast<v4u*>(qr + c * 16) = out;
    }
  }
  if (threadIdx.x == 0) s[row] = (amax != 0.0f) ? sc : 0.0f;
}

hipError_t launch_quant_rows_packed(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                    int8_t* q, float* s, hipStream_t stream) {
  hipLaunchKernelGGL((k_quant_rows<uint16_t, true>), dim3((unsigned)M), dim3(256), 0, stream, x,
                     ldx, (int)K, q, (int64_t)0, s);
  return hipGetLastError();
}

hipError_t launch_quant_rows(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                             int8_t* q, int64_t ldq, float* s, hipStream_t stream) {
  dim3 grid((unsigned)M), block(256);
  if (x_dtype == 0)
    hipLaunchKernelGGL(k_quant_rows<uint16_t>, grid, block, 0, stream,
                       static_cast<const uint16_t*>(x), ldx, (int)K, q, ldq, s);
  else
    hipLaunchKernelGGL(k_quant_rows<float>, grid, block, 0, stream,
                       static_cast<const float*>(x), ldx, (int)K, q, ldq, s);
  return hipGetLastError();
}

}  // namespace w8a8
