// Per-row dynamic int8 quantisation (per token for activations, per output
// channel for weights).  Source: "Qwen3.6-27B-Quark-W8A8-INT8" model card,
// Quantization Scheme table (symmetric INT8, per token / per channel);
// "Qwen3.6-35B-A3B IQ8R - radiance container", Trunk row (codes -127..127,
// round to nearest).  scale = amax/127 in fp32, code = rint(x / scale).
//
// One 256-thread workgroup per row.  The row maximum of |x| is reduced with
// wave shuffles, then 4 partials through LDS; the codes go out 16 per
// thread-iteration as one 16-byte store.  HBM-bound: 2 (bf16) or 4 (fp32)
// bytes in and 1 byte out per element.
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

// Fast quotient for bf16 rows: with r = 1/s (IEEE), q0 = x*r,
// e = fma(-q0, s, x) (exact), q = fma(e, r, q0).  For bf16 x with
// |x| <= amax and s = amax/127 >= 2^-100, rint(q) equals rint of the IEEE
// quotient x/s: checked exhaustively over every such (x, amax) pair.  fp32
// rows, and rows with a smaller scale, use the IEEE division.
__device__ __forceinline__ int quant_code_recip(float x, float s, float r) {
  const float q0 = x * r;
  const float e = __builtin_fmaf(-q0, s, x);
  const float q = __builtin_fmaf(e, r, q0);
  return (int)fminf(fmaxf(__builtin_rintf(q), -127.0f), 127.0f);
}

// PACKED_OUT: write the codes in the 16-row x 64-byte MFMA tile layout of
// pack.hip (row m, bytes 16c..16c+15 of k chunk kc go to tile m/16, block kc,
// slot (m % 16) + 16 * (c % 4)) instead of row-major; ldq is then unused.
// Rows of up to kQuantHeld chunks of 16 per thread are read once and held in
// registers; longer rows are read a second time (from L2) for the codes.
constexpr int kQuantHeld = 4;

template <typename T, bool PACKED_OUT = false>
__global__ __launch_bounds__(256) void k_quant_rows(const T* __restrict__ x, int64_t ldx, int K,
                                                    int8_t* __restrict__ q, int64_t ldq,
                                                    float* __restrict__ s) {
  __shared__ float part[4];
  const int64_t row = blockIdx.x;
  const T* xr = x + row * ldx;
  int8_t* qr = PACKED_OUT ? nullptr : q + row * ldq;
  const int nchunk = K >> 4;
  const bool held = nchunk <= 256 * kQuantHeld;

  Chunk16<T> ch[kQuantHeld];
  float amax = 0.0f;
  if (held) {
#pragma unroll
    for (int i = 0; i < kQuantHeld; i++) {
      const int c = threadIdx.x + 256 * i;
      if (c < nchunk) {
        ch[i].load(xr + c * 16);
#pragma unroll
        for (int e = 0; e < 16; e++) amax = fmaxf(amax, fabsf(ch[i].v[e]));
      }
    }
  } else {
    for (int c = threadIdx.x; c < nchunk; c += 256) {
      Chunk16<T> t;
      t.load(xr + c * 16);
#pragma unroll
      for (int e = 0; e < 16; e++) amax = fmaxf(amax, fabsf(t.v[e]));
    }
  }
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
  const float sc = amax / 127.0f;
  const bool recip = sizeof(T) == 2 && sc >= 0x1p-100f;
  const float rc = 1.0f / sc;

  auto emit = [&](const Chunk16<T>& cv, int c) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      int c4[4] = {0, 0, 0, 0};
      if (recip) {
#pragma unroll
        for (int e = 0; e < 4; e++) c4[e] = quant_code_recip(cv.v[4 * i + e], sc, rc);
      } else if (amax != 0.0f) {
#pragma unroll
        for (int e = 0; e < 4; e++) c4[e] = quant_code(cv.v[4 * i + e], sc);
      }
      w[i] = pack4_i8(c4[0], c4[1], c4[2], c4[3]);
    }
    v4u out = {w[0], w[1], w[2], w[3]};
    if (PACKED_OUT) {
      const int64_t off = ((row >> 4) * (int64_t)(K >> 6) + (c >> 2)) * 1024 +
                          ((row & 15) + 16 * (c & 3)) * 16;
      *reinterpret_cast<v4u*>(q + off) = out;
    } else {
      *reinterpret_cast<v4u*>(qr + c * 16) = out;
    }
  };
  if (held) {
#pragma unroll
    for (int i = 0; i < kQuantHeld; i++) {
      const int c = threadIdx.x + 256 * i;
      if (c < nchunk) emit(ch[i], c);
    }
  } else {
    for (int c = threadIdx.x; c < nchunk; c += 256) {
      Chunk16<T> t;
      t.load(xr + c * 16);
      emit(t, c);
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
