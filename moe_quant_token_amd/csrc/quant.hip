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

// PACKED_OUT: write the codes in the 16-row x 64-byte MFMA tile layout of
// pack.hip (row m, bytes 16c..16c+15 of k chunk kc go to tile m/16, block kc,
// slot (m % 16) + 16 * (c % 4)) instead of row-major; ldq is then unused.
// Rows of up to kQuantHeld chunks of 16 per thread are read once and held in
// registers; longer rows are read a second time (from L2) for the codes.
constexpr int kQuantHeld = 4;

template <typename T, bool PACKED_OUT = false, int NT = 256>
__global__ __launch_bounds__(NT) void k_quant_rows(const T* __restrict__ x, int64_t ldx, int K,
                                                   int8_t* __restrict__ q, int64_t ldq,
                                                   float* __restrict__ s) {
  constexpr int NW = NT / 64;
  __shared__ float part[NW];
  const int64_t row = blockIdx.x;
  const T* xr = x + row * ldx;
  int8_t* qr = PACKED_OUT ? nullptr : q + row * ldq;
  const int nchunk = K >> 4;
  const bool held = nchunk <= NT * kQuantHeld;

  Chunk16<T> ch[kQuantHeld];
  float amax = 0.0f;
  if (held) {
#pragma unroll
    for (int i = 0; i < kQuantHeld; i++) {
      const int c = threadIdx.x + NT * i;
      if (c < nchunk) {
        ch[i].load(xr + c * 16);
#pragma unroll
        for (int e = 0; e < 16; e++) amax = fmaxf(amax, fabsf(ch[i].v[e]));
      }
    }
  } else {
    for (int c = threadIdx.x; c < nchunk; c += NT) {
      Chunk16<T> t;
      t.load(xr + c * 16);
#pragma unroll
      for (int e = 0; e < 16; e++) amax = fmaxf(amax, fabsf(t.v[e]));
    }
  }
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = part[0];
#pragma unroll
  for (int w = 1; w < NW; w++) amax = fmaxf(amax, part[w]);
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
      const int c = threadIdx.x + NT * i;
      if (c < nchunk) emit(ch[i], c);
    }
  } else {
    for (int c = threadIdx.x; c < nchunk; c += NT) {
      Chunk16<T> t;
      t.load(xr + c * 16);
      emit(t, c);
    }
  }
  if (threadIdx.x == 0) s[row] = (amax != 0.0f) ? sc : 0.0f;
}

// Many rows (prefill): one wave per row, the row held in registers as raw
// bf16 (8 values a 16-byte chunk, up to NCH chunks a lane: K <= 512 * NCH),
// the maximum through DPP, no barrier.  A workgroup of 4 waves has four rows
// in flight, and a CU up to ~24 waves, so far more bytes are in flight than
// with a 256-thread workgroup per row.  Same arithmetic as k_quant_rows.
// PACKED_OUT: lane pairs (2i, 2i+1) hold the two halves of a 16-code k slice
// and store them as 8-byte pieces of the tile layout.
template <int NCH, bool PACKED_OUT>
__global__ __launch_bounds__(256) void k_quant_rows_wave(const uint16_t* __restrict__ x,
                                                         int64_t ldx, int M, int K,
                                                         int8_t* __restrict__ q, int64_t ldq,
                                                         float* __restrict__ s) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const uint16_t* xr = x + row * ldx;
  const int nc = K >> 3;  // 8-value chunks
  v4u raw[NCH];
  uint32_t m2 = 0u;
#pragma unroll
  for (int u = 0; u < NCH; u++) {
    const int c = lane + 64 * u;
    raw[u] = c < nc ? *reinterpret_cast<const v4u*>(xr + c * 8) : v4u{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; i++) m2 = bf16x2_absmax(m2, raw[u][i]);
  }
  const float amax = wave_max(bf16x2_absmax_value(m2));
  const float sc = amax / 127.0f;
  const float rc = 1.0f / sc;
  auto emit = [&](auto code) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < NCH; u++) {
      const int c = lane + 64 * u;
      if (c >= nc) break;
      uint32_t w[2];
#pragma unroll
      for (int i = 0; i < 2; i++)
        w[i] = pack4_i8(code(raw[u][2 * i] & 0xffffu), code(raw[u][2 * i] >> 16),
                        code(raw[u][2 * i + 1] & 0xffffu), code(raw[u][2 * i + 1] >> 16));
      int8_t* dst;
      if (PACKED_OUT) {
        const int c16 = c >> 1;  // 16-code slice: k bytes 16*c16 .. +15
        dst = q + ((row >> 4) * (int64_t)(K >> 6) + (c16 >> 2)) * 1024 +
              ((row & 15) + 16 * (c16 & 3)) * 16 + (c & 1) * 8;
      } else {
        dst = q + row * ldq + c * 8;
      }
      *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
    }
  };
  // the scale test is wave-uniform: one branch for the whole row
  if (sc >= 0x1p-100f)
    emit([&](uint32_t h) __attribute__((always_inline)) {
      return quant_code_recip(bf16_bits_to_f32(h), sc, rc);
    });
  else
    emit([&](uint32_t h) __attribute__((always_inline)) {
      return amax != 0.0f ? quant_code(bf16_bits_to_f32(h), sc) : 0;
    });
  if (lane == 0) s[row] = amax != 0.0f ? sc : 0.0f;
}

// bf16 rows of up to 8192 values, more than 16 rows: the wave-per-row kernel,
// holding as few chunks a lane as the row needs (registers bound how many
// rows a CU keeps in flight)
constexpr int kQuantWaveNch = 16;
static bool use_wave_quant(int64_t M, int64_t K) { return M > 16 && K <= 512 * kQuantWaveNch; }

template <bool PACKED_OUT>
static void launch_quant_wave(const uint16_t* x, int64_t ldx, int64_t M, int64_t K, int8_t* q,
                              int64_t ldq, float* s, hipStream_t stream) {
  const int need = (int)((K + 511) / 512);
  const dim3 grid((unsigned)((M + 3) / 4)), block(256);
#define W8A8_QW(n)                                                                            \
  hipLaunchKernelGGL((k_quant_rows_wave<n, PACKED_OUT>), grid, block, 0, stream, x, ldx, (int)M, \
                     (int)K, q, ldq, s)
  if (need <= 2) W8A8_QW(2);
  else if (need <= 4) W8A8_QW(4);
  else if (need <= 8) W8A8_QW(8);
  else if (need <= 10) W8A8_QW(10);
  else if (need <= 12) W8A8_QW(12);
  else W8A8_QW(16);
#undef W8A8_QW
}

hipError_t launch_quant_rows_packed(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                    int8_t* q, float* s, hipStream_t stream) {
  if (use_wave_quant(M, K)) {
    launch_quant_wave<true>(x, ldx, M, K, q, 0, s, stream);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((k_quant_rows<uint16_t, true>), dim3((unsigned)M), dim3(256), 0, stream, x,
                     ldx, (int)K, q, (int64_t)0, s);
  return hipGetLastError();
}

hipError_t launch_quant_rows_f32(const float* x, int64_t M, int64_t K, int64_t ldx, int8_t* q,
                                 int64_t ldq, float* s, bool packed, hipStream_t stream) {
  if (packed)
    hipLaunchKernelGGL((k_quant_rows<float, true>), dim3((unsigned)M), dim3(256), 0, stream, x,
                       ldx, (int)K, q, (int64_t)0, s);
  else if (M <= 16)
    hipLaunchKernelGGL((k_quant_rows<float, false, 1024>), dim3((unsigned)M), dim3(1024), 0,
                       stream, x, ldx, (int)K, q, ldq, s);
  else
    hipLaunchKernelGGL((k_quant_rows<float, false>), dim3((unsigned)M), dim3(256), 0, stream, x,
                       ldx, (int)K, q, ldq, s);
  return hipGetLastError();
}

hipError_t launch_quant_rows(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                             int8_t* q, int64_t ldq, float* s, hipStream_t stream) {
  dim3 grid((unsigned)M), block(256);
  if (x_dtype == 0 && use_wave_quant(M, K)) {
    launch_quant_wave<false>(static_cast<const uint16_t*>(x), ldx, M, K, q, ldq, s, stream);
    return hipGetLastError();
  }
  if (x_dtype == 0 && M <= 16)
    hipLaunchKernelGGL((k_quant_rows<uint16_t, false, 1024>), grid, dim3(1024), 0, stream,
                       static_cast<const uint16_t*>(x), ldx, (int)K, q, ldq, s);
  else if (x_dtype == 0)
    hipLaunchKernelGGL(k_quant_rows<uint16_t>, grid, block, 0, stream,
                       static_cast<const uint16_t*>(x), ldx, (int)K, q, ldq, s);
  else
    hipLaunchKernelGGL(k_quant_rows<float>, grid, block, 0, stream,
                       static_cast<const float*>(x), ldx, (int)K, q, ldq, s);
  return hipGetLastError();
}

}  // namespace w8a8
