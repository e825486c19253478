// Hadamard-domain (fwht128) W8A8: activation rotation + quant, rotated weight
// preparation with a u8 scale per 256 of K under a bf16 row scale, and the
// decode-shaped g256 GEMM.
//
// Source: "Qwen3.6-35B-A3B IQ8R - radiance container": Trunk row (int8 codes
// -127..127, a u8 scale per row and 256 of K under a bf16 scale per row, each
// 128 of K rotated by the unnormalised Hadamard, round to nearest);
// Activations row (int8 activations under the same rotation); the recipe
// under "How this file was made" (group=256 scale=u8 scale2=bf16 block2=1x*
// transform=fwht128 clamp=sym).
//
// The transform is the fp32 fast Walsh-Hadamard butterfly in natural
// (Sylvester) order with stages h = 1, 2, ..., 64; pair (i, i+h) becomes
// (a + b, a - b).  Every stage performs exactly those additions, in that
// order, so the rotated values are reproducible bit for bit.  Register
// layout: 16 lanes hold one 128-block, 8 consecutive elements per lane;
// stages 1, 2, 4 stay inside a lane, stages 8..64 exchange with lane ^ (h/8).
#include "kernels.h"

namespace w8a8 {

namespace {

__device__ __forceinline__ float block_max_256(float v, float* part) {
  v = wave_max(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
}

}  // namespace

constexpr int kMaxK = 16384;

// One 256-thread workgroup per row: rotate into LDS, reduce amax, quantise.
// PACKED_OUT: codes in the 16-row x 64-byte MFMA tile layout of pack.hip
// (row m, k bytes 16c..16c+15 -> tile m/16, block c/4, slot m%16 + 16*(c%4)),
// the operand layout of the tiled GEMM; ldq is then unused.
template <bool PACKED_OUT>
__global__ __launch_bounds__(256) void k_fwht128_quant(const uint16_t* __restrict__ x,
                                                       int64_t ldx, int K,
                                                       int8_t* __restrict__ q, int64_t ldq,
                                                       float* __restrict__ s) {
  __shared__ __attribute__((aligned(16))) float rot[kMaxK];
  __shared__ float part[4];
  const int64_t row = blockIdx.x;
  const uint16_t* xr = x + row * ldx;
  const int l16 = threadIdx.x & 15;
  const int nblk = K >> 7;
  float amax = 0.0f;
  for (int b0 = 0; b0 < nblk; b0 += 16) {
    const int blk = b0 + (threadIdx.x >> 4);
    const bool ok = blk < nblk;
    Block8 b;
    if (ok) {
      const v4u raw = *reinterpret_cast<const v4u*>(xr + blk * 128 + l16 * 8);
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int i = 0; i < 4; i++) {
        b.v[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
        b.v[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
      }
    } else {
#pragma unroll
      for (int c = 0; c < 8; c++) b.v[c] = 0.0f;
    }
    fwht128_lanes(b, l16);
    if (ok) {
      float* dst = rot + blk * 128 + l16 * 8;
#pragma unroll
      for (int c = 0; c < 8; c++) {
        dst[c] = b.v[c];
        amax = fmaxf(amax, fabsf(b.v[c]));
      }
    }
  }
  amax = block_max_256(amax, part);
  const float sc = amax / 127.0f;
  // codes: 16 per thread-iteration, one 16-byte store
  for (int c16 = threadIdx.x; c16 < (K >> 4); c16 += 256) {
    const float* src = rot + c16 * 16;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      int a0 = 0, a1 = 0, a2 = 0, a3 = 0;
      if (amax != 0.0f) {
        a0 = quant_code(src[4 * i], sc);
        a1 = quant_code(src[4 * i + 1], sc);
        a2 = quant_code(src[4 * i + 2], sc);
        a3 = quant_code(src[4 * i + 3], sc);
      }
      w[i] = pack4_i8(a0, a1, a2, a3);
    }
    const int64_t off = PACKED_OUT ? ((row >> 4) * (int64_t)(K >> 6) + (c16 >> 2)) * 1024 +
                                         ((row & 15) + 16 * (c16 & 3)) * 16
                                   : row * ldq + c16 * 16;
    *reinterpret_cast<v4u*>(q + off) = v4u{w[0], w[1], w[2], w[3]};
  }
  if (threadIdx.x == 0) s[row] = amax != 0.0f ? sc : 0.0f;
}

// Rotated weight preparation, one 256-thread workgroup per weight row.
__global__ __launch_bounds__(256) void k_fwht128_wprep(const float* __restrict__ W, int K,
                                                       int8_t* __restrict__ qw,
                                                       uint8_t* __restrict__ su8,
                                                       uint16_t* __restrict__ s2) {
  __shared__ __attribute__((aligned(16))) float rot[kMaxK];
  __shared__ float gmax[kMaxK / 256];
  __shared__ float eff_s[kMaxK / 256];
  __shared__ float part[4];
  const int64_t row = blockIdx.x;
  const float* wr = W + row * K;
  const int l16 = threadIdx.x & 15;
  const int lane = threadIdx.x & 63;
  const int nblk = K >> 7;
  const int G = K >> 8;
  for (int b0 = 0; b0 < nblk; b0 += 16) {
    const int blk = b0 + (threadIdx.x >> 4);
    const bool ok = blk < nblk;
    Block8 b;
    if (ok) {
      const v4f lo = *reinterpret_cast<const v4f*>(wr + blk * 128 + l16 * 8);
      const v4f hi = *reinterpret_cast<const v4f*>(wr + blk * 128 + l16 * 8 + 4);
      b.v[0] = lo.x; b.v[1] = lo.y; b.v[2] = lo.z; b.v[3] = lo.w;
      b.v[4] = hi.x; b.v[5] = hi.y; b.v[6] = hi.z; b.v[7] = hi.w;
    } else {
#pragma unroll
      for (int c = 0; c < 8; c++) b.v[c] = 0.0f;
    }
    fwht128_lanes(b, l16);
    float m = 0.0f;
    if (ok) {
      float* dst = rot + blk * 128 + l16 * 8;
#pragma unroll
      for (int c = 0; c < 8; c++) {
        dst[c] = b.v[c];
        m = fmaxf(m, fabsf(b.v[c]));
      }
    }
    // a 256-group is two consecutive blocks = 32 consecutive lanes
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    if (ok && (lane & 31) == 0) gmax[blk >> 1] = m;
  }
  __syncthreads();
  // per-group scale a_g / 127 and the row maximum of those scales
  float smax = 0.0f;
  for (int gi = threadIdx.x; gi < G; gi += 256) smax = fmaxf(smax, gmax[gi] / 127.0f);
  smax = block_max_256(smax, part);
  const uint32_t s2b = f32_to_bf16_bits(smax / 255.0f);
  const float s2f = bf16_bits_to_f32(s2b);
  for (int gi = threadIdx.x; gi < G; gi += 256) {
    const float sg = gmax[gi] / 127.0f;
    int u = 0;
    if (s2f != 0.0f && sg != 0.0f) {
      float r = __builtin_rintf(sg / s2f);
      r = fminf(fmaxf(r, 1.0f), 255.0f);
      u = (int)r;
    }
    su8[row * G + gi] = (uint8_t)u;
    eff_s[gi] = s2f * (float)u;
  }
  if (threadIdx.x == 0) s2[row] = (uint16_t)s2b;
  __syncthreads();
  for (int c16 = threadIdx.x; c16 < (K >> 4); c16 += 256) {
    const float eff = eff_s[c16 >> 4];
    const float* src = rot + c16 * 16;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      int a[4] = {0, 0, 0, 0};
      if (eff != 0.0f) {
#pragma unroll
        for (int t = 0; t < 4; t++) a[t] = quant_code(src[4 * i + t], eff);
      }
      w[i] = pack4_i8(a[0], a[1], a[2], a[3]);
    }
    *reinterpret_cast<v4u*>(qw + row * K + c16 * 16) = v4u{w[0], w[1], w[2], w[3]};
  }
}

// Rotated weight preparation with a bf16 scale per row per 128 of K (each
// 128-group is one rotated block): one 16-lane group owns a block, so the
// block maximum is a 16-lane reduction and no LDS is needed.  s = bf16(amax /
// 127) rounded to nearest even; the codes are taken against the stored bf16
// scale (zero codes where it is zero).  Workgroup b takes rows 16 b .. (one
// 16-lane group per row, the row's blocks in turn); W fp32 [N, K], qw
// row-major [N, K], s [N, K / 128].
__global__ __launch_bounds__(256) void k_fwht128_wprep_g128(const float* __restrict__ W,
                                                            int64_t N, int K,
                                                            int8_t* __restrict__ qw,
                                                            uint16_t* __restrict__ s) {
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  if (row >= N) return;  // 16-lane-uniform; the shuffles below stay within a group
  const int l16 = threadIdx.x & 15;
  const float* wr = W + row * K;
  const int G = K >> 7;
  for (int blk = 0; blk < G; blk++) {
    Block8 b;
    const v4f lo = *reinterpret_cast<const v4f*>(wr + blk * 128 + l16 * 8);
    const v4f hi = *reinterpret_cast<const v4f*>(wr + blk * 128 + l16 * 8 + 4);
    b.v[0] = lo.x; b.v[1] = lo.y; b.v[2] = lo.z; b.v[3] = lo.w;
    b.v[4] = hi.x; b.v[5] = hi.y; b.v[6] = hi.z; b.v[7] = hi.w;
    fwht128_lanes(b, l16);
    float m = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; c++) m = fmaxf(m, fabsf(b.v[c]));
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, 16));
    const uint32_t sb = f32_to_bf16_bits(m / 127.0f);
    const float sf = bf16_bits_to_f32(sb);
    int a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (sf != 0.0f) {
#pragma unroll
      for (int c = 0; c < 8; c++) a[c] = quant_code(b.v[c], sf);
    }
    *reinterpret_cast<uint2*>(qw + row * K + blk * 128 + l16 * 8) =
        make_uint2(pack4_i8(a[0], a[1], a[2], a[3]), pack4_i8(a[4], a[5], a[6], a[7]));
    if (l16 == 0) s[row * G + blk] = (uint16_t)sb;
  }
}

// g256 epilogue: exact int64 group sum -> fp64 scaling -> fp32 -> bf16.
__device__ __forceinline__ uint16_t g256_out(long long tsum, float sa, float s2f) {
  double v = (double)tsum * (double)sa;
  v = v * (double)s2f;
  v = v * 0.0078125;
  return (uint16_t)f32_to_bf16_bits((float)v);
}

// Weight-streaming g256 GEMM for M <= 16 (same operand mapping as the dense
// decode kernel).  Wave w takes the 256-groups w, w + WAVES, ...; each group
// is four 64-byte k steps (four 1 KiB loads with packed weights), and the
// loads of two groups are in flight at once.  After each group the exact
// int32 MFMA sum times that group's u8 (< 2^31: |sum| <= 256 * 127^2) is added
// to an int64 running sum; the waves' sums are added through LDS.
template <int WAVES, bool PACKED>
__global__ __launch_bounds__(WAVES * 64) void k_gemm_g256_skinny(
    const int8_t* __restrict__ qa, const float* __restrict__ sa, int M, int K,
    const int8_t* __restrict__ qw, const uint8_t* __restrict__ su8,
    const uint16_t* __restrict__ s2, uint16_t* __restrict__ y, int64_t ldy) {
  __shared__ long long red[WAVES][64][4];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int j = lane & 15;
  const int g = lane >> 4;
  const int64_t tile = blockIdx.x;
  const int64_t n0 = tile * 16;
  const int G = K >> 8;
  const int nk = K >> 6;
  // k step c of this lane's weight fragment
  const int8_t* wp = PACKED ? qw + tile * nk * 1024 + lane * 16 : qw + (n0 + j) * K + g * 16;
  constexpr int64_t wstep = PACKED ? 1024 : 64;
  const bool a_ok = j < M;
  const int8_t* ap = qa + (int64_t)(a_ok ? j : 0) * K + g * 16;
  const uint8_t* sp = su8 + (n0 + j) * G;

  long long ts[4] = {0, 0, 0, 0};
  for (int g0 = wv; g0 < G; g0 += 2 * WAVES) {
    v4i b[2][4], a[2][4];
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const int gr = g0 + h * WAVES;
      const bool in = gr < G;
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const int c = gr * 4 + u;
        b[h][u] = in ? ld_stream(wp + c * wstep) : v4i{0, 0, 0, 0};
        a[h][u] = (in && a_ok) ? *reinterpret_cast<const v4i*>(ap + (int64_t)c * 64)
                               : v4i{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const int gr = g0 + h * WAVES;
      if (gr >= G) break;
      v4i acc = {0, 0, 0, 0};
#pragma unroll
      for (int u = 0; u < 4; u++) acc = mfma_16x16x64_i8(a[h][u], b[h][u], acc);
      const int u8 = sp[gr];
#pragma unroll
      for (int v = 0; v < 4; v++) ts[v] += (long long)(acc[v] * u8);
    }
  }
  // wave 0 writes the tile: its scales are loaded before the reduction (row
  // index clamped into range) and waited for once, so no store waits on a
  // scale load
  const int64_t n = n0 + j;
  float sam[4] = {0.0f, 0.0f, 0.0f, 0.0f}, s2f = 0.0f;
  if (wv == 0) {
#pragma unroll
    for (int v = 0; v < 4; v++) sam[v] = sa[min(4 * g + v, M - 1)];
    s2f = bf16_bits_to_f32(s2[n]);
  }
  if (WAVES > 1) {
#pragma unroll
    for (int v = 0; v < 4; v++) red[wv][lane][v] = ts[v];
    __syncthreads();
    if (wv != 0) return;
    for (int w = 1; w < WAVES; w++)
#pragma unroll
      for (int v = 0; v < 4; v++) ts[v] += red[w][lane][v];
  }
#pragma unroll
  for (int v = 0; v < 4; v++) keep_live(sam[v]);
  keep_live(s2f);
#pragma unroll
  for (int v = 0; v < 4; v++) {
    const int m = 4 * g + v;
    if (m >= M) break;
    y[(int64_t)m * ldy + n] = g256_out(ts[v], sam[v], s2f);
  }
}

// The single-token Hadamard-domain linear in one launch (packed weights,
// K <= kFusedG256MaxK): every workgroup rotates and quantises the token row
// itself (a few hundred instructions a wave) while its weight loads are in
// flight, then runs the g256 GEMM of k_gemm_g256_skinny on those codes.  The
// rotation, the row maximum and the codes are those of k_fwht128_quant (same
// butterfly, same quotient); workgroup 0 also stores the codes and the scale.
// Lane layout of the rotation: wave w holds the 128-blocks 4w .. 4w+3, 16
// lanes a block, 8 values a lane.  The row's loads are issued before the
// weight loads: loads retire in order, so the rotation then waits for the row
// only.
constexpr int kFusedG256MaxK = 4096;
__global__ __launch_bounds__(512) void k_linear_g256_one(
    const uint16_t* __restrict__ x, int K, const int8_t* __restrict__ qw,
    const uint8_t* __restrict__ su8, const uint16_t* __restrict__ s2,
    uint16_t* __restrict__ y, int8_t* __restrict__ q, float* __restrict__ s) {
  constexpr int WAVES = 8;
  __shared__ long long red[WAVES][16];
  __shared__ float part[WAVES];
  __shared__ __attribute__((aligned(16))) int8_t q_lds[kFusedG256MaxK];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int j = lane & 15;
  const int g = lane >> 4;
  const int64_t tile = blockIdx.x;
  const int64_t n0 = tile * 16;
  const int G = K >> 8;
  const int nk = K >> 6;
  const int nblk = K >> 7;

  // the token row: this lane's 8 values of block 4w + lane/16
  const int blk = wv * 4 + (lane >> 4);
  const int l16 = lane & 15;
  const bool xin = blk < nblk;
  const v4u raw = xin ? *reinterpret_cast<const v4u*>(x + blk * 128 + l16 * 8)
                      : v4u{0u, 0u, 0u, 0u};
  // the tile's weights (wave w: groups w and w + 8, four 1 KiB steps each),
  // their u8 group scales, and the row scale of the tile's channels
  const int8_t* wp = qw + tile * nk * 1024 + lane * 16;
  const uint8_t* sp = su8 + (n0 + j) * G;
  v4i b[2][4];
  int u8[2];
#pragma unroll
  for (int h = 0; h < 2; h++) {
    const int gr = wv + h * WAVES;
    const bool in = gr < G;
#pragma unroll
    for (int u = 0; u < 4; u++)
      b[h][u] = in ? ld_stream(wp + (gr * 4 + u) * 1024)
                   : v4i{0, 0, 0, 0};
    u8[h] = in ? sp[gr] : 0;
  }
  const float s2f = wv == 0 ? bf16_bits_to_f32(s2[n0 + j]) : 0.0f;

  // rotate, row maximum, codes into LDS
  Block8 bv;
  const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    bv.v[2 * i] = bf16_bits_to_f32(w4[i] & 0xffffu);
    bv.v[2 * i + 1] = bf16_bits_to_f32(w4[i] >> 16);
  }
  fwht128_lanes(bv, l16);
  float am = 0.0f;
  if (xin) {
#pragma unroll
    for (int c = 0; c < 8; c++) am = fmaxf(am, fabsf(bv.v[c]));
  }
  am = wave_max(am);
  if (lane == 0) part[wv] = am;
  __syncthreads();
  am = part[0];
#pragma unroll
  for (int w = 1; w < WAVES; w++) am = fmaxf(am, part[w]);
  const float sc = am / 127.0f;
  if (xin) {
    int cd[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (am != 0.0f) {
#pragma unroll
      for (int c = 0; c < 8; c++) cd[c] = quant_code(bv.v[c], sc);
    }
    const uint2 wd = make_uint2(pack4_i8(cd[0], cd[1], cd[2], cd[3]),
                                pack4_i8(cd[4], cd[5], cd[6], cd[7]));
    *reinterpret_cast<uint2*>(q_lds + blk * 128 + l16 * 8) = wd;
    if (tile == 0) *reinterpret_cast<uint2*>(q + blk * 128 + l16 * 8) = wd;
  }
  const float sa = am != 0.0f ? sc : 0.0f;
  if (tile == 0 && threadIdx.x == 0) s[0] = sa;
  __syncthreads();

  // g256 GEMM: row 0 of the A operand (lanes j == 0) holds the codes; the
  // result's row 0 is element 0 of lanes 0..15
  long long ts = 0;
#pragma unroll
  for (int h = 0; h < 2; h++) {
    const int gr = wv + h * WAVES;
    if (gr >= G) break;
    v4i acc = {0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const v4i a = j == 0 ? *reinterpret_cast<const v4i*>(q_lds + (gr * 4 + u) * 64 + g * 16)
                           : v4i{0, 0, 0, 0};
      acc = mfma_16x16x64_i8(a, b[h][u], acc);
    }
    ts += (long long)(acc[0] * u8[h]);
  }
  if (g == 0) red[wv][j] = ts;
  __syncthreads();
  if (wv == 0 && g == 0) {
#pragma unroll
    for (int w = 1; w < WAVES; w++) ts += red[w][j];
    y[n0 + j] = g256_out(ts, sa, s2f);
  }
}

hipError_t launch_gemm_g256_tile(const int8_t* qa, const float* sa, int64_t M, int64_t K,
                                 const int8_t* qw, const uint8_t* su8, const uint16_t* s2,
                                 int64_t N, bool packed, bool apacked, uint16_t* y, int64_t ldy,
                                 hipStream_t stream);

hipError_t launch_fwht128_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int8_t* q,
                                int64_t ldq, float* s, hipStream_t stream) {
  hipLaunchKernelGGL(k_fwht128_quant<false>, dim3((unsigned)M), dim3(256), 0, stream, x, ldx,
                     (int)K, q, ldq, s);
  return hipGetLastError();
}

hipError_t launch_fwht128_quant_packed(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                       int8_t* q, float* s, hipStream_t stream) {
  hipLaunchKernelGGL(k_fwht128_quant<true>, dim3((unsigned)M), dim3(256), 0, stream, x, ldx,
                     (int)K, q, (int64_t)0, s);
  return hipGetLastError();
}

hipError_t launch_fwht128_weight_prep(const float* W, int64_t N, int64_t K, int8_t* qw,
                                      uint8_t* su8, uint16_t* s2, hipStream_t stream) {
  hipLaunchKernelGGL(k_fwht128_wprep, dim3((unsigned)N), dim3(256), 0, stream, W, (int)K, qw,
                     su8, s2);
  return hipGetLastError();
}

hipError_t launch_fwht128_weight_prep_g128(const float* W, int64_t N, int64_t K, int8_t* qw,
                                           uint16_t* s, hipStream_t stream) {
  hipLaunchKernelGGL(k_fwht128_wprep_g128, dim3((unsigned)((N + 15) / 16)), dim3(256), 0, stream,
                     W, N, (int)K, qw, s);
  return hipGetLastError();
}

size_t g256_workspace_bytes(int64_t, int64_t, int64_t) { return 0; }

hipError_t launch_gemm_g256(const int8_t* qa, const float* sa, int64_t M, int64_t K,
                            const int8_t* qw, const uint8_t* su8, const uint16_t* s2, int64_t N,
                            bool packed, uint16_t* y, int64_t ldy, void*, hipStream_t stream) {
  if (M <= 16) {
    if (packed)
      hipLaunchKernelGGL((k_gemm_g256_skinny<8, true>), dim3((unsigned)(N / 16)), dim3(512), 0,
                         stream, qa, sa, (int)M, (int)K, qw, su8, s2, y, ldy);
    else
      hipLaunchKernelGGL((k_gemm_g256_skinny<8, false>), dim3((unsigned)(N / 16)), dim3(512), 0,
                         stream, qa, sa, (int)M, (int)K, qw, su8, s2, y, ldy);
    return hipGetLastError();
  }
  return launch_gemm_g256_tile(qa, sa, M, K, qw, su8, s2, N, packed, false, y, ldy, stream);
}

// The whole Hadamard-domain linear: fwht128 + per-token quant into the
// workspace (codes in the tile layout when the tiled GEMM runs), then the
// g256 GEMM on packed weights.
hipError_t launch_linear_g256(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                              const int8_t* qw_packed, const uint8_t* su8, const uint16_t* s2,
                              int64_t N, uint16_t* y, int64_t ldy, int8_t* q, float* s,
                              hipStream_t stream) {
  hipError_t e;
  if (M == 1 && K <= kFusedG256MaxK) {
    hipLaunchKernelGGL(k_linear_g256_one, dim3((unsigned)(N / 16)), dim3(512), 0, stream, x,
                       (int)K, qw_packed, su8, s2, y, q, s);
    return hipGetLastError();
  }
  if (M <= 16) {
    if ((e = launch_fwht128_quant(x, M, K, ldx, q, K, s, stream)) != hipSuccess) return e;
    return launch_gemm_g256(q, s, M, K, qw_packed, su8, s2, N, true, y, ldy, nullptr, stream);
  }
  if ((e = launch_fwht128_quant_packed(x, M, K, ldx, q, s, stream)) != hipSuccess) return e;
  return launch_gemm_g256_tile(q, s, M, K, qw_packed, su8, s2, N, true, true, y, ldy, stream);
}

}  // namespace w8a8
