// Weight-streaming W8A8 GEMM for decode-shaped inputs (M <= 16 tokens).
//
// Source: "[gfx1151] Online INT8 W8A8 for Qwen3.6 27B / 35B-A3B on RDNA3.5,
// with working MTP" (ATOM pull request): halving weight bytes matters because
// they are the decode bottleneck (intro, precision split); Changes, linear.py
// bullet: per-token int8 activations x per-channel int8 weights, bf16 out.
//
// At M <= 16 every weight byte is used once, so the kernel is bound by HBM
// reads of the [N, K] int8 weights.  Each workgroup owns 16 output channels
// (one 16x16x64 MFMA column tile).  Its waves take the tile's 64-byte k
// steps round-robin (wave w of W: steps w, w+W, ...), so at any moment the
// workgroup streams one contiguous stretch of the tile; every wave keeps U
// 1 KiB weight loads in flight, non-temporal (the weights are read once:
// measured on MI355X 7% faster than plain loads over the decode step).  The
// waves' int32 partial sums are added exactly through LDS and the fp32
// epilogue runs in registers: no workspace and no cross-workgroup traffic.
//
// Weight layouts: row-major [N, K], or the packed tile layout (see pack.hip)
// in which each 16-row x 64-byte MFMA operand tile is one contiguous 1 KiB
// block, so every wave-wide load reads 1 KiB of consecutive bytes.
//
// MFMA operand mapping (v_mfma_i32_16x16x64_i8): lane l supplies 16 bytes of
// A row (l % 16) and of B column (l % 16) for k-slice (l / 16); the same
// k-slice is used for A and B, so the sum over k is exact whatever the
// hardware's byte order inside the slice.  Result lane l holds rows
// 4*(l/16) + v (v = 0..3) of column l % 16.  Rows >= M are fed zeros.
#include "kernels.h"

namespace w8a8 {

// Epilogues of the decode GEMM: bf16 y = (float(acc) * sa) * sw; the int32
// sums; or the gated SiLU of an interleaved gate/up weight (rows 2i = gate_i,
// 2i+1 = up_i): act[m, i] = silu(h[m, 2i]) * h[m, 2i+1] in fp32 with h the
// fp32-dequantised sums (SiLU in fp64, rounded once).
enum { kSkEpiBf16 = 0, kSkEpiI32 = 1, kSkEpiSilu = 2 };

__device__ __forceinline__ float silu_times(float gate, float up) {
  const float sg = (float)((double)gate / (1.0 + exp(-(double)gate)));
  return sg * up;
}

template <int WAVES, int U, bool PACKED, int EPI>
__global__ __launch_bounds__(WAVES * 64) void k_gemm_skinny(
    const int8_t* __restrict__ qa, const float* __restrict__ sa, int M, int K, int64_t lda,
    const int8_t* __restrict__ qw, const float* __restrict__ sw, int64_t ldw,
    void* __restrict__ out, int64_t ldo) {
  __shared__ v4i red[WAVES][64];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int j = lane & 15;  // A row (token) / B column (output channel)
  const int g = lane >> 4;  // 16-byte k-slice inside a 64-wide k step
  const int64_t tile = blockIdx.x;
  const int nchunk = K >> 6;  // 64-wide k steps

  const int8_t* wp = PACKED ? qw + tile * nchunk * 1024 + lane * 16
                            : qw + (tile * 16 + j) * ldw + g * 16;
  constexpr int64_t wstep = PACKED ? 1024 : 64;
  const bool a_ok = j < M;
  const int8_t* ap = qa + (int64_t)(a_ok ? j : 0) * lda + g * 16;

  v4i acc = {0, 0, 0, 0};
  for (int c0 = wv; c0 < nchunk; c0 += WAVES * U) {
    v4i b[U], a[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int c = c0 + u * WAVES;
      const bool in = c < nchunk;
      b[u] = in ? ld_stream(wp + c * wstep) : v4i{0, 0, 0, 0};
      a[u] = (in && a_ok) ? *reinterpret_cast<const v4i*>(ap + (int64_t)c * 64)
                          : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; u++) acc = mfma_16x16x64_i8(a[u], b[u], acc);
  }

  // wave 0 writes the tile: its scales are loaded before the reduction
  // (row index clamped into range) and waited for once, so no store waits
  // on a scale load (a load between two stores would also wait for the
  // earlier store)
  constexpr bool STORE_I32 = EPI == kSkEpiI32;
  const int64_t n = tile * 16 + j;
  float sam[4] = {0.0f, 0.0f, 0.0f, 0.0f}, swn = 0.0f;
  if (!STORE_I32 && wv == 0) {
#pragma unroll
    for (int v = 0; v < 4; v++) sam[v] = sa[min(4 * g + v, M - 1)];
    swn = sw[n];
  }
  red[wv][lane] = acc;
  __syncthreads();
  if (wv != 0) return;
#pragma unroll
  for (int w = 1; w < WAVES; w++) acc += red[w][lane];
  if (!STORE_I32) {
#pragma unroll
    for (int v = 0; v < 4; v++) keep_live(sam[v]);
    keep_live(swn);
  }
  if (EPI == kSkEpiSilu) {
    // lanes j and j ^ 1 hold the gate and up rows of one channel for the same
    // tokens; the even lane forms the activation
    float h[4], up[4];
#pragma unroll
    for (int v = 0; v < 4; v++) {
      h[v] = (float)acc[v];
      h[v] = h[v] * sam[v];
      h[v] = h[v] * swn;
      up[v] = __shfl_xor(h[v], 1, 64);
    }
    if ((j & 1) == 0) {
#pragma unroll
      for (int v = 0; v < 4; v++) {
        const int m = 4 * g + v;
        if (m >= M) break;
        static_cast<float*>(out)[(int64_t)m * ldo + (n >> 1)] = silu_times(h[v], up[v]);
      }
    }
    return;
  }
#pragma unroll
  for (int v = 0; v < 4; v++) {
    const int m = 4 * g + v;
    if (m >= M) break;
    if (STORE_I32) {
      static_cast<int32_t*>(out)[(int64_t)m * ldo + n] = acc[v];
    } else {
      float r = (float)acc[v];
      r = r * sam[v];
      r = r * swn;
      static_cast<uint16_t*>(out)[(int64_t)m * ldo + n] = (uint16_t)f32_to_bf16_bits(r);
    }
  }
}

// 8 waves x 8 loads of 1 KiB in flight per wave (measured on MI355X over
// waves in {4, 8, 16} and depths 4..24 at the decode shapes)
constexpr int kSkinnyWaves = 8;
constexpr int kSkinnyU = 8;

// The decode linear for one or two tokens in one launch (packed weights): every
// workgroup quantises the bf16 rows itself into LDS while its first weight
// batch is in flight, then runs the k_gemm_skinny main loop with the codes
// read from LDS.  The row loads are issued before the weight loads (loads
// retire in order, so the quantisation waits for the rows only).  Codes and
// scales are those of k_quant_rows (row maximum, amax / 127, the same
// quotient).  Every workgroup repeats the quantisation, which pays only while
// a CU holds few workgroups: the launcher takes this kernel for at most two
// 16-channel tiles per CU (the down projection of the decode workload: one
// token 14.1 -> 11.8 us, two 14.1 -> 13.4 us; with four workgroups a CU, as
// for the gate_up projection, it is slower).
// Eight consecutive values of a row: bf16 as one 16-byte load, fp32 as two.
template <typename T>
struct Row8;
template <>
struct Row8<uint16_t> {
  v4u r;
  __device__ __forceinline__ void load(const uint16_t* p) { r = *reinterpret_cast<const v4u*>(p); }
  __device__ __forceinline__ void zero() { r = v4u{0u, 0u, 0u, 0u}; }
  __device__ __forceinline__ float at(int i) const {
    const uint32_t w = r[i >> 1];
    return bf16_bits_to_f32((i & 1) ? (w >> 16) : (w & 0xffffu));
  }
  __device__ __forceinline__ float absmax() const {
    uint32_t m = 0u;
#pragma unroll
    for (int i = 0; i < 4; i++) m = bf16x2_absmax(m, r[i]);
    return bf16x2_absmax_value(m);
  }
};
template <>
struct Row8<float> {
  v4f a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const v4f*>(p);
    b = *reinterpret_cast<const v4f*>(p + 4);
  }
  __device__ __forceinline__ void zero() {
    a = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    b = a;
  }
  __device__ __forceinline__ float at(int i) const { return i < 4 ? a[i] : b[i - 4]; }
  __device__ __forceinline__ float absmax() const {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++) m = fmaxf(m, fabsf(at(i)));
    return m;
  }
};

// TIN: bf16 rows (the linear entry points) or fp32 rows (the MLP block's
// activation, quantised as k_quant_rows<float>: IEEE quotient always).  With
// q_out / s_out, workgroup 0 also writes the codes (row-major, row stride K)
// and the scales.
template <int MMAX, int XH, typename TIN>
__global__ __launch_bounds__(kSkinnyWaves * 64) void k_linear_skinny_fused(
    const TIN* __restrict__ x, int64_t ldx, int M, int K, const int8_t* __restrict__ qw,
    const float* __restrict__ sw, uint16_t* __restrict__ out, int64_t ldo,
    int8_t* __restrict__ q_out, float* __restrict__ s_out) {
  constexpr int WAVES = kSkinnyWaves, U = kSkinnyU, NT = WAVES * 64;
  __shared__ v4i red[WAVES][64];
  __shared__ float part[WAVES][MMAX];
  extern __shared__ __attribute__((aligned(16))) int8_t q_lds[];  // M rows of K codes
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int tid = threadIdx.x;
  const int j = lane & 15;
  const int g = lane >> 4;
  const int64_t tile = blockIdx.x;
  const int nchunk = K >> 6;
  const int nc8 = K >> 3;  // 8-value chunks a row
  const int tot = M * nc8;

  // the rows: chunk c = tid + NT * i of the M x nc8 chunks
  Row8<TIN> xr[XH];
#pragma unroll
  for (int i = 0; i < XH; i++) {
    const int c = tid + NT * i;
    const int r = c / nc8, col = c - r * nc8;
    if (c < tot)
      xr[i].load(x + (int64_t)r * ldx + col * 8);
    else
      xr[i].zero();
  }
  // the first weight batch
  const int8_t* wp = qw + tile * nchunk * 1024 + lane * 16;
  v4i b0[U];
#pragma unroll
  for (int u = 0; u < U; u++) {
    const int c = wv + u * WAVES;
    b0[u] = c < nchunk ? ld_stream(wp + (int64_t)c * 1024) : v4i{0, 0, 0, 0};
  }
  const int64_t n = tile * 16 + j;
  const float swn = wv == 0 ? sw[n] : 0.0f;

  // row maxima: per thread, per wave, then across the waves
  float am[MMAX];
#pragma unroll
  for (int r = 0; r < MMAX; r++) am[r] = 0.0f;
#pragma unroll
  for (int i = 0; i < XH; i++) {
    const int r = (tid + NT * i) / nc8;
    const float m8 = xr[i].absmax();
#pragma unroll
    for (int rr = 0; rr < MMAX; rr++)
      if (rr == r) am[rr] = fmaxf(am[rr], m8);
  }
#pragma unroll
  for (int r = 0; r < MMAX; r++) {
    const float v = wave_max(am[r]);
    if (lane == 0) part[wv][r] = v;
  }
  __syncthreads();
  float sc[MMAX], rc[MMAX];
#pragma unroll
  for (int r = 0; r < MMAX; r++) {
    am[r] = part[0][r];
#pragma unroll
    for (int w = 1; w < WAVES; w++) am[r] = fmaxf(am[r], part[w][r]);
    sc[r] = am[r] / 127.0f;
    rc[r] = 1.0f / sc[r];
  }
  if (s_out && tile == 0 && tid < M) {
#pragma unroll
    for (int rr = 0; rr < MMAX; rr++)
      if (rr == tid) s_out[rr] = am[rr] != 0.0f ? sc[rr] : 0.0f;
  }
  // codes into LDS, row r at r * K
#pragma unroll
  for (int i = 0; i < XH; i++) {
    const int c = tid + NT * i;
    if (c >= tot) break;
    const int r = c / nc8, col = c - r * nc8;
    float s_ = sc[0], r_ = rc[0], a_ = am[0];
#pragma unroll
    for (int rr = 1; rr < MMAX; rr++)
      if (rr == r) {
        s_ = sc[rr];
        r_ = rc[rr];
        a_ = am[rr];
      }
    // the reciprocal form is exact for bf16 rows only (k_quant_rows)
    const bool recip = sizeof(TIN) == 2 && s_ >= 0x1p-100f;
    uint32_t pk[2] = {0u, 0u};
    if (recip) {
#pragma unroll
      for (int hh = 0; hh < 2; hh++)
        pk[hh] = pack4_i8(quant_code_recip(xr[i].at(4 * hh), s_, r_),
                          quant_code_recip(xr[i].at(4 * hh + 1), s_, r_),
                          quant_code_recip(xr[i].at(4 * hh + 2), s_, r_),
                          quant_code_recip(xr[i].at(4 * hh + 3), s_, r_));
    } else if (a_ != 0.0f) {
#pragma unroll
      for (int hh = 0; hh < 2; hh++)
        pk[hh] = pack4_i8(quant_code(xr[i].at(4 * hh), s_), quant_code(xr[i].at(4 * hh + 1), s_),
                          quant_code(xr[i].at(4 * hh + 2), s_),
                          quant_code(xr[i].at(4 * hh + 3), s_));
    }
    *reinterpret_cast<uint2*>(q_lds + r * K + col * 8) = make_uint2(pk[0], pk[1]);
    if (q_out && tile == 0)
      *reinterpret_cast<uint2*>(q_out + (int64_t)r * K + col * 8) = make_uint2(pk[0], pk[1]);
  }
  __syncthreads();

  // the k_gemm_skinny main loop, A from LDS
  const bool a_ok = j < M;
  const int8_t* ap = q_lds + (a_ok ? j : 0) * K + g * 16;
  v4i acc = {0, 0, 0, 0};
  for (int c0 = wv; c0 < nchunk; c0 += WAVES * U) {
    v4i b[U], a[U];
    const bool first = c0 == wv;
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int c = c0 + u * WAVES;
      const bool in = c < nchunk;
      b[u] = first ? b0[u]
                   : (in ? ld_stream(wp + (int64_t)c * 1024) : v4i{0, 0, 0, 0});
      a[u] = (in && a_ok) ? *reinterpret_cast<const v4i*>(ap + c * 64) : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; u++) acc = mfma_16x16x64_i8(a[u], b[u], acc);
  }
  red[wv][lane] = acc;
  __syncthreads();
  if (wv != 0) return;
#pragma unroll
  for (int w = 1; w < WAVES; w++) acc += red[w][lane];
  keep_live(swn);
#pragma unroll
  for (int v = 0; v < 4; v++) {
    const int m = 4 * g + v;
    if (m >= M) break;
    float sv = 0.0f;
#pragma unroll
    for (int rr = 0; rr < MMAX; rr++)
      if (rr == m) sv = am[rr] != 0.0f ? sc[rr] : 0.0f;
    float r = (float)acc[v];
    r = r * sv;
    r = r * swn;
    out[(int64_t)m * ldo + n] = (uint16_t)f32_to_bf16_bits(r);
  }
}

bool linear_fused_fits(int64_t M, int64_t N, int64_t K) {
  return M >= 1 && M <= 2 && K <= 16384 && N / 16 <= 2 * (int64_t)device_cus();
}

template <typename TIN>
static hipError_t launch_fused_impl(const TIN* x, int64_t ldx, int64_t M, int64_t K,
                                    const int8_t* qw_packed, const float* sw, int64_t N,
                                    uint16_t* y, int64_t ldy, int8_t* q_out, float* s_out,
                                    hipStream_t stream) {
  // 8-value row chunks held a thread: ceil(M * K / 8 / 512), at most 4 for
  // one row and 8 for two.  Two bf16 rows hold 5 up to K = 10240 (110
  // VGPRs: two workgroups a CU); holding 8 takes 150 VGPRs and one
  // workgroup a CU.
  const size_t lds = (size_t)(M * K);
  const int64_t need = (M * (K / 8) + kSkinnyWaves * 64 - 1) / (kSkinnyWaves * 64);
  const dim3 grid((unsigned)(N / 16)), block(kSkinnyWaves * 64);
  // (12 loads a wave for the down projection, as launch_skinny_impl: 12.38 ->
  // 12.29 us at one token, 13.67 -> 18.66 us at two; kept at 8)
  if (M == 1)
    hipLaunchKernelGGL((k_linear_skinny_fused<1, 4, TIN>), grid, block, lds, stream, x, ldx,
                       (int)M, (int)K, qw_packed, sw, y, ldy, q_out, s_out);
  else if (need <= 5)
    hipLaunchKernelGGL((k_linear_skinny_fused<2, 5, TIN>), grid, block, lds, stream, x, ldx,
                       (int)M, (int)K, qw_packed, sw, y, ldy, q_out, s_out);
  else
    hipLaunchKernelGGL((k_linear_skinny_fused<2, 8, TIN>), grid, block, lds, stream, x, ldx,
                       (int)M, (int)K, qw_packed, sw, y, ldy, q_out, s_out);
  return hipGetLastError();
}

hipError_t launch_linear_skinny_fused(const uint16_t* x, int64_t ldx, int64_t M, int64_t K,
                                      const int8_t* qw_packed, const float* sw, int64_t N,
                                      uint16_t* y, int64_t ldy, hipStream_t stream) {
  return launch_fused_impl(x, ldx, M, K, qw_packed, sw, N, y, ldy, nullptr, nullptr, stream);
}

hipError_t launch_linear_skinny_fused_f32(const float* x, int64_t ldx, int64_t M, int64_t K,
                                          const int8_t* qw_packed, const float* sw, int64_t N,
                                          uint16_t* y, int64_t ldy, int8_t* q_out, float* s_out,
                                          hipStream_t stream) {
  return launch_fused_impl(x, ldx, M, K, qw_packed, sw, N, y, ldy, q_out, s_out, stream);
}

template <bool PACKED, int EPI>
static hipError_t launch_skinny_impl(const int8_t* qa, const float* sa, int64_t M, int64_t K,
                                     int64_t lda, const int8_t* qw, const float* sw, int64_t N,
                                     int64_t ldw, void* out, int64_t ldo, hipStream_t stream) {
  // loads in flight per wave by the tile's k-step count: 65..80 steps take one
  // round of 10 (the gate_up projection, K=5120: 17.0 -> 16.5 us at one
  // token, 19.3 -> 18.1 at eight), 129..144 steps two rounds of 12 (the down
  // projection, K=8704: 11.57 -> 11.44 us, 13.6 -> 13.2), else 8 (measured on
  // MI355X, two interleaved rounds; one round of 17 for the down projection
  // was slower, 11.8 us)
  const int64_t nc = K >> 6;
  const dim3 grid((unsigned)(N / 16)), block(kSkinnyWaves * 64);
  if (nc > 64 && nc <= 80)
    hipLaunchKernelGGL((k_gemm_skinny<kSkinnyWaves, 10, PACKED, EPI>), grid, block, 0, stream,
                       qa, sa, (int)M, (int)K, lda, qw, sw, ldw, out, ldo);
  else if (nc > 128 && nc <= 144)
    hipLaunchKernelGGL((k_gemm_skinny<kSkinnyWaves, 12, PACKED, EPI>), grid, block, 0, stream,
                       qa, sa, (int)M, (int)K, lda, qw, sw, ldw, out, ldo);
  else
    hipLaunchKernelGGL((k_gemm_skinny<kSkinnyWaves, kSkinnyU, PACKED, EPI>), grid, block, 0,
                       stream, qa, sa, (int)M, (int)K, lda, qw, sw, ldw, out, ldo);
  return hipGetLastError();
}

hipError_t launch_gemm_skinny(const int8_t* qa, const float* sa, int64_t M, int64_t K,
                              int64_t lda, const int8_t* qw, const float* sw, int64_t N,
                              int64_t ldw, bool packed, uint16_t* y, int64_t ldy,
                              hipStream_t stream) {
  return packed ? launch_skinny_impl<true, kSkEpiBf16>(qa, sa, M, K, lda, qw, sw, N, ldw, y,
                                                        ldy, stream)
                : launch_skinny_impl<false, kSkEpiBf16>(qa, sa, M, K, lda, qw, sw, N, ldw, y,
                                                         ldy, stream);
}

hipError_t launch_gemm_skinny_silu(const int8_t* qa, const float* sa, int64_t M, int64_t K,
                                   int64_t lda, const int8_t* qw_packed, const float* sw,
                                   int64_t N, float* act, int64_t ldact, hipStream_t stream) {
  return launch_skinny_impl<true, kSkEpiSilu>(qa, sa, M, K, lda, qw_packed, sw, N, K, act,
                                              ldact, stream);
}

hipError_t launch_gemm_skinny_i32(const int8_t* qa, int64_t M, int64_t K, int64_t lda,
                                  const int8_t* qw, int64_t N, int64_t ldw, bool packed,
                                  int32_t* acc, int64_t ldacc, hipStream_t stream) {
  return packed ? launch_skinny_impl<true, kSkEpiI32>(qa, nullptr, M, K, lda, qw, nullptr, N,
                                                       ldw, acc, ldacc, stream)
                : launch_skinny_impl<false, kSkEpiI32>(qa, nullptr, M, K, lda, qw, nullptr, N,
                                                        ldw, acc, ldacc, stream);
}

}  // namespace w8a8
