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
// 1 KiB weight loads in flight.  The waves' int32 partial sums are added
// exactly through LDS and the fp32 epilogue runs in registers: no workspace
// and no cross-workgroup traffic.
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

template <int WAVES, int U, bool PACKED, bool STORE_I32>
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
      b[u] = in ? *reinterpret_cast<const v4i*>(wp + c * wstep) : v4i{0, 0, 0, 0};
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

template <bool PACKED, bool STORE_I32>
static hipError_t launch_skinny_impl(const int8_t* qa, const float* sa, int64_t M, int64_t K,
                                     int64_t lda, const int8_t* qw, const float* sw, int64_t N,
                                     int64_t ldw, void* out, int64_t ldo, hipStream_t stream) {
  hipLaunchKernelGGL((k_gemm_skinny<kSkinnyWaves, kSkinnyU, PACKED, STORE_I32>),
                     dim3((unsigned)(N / 16)), dim3(kSkinnyWaves * 64), 0, stream, qa, sa, (int)M,
                     (int)K, lda, qw, sw, ldw, out, ldo);
  return hipGetLastError();
}

hipError_t launch_gemm_skinny(const int8_t* qa, const float* sa, int64_t M, int64_t K,
                              int64_t lda, const int8_t* qw, const float* sw, int64_t N,
                              int64_t ldw, bool packed, uint16_t* y, int64_t ldy,
                              hipStream_t stream) {
  return packed ? launch_skinny_impl<true, false>(qa, sa, M, K, lda, qw, sw, N, ldw, y, ldy,
                                                  stream)
                : launch_skinny_impl<false, false>(qa, sa, M, K, lda, qw, sw, N, ldw, y, ldy,
                                                   stream);
}

hipError_t launch_gemm_skinny_i32(const int8_t* qa, int64_t M, int64_t K, int64_t lda,
                                  const int8_t* qw, int64_t N, int64_t ldw, bool packed,
                                  int32_t* acc, int64_t ldacc, hipStream_t stream) {
  return packed ? launch_skinny_impl<true, true>(qa, nullptr, M, K, lda, qw, nullptr, N, ldw,
                                                 acc, ldacc, stream)
                : launch_skinny_impl<false, true>(qa, nullptr, M, K, lda, qw, nullptr, N, ldw,
                                                  acc, ldacc, stream);
}

}  // namespace w8a8
