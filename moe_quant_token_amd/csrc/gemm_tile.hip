// LDS-tiled int8 MFMA GEMM with the fused per-token x per-channel epilogue
// (prefill-shaped inputs, M > 16).
//
// Source: "[gfx1151] Online INT8 W8A8 for Qwen3.6 27B / 35B-A3B on RDNA3.5,
// with working MTP" (ATOM pull request), Changes, linear.py bullet (int8
// activations per token x int8 weights per channel, fp32 scales, bf16 out);
// the Performance section notes prefill is compute-bound.
//
// Layout: both operands are K-contiguous ([M, K] activations, [N, K] weights),
// which is the native operand order of v_mfma_i32_16x16x64_i8: every lane
// reads 16 consecutive k bytes of one row, so no transposes are needed.
//
// Workgroup tile BM x BN, k step 64, WAVES_M x WAVES_N waves.  Each k step the
// block copies a BM x 64 and a BN x 64 byte tile to LDS (16-byte loads and
// stores, double buffered: the next step's global loads are in flight while
// the current step's MFMAs run).  Inside a 64-byte LDS row the four 16-byte
// chunks are XOR-swizzled by (row / 2) % 4 so the 16-byte reads of eight
// consecutive rows fall in distinct banks.
#include "kernels.h"

namespace w8a8 {

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * 64 + ((chunk ^ ((row >> 1) & 3)) << 4);
}

// MODE 0: bf16 epilogue (float(acc) * sa[m]) * sw[n]; MODE 1: store the int32
// sums; MODE 2: Hadamard-domain g256 epilogue (every four k steps = one group
// of 256, the exact int32 sum is scaled by su8[n, group] into an int64 sum).
enum { kEpiBf16 = 0, kEpiI32 = 1, kEpiG256 = 2 };

template <int BM, int BN, int WAVES_M, int WAVES_N, int MODE>
__global__ __launch_bounds__(WAVES_M* WAVES_N * 64) void k_gemm_tile(
    const int8_t* __restrict__ qa, const float* __restrict__ sa, int M, int K, int64_t lda,
    const int8_t* __restrict__ qw, const float* __restrict__ sw, int N, int64_t ldw,
    void* __restrict__ out, int64_t ldo, int tiles_n, int group_m,
    const uint8_t* __restrict__ su8, const uint16_t* __restrict__ s2) {
  constexpr int NT = WAVES_M * WAVES_N * 64;
  constexpr int WM = BM / WAVES_M;  // rows of the wave tile
  constexpr int WN = BN / WAVES_N;  // columns of the wave tile
  constexpr int TM = WM / 16;
  constexpr int TN = WN / 16;
  constexpr int A_CH = BM * 4;  // 16-byte chunks per k step
  constexpr int B_CH = BN * 4;
  constexpr int A_PER = (A_CH + NT - 1) / NT;
  constexpr int B_PER = (B_CH + NT - 1) / NT;
  static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile must be a multiple of 16");

  __shared__ __attribute__((aligned(16))) int8_t sA[2][BM * 64];
  __shared__ __attribute__((aligned(16))) int8_t sB[2][BN * 64];

  // Tile order: groups of `group_m` row tiles sweep all column tiles, so
  // workgroups running together share activation rows and weight rows in L2.
  const int tiles_m = (M + BM - 1) / BM;
  const int bid = blockIdx.x;
  const int per_group = group_m * tiles_n;
  const int grp = bid / per_group;
  const int first_m = grp * group_m;
  const int gm = min(tiles_m - first_m, group_m);
  const int in_grp = bid - grp * per_group;
  const int tm = first_m + in_grp % gm;
  const int tn = in_grp / gm;
  const int m0 = tm * BM;
  const int n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int wm = wv / WAVES_N;
  const int wn = wv % WAVES_N;
  const int j = lane & 15;
  const int g = lane >> 4;

  // global -> register staging of one k step
  v4i ra[A_PER], rb[B_PER];
  auto load_tiles = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_PER; i++) {
      const int ch = tid + i * NT;
      if (ch < A_CH) {
        const int r = ch >> 2, c = ch & 3;
        const int gr = min(m0 + r, M - 1);
        ra[i] = *reinterpret_cast<const v4i*>(qa + (int64_t)gr * lda + k0 + c * 16);
      }
    }
#pragma unroll
    for (int i = 0; i < B_PER; i++) {
      const int ch = tid + i * NT;
      if (ch < B_CH) {
        const int r = ch >> 2, c = ch & 3;
        const int gr = min(n0 + r, N - 1);
        rb[i] = *reinterpret_cast<const v4i*>(qw + (int64_t)gr * ldw + k0 + c * 16);
      }
    }
  };
  auto store_tiles = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_PER; i++) {
      const int ch = tid + i * NT;
      if (ch < A_CH) *reinterpret_cast<v4i*>(&sA[buf][swz(ch >> 2, ch & 3)]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_PER; i++) {
      const int ch = tid + i * NT;
      if (ch < B_CH) *reinterpret_cast<v4i*>(&sB[buf][swz(ch >> 2, ch & 3)]) = rb[i];
    }
  };

  v4i acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; i++)
#pragma unroll
    for (int n = 0; n < TN; n++) acc[i][n] = v4i{0, 0, 0, 0};
  long long ts[MODE == kEpiG256 ? TM : 1][MODE == kEpiG256 ? TN : 1][4];
  if (MODE == kEpiG256) {
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
      for (int n = 0; n < TN; n++)
#pragma unroll
        for (int v = 0; v < 4; v++) ts[i][n][v] = 0;
  }
  const int G = K >> 8;

  const int nk = K >> 6;
  load_tiles(0);
  store_tiles(0);
  __syncthreads();

  for (int kt = 0; kt < nk; kt++) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_tiles((kt + 1) << 6);

    v4i fa[TM], fb[TN];
#pragma unroll
    for (int i = 0; i < TM; i++)
      fa[i] = *reinterpret_cast<const v4i*>(&sA[cur][swz(wm * WM + i * 16 + j, g)]);
#pragma unroll
    for (int n = 0; n < TN; n++)
      fb[n] = *reinterpret_cast<const v4i*>(&sB[cur][swz(wn * WN + n * 16 + j, g)]);
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
      for (int n = 0; n < TN; n++) acc[i][n] = mfma_16x16x64_i8(fa[i], fb[n], acc[i][n]);

    if (MODE == kEpiG256 && (kt & 3) == 3) {
#pragma unroll
      for (int n = 0; n < TN; n++) {
        const int col = min(n0 + wn * WN + n * 16 + j, N - 1);
        const long long u8 = su8[(int64_t)col * G + (kt >> 2)];
#pragma unroll
        for (int i = 0; i < TM; i++) {
#pragma unroll
          for (int v = 0; v < 4; v++) ts[i][n][v] += (long long)acc[i][n][v] * u8;
          acc[i][n] = v4i{0, 0, 0, 0};
        }
      }
    }

    if (kt + 1 < nk) store_tiles(cur ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds rows 4g+v of column j of every 16x16 block
#pragma unroll
  for (int n = 0; n < TN; n++) {
    const int col = n0 + wn * WN + n * 16 + j;
    if (col >= N) continue;
    const float swn = MODE == kEpiBf16 ? sw[col] : 0.0f;
    const float s2f = MODE == kEpiG256 ? __uint_as_float((uint32_t)s2[col] << 16) : 0.0f;
#pragma unroll
    for (int i = 0; i < TM; i++) {
#pragma unroll
      for (int v = 0; v < 4; v++) {
        const int row = m0 + wm * WM + i * 16 + 4 * g + v;
        if (row >= M) continue;
        if (MODE == kEpiI32) {
          static_cast<int32_t*>(out)[(int64_t)row * ldo + col] = acc[i][n][v];
        } else if (MODE == kEpiG256) {
          double r = (double)ts[i][n][v] * (double)sa[row];
          r = r * (double)s2f;
          r = r * 0.0078125;
          static_cast<uint16_t*>(out)[(int64_t)row * ldo + col] =
              (uint16_t)f32_to_bf16_bits((float)r);
        } else {
          float r = (float)acc[i][n][v];
          r = r * sa[row];
          r = r * swn;
          static_cast<uint16_t*>(out)[(int64_t)row * ldo + col] = (uint16_t)f32_to_bf16_bits(r);
        }
      }
    }
  }
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int MODE>
static hipError_t launch_tile_cfg(const int8_t* qa, const float* sa, int64_t M, int64_t K,
                                  int64_t lda, const int8_t* qw, const float* sw, int64_t N,
                                  int64_t ldw, void* out, int64_t ldo, const uint8_t* su8,
                                  const uint16_t* s2, hipStream_t stream) {
  const int tiles_m = (int)((M + BM - 1) / BM);
  const int tiles_n = (int)((N + BN - 1) / BN);
  const int group_m = 8;
  dim3 grid((unsigned)(tiles_m * tiles_n)), block(WAVES_M * WAVES_N * 64);
  hipLaunchKernelGGL((k_gemm_tile<BM, BN, WAVES_M, WAVES_N, MODE>), grid, block, 0, stream, qa,
                     sa, (int)M, (int)K, lda, qw, sw, (int)N, ldw, out, ldo, tiles_n, group_m,
                     su8, s2);
  return hipGetLastError();
}

template <int MODE>
static hipError_t launch_tile_impl(const int8_t* qa, const float* sa, int64_t M, int64_t K,
                                   int64_t lda, const int8_t* qw, const float* sw, int64_t N,
                                   int64_t ldw, void* out, int64_t ldo, hipStream_t stream) {
  if (M >= 2048 && N >= 2048)
    return launch_tile_cfg<256, 256, 2, 2, MODE>(qa, sa, M, K, lda, qw, sw, N, ldw, out, ldo,
                                                 nullptr, nullptr, stream);
  return launch_tile_cfg<64, 64, 2, 2, MODE>(qa, sa, M, K, lda, qw, sw, N, ldw, out, ldo,
                                             nullptr, nullptr, stream);
}

hipError_t launch_gemm_tile(const int8_t* qa, const float* sa, int64_t M, int64_t K,
                            int64_t lda, const int8_t* qw, const float* sw, int64_t N,
                            int64_t ldw, uint16_t* y, int64_t ldy, hipStream_t stream) {
  return launch_tile_impl<kEpiBf16>(qa, sa, M, K, lda, qw, sw, N, ldw, y, ldy, stream);
}

hipError_t launch_gemm_tile_i32(const int8_t* qa, int64_t M, int64_t K, int64_t lda,
                                const int8_t* qw, int64_t N, int64_t ldw, int32_t* acc,
                                int64_t ldacc, hipStream_t stream) {
  return launch_tile_impl<kEpiI32>(qa, nullptr, M, K, lda, qw, nullptr, N, ldw, acc, ldacc,
                                   stream);
}

hipError_t launch_gemm_g256_tile(const int8_t* qa, const float* sa, int64_t M, int64_t K,
                                 const int8_t* qw, const uint8_t* su8, const uint16_t* s2,
                                 int64_t N, uint16_t* y, int64_t ldy, hipStream_t stream) {
  return launch_tile_cfg<64, 64, 2, 2, kEpiG256>(qa, sa, M, K, K, qw, nullptr, N, K, y, ldy,
                                                 su8, s2, stream);
}

}  // namespace w8a8
