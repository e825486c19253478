// LDS-tiled int8 MFMA GEMM with the fused per-token x per-channel epilogue
// (prefill-shaped inputs, M > 16).
//
// Source: "[gfx1151] Online INT8 W8A8 for Qwen3.6 27B / 35B-A3B on RDNA3.5,
// with working MTP" (ATOM pull request), Changes, linear.py bullet (int8
// activations per token x int8 weights per channel, fp32 scales, bf16 out);
// its Performance section notes that prefill is compute-bound.
//
// Both operands are K-contiguous, the native operand order of
// v_mfma_i32_16x16x64_i8 (each lane feeds 16 consecutive k bytes of one row).
// Every 64-byte k step the workgroup stages a BM x 64 activation tile and a
// BN x 64 weight tile in LDS as 1 KiB blocks in MFMA lane order (16 rows x 4
// k-slices, lane l's 16 bytes at offset 16*l), so the operand reads are
// consecutive 16-byte LDS reads with no bank conflicts and no swizzle.  A wave
// fetches one block per global load: 16 rows x 64 bytes for row-major
// operands, or 1 KiB of consecutive bytes for packed weights (pack.hip).
//
// Pipeline: an NSTAGE-deep ring of LDS stages filled by global_load_lds_dwordx4
// (global memory straight into LDS, no staging registers): each wave's load
// lands as one 1 KiB block at lane-order offsets.  Loads run NSTAGE-1 k steps
// ahead; before a step is read, each wave waits for its own loads of that step
// (s_waitcnt vmcnt) and a barrier makes every wave's blocks visible.
// Workgroups are dispatched round-robin over the 8 XCDs; the tile order gives
// each XCD a contiguous range of tiles, grouped by rows, so tiles that share
// operands share an L2.
#include "kernels.h"

namespace w8a8 {

// MODE 0: bf16 epilogue (float(acc) * sa[m]) * sw[n]; MODE 1: store the int32
// sums; MODE 2: Hadamard-domain g256 epilogue (every four k steps = one group
// of 256, the exact int32 sum is scaled by su8[n, group] into an int64 sum).
enum { kEpiBf16 = 0, kEpiI32 = 1, kEpiG256 = 2 };

constexpr int kXcds = 8;

// s_waitcnt immediate that waits for vmcnt <= v and leaves the other counters
// unconstrained (gfx9 encoding: vmcnt[3:0] at bits 3:0 and vmcnt[5:4] at bits
// 15:14, expcnt at 6:4, lgkmcnt at 11:8).
constexpr int vmcnt_imm(int v) { return (v & 15) | ((v >> 4) << 14) | (7 << 4) | (15 << 8); }

template <int BM, int BN, int WAVES_M, int WAVES_N, int NSTAGE, int MODE, bool BPACKED>
__global__ __launch_bounds__(WAVES_M* WAVES_N * 64) void k_gemm_tile(
    const int8_t* __restrict__ qa, const float* __restrict__ sa, int M, int K, int64_t lda,
    const int8_t* __restrict__ qw, const float* __restrict__ sw, int N, int64_t ldw,
    void* __restrict__ out, int64_t ldo, int tiles_m, int tiles_n, int group_m,
    const uint8_t* __restrict__ su8, const uint16_t* __restrict__ s2) {
  constexpr int W = WAVES_M * WAVES_N;
  constexpr int WM = BM / WAVES_M;  // rows of the wave tile
  constexpr int WN = BN / WAVES_N;  // columns of the wave tile
  constexpr int TM = WM / 16;
  constexpr int TN = WN / 16;
  constexpr int NA = BM / 16;  // 1 KiB blocks per k step
  constexpr int NB = BN / 16;
  static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile must be a multiple of 16");

  constexpr int STAGE_BYTES = (NA + NB) * 1024;
  __shared__ __attribute__((aligned(1024))) int8_t smem[NSTAGE * STAGE_BYTES];

  // ---- tile selection: XCD-contiguous ranges, then row groups
  const int nwg = tiles_m * tiles_n;
  const int bid = blockIdx.x;
  const int xcd = bid % kXcds, local = bid / kXcds;
  const int q = nwg / kXcds, r = nwg % kXcds;
  const int logical = xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
  const int per_group = group_m * tiles_n;
  const int grp = logical / per_group;
  const int first_m = grp * group_m;
  const int gm = min(tiles_m - first_m, group_m);
  const int in_grp = logical - grp * per_group;
  const int tm = first_m + in_grp % gm;
  const int tn = in_grp / gm;
  const int m0 = tm * BM;
  const int n0 = tn * BN;

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int wm = wv / WAVES_N;
  const int wn = wv % WAVES_N;
  const int j = lane & 15;
  const int g = lane >> 4;
  const int nk = K >> 6;
  const int ntile_n = N >> 4;

  // per-wave block assignment: wave wv loads A blocks wv, wv+W, ... (< NA) and
  // B blocks wv, wv+W, ... (< NB) of every k step.  One row pointer per slot;
  // the k offset advances by 64 bytes (row-major) or 1 KiB (packed) a step.
  constexpr int LA = (NA + W - 1) / W;
  constexpr int LB = (NB + W - 1) / W;
  constexpr int BSTEP = BPACKED ? 1024 : 64;
  const int8_t* srcA[LA];
  const int8_t* srcB[LB];
#pragma unroll
  for (int i = 0; i < LA; i++) {
    const int b = min(wv + i * W, NA - 1);
    srcA[i] = qa + (int64_t)min(m0 + b * 16 + j, M - 1) * lda + g * 16;
  }
#pragma unroll
  for (int i = 0; i < LB; i++) {
    const int b = min(wv + i * W, NB - 1);
    if (BPACKED)
      srcB[i] = qw + (int64_t)min(n0 / 16 + b, ntile_n - 1) * nk * 1024 + lane * 16;
    else
      srcB[i] = qw + (int64_t)min(n0 + b * 16 + j, N - 1) * ldw + g * 16;
  }

  // global -> LDS for k step kt into ring stage st (each wave its own blocks)
  auto issue = [&](int kt, int st) {
    int8_t* stage = smem + st * STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < LA; i++)
      if (NA % W == 0 || wv + i * W < NA)
        __builtin_amdgcn_global_load_lds(
            (const void*)(srcA[i] + kt * 64),
            (__attribute__((address_space(3))) void*)(stage + (wv + i * W) * 1024), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < LB; i++)
      if (NB % W == 0 || wv + i * W < NB)
        __builtin_amdgcn_global_load_lds(
            (const void*)(srcB[i] + kt * BSTEP),
            (__attribute__((address_space(3))) void*)(stage + (NA + wv + i * W) * 1024), 16, 0,
            0);
  };
  // loads every wave issues per k step, at least (waves 0.. may issue one
  // more of each operand when W does not divide the block counts); waiting
  // on this lower bound is conservative for the waves that issue more
  constexpr int PER_STEP_MIN = NA / W + NB / W;
  static_assert(PER_STEP_MIN >= 1, "every wave must load at least one block per step");

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

  auto compute = [&](int st, int kt) {
    const int8_t* stage = smem + st * STAGE_BYTES;
    v4i fa[TM], fb[TN];
#pragma unroll
    for (int i = 0; i < TM; i++)
      fa[i] = *reinterpret_cast<const v4i*>(stage + (wm * TM + i) * 1024 + lane * 16);
#pragma unroll
    for (int n = 0; n < TN; n++)
      fb[n] = *reinterpret_cast<const v4i*>(stage + (NA + wn * TN + n) * 1024 + lane * 16);
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
  };

  // prologue: steps 0 .. NSTAGE-2 in flight
#pragma unroll
  for (int p = 0; p < NSTAGE - 1; p++)
    if (p < nk) issue(p, p);

  for (int kt = 0; kt < nk; kt++) {
    // this wave's loads of step kt are done once at most (NSTAGE-2) steps'
    // worth of newer loads are still outstanding
    const int newer = min(NSTAGE - 2, nk - 1 - kt);
    if (newer >= 2)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * PER_STEP_MIN));
    else if (newer == 1)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER_STEP_MIN));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    // a bare barrier: __syncthreads() would also wait for every outstanding
    // load (vmcnt(0)), draining the prefetch of the later stages
    __builtin_amdgcn_s_barrier();
    // the stage that step kt+NSTAGE-1 overwrites was read in step kt-1, which
    // every wave finished before the barrier above
    if (kt + NSTAGE - 1 < nk) issue(kt + NSTAGE - 1, (kt + NSTAGE - 1) % NSTAGE);
    compute(kt % NSTAGE, kt);
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
          double rr = (double)ts[i][n][v] * (double)sa[row];
          rr = rr * (double)s2f;
          rr = rr * 0.0078125;
          static_cast<uint16_t*>(out)[(int64_t)row * ldo + col] =
              (uint16_t)f32_to_bf16_bits((float)rr);
        } else {
          float rr = (float)acc[i][n][v];
          rr = rr * sa[row];
          rr = rr * swn;
          static_cast<uint16_t*>(out)[(int64_t)row * ldo + col] =
              (uint16_t)f32_to_bf16_bits(rr);
        }
      }
    }
  }
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int NSTAGE, int MODE, bool BPACKED>
hipError_t launch_tile_cfg(const int8_t* qa, const float* sa, int64_t M, int64_t K, int64_t lda,
                           const int8_t* qw, const float* sw, int64_t N, int64_t ldw, void* out,
                           int64_t ldo, const uint8_t* su8, const uint16_t* s2,
                           hipStream_t stream) {
  const int tiles_m = (int)((M + BM - 1) / BM);
  const int tiles_n = (int)((N + BN - 1) / BN);
  const int group_m = 4;
  dim3 grid((unsigned)(tiles_m * tiles_n)), block(WAVES_M * WAVES_N * 64);
  hipLaunchKernelGGL((k_gemm_tile<BM, BN, WAVES_M, WAVES_N, NSTAGE, MODE, BPACKED>), grid, block,
                     0,
                     stream, qa, sa, (int)M, (int)K, lda, qw, sw, (int)N, ldw, out, ldo, tiles_m,
                     tiles_n, group_m, su8, s2);
  return hipGetLastError();
}

// Tile shape per problem: large problems use 256-row tiles (256 x 160 when N
// is a multiple of 160 and 256 x 256 tiles would leave a partial last wave of
// workgroups, else 256 x 256); small ones 64 x 64 so there are enough tiles.
template <int MODE, bool BPACKED>
static hipError_t launch_tile_impl(const int8_t* qa, const float* sa, int64_t M, int64_t K,
                                   int64_t lda, const int8_t* qw, const float* sw, int64_t N,
                                   int64_t ldw, void* out, int64_t ldo, hipStream_t stream) {
  if (M >= 1024 && N >= 1024) {
    const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256);
    if (N % 160 == 0 && (t256 % 256) != 0 && (t256 % 256) < 192)
      return launch_tile_cfg<256, 160, 4, 2, 3, MODE, BPACKED>(qa, sa, M, K, lda, qw, sw, N, ldw,
                                                            out, ldo, nullptr, nullptr, stream);
    return launch_tile_cfg<256, 256, 4, 2, 3, MODE, BPACKED>(qa, sa, M, K, lda, qw, sw, N, ldw, out,
                                                          ldo, nullptr, nullptr, stream);
  }
  return launch_tile_cfg<64, 64, 2, 2, 3, MODE, BPACKED>(qa, sa, M, K, lda, qw, sw, N, ldw, out,
                                                      ldo, nullptr, nullptr, stream);
}

hipError_t launch_gemm_tile(const int8_t* qa, const float* sa, int64_t M, int64_t K,
                            int64_t lda, const int8_t* qw, const float* sw, int64_t N,
                            int64_t ldw, bool packed, uint16_t* y, int64_t ldy,
                            hipStream_t stream) {
  return packed ? launch_tile_impl<kEpiBf16, true>(qa, sa, M, K, lda, qw, sw, N, ldw, y, ldy,
                                                   stream)
                : launch_tile_impl<kEpiBf16, false>(qa, sa, M, K, lda, qw, sw, N, ldw, y, ldy,
                                                    stream);
}

hipError_t launch_gemm_tile_i32(const int8_t* qa, int64_t M, int64_t K, int64_t lda,
                                const int8_t* qw, int64_t N, int64_t ldw, bool packed,
                                int32_t* acc, int64_t ldacc, hipStream_t stream) {
  return packed ? launch_tile_impl<kEpiI32, true>(qa, nullptr, M, K, lda, qw, nullptr, N, ldw,
                                                  acc, ldacc, stream)
                : launch_tile_impl<kEpiI32, false>(qa, nullptr, M, K, lda, qw, nullptr, N, ldw,
                                                   acc, ldacc, stream);
}

hipError_t launch_gemm_g256_tile(const int8_t* qa, const float* sa, int64_t M, int64_t K,
                                 const int8_t* qw, const uint8_t* su8, const uint16_t* s2,
                                 int64_t N, uint16_t* y, int64_t ldy, hipStream_t stream) {
  return launch_tile_cfg<64, 64, 2, 2, 3, kEpiG256, false>(qa, sa, M, K, K, qw, nullptr, N, K, y,
                                                        ldy, su8, s2, stream);
}

}  // namespace w8a8
