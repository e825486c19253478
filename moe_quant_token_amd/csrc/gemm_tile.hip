// LDS-tiled int8 MFMA GEMM with the fused per-token x per-channel epilogue
// (prefill-shaped inputs, M > 16).
//
// Source: "[gfx1151] Online INT8 W8A8 for Qwen3.6 27B / 35B-A3B on RDNA3.5,
// with working MTP" (ATOM pull request), Changes, linear.py bullet (int8
// activations per token x int8 weights per channel, fp32 scales, bf16 out);
// its Performance section notes that prefill is compute-bound.
//
// Both operands are K-contiguous, the native operand order of the int8 MFMAs
// (each lane feeds 16 consecutive k bytes of one row).  The compute uses
// v_mfma_i32_32x32x32_i8, which on gfx950 does the same work as the 16x16x64
// form at twice the issue rate.
// Every 64-byte k step the workgroup stages a BM x 64 activation tile and a
// BN x 64 weight tile in LDS as 1 KiB blocks of 16 rows x 4 k-slices (slot
// j + 16*s holds row j, k bytes 16s..16s+15).  A 32x32x32 operand fragment
// (32 rows, one 32-byte k half) is then four runs of 256 consecutive bytes,
// read without bank conflicts and without a swizzle.  A wave
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
// of 256, the exact int32 sum is scaled by su8[n, group] into an int64 sum);
// MODE 3: gated SiLU over an interleaved gate/up weight (columns 2i = gate_i,
// 2i+1 = up_i of the product): out[m, i] = silu(h[m, 2i]) * h[m, 2i+1] in
// fp32, h = (float(acc) * sa[m]) * sw[n], SiLU in fp64 rounded once.
enum { kEpiBf16 = 0, kEpiI32 = 1, kEpiG256 = 2, kEpiSilu = 3 };

constexpr int kXcds = 8;

// One wave-wide 1 KiB copy global -> LDS (lane l: 16 bytes to dst + 16 l).
// buf: as a buffer load at byte offset voff + soff of [base, base + span);
// else as a global load from src.  The compiler counts global_load_lds as a
// possible LDS access that completes out of order, so with those in flight
// every LDS wait is a full lgkmcnt(0) (each step's MFMAs then wait for all of
// the step's fragment reads); buffer loads to LDS are not counted that way.
__device__ __forceinline__ void lds_dma(bool buf, const int8_t* base, int span, int voff,
                                        int soff, const int8_t* src, int8_t* dst) {
  auto* d = (__attribute__((address_space(3))) void*)dst;
  if (buf) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, span, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, d, 16, voff, soff, 0, 0);
  } else {
    __builtin_amdgcn_global_load_lds((const void*)src, d, 16, 0, 0);
  }
}

// MINB: workgroups that must fit on one CU at once (the register budget the
// compiler gets follows from it).
template <int BM, int BN, int WAVES_M, int WAVES_N, int NSTAGE, int MODE, bool BPACKED,
          bool APACKED = false, int KSUB = 1, int MINB = 1, bool BUF = false>
__global__ __launch_bounds__(WAVES_M* WAVES_N * 64, MINB) void k_gemm_tile(
    const int8_t* __restrict__ qa, const float* __restrict__ sa, int M, int K, int64_t lda,
    const int8_t* __restrict__ qw, const float* __restrict__ sw, int N, int64_t ldw,
    void* __restrict__ out, int64_t ldo, int tiles_m, int tiles_n, int group_m,
    const uint8_t* __restrict__ su8, const uint16_t* __restrict__ s2) {
  constexpr int W = WAVES_M * WAVES_N;
  constexpr int WM = BM / WAVES_M;  // rows of the wave tile
  constexpr int WN = BN / WAVES_N;  // columns of the wave tile
  constexpr int TM = WM / 32;       // 32x32 MFMA blocks per wave
  constexpr int TN = WN / 32;
  constexpr int NA = BM / 16;  // 1 KiB blocks per k step
  constexpr int NB = BN / 16;
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be a multiple of 32");

  // a pipeline step covers KSUB 64-byte k chunks
  constexpr int CHUNK_BYTES = (NA + NB) * 1024;
  constexpr int STAGE_BYTES = KSUB * CHUNK_BYTES;
  // g256: the tile's u8 group scales (K <= 16384: at most 64 groups a row)
  // sit after the stages in the same LDS array (a second LDS array makes the
  // compiler wait for every LDS DMA in flight before each fragment read)
  constexpr int SU8_BYTES = MODE == kEpiG256 ? BN * 64 : 0;
  __shared__ __attribute__((aligned(1024))) int8_t smem[NSTAGE * STAGE_BYTES + SU8_BYTES];

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
  // g256: the group scales are read once into LDS, so the main loop issues
  // no other global loads
  uint8_t* su8_lds = reinterpret_cast<uint8_t*>(smem + NSTAGE * STAGE_BYTES);
  if (MODE == kEpiG256) {
    const int G = K >> 8;
    for (int i = threadIdx.x; i < BN * G; i += W * 64) {
      const int c = i / G, gg = i - c * G;
      su8_lds[c * 64 + gg] = su8[(int64_t)min(n0 + c, N - 1) * G + gg];
    }
    __syncthreads();
  }
  const int wm = wv / WAVES_N;
  const int wn = wv % WAVES_N;
  const int j = lane & 15;
  const int g = lane >> 4;
  const int nk = K >> 6;          // 64-byte k chunks
  const int nsteps = nk / KSUB;   // pipeline steps (K % (64 * KSUB) == 0)
  const int ntile_n = N >> 4;

  // per-wave block assignment: wave wv loads A blocks wv, wv+W, ... (< NA) and
  // B blocks wv, wv+W, ... (< NB) of every k step.  One row pointer per slot;
  // the k offset advances by 64 bytes (row-major) or 1 KiB (packed) a step.
  constexpr int LA = (NA + W - 1) / W;
  constexpr int LB = (NB + W - 1) / W;
  constexpr int BSTEP = BPACKED ? 1024 : 64;
  const int8_t* srcA[LA];
  const int8_t* srcB[LB];
  constexpr int ASTEP = APACKED ? 1024 : 64;
  const int ntile_m = (M + 15) >> 4;
  // BUF: the same loads as buffer loads from the workgroup's own operand
  // ranges (32-bit offsets; the host picks BUF only when they fit)
  const int8_t* baseA = APACKED ? qa + (int64_t)(m0 / 16) * nk * 1024 : qa + (int64_t)m0 * lda;
  const int8_t* baseB = BPACKED ? qw + (int64_t)(n0 / 16) * nk * 1024 : qw + (int64_t)n0 * ldw;
  int voffA[LA], voffB[LB];
#pragma unroll
  for (int i = 0; i < LA; i++) {
    const int b = min(wv + i * W, NA - 1);
    if (APACKED)
      srcA[i] = qa + (int64_t)min(m0 / 16 + b, ntile_m - 1) * nk * 1024 + lane * 16;
    else
      srcA[i] = qa + (int64_t)min(m0 + b * 16 + j, M - 1) * lda + g * 16;
    voffA[i] = (int)(srcA[i] - baseA);
  }
#pragma unroll
  for (int i = 0; i < LB; i++) {
    const int b = min(wv + i * W, NB - 1);
    if (BPACKED)
      srcB[i] = qw + (int64_t)min(n0 / 16 + b, ntile_n - 1) * nk * 1024 + lane * 16;
    else
      srcB[i] = qw + (int64_t)min(n0 + b * 16 + j, N - 1) * ldw + g * 16;
    voffB[i] = (int)(srcB[i] - baseB);
  }
  // byte ranges the offsets above stay in (clamped rows)
  const int spanA = !BUF ? 0 : APACKED ? NA * nk * 1024 : (BM - 1) * (int)lda + K;
  const int spanB = !BUF ? 0 : BPACKED ? NB * nk * 1024 : (BN - 1) * (int)ldw + K;

  // global -> LDS for pipeline step ks (KSUB chunks) into ring stage st
  auto issue = [&](int ks, int st) {
#pragma unroll
    for (int c = 0; c < KSUB; c++) {
      const int kt = ks * KSUB + c;
      int8_t* stage = smem + st * STAGE_BYTES + c * CHUNK_BYTES;
#pragma unroll
      for (int i = 0; i < LA; i++)
        if (NA % W == 0 || wv + i * W < NA)
          lds_dma(BUF, baseA, spanA, voffA[i], kt * ASTEP, srcA[i] + kt * ASTEP,
                  stage + (wv + i * W) * 1024);
#pragma unroll
      for (int i = 0; i < LB; i++)
        if (NB % W == 0 || wv + i * W < NB)
          lds_dma(BUF, baseB, spanB, voffB[i], kt * BSTEP, srcB[i] + kt * BSTEP,
                  stage + (NA + wv + i * W) * 1024);
    }
  };
  // loads every wave issues per k step, at least (waves 0.. may issue one
  // more of each operand when W does not divide the block counts); waiting
  // on this lower bound is conservative for the waves that issue more
  constexpr int PER_STEP_MIN = KSUB * (NA / W + NB / W);
  static_assert(PER_STEP_MIN >= 1, "every wave must load at least one block per step");
  static_assert(NSTAGE >= 2, "the pipeline needs at least two stages");

  v16i acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; i++)
#pragma unroll
    for (int n = 0; n < TN; n++) acc[i][n] = v16i{0};
  long long ts[MODE == kEpiG256 ? TM : 1][MODE == kEpiG256 ? TN : 1][16];
  if (MODE == kEpiG256) {
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
      for (int n = 0; n < TN; n++)
#pragma unroll
        for (int v = 0; v < 16; v++) ts[i][n][v] = 0;
  }

  // Operand fragments of one 32-byte k half: LDS -> registers.  Lane l reads
  // row (l % 32) of a 32-row block, k-slice 2h + l/32: 16-row block
  // (l % 32) / 16, slot (l % 16) + 16 * (2h + l/32).
  const int frag_off = ((lane >> 4) & 1) * 1024 + ((lane & 15) + 16 * (lane >> 5)) * 16;
  // One k step: every fragment of both 32-byte halves is read first, then
  // the MFMAs run; the scheduling groups keep the compiler from interleaving
  // a wait for each read into the MFMA stream (one wave per SIMD has nothing
  // else to hide LDS latency with).
  auto k_step = [&](int st) {
#pragma unroll
    for (int c = 0; c < KSUB; c++) {
      const int8_t* stage = smem + st * STAGE_BYTES + c * CHUNK_BYTES + frag_off;
      v4i fa[2][TM], fb[2][TN];
#pragma unroll
      for (int h = 0; h < 2; h++) {
#pragma unroll
        for (int i = 0; i < TM; i++)
          fa[h][i] = *reinterpret_cast<const v4i*>(stage + h * 512 + (wm * TM + i) * 2048);
#pragma unroll
        for (int n = 0; n < TN; n++)
          fb[h][n] = *reinterpret_cast<const v4i*>(stage + h * 512 +
                                                   (NA + (wn * TN + n) * 2) * 1024);
      }
#pragma unroll
      for (int h = 0; h < 2; h++)
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
          for (int n = 0; n < TN; n++)
            acc[i][n] = mfma_32x32x32_i8(fa[h][i], fb[h][n], acc[i][n]);
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * (TM + TN), 0);  // LDS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * TM * TN, 0);    // MFMAs
    }
  };
  auto fold_g256 = [&](int kt) {
    if (MODE == kEpiG256 && (kt & 3) == 3) {
#pragma unroll
      for (int n = 0; n < TN; n++) {
        // |acc| <= 256 * 127^2 per group, so acc * u8 < 2^31 is exact in int32
        const int u8 = su8_lds[(wn * WN + n * 32 + (lane & 31)) * 64 + (kt >> 2)];
#pragma unroll
        for (int i = 0; i < TM; i++) {
#pragma unroll
          for (int v = 0; v < 16; v++) ts[i][n][v] += (long long)(acc[i][n][v] * u8);
          acc[i][n] = v16i{0};
        }
      }
    }
  };
  // Steps issued before arrive(kt): 0..NSTAGE-2 by the prologue, then one more
  // after each earlier arrive: NSTAGE-2 newer steps than kt (fewer near the
  // end of K).
  auto arrive = [&](int kt) {
    const int newer = min(NSTAGE - 2, nsteps - 1 - kt);
    if (newer >= 3)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * PER_STEP_MIN));
    else if (newer == 2)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * PER_STEP_MIN));
    else if (newer == 1)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER_STEP_MIN));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __builtin_amdgcn_s_barrier();
  };

  // Pipeline.  Step ks: wait for its blocks (arrive), send the loads of step
  // ks+NSTAGE-1 into the stage step ks-1 used (every wave finished reading it
  // before the barrier in arrive), then run step ks.
#pragma unroll
  for (int p = 0; p < NSTAGE - 1; p++)
    if (p < nsteps) issue(p, p);
  for (int ks = 0; ks < nsteps; ks++) {
    // Scalar loads still in flight (the compiler issues the epilogue's
    // argument loads before this loop) return out of order, and while any
    // is pending every LDS wait must be a full lgkmcnt(0): each step's MFMAs
    // would then wait for all of its fragment reads.  Retiring them here
    // (free after the first step) lets each MFMA wait only for its own.
    __builtin_amdgcn_s_waitcnt(lgkmcnt0_imm());
    arrive(ks);
    if (ks + NSTAGE - 1 < nsteps) issue(ks + NSTAGE - 1, (ks + NSTAGE - 1) % NSTAGE);
    k_step(ks % NSTAGE);
#pragma unroll
    for (int c = 0; c < KSUB; c++) fold_g256(ks * KSUB + c);
  }

  // epilogue: lane holds column (lane % 32) of every 32x32 block, rows
  // 8*(r/4) + 4*(lane/32) + r%4 for r < 16.  The scales of the lane's rows
  // and columns are loaded up front (indices clamped into range), so the
  // stores never wait on a scale load.
  const int row0 = m0 + wm * WM + 4 * (lane >> 5);
  const int col0 = n0 + wn * WN + (lane & 31);
  float sar[MODE == kEpiI32 ? 1 : TM][MODE == kEpiI32 ? 1 : 16];
  float scol[MODE == kEpiI32 ? 1 : TN];
  if (MODE != kEpiI32) {
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
      for (int v = 0; v < 16; v++)
        sar[i][v] = sa[min(row0 + i * 32 + 8 * (v >> 2) + (v & 3), M - 1)];
#pragma unroll
    for (int n = 0; n < TN; n++) {
      const int c = min(col0 + n * 32, N - 1);
      scol[n] = MODE == kEpiG256 ? __uint_as_float((uint32_t)s2[c] << 16) : sw[c];
    }
    // one wait for all of them: the stores below sit in per-element
    // branches, across which the compiler would otherwise wait again
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
      for (int v = 0; v < 16; v++) keep_live(sar[i][v]);
#pragma unroll
    for (int n = 0; n < TN; n++) keep_live(scol[n]);
  }
  if (MODE == kEpiSilu) {
    // lanes l and l ^ 1 hold adjacent product columns (gate, up) of the same
    // 16 rows; the pair splits the rows so that each lane forms 8 of the 16
    // activations (the even lane rows v < 8, the odd lane v >= 8): one fp64
    // exp per output instead of two lanes' worth.  N is even, so both lanes
    // of a pair are in range or out of range together.
    const bool odd = (lane & 1) != 0;
#pragma unroll
    for (int n = 0; n < TN; n++) {
      const int col = col0 + n * 32;
      const bool col_ok = col < N;
#pragma unroll
      for (int i = 0; i < TM; i++) {
        float h[16], x[16];
#pragma unroll
        for (int v = 0; v < 16; v++) {
          h[v] = (float)acc[i][n][v];
          h[v] = h[v] * sar[i][v];
          h[v] = h[v] * scol[n];
        }
#pragma unroll
        for (int v = 0; v < 16; v++) x[v] = __shfl_xor(h[v], 1, 64);
#pragma unroll
        for (int q = 0; q < 8; q++) {
          const float gate = odd ? x[q + 8] : h[q];
          const float up = odd ? h[q + 8] : x[q];
          const int v = odd ? q + 8 : q;
          const int row = row0 + i * 32 + 8 * (v >> 2) + (v & 3);
          const float sg = (float)((double)gate / (1.0 + exp(-(double)gate)));
          if (col_ok && row < M)
            static_cast<float*>(out)[(int64_t)row * ldo + (col >> 1)] = sg * up;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    return;
  }
#pragma unroll
  for (int n = 0; n < TN; n++) {
    const int col = col0 + n * 32;
    const bool col_ok = col < N;
#pragma unroll
    for (int i = 0; i < TM; i++) {
#pragma unroll
      for (int v = 0; v < 16; v++) {
        const int row = row0 + i * 32 + 8 * (v >> 2) + (v & 3);
        if (!col_ok || row >= M) continue;
        if (MODE == kEpiI32) {
          static_cast<int32_t*>(out)[(int64_t)row * ldo + col] = acc[i][n][v];
        } else if (MODE == kEpiG256) {
          double rr = (double)ts[i][n][v] * (double)sar[i][v];
          rr = rr * (double)scol[n];
          rr = rr * 0.0078125;
          static_cast<uint16_t*>(out)[(int64_t)row * ldo + col] =
              (uint16_t)f32_to_bf16_bits((float)rr);
        } else {
          float rr = (float)acc[i][n][v];
          rr = rr * sar[i][v];
          rr = rr * scol[n];
          static_cast<uint16_t*>(out)[(int64_t)row * ldo + col] =
              (uint16_t)f32_to_bf16_bits(rr);
        }
      }
      // one 32x32 block at a time: keeps the accumulators in AGPRs until
      // their block is stored, so the epilogue does not raise the kernel's
      // VGPR count (and with it the workgroups that fit on a CU)
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int NSTAGE, int MODE, bool BPACKED,
          bool APACKED = false, int KSUB = 1, int MINB = 1>
hipError_t launch_tile_cfg(const int8_t* qa, const float* sa, int64_t M, int64_t K, int64_t lda,
                           const int8_t* qw, const float* sw, int64_t N, int64_t ldw, void* out,
                           int64_t ldo, const uint8_t* su8, const uint16_t* s2,
                           hipStream_t stream) {
  const int tiles_m = (int)((M + BM - 1) / BM);
  const int tiles_n = (int)((N + BN - 1) / BN);
  const int group_m = 4;
  dim3 grid((unsigned)(tiles_m * tiles_n)), block(WAVES_M * WAVES_N * 64);
  // buffer-load operand feed when a workgroup's operand bytes span < 2 GiB
  // (always for packed operands: BM x K or BN x K bytes)
  constexpr int64_t kSpan = (int64_t)1 << 31;
  const bool buf = (APACKED || (BM - 1) * lda + K < kSpan) && (BPACKED || (BN - 1) * ldw + K < kSpan);
  if (buf)
    hipLaunchKernelGGL(
        (k_gemm_tile<BM, BN, WAVES_M, WAVES_N, NSTAGE, MODE, BPACKED, APACKED, KSUB, MINB, true>),
        grid, block, 0, stream, qa, sa, (int)M, (int)K, lda, qw, sw, (int)N, ldw, out, ldo,
        tiles_m, tiles_n, group_m, su8, s2);
  else
    hipLaunchKernelGGL(
        (k_gemm_tile<BM, BN, WAVES_M, WAVES_N, NSTAGE, MODE, BPACKED, APACKED, KSUB, MINB, false>),
        grid, block, 0, stream, qa, sa, (int)M, (int)K, lda, qw, sw, (int)N, ldw, out, ldo,
        tiles_m, tiles_n, group_m, su8, s2);
  return hipGetLastError();
}

// Output columns [n0, n0 + nn) as a launch of their own: the weight rows,
// channel scales and output columns move by n0 (n0 % 16 == 0, so packed
// weights keep whole 16-row tiles); the activations are shared.
template <int BM, int BN, int WAVES_M, int WAVES_N, int NSTAGE, int MODE, bool BPACKED,
          bool APACKED, int KSUB, int MINB>
static hipError_t launch_cols(const int8_t* qa, const float* sa, int64_t M, int64_t K,
                              int64_t lda, const int8_t* qw, const float* sw, int64_t ldw,
                              void* out, int64_t ldo, int64_t n0, int64_t nn,
                              hipStream_t stream) {
  // bytes per product column of the output: int32, bf16, or half an fp32
  // activation (two product columns make one)
  const int64_t off = MODE == kEpiI32 ? n0 * 4 : MODE == kEpiSilu ? n0 / 2 * 4 : n0 * 2;
  return launch_tile_cfg<BM, BN, WAVES_M, WAVES_N, NSTAGE, MODE, BPACKED, APACKED, KSUB, MINB>(
      qa, sa, M, K, lda, qw + n0 * (BPACKED ? K : ldw), sw ? sw + n0 : nullptr, nn, ldw,
      static_cast<char*>(out) + off, ldo, nullptr, nullptr, stream);
}

static int64_t gcd64(int64_t a, int64_t b) {
  while (b) {
    const int64_t t = a % b;
    a = b;
    b = t;
  }
  return a;
}

// 256 x 256 tiles (8 waves of 64 x 128): two 64-byte k chunks per pipeline
// step and two stages when K % 128 == 0 (half the barriers per MFMA; measured
// on MI355X ~8% faster than one chunk and four stages), else one chunk and
// four stages.
template <int MODE, bool BPACKED, bool APACKED>
static hipError_t launch_256(const int8_t* qa, const float* sa, int64_t M, int64_t K,
                             int64_t lda, const int8_t* qw, const float* sw, int64_t ldw,
                             void* out, int64_t ldo, int64_t n0, int64_t nn, hipStream_t stream) {
  if (K % 128 == 0)
    return launch_cols<256, 256, 4, 2, 2, MODE, BPACKED, APACKED, 2, 1>(
        qa, sa, M, K, lda, qw, sw, ldw, out, ldo, n0, nn, stream);
  return launch_cols<256, 256, 4, 2, 4, MODE, BPACKED, APACKED, 1, 1>(
      qa, sa, M, K, lda, qw, sw, ldw, out, ldo, n0, nn, stream);
}

// Launch plan per problem.  A 256 x 256 tile needs a whole CU (one workgroup
// per CU), so the tile count should be a multiple of the CU count: a partial
// last round leaves most CUs idle for a whole tile time.  In order:
//  - 256 x 256 when the tiles fill whole rounds;
//  - 256 x 160, two workgroups per CU, when N is a multiple of 160 and the
//    256 x 256 tiling would leave under 3/4 of a round (N=5120: 512 tiles,
//    one round of 2 x 256);
//  - otherwise the widest column range whose 256 x 256 tiles fill whole
//    rounds, then the remaining columns as 128 x 64 tiles (two per CU), when
//    that is cheaper than the partial round.  Measured on MI355X at
//    M=4096, K=5120: one round of 128 x 64 tiles takes ~0.4 of a 256 x 256
//    round (N=17408: 492 -> ~395 us);
//  - small problems: 64 x 64 tiles so there are enough of them.
template <int MODE, bool BPACKED, bool APACKED = false>
static hipError_t launch_tile_impl(const int8_t* qa, const float* sa, int64_t M, int64_t K,
                                   int64_t lda, const int8_t* qw, const float* sw, int64_t N,
                                   int64_t ldw, void* out, int64_t ldo, hipStream_t stream) {
  if (M >= 1024 && N >= 1024) {
    const int64_t cus = device_cus();
    const int64_t tm = (M + 255) / 256, tn = (N + 255) / 256, t256 = tm * tn;
    const int64_t rounds = (t256 + cus - 1) / cus;
    if (t256 % cus != 0) {
      if (N % 160 == 0 && (t256 % cus) * 4 < cus * 3)
        return launch_cols<256, 160, 4, 1, 3, MODE, BPACKED, APACKED, 1, 2>(
            qa, sa, M, K, lda, qw, sw, ldw, out, ldo, 0, N, stream);
      const int64_t q = cus / gcd64(tm, cus);  // column tiles per whole number of rounds
      const int64_t tn_main = tn / q * q;      // < tn, so the main range ends before N
      if (tn_main > 0) {
        const int64_t n_main = tn_main * 256;
        const int64_t rem_tiles =
            APACKED ? ((M + 127) / 128) * ((N - n_main + 63) / 64)
                    : ((M + 63) / 64) * ((N - n_main + 127) / 128);
        const int64_t rem_rounds = (rem_tiles + 2 * cus - 1) / (2 * cus);
        // in tenths of a 256 x 256 round
        if (10 * (tm * tn_main / cus) + 4 * rem_rounds < 10 * rounds) {
          hipError_t e = launch_256<MODE, BPACKED, APACKED>(qa, sa, M, K, lda, qw, sw, ldw, out,
                                                            ldo, 0, n_main, stream);
          if (e != hipSuccess) return e;
          // row-major activations cost more per row than packed ones (16
          // separate 64-byte pieces per 1 KiB load), so their remainder tiles
          // take fewer rows and more columns
          if (!APACKED)
            return launch_cols<64, 128, 2, 2, 4, MODE, BPACKED, APACKED, 1, 2>(
                qa, sa, M, K, lda, qw, sw, ldw, out, ldo, n_main, N - n_main, stream);
          return launch_cols<128, 64, 2, 2, 4, MODE, BPACKED, APACKED, 1, 2>(
              qa, sa, M, K, lda, qw, sw, ldw, out, ldo, n_main, N - n_main, stream);
        }
      }
    }
    return launch_256<MODE, BPACKED, APACKED>(qa, sa, M, K, lda, qw, sw, ldw, out, ldo, 0, N,
                                              stream);
  }
  if constexpr (BPACKED && APACKED) {
    if (M < 1024) {
      // mid-size problems, both operands in the tile layout (measured on
      // MI355X with the weights coming from HBM; the first figure is the
      // 64 x 64 one-chunk tiling below):
      //  - M >= 128 and K >= 4096: 128 x 128 tiles (512x5120x5120 33.1 -> 28.0
      //    us, 128x5120x17408 40.0 -> 29.6 us);
      //  - M >= 128, shorter K: 128 x 64 tiles of 8 waves, two chunks a step
      //    (256x2048x8192 11.6 -> 10.6 us);
      //  - 33 to 127 rows: 64 x 64 tiles, two chunks a step, two workgroups a
      //    CU (64x8704x5120 31.8 -> 22.7 us);
      //  - up to 32 rows: one-wave 32 x 32 tiles, two chunks a step, up to
      //    five workgroups a CU (32 KiB of LDS each), so a CU has many weight
      //    streams in flight (32x5120x17408 27.2 -> 20.7 us, 17x5120x17408
      //    25.6 -> 20.6 us, 32x8704x5120 21.6 -> 19.1 us).
      if (M >= 128 && K >= 4096)
        return launch_cols<128, 128, 4, 2, 4, MODE, BPACKED, APACKED, 1, 1>(
            qa, sa, M, K, lda, qw, sw, ldw, out, ldo, 0, N, stream);
      if (K % 128 == 0) {
        if (M >= 128)
          return launch_cols<128, 64, 4, 2, 4, MODE, BPACKED, APACKED, 2, 1>(
              qa, sa, M, K, lda, qw, sw, ldw, out, ldo, 0, N, stream);
        if (M <= 32)
          return launch_cols<32, 32, 1, 1, 4, MODE, BPACKED, APACKED, 2, 2>(
              qa, sa, M, K, lda, qw, sw, ldw, out, ldo, 0, N, stream);
        return launch_cols<64, 64, 2, 2, 4, MODE, BPACKED, APACKED, 2, 2>(
            qa, sa, M, K, lda, qw, sw, ldw, out, ldo, 0, N, stream);
      }
    }
  }
  return launch_cols<64, 64, 2, 2, 4, MODE, BPACKED, APACKED, 1, 1>(
      qa, sa, M, K, lda, qw, sw, ldw, out, ldo, 0, N, stream);
}

hipError_t launch_gemm_tile_apacked(const int8_t* qa_packed, const float* sa, int64_t M,
                                    int64_t K, const int8_t* qw_packed, const float* sw,
                                    int64_t N, uint16_t* y, int64_t ldy, hipStream_t stream) {
  return launch_tile_impl<kEpiBf16, true, true>(qa_packed, sa, M, K, K, qw_packed, sw, N, K, y,
                                                ldy, stream);
}

hipError_t launch_gemm_tile_apacked_silu(const int8_t* qa_packed, const float* sa, int64_t M,
                                         int64_t K, const int8_t* qw_packed, const float* sw,
                                         int64_t N, float* act, int64_t ldact,
                                         hipStream_t stream) {
  return launch_tile_impl<kEpiSilu, true, true>(qa_packed, sa, M, K, K, qw_packed, sw, N, K, act,
                                                ldact, stream);
}

hipError_t launch_gemm_tile_apacked_i32(const int8_t* qa_packed, int64_t M, int64_t K,
                                        const int8_t* qw_packed, int64_t N, int32_t* acc,
                                        int64_t ldacc, hipStream_t stream) {
  return launch_tile_impl<kEpiI32, true, true>(qa_packed, nullptr, M, K, K, qw_packed, nullptr, N,
                                               K, acc, ldacc, stream);
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
                                 int64_t N, bool packed, bool apacked, uint16_t* y, int64_t ldy,
                                 hipStream_t stream) {
  // 64 x 64 tiles, one 256-byte group (four 64-byte k chunks) per pipeline
  // step over two stages, two workgroups per CU.  Measured on MI355X at
  // 256 x 2048 x 8192: 14.4 us with two chunks per step over four stages,
  // 13.0 us like this.  Up to 32 rows: one-wave 32 x 32 tiles over three
  // stages, up to three workgroups a CU (50 KiB of LDS each; 32 x 2048 x
  // 8192: 10.4 -> 8.1 us).
  if (M <= 32) {
    if (packed && apacked)
      return launch_tile_cfg<32, 32, 1, 1, 3, kEpiG256, true, true, 4, 1>(
          qa, sa, M, K, K, qw, nullptr, N, K, y, ldy, su8, s2, stream);
    if (packed)
      return launch_tile_cfg<32, 32, 1, 1, 3, kEpiG256, true, false, 4, 1>(
          qa, sa, M, K, K, qw, nullptr, N, K, y, ldy, su8, s2, stream);
    return launch_tile_cfg<32, 32, 1, 1, 3, kEpiG256, false, false, 4, 1>(
        qa, sa, M, K, K, qw, nullptr, N, K, y, ldy, su8, s2, stream);
  }
  if (packed && apacked)
    return launch_tile_cfg<64, 64, 2, 2, 2, kEpiG256, true, true, 4, 2>(
        qa, sa, M, K, K, qw, nullptr, N, K, y, ldy, su8, s2, stream);
  if (packed)
    return launch_tile_cfg<64, 64, 2, 2, 2, kEpiG256, true, false, 4, 2>(
        qa, sa, M, K, K, qw, nullptr, N, K, y, ldy, su8, s2, stream);
  return launch_tile_cfg<64, 64, 2, 2, 2, kEpiG256, false, false, 4, 2>(
      qa, sa, M, K, K, qw, nullptr, N, K, y, ldy, su8, s2, stream);
}

}  // namespace w8a8
