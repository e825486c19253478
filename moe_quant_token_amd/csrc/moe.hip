// Routed int8 MoE layer on gfx950.
//
// Source: "[gfx1151] Online INT8 W8A8 for Qwen3.6 27B / 35B-A3B on RDNA3.5,
// with working MTP" (ATOM pull request), Changes: the fused_moe_triton.py
// bullet gives the order routing -> per-token int8 quant -> gemm1 with fused
// gated SiLU over interleaved w13 rows -> per-token int8 quant -> gemm2 with
// scatter/combine; the moe.py bullet gives int8 w13/w2 with per-channel fp32
// scales.
//
// Kernels, in launch order (all on the caller's stream, no host sync; every
// count that depends on the routing stays on the device).
// Small batches (at most 2048 routed pairs):
//   k_moe_prep     one workgroup: routing (one wave per token), per-token int8
//                  codes of x, and the sort of the pairs by expert (up to 16
//                  tokens; beyond, k_moe_route_quant and the one-workgroup
//                  k_moe_sort)
//   k_moe_skinny<1> grouped gemm1 streaming each touched expert's w13 once,
//                  SiLU(gate)*up epilogue, per-pair |act| maximum (atomic max)
//   k_moe_skinny<2> grouped gemm2; its prologue requantises the pairs' rows
//   k_moe_combine  out[t] = sum over the k slots, in slot order, one bf16
//                  rounding; deterministic (no floating-point atomics)
// Large batches:
//   k_moe_route_quant  routing and per-token int8 codes of x, four tokens per
//                  8-wave workgroup (routing waves beside quantising waves)
//   k_moe_sort_hist / k_moe_sort_scatter  the sort over chunks of pairs, one
//                  workgroup per chunk: per-chunk expert counts, then segment
//                  offsets, the list of experts that received pairs, the
//                  pairs grouped by expert and the table of 128-pair m-blocks
//   k_moe_tile<1>  grouped gemm1 (32x32x32 MFMA): gathered activation rows
//                  through LDS, weights prefetched into registers,
//                  SiLU(gate)*up epilogue
//   k_moe_requant  per-pair int8 codes of the activation, one wave per pair
//   k_moe_tile<2>  grouped gemm2, epilogue writes dequantised fp32 rows
//   k_moe_combine  as above
#include <algorithm>
#include <type_traits>

#include "kernels.h"

namespace w8a8 {

namespace {

constexpr size_t kAlign = 256;
// pair rows per workgroup of the large-batch grouped GEMMs
constexpr int kMoeBM = 128;
// largest number of weight blocks one gemm2 workgroup walks (npw)
constexpr int kMoeMaxNpw = 8;
// batches up to this many tokens run routing, quantisation and the sort in
// one workgroup (k_moe_prep); top-k is at most kMoeMaxTopk (checked at the
// entry point)
constexpr int kMoePrepTokens = 16;
constexpr int kMoeMaxTopk = 16;
constexpr int kMoeMaxH = 16384;  // hidden size limit (checked at the entry point)
// the large-batch sort splits the pairs into at most this many chunks
constexpr int kMoeSortChunks = 64;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct MoeWs {
  int32_t* expert_list;   // [E]
  int32_t* seg_off;       // [E + 1]
  int32_t* n_active;      // [1]
  int32_t* sorted_pairs;  // [P]
  int8_t* qx;             // [T, H]
  float* sx;              // [T]
  float* act;             // [P, I]
  uint32_t* amax;         // [P]  (fp32 bit patterns of non-negative values)
  int8_t* qa;             // [P, I]
  float* sa2;             // [P]
  float* y2;              // [P, H]
  int32_t* blk_slot;      // [P / kMoeBM + E + 1]  m-block -> expert slot
  int32_t* blk_row0;      // [P / kMoeBM + E + 1]  m-block -> first sorted pair
  int32_t* n_blocks;      // [1]
  int32_t* rank;          // [P]  a pair's place among its sort chunk's pairs of its expert
  int32_t* hist;          // [kMoeSortChunks, E]  per-chunk expert counts of the sort
  uint32_t* amax_part;    // [P, 2I/16] (T == 1 only) per-tile partial |act| maxima
  size_t bytes;
};

MoeWs carve(void* base, int64_t T, int64_t H, int64_t E, int64_t I, int k) {
  const int64_t P = T * k;
  MoeWs w;
  size_t off = 0;
  char* b = static_cast<char*>(base);
  auto take = [&](size_t bytes) {
    char* p = b ? b + off : nullptr;
    off += align_up(bytes);
    return p;
  };
  w.expert_list = reinterpret_cast<int32_t*>(take(E * 4));
  w.seg_off = reinterpret_cast<int32_t*>(take((E + 1) * 4));
  w.n_active = reinterpret_cast<int32_t*>(take(4));
  w.sorted_pairs = reinterpret_cast<int32_t*>(take(P * 4));
  w.qx = reinterpret_cast<int8_t*>(take(T * H));
  w.sx = reinterpret_cast<float*>(take(T * 4));
  w.act = reinterpret_cast<float*>(take(P * I * 4));
  w.amax = reinterpret_cast<uint32_t*>(take(P * 4));
  w.qa = reinterpret_cast<int8_t*>(take(P * I));
  w.sa2 = reinterpret_cast<float*>(take(P * 4));
  w.y2 = reinterpret_cast<float*>(take(P * H * 4));
  w.blk_slot = reinterpret_cast<int32_t*>(take((P / kMoeBM + E + 1) * 4));
  w.blk_row0 = reinterpret_cast<int32_t*>(take((P / kMoeBM + E + 1) * 4));
  w.n_blocks = reinterpret_cast<int32_t*>(take(4));
  w.rank = reinterpret_cast<int32_t*>(take(P * 4));
  w.hist = reinterpret_cast<int32_t*>(take(kMoeSortChunks * E * 4));
  w.amax_part = reinterpret_cast<uint32_t*>(take(T == 1 ? P * (2 * I / 16) * 4 : 0));
  w.bytes = off;
  return w;
}

}  // namespace

// Wave-wide maximum of a 32-bit unsigned key through DPP row shifts and row
// broadcasts (no LDS traffic); every lane gets the result.  Lanes a shift
// reads past the row edge get 0, the identity of the maximum.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#define W8A8_DPP_MAX(ctrl, rmask) \
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, ctrl, rmask, 0xf, true))
  W8A8_DPP_MAX(0x111, 0xf);  // row_shr:1
  W8A8_DPP_MAX(0x112, 0xf);  // row_shr:2
  W8A8_DPP_MAX(0x114, 0xf);  // row_shr:4
  W8A8_DPP_MAX(0x118, 0xf);  // row_shr:8
  W8A8_DPP_MAX(0x142, 0xa);  // row_bcast:15
  W8A8_DPP_MAX(0x143, 0xc);  // row_bcast:31
#undef W8A8_DPP_MAX
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Order-preserving map of a finite fp32 value to an unsigned key.
__device__ __forceinline__ uint32_t float_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// ---------------------------------------------------------------------------
// Routing of one token by one wave: softmax over E, top-k, renormalise.
// Selection compares the fp32 logits (softmax is monotonic): slot s gets the
// s-th largest, equal logits go to the lower expert index.  Each round takes
// the wave maximum of the key (logit, then 2^32-1-index) over the experts not
// yet taken; lane s keeps slot s.  The rounds hold no floating-point work.
// Weights: w_s = p_s / (sum of the kept p) with p = softmax; the softmax
// denominator cancels, so lane s forms e_s = exp(l_s - max) in fp64, the
// kept e are summed in slot order and w_s = e_s / sum is rounded once to
// fp32 (within one fp32 ulp of the quotient of the rounded fp64 softmax
// probabilities).
// ---------------------------------------------------------------------------
// Routing of one token by one wave: lane s < k ends with the expert of slot
// s and its renormalised weight.  VPL logits per lane (E <= 64 * VPL).
template <int VPL>
__device__ __forceinline__ void route_select_v(const float* __restrict__ lt, int E, int k,
                                               int lane, int& sel_e, float& sel_w) {
  uint32_t kv[VPL];  // order-preserving keys of the lane's logits; 0 = none
  uint32_t kmax = 0;
  // every load is issued before any is used (a load whose value is used
  // inside its own bounds branch gets a wait of its own: VPL round trips)
  float lv[VPL];
#pragma unroll
  for (int i = 0; i < VPL; i++) lv[i] = lt[min(lane + 64 * i, E - 1)];
#pragma unroll
  for (int i = 0; i < VPL; i++) {
    kv[i] = lane + 64 * i < E ? float_key(lv[i]) : 0u;
    kmax = max(kmax, kv[i]);
  }
  const double mx = (double)key_float(wave_max_u32(kmax));  // the largest logit

  uint32_t taken = 0;
  int my_e = 0;
  float my_l = 0.0f;
  for (int s = 0; s < k; s++) {
    uint32_t hi = 0, lo = 0;  // best local key; 0 = none
#pragma unroll
    for (int i = 0; i < VPL; i++) {
      // ascending e: ties keep the lower index
      if (!(taken & (1u << i)) && kv[i] > hi) {
        hi = kv[i];
        lo = 0xffffffffu - (uint32_t)(lane + 64 * i);
      }
    }
    const uint32_t mh = wave_max_u32(hi);
    // the lane holding the maximum; equal keys on several lanes (tied
    // logits) take a second reduction for the lowest index
    const uint64_t holders = __ballot(hi == mh);
    uint32_t ml;
    if (__popcll(holders) == 1)
      ml = (uint32_t)__builtin_amdgcn_readlane((int)lo, __ffsll((long long)holders) - 1);
    else
      ml = wave_max_u32(hi == mh ? lo : 0u);
    const int be = (int)(0xffffffffu - ml);
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == s) {
      my_e = be;
      my_l = key_float(mh);
    }
  }
  const double myp = exp((double)my_l - mx);
  // kept probabilities summed in slot order (lane reads, no LDS traffic)
  const uint64_t pb = (uint64_t)__double_as_longlong(myp);
  double kept = 0.0;
  for (int s = 0; s < k; s++) {
    const uint32_t plo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)pb, s);
    const uint32_t phi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(pb >> 32), s);
    kept += __longlong_as_double((long long)(((uint64_t)phi << 32) | plo));
  }
  sel_e = my_e;
  sel_w = (float)(myp / kept);
}

// Up to 256 experts: each lane first orders its four (logit, expert) pairs
// (logit descending, expert ascending), so a round needs no scan of the
// lane's entries: the wave maximum of the lanes' first keys, then among the
// lanes holding it the lowest expert (a second maximum, of the inverted
// index), and the winning lane drops its first entry.  Same selection and
// weights as route_select_v.
__device__ __forceinline__ void order_pair(uint32_t& ka, int& ea, uint32_t& kb, int& eb) {
  const bool sw = kb > ka || (kb == ka && eb < ea);
  const uint32_t k0 = sw ? kb : ka, k1 = sw ? ka : kb;
  const int e0 = sw ? eb : ea, e1 = sw ? ea : eb;
  ka = k0;
  kb = k1;
  ea = e0;
  eb = e1;
}
__device__ __forceinline__ void route_select_sorted4(const float* __restrict__ lt, int E, int k,
                                                     int lane, int& sel_e, float& sel_w) {
  float lv[4];
#pragma unroll
  for (int i = 0; i < 4; i++) lv[i] = lt[min(lane + 64 * i, E - 1)];
  uint32_t q[4];  // order-preserving keys; 0 = none
  int ee[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    ee[i] = lane + 64 * i;
    q[i] = ee[i] < E ? float_key(lv[i]) : 0u;
  }
  // a sorting network over the four pairs (the pairs are distinct)
  order_pair(q[0], ee[0], q[1], ee[1]);
  order_pair(q[2], ee[2], q[3], ee[3]);
  order_pair(q[0], ee[0], q[2], ee[2]);
  order_pair(q[1], ee[1], q[3], ee[3]);
  order_pair(q[1], ee[1], q[2], ee[2]);
  int my_e = 0;
  float my_l = 0.0f;
  double mx = 0.0;
  for (int s = 0; s < k; s++) {
    const uint32_t mh = wave_max_u32(q[0]);
    const uint32_t ml = wave_max_u32(q[0] == mh ? 0xffffffffu - (uint32_t)ee[0] : 0u);
    const int be = (int)(0xffffffffu - ml);
    if (s == 0) mx = (double)key_float(mh);  // the largest logit
    if ((be & 63) == lane) {
      q[0] = q[1];
      ee[0] = ee[1];
      q[1] = q[2];
      ee[1] = ee[2];
      q[2] = q[3];
      ee[2] = ee[3];
      q[3] = 0u;
      ee[3] = 0x7fffffff;
    }
    if (lane == s) {
      my_e = be;
      my_l = key_float(mh);
    }
  }
  const double myp = exp((double)my_l - mx);
  const uint64_t pb = (uint64_t)__double_as_longlong(myp);
  double kept = 0.0;
  for (int s = 0; s < k; s++) {
    const uint32_t plo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)pb, s);
    const uint32_t phi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(pb >> 32), s);
    kept += __longlong_as_double((long long)(((uint64_t)phi << 32) | plo));
  }
  sel_e = my_e;
  sel_w = (float)(myp / kept);
}

__device__ __forceinline__ void route_select(const float* __restrict__ lt, int E, int k,
                                             int lane, int& sel_e, float& sel_w) {
  if (E <= 256)
    route_select_sorted4(lt, E, k, lane, sel_e, sel_w);
  else
    route_select_v<16>(lt, E, k, lane, sel_e, sel_w);
}

__device__ __forceinline__ void route_token(const float* __restrict__ lt, int E, int k,
                                            int32_t* __restrict__ ids, float* __restrict__ w,
                                            int lane, int32_t* ids_copy = nullptr) {
  int my_e;
  float my_w;
  route_select(lt, E, k, lane, my_e, my_w);
  if (lane < k) {
    ids[lane] = my_e;
    w[lane] = my_w;
    if (ids_copy) ids_copy[lane] = my_e;
  }
}


// One wave quantises one bf16 row of length K (K % 16 == 0), exactly as
// k_quant_rows does: amax / 127 in fp32, round-half-even of the quotient.
// Rows up to 4096 are held in registers (one read); longer rows are read
// twice (the second time from L2).
// Codes of four bf16 values.  Quotient: with r = 1/s (IEEE), q0 = x*r,
// e = fma(-q0, s, x), q = fma(e, r, q0); for bf16 x with |x| <= amax and
// s = amax/127 >= 2^-100, rint(q) equals rint of the IEEE quotient x/s
// (checked exhaustively over every such pair); smaller scales divide.
__device__ __forceinline__ int code_bf16(uint32_t h, float sc, float rc) {
  const float x = bf16_bits_to_f32(h);
  if (sc < 0x1p-100f) return quant_code(x, sc);
  const float q0 = x * rc;
  const float e = __builtin_fmaf(-q0, sc, x);
  const float q = __builtin_fmaf(e, rc, q0);
  return (int)fminf(fmaxf(__builtin_rintf(q), -127.0f), 127.0f);
}
__device__ __forceinline__ uint32_t quant_pack4_bf16(uint32_t w0, uint32_t w1, float sc,
                                                     float rc) {
  return pack4_i8(code_bf16(w0 & 0xffffu, sc, rc), code_bf16(w0 >> 16, sc, rc),
                  code_bf16(w1 & 0xffffu, sc, rc), code_bf16(w1 >> 16, sc, rc));
}
__device__ __forceinline__ float amax8_bf16(v4u raw) {
  const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; i++)
    a = fmaxf(a, fmaxf(fabsf(bf16_bits_to_f32(wd[i] & 0xffffu)),
                       fabsf(bf16_bits_to_f32(wd[i] >> 16))));
  return a;
}
__device__ __forceinline__ void quant_row_wave(const uint16_t* __restrict__ x, int K,
                                               int8_t* __restrict__ q, float* __restrict__ s,
                                               int lane) {
  const int nc = K >> 3;  // 8-element (16-byte) chunks
  if (nc <= 512) {
    v4u raw[8];
    float amax = 0.0f;
#pragma unroll
    for (int u = 0; u < 8; u++) {
      const int c = lane + 64 * u;
      raw[u] = c < nc ? *reinterpret_cast<const v4u*>(x + c * 8) : v4u{0u, 0u, 0u, 0u};
      amax = fmaxf(amax, amax8_bf16(raw[u]));
    }
    amax = wave_max(amax);
    const float sc = amax / 127.0f;
    const float rc = 1.0f / sc;
#pragma unroll
    for (int u = 0; u < 8; u++) {
      const int c = lane + 64 * u;
      if (c >= nc) break;
      uint32_t lo = 0, hi = 0;
      if (amax != 0.0f) {
        lo = quant_pack4_bf16(raw[u].x, raw[u].y, sc, rc);
        hi = quant_pack4_bf16(raw[u].z, raw[u].w, sc, rc);
      }
      uint32_t* o = reinterpret_cast<uint32_t*>(q + c * 8);
      o[0] = lo;
      o[1] = hi;
    }
    if (lane == 0) s[0] = amax != 0.0f ? sc : 0.0f;
    return;
  }
  float amax = 0.0f;
  for (int c = lane; c < nc; c += 64)
    amax = fmaxf(amax, amax8_bf16(*reinterpret_cast<const v4u*>(x + c * 8)));
  amax = wave_max(amax);
  const float sc = amax / 127.0f;
  const float rc = 1.0f / sc;
  for (int c = lane; c < nc; c += 64) {
    const v4u raw = *reinterpret_cast<const v4u*>(x + c * 8);
    uint32_t lo = 0, hi = 0;
    if (amax != 0.0f) {
      lo = quant_pack4_bf16(raw.x, raw.y, sc, rc);
      hi = quant_pack4_bf16(raw.z, raw.w, sc, rc);
    }
    uint32_t* o = reinterpret_cast<uint32_t*>(q + c * 8);
    o[0] = lo;
    o[1] = hi;
  }
  if (lane == 0) s[0] = amax != 0.0f ? sc : 0.0f;
}

// ---------------------------------------------------------------------------
// Sort / align by expert.  Pairs with an id outside [0, E) are dropped; the
// order of the pairs inside an expert's segment is not fixed (every pair's
// row is computed on its own, so results do not depend on it).
// ---------------------------------------------------------------------------
// Exclusive scans over the experts, one thread per expert (a whole 1024-thread
// workgroup; E <= 1024): c = the expert's pair count.  Returns the expert's
// segment offset.  With write set the workgroup also stores the list of
// experts that received pairs (ascending), their segment offsets, the active
// count and the end of the last segment, and, with blk_slot set, the table of
// kMoeBM-pair m-blocks of the large-batch GEMMs (each segment split into
// blocks of kMoeBM sorted pairs) and its length.
__device__ __forceinline__ int expert_scan(int c, bool write, int32_t* __restrict__ expert_list,
                                           int32_t* __restrict__ seg_off,
                                           int32_t* __restrict__ n_active,
                                           int32_t* __restrict__ blk_slot,
                                           int32_t* __restrict__ blk_row0,
                                           int32_t* __restrict__ n_blocks) {
  __shared__ int wsum_c[16], wsum_f[16], wsum_b[16];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int f = c > 0 ? 1 : 0;
  const int nb = (c + kMoeBM - 1) / kMoeBM;
  int ic = c, iflag = f, ib = nb;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int oc = __shfl_up(ic, off, 64);
    const int of = __shfl_up(iflag, off, 64);
    const int ob = __shfl_up(ib, off, 64);
    if (lane >= off) {
      ic += oc;
      iflag += of;
      ib += ob;
    }
  }
  if (lane == 63) {
    wsum_c[wv] = ic;
    wsum_f[wv] = iflag;
    wsum_b[wv] = ib;
  }
  __syncthreads();
  int base_c = 0, base_f = 0, base_b = 0, tot_c = 0, tot_f = 0, tot_b = 0;
  for (int i = 0; i < 16; i++) {
    if (i < wv) {
      base_c += wsum_c[i];
      base_f += wsum_f[i];
      base_b += wsum_b[i];
    }
    tot_c += wsum_c[i];
    tot_f += wsum_f[i];
    tot_b += wsum_b[i];
  }
  const int off_c = base_c + ic - c;
  if (write) {
    const int slot = base_f + iflag - f;
    if (f) {
      expert_list[slot] = tid;
      seg_off[slot] = off_c;
    }
    if (blk_slot) {
      const int off_b = base_b + ib - nb;
      for (int i = 0; i < nb; i++) {
        blk_slot[off_b + i] = slot;
        blk_row0[off_b + i] = off_c + i * kMoeBM;
      }
      if (tid == 0) n_blocks[0] = tot_b;
    }
    if (tid == 0) {
      n_active[0] = tot_f;
      seg_off[tot_f] = tot_c;
    }
  }
  return off_c;
}

// Small batches: the whole sort in one 1024-thread workgroup, for at most
// kMoeSortOneWg pairs (16 a thread, held in registers between the count and
// the scatter).  Also clears the per-pair |act| maxima.
constexpr int kMoeSortOneWg = 16 * 1024;
__device__ __forceinline__ void sort_pairs(const int32_t* __restrict__ ids, int P, int E,
                                           int32_t* __restrict__ expert_list,
                                           int32_t* __restrict__ seg_off,
                                           int32_t* __restrict__ n_active,
                                           int32_t* __restrict__ sorted_pairs,
                                           uint32_t* __restrict__ amax) {
  __shared__ int cnt[1024];
  __shared__ int cursor[1024];
  const int tid = threadIdx.x;
  cnt[tid] = 0;
  __syncthreads();
  // counts; each pair keeps the count it saw (its place in its expert's
  // segment); the id loads are all in flight before the first atomic
  constexpr int B = kMoeSortOneWg / 1024;
  int e1[B], k1[B];
#pragma unroll
  for (int b = 0; b < B; b++) {
    const int r = tid + 1024 * b;
    e1[b] = r < P ? ids[r] : -1;
    k1[b] = 0;
  }
#pragma unroll
  for (int b = 0; b < B; b++) {
    const int r = tid + 1024 * b;
    if (e1[b] >= 0 && e1[b] < E)
      k1[b] = atomicAdd(&cnt[e1[b]], 1);
    else
      e1[b] = -1;
    if (amax && r < P) amax[r] = 0u;
  }
  __syncthreads();
  const int off_c = expert_scan(tid < E ? cnt[tid] : 0, true, expert_list, seg_off, n_active,
                                nullptr, nullptr, nullptr);
  if (tid < E) cursor[tid] = off_c;
  __syncthreads();
#pragma unroll
  for (int b = 0; b < B; b++)
    if (e1[b] >= 0) sorted_pairs[cursor[e1[b]] + k1[b]] = tid + 1024 * b;
}

__global__ __launch_bounds__(1024) void k_moe_sort(
    const int32_t* __restrict__ ids, int P, int E, int32_t* __restrict__ expert_list,
    int32_t* __restrict__ seg_off, int32_t* __restrict__ n_active,
    int32_t* __restrict__ sorted_pairs, uint32_t* __restrict__ amax) {
  sort_pairs(ids, P, E, expert_list, seg_off, n_active, sorted_pairs, amax);
}

// Large batches: the sort in two launches over chunks of pairs, one
// workgroup per chunk (at most kMoeSortChunks chunks).
// k_moe_sort_hist: the chunk's per-expert counts (LDS atomics); each pair
// keeps the count it saw, its place among the chunk's pairs of its expert.
__global__ __launch_bounds__(1024) void k_moe_sort_hist(const int32_t* __restrict__ ids, int P,
                                                        int E, int chunk,
                                                        int32_t* __restrict__ hist,
                                                        int32_t* __restrict__ rank) {
  __shared__ int cnt[1024];
  const int tid = threadIdx.x;
  cnt[tid] = 0;
  __syncthreads();
  const int p0 = blockIdx.x * chunk, p1 = min(P, p0 + chunk);
  for (int p = p0 + tid; p < p1; p += 1024) {
    const int e = ids[p];
    if (e >= 0 && e < E) rank[p] = atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  if (tid < E) hist[blockIdx.x * E + tid] = cnt[tid];
}

// k_moe_sort_scatter: every workgroup reads all nb chunk counts, forms the
// segment offsets (workgroup 0 also writes the expert list and the m-block
// table) and places its chunk's pairs: pair p of expert e goes to
// seg_off(e) + (pairs of e in earlier chunks) + its place in its chunk.
__global__ __launch_bounds__(1024) void k_moe_sort_scatter(
    const int32_t* __restrict__ ids, int P, int E, int chunk, int nb,
    const int32_t* __restrict__ hist, const int32_t* __restrict__ rank,
    int32_t* __restrict__ expert_list, int32_t* __restrict__ seg_off,
    int32_t* __restrict__ n_active, int32_t* __restrict__ sorted_pairs,
    int32_t* __restrict__ blk_slot, int32_t* __restrict__ blk_row0,
    int32_t* __restrict__ n_blocks) {
  __shared__ int cursor[1024];
  const int tid = threadIdx.x;
  const int p0 = blockIdx.x * chunk, p1 = min(P, p0 + chunk);
  // the thread's first pair is read before the counts (independent loads)
  const int pf = p0 + tid;
  const int e_first = pf < p1 ? ids[pf] : -1;
  const int r_first = pf < p1 ? rank[pf] : 0;
  int c = 0, before = 0;
  if (tid < E) {
    for (int b0 = 0; b0 < nb; b0 += 16) {
      int h[16];
#pragma unroll
      for (int i = 0; i < 16; i++) h[i] = b0 + i < nb ? hist[(b0 + i) * E + tid] : 0;
#pragma unroll
      for (int i = 0; i < 16; i++) {
        if (b0 + i < (int)blockIdx.x) before += h[i];
        c += h[i];
      }
    }
  }
  const int off_c = expert_scan(c, blockIdx.x == 0, expert_list, seg_off, n_active, blk_slot,
                                blk_row0, n_blocks);
  if (tid < E) cursor[tid] = off_c + before;
  __syncthreads();
  if (e_first >= 0 && e_first < E) sorted_pairs[cursor[e_first] + r_first] = pf;
  for (int p = pf + 1024; p < p1; p += 1024) {
    const int e = ids[p];
    if (e >= 0 && e < E) sorted_pairs[cursor[e] + rank[p]] = p;
  }
}

// Routing and per-token quant for batches beyond the single-workgroup prep:
// workgroup b takes tokens 4b..4b+3; waves 0-3 route them while waves 4-7
// quantise them, so a token costs the longer of the two, not their sum.
__global__ __launch_bounds__(512) void k_moe_route_quant(
    const uint16_t* __restrict__ x, const float* __restrict__ logits, int T, int H, int E, int k,
    int32_t* __restrict__ ids, float* __restrict__ w, int8_t* __restrict__ qx,
    float* __restrict__ sx) {
  const int wv = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + (wv & 3);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  if (wv < 4) {
    if (logits)
      route_token(logits + (int64_t)t * E, E, k, ids + (int64_t)t * k, w + (int64_t)t * k, lane);
  } else {
    quant_row_wave(x + (int64_t)t * H, H, qx + (int64_t)t * H, sx + t, lane);
  }
}

// Small batches: routing, per-token quant of x and the sort in one
// 1024-thread workgroup (one launch instead of three).
__global__ __launch_bounds__(1024) void k_moe_prep(
    const uint16_t* __restrict__ x, const float* __restrict__ logits, int T, int H, int E, int k,
    int32_t* __restrict__ ids, float* __restrict__ w, int8_t* __restrict__ qx,
    float* __restrict__ sx, int32_t* __restrict__ expert_list, int32_t* __restrict__ seg_off,
    int32_t* __restrict__ n_active, int32_t* __restrict__ sorted_pairs,
    uint32_t* __restrict__ amax) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  // routed ids also go to LDS, where the sort reads them (no round trip
  // through global memory); caller-provided ids are read from global memory
  __shared__ int32_t ids_lds[kMoePrepTokens * kMoeMaxTopk];
  // waves 0-7 route tokens, waves 8-15 quantise them, side by side
  const int t0 = wv & 7;
  for (int t = t0; t < T; t += 8) {
    if (wv < 8) {
      if (logits)
        route_token(logits + (int64_t)t * E, E, k, ids + (int64_t)t * k, w + (int64_t)t * k,
                    lane, ids_lds + t * k);
    } else {
      quant_row_wave(x + (int64_t)t * H, H, qx + (int64_t)t * H, sx + t, lane);
    }
  }
  __syncthreads();  // the routing ids written above are read by the sort
  sort_pairs(logits ? ids_lds : ids, T * k, E, expert_list, seg_off, n_active, sorted_pairs,
             amax);
}

// ---------------------------------------------------------------------------
// Grouped GEMM for small batches (few pairs per expert): the weight-streaming
// structure of the dense decode kernel.  Workgroup = (16 weight rows of one
// expert, that expert's pairs in blocks of 16); its WAVES waves take the k
// steps round-robin and their int32 partials are added through LDS.
// MODE 1 = gemm1 (A = the pairs' token rows of qx; epilogue dequantises,
// applies SiLU(gate) * up on the interleaved rows, stores the fp32 activation
// and records the pair's |act| maximum with an integer atomic max).
// MODE 2 = gemm2 (prologue requantises the block's activation rows into LDS
// from that maximum; epilogue stores dequantised fp32 rows).
// Operand mapping as in gemm_skinny.hip (16x16x64 MFMA).
// ---------------------------------------------------------------------------
constexpr int kMoeSkinnyMaxK2 = 2048;  // gemm2 reduction length (I) staged in LDS

// NT: consecutive 16-row weight tiles per workgroup (amortises the chain of
// dependent reads -- active count, expert id, segment, pair ids -- over more
// weight bytes).  The first batch of weight loads is issued as soon as the
// expert id is known, before the pair data is read, and every batch's MFMAs
// run while the next batch's weight loads are in flight.
template <int WAVES, int NT, int MODE, bool PACKED, int MINB = 1>
__global__ __launch_bounds__(WAVES * 64, MINB) void k_moe_skinny(
    const int8_t* __restrict__ qx, const float* __restrict__ sx, const float* __restrict__ act,
    const uint32_t* __restrict__ amax_in, int k, const int8_t* __restrict__ W,
    const float* __restrict__ sW, int Nw, int K, const int32_t* __restrict__ expert_list,
    const int32_t* __restrict__ seg_off, const int32_t* __restrict__ n_active,
    const int32_t* __restrict__ sorted_pairs, float* __restrict__ out, int ldo,
    uint32_t* __restrict__ amax_out, int8_t* __restrict__ qa_rec, float* __restrict__ sa2_rec,
    int32_t* __restrict__ dbg_acc, int amax_parts = 1) {
  constexpr int U = NT >= 4 ? 2 : 4;  // 64-byte k steps per batch
  __shared__ v4i red[NT][WAVES][64];
  // gemm2: the block's requantised rows, 16 x K bytes of dynamic LDS (sized
  // at launch, so short rows leave room for more workgroups per CU)
  extern __shared__ __attribute__((aligned(16))) int8_t a_lds[];
  __shared__ float sa2_lds[16];
  __shared__ int pair_lds[16];
  const int slot = blockIdx.y;
  const int nact = n_active[0];
  const int e = expert_list[slot];
  if (slot >= nact) return;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int j = lane & 15;
  const int g = lane >> 4;
  const int nk = K >> 6;
  const int ntile0 = blockIdx.x * NT;
  const int8_t* wbase = PACKED
                            ? W + ((int64_t)e * (Nw >> 4) + ntile0) * nk * 1024 + lane * 16
                            : W + ((int64_t)e * Nw + ntile0 * 16 + j) * K + g * 16;
  constexpr int64_t wstep = PACKED ? 1024 : 64;
  const int64_t tstep = PACKED ? (int64_t)nk * 1024 : (int64_t)16 * K;

  auto load_w = [&](v4i (*b)[NT], int c0) {
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int c = c0 + u * WAVES;
#pragma unroll
      for (int t = 0; t < NT; t++)
        b[u][t] = c < nk ? ld_stream(wbase + t * tstep + c * wstep)
                         : v4i{0, 0, 0, 0};
    }
  };
  v4i bq[U][NT];
  load_w(bq, wv);  // first batch, in flight while the pair data is read
  // wave w finishes tile w (NT <= WAVES): its column scale is loaded now, so
  // the epilogue issues no global load behind the next weight prefetch
  static_assert(NT <= WAVES, "each wave finishes at most one tile");
  const float swc_w = wv < NT ? sW[(int64_t)e * Nw + (ntile0 + wv) * 16 + j] : 0.0f;

  const int seg_begin = seg_off[slot];
  const int seg_end = seg_off[slot + 1];
  for (int pb = seg_begin; pb < seg_end; pb += 16) {
    const int nrows = min(16, seg_end - pb);
    __syncthreads();  // LDS of the previous block fully consumed
    if (threadIdx.x < 16)
      pair_lds[threadIdx.x] = threadIdx.x < nrows ? sorted_pairs[pb + threadIdx.x] : 0;
    if (MODE == 2) {
      __syncthreads();
      // each pair's |act| maximum, kept as amax_parts partial maxima
      // (non-negative fp32 bit patterns, so the integer maximum is theirs):
      // one wave per row, the parts spread over its lanes
      for (int r = wv; r < nrows; r += WAVES) {
        const uint32_t* ap = amax_in + (int64_t)pair_lds[r] * amax_parts;
        uint32_t mb = 0u;
        for (int i = lane; i < amax_parts; i += 64) mb = max(mb, ap[i]);
        mb = wave_max_u32(mb);
        if (lane == 0) {
          const float am = __uint_as_float(mb);
          sa2_lds[r] = am != 0.0f ? am / 127.0f : 0.0f;
        }
      }
      __syncthreads();
      // requantise the block's activation rows straight into the packed
      // operand layout: row r, bytes 16s..16s+15 of k step c at c*1024 + (r + 16s)*16
      const int per_row = K >> 2;
      for (int idx = threadIdx.x; idx < nrows * per_row; idx += WAVES * 64) {
        const int r = idx / per_row;
        const int kk = (idx - r * per_row) * 4;
        const int p = pair_lds[r];
        const float sc = sa2_lds[r];
        const v4f a = *reinterpret_cast<const v4f*>(act + (int64_t)p * K + kk);
        uint32_t wd = 0;
        if (sc != 0.0f)
          wd = pack4_i8(quant_code(a.x, sc), quant_code(a.y, sc), quant_code(a.z, sc),
                        quant_code(a.w, sc));
        const int c = kk >> 6, sl = (kk & 63) >> 4;
        *reinterpret_cast<uint32_t*>(&a_lds[c * 1024 + (r + 16 * sl) * 16 + (kk & 15)]) = wd;
        if (blockIdx.x == 0 && qa_rec)
          *reinterpret_cast<uint32_t*>(qa_rec + (int64_t)p * K + kk) = wd;
      }
      if (blockIdx.x == 0 && sa2_rec && threadIdx.x < nrows)
        sa2_rec[pair_lds[threadIdx.x]] = sa2_lds[threadIdx.x];
    }
    __syncthreads();

    const bool a_ok = j < nrows;
    const int8_t* ap = qx + (int64_t)(pair_lds[a_ok ? j : 0] / k) * K + g * 16;
    // gemm1: the token scales of the lane's four pair rows (rows past the
    // block read pair id 0), loaded before the k loop
    float sxv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (MODE == 1) {
#pragma unroll
      for (int v = 0; v < 4; v++) sxv[v] = sx[pair_lds[4 * g + v] / k];
    }
    v4i acc[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) acc[t] = v4i{0, 0, 0, 0};
    for (int c0 = wv; c0 < nk; c0 += WAVES * U) {
      v4i bn[U][NT];
      if (c0 + WAVES * U < nk) load_w(bn, c0 + WAVES * U);
      v4i a[U];
#pragma unroll
      for (int u = 0; u < U; u++) {
        const int c = c0 + u * WAVES;
        const bool in = c < nk;
        if (MODE == 1)
          a[u] = (in && a_ok) ? *reinterpret_cast<const v4i*>(ap + (int64_t)c * 64)
                              : v4i{0, 0, 0, 0};
        else
          a[u] = in ? *reinterpret_cast<const v4i*>(&a_lds[c * 1024 + lane * 16])
                    : v4i{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < U; u++)
#pragma unroll
        for (int t = 0; t < NT; t++) acc[t] = mfma_16x16x64_i8(a[u], bq[u][t], acc[t]);
      if (c0 + WAVES * U < nk) {
#pragma unroll
        for (int u = 0; u < U; u++)
#pragma unroll
          for (int t = 0; t < NT; t++) bq[u][t] = bn[u][t];
      }
    }
    if (pb + 16 < seg_end) load_w(bq, wv);  // the next pair block streams the tiles again
#pragma unroll
    for (int t = 0; t < NT; t++) red[t][wv][lane] = acc[t];
    __syncthreads();
    // wave w finishes tiles w, w + WAVES, ...
    for (int t = wv; t < NT; t += WAVES) {
      v4i sum = red[t][0][lane];
#pragma unroll
      for (int w2 = 1; w2 < WAVES; w2++) sum += red[t][w2][lane];
      const int col = (ntile0 + t) * 16 + j;
      const float swc = swc_w;
#pragma unroll
      for (int v = 0; v < 4; v++) {
        const int r = 4 * g + v;
        const bool valid = r < nrows;
        const int p = pair_lds[valid ? r : 0];
        if (dbg_acc && valid) dbg_acc[(int64_t)p * Nw + col] = sum[v];
        if (MODE == 1) {
          float h = 0.0f;
          if (valid) {
            h = (float)sum[v];
            h = h * sxv[v];
            h = h * swc;
          }
          const float partner = __shfl_xor(h, 1, 64);
          float mag = 0.0f;
          if ((j & 1) == 0 && valid) {
            // SiLU(gate) * up; the gate is the even interleaved row
            const float sg = (float)((double)h / (1.0 + exp(-(double)h)));
            const float av = sg * partner;
            out[(int64_t)p * ldo + (col >> 1)] = av;
            mag = fabsf(av);
          }
#pragma unroll
          for (int off = 1; off < 16; off <<= 1) mag = fmaxf(mag, __shfl_xor(mag, off, 64));
          if (j == 0 && valid) atomicMax(&amax_out[p], __float_as_uint(mag));
        } else if (valid) {
          float yv = (float)sum[v];
          yv = yv * sa2_lds[r];
          yv = yv * swc;
          out[(int64_t)p * ldo + col] = yv;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// One routed token (T == 1, router logits given): routing, the token's
// quantisation and gemm1 in one launch.  With one token the k selected
// experts are distinct, so slot s is pair s of expert ids[s] and no sort is
// needed.  Every workgroup routes the token (wave 0) and every wave finds the
// row maximum itself (the logits and the row are small and come from L2), so
// each workgroup requests its expert's weights without waiting on another
// launch.  Workgroup (tile,
// slot) = one 16-row tile of that expert's interleaved w13, 8 waves over K
// as in k_moe_skinny, epilogue SiLU(gate) * up.  The pair's |act| maximum is
// left as one partial maximum per tile (gemm2's prologue takes their
// maximum), so nothing needs clearing before the launch.  Workgroup
// (tile 0, slot s) also writes the slot's segment record for gemm2, and
// (tile 0, slot 0) the routing outputs and the token's codes and scale.
// ---------------------------------------------------------------------------
template <bool PACKED>
__global__ __launch_bounds__(512) void k_moe_t1_gemm1(
    const uint16_t* __restrict__ x, const float* __restrict__ logits, int H, int E, int k,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_w, const int8_t* __restrict__ W,
    const float* __restrict__ sW, int Nw, int8_t* __restrict__ qx, float* __restrict__ sx,
    int32_t* __restrict__ expert_list, int32_t* __restrict__ seg_off,
    int32_t* __restrict__ n_active, int32_t* __restrict__ sorted_pairs,
    float* __restrict__ out, int ldo, uint32_t* __restrict__ amax_part,
    int32_t* __restrict__ dbg_acc) {
  constexpr int WAVES = 8, U = 4;
  __shared__ v4i red[WAVES][64];
  __shared__ __attribute__((aligned(16))) int8_t q_lds[kMoeMaxH];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int j = lane & 15;
  const int g = lane >> 4;
  const int tile = blockIdx.x, slot = blockIdx.y, ntiles = gridDim.x;
  const int nk = H >> 6;

  // the token row goes out first (held for the row maximum: 8 16-byte
  // chunks a lane cover H <= 4096), then the logits with the routing
  constexpr int XR = 8;
  const int nc8 = H >> 3;
  v4u xr[XR];
#pragma unroll
  for (int u = 0; u < XR; u++) {
    const int c = lane + 64 * u;
    xr[u] = c < nc8 ? *reinterpret_cast<const v4u*>(x + c * 8) : v4u{0u, 0u, 0u, 0u};
  }
  // wave 0 routes the token (the selection is a chain of k wave-wide
  // maximum rounds; on every wave it would fill the SIMDs for microseconds);
  // the others wait at the barrier
  __shared__ int e_lds;
  int sel_e = 0;
  float sel_w = 0.0f;
  if (wv == 0) {
    route_select(logits, E, k, lane, sel_e, sel_w);
    const int es = __shfl(sel_e, slot, 64);
    if (lane == 0) e_lds = es;
  }
  __syncthreads();
  const int e = __builtin_amdgcn_readfirstlane(e_lds);

  const int8_t* wbase = PACKED ? W + ((int64_t)e * (Nw >> 4) + tile) * nk * 1024 + lane * 16
                               : W + ((int64_t)e * Nw + tile * 16 + j) * H + g * 16;
  constexpr int64_t wstep = PACKED ? 1024 : 64;
  auto load_w = [&](v4i* b, int c0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int c = c0 + u * WAVES;
      b[u] = c < nk ? ld_stream(wbase + c * wstep) : v4i{0, 0, 0, 0};
    }
  };
  v4i bq[U];
  load_w(bq, wv);
  const int col = tile * 16 + j;
  const float swc = wv == 0 ? sW[(int64_t)e * Nw + col] : 0.0f;  // wave 0's epilogue

  // the token's scale: maximum of |x| over the row (every wave), as k_quant_rows
  float amax = 0.0f;
#pragma unroll
  for (int u = 0; u < XR; u++) amax = fmaxf(amax, amax8_bf16(xr[u]));
  for (int c = lane + 64 * XR; c < nc8; c += 64)
    amax = fmaxf(amax, amax8_bf16(*reinterpret_cast<const v4u*>(x + c * 8)));
  amax = wave_max(amax);
  const float sc = amax / 127.0f;
  const float rc = 1.0f / sc;
  const float sxv = amax != 0.0f ? sc : 0.0f;
  // the token's codes, by the whole workgroup (8 per thread), into LDS;
  // workgroup (0, 0) also writes them out with the scale
  for (int c8 = threadIdx.x; c8 < nc8; c8 += WAVES * 64) {
    const v4u raw = *reinterpret_cast<const v4u*>(x + c8 * 8);
    uint32_t lo = 0, hi = 0;
    if (amax != 0.0f) {
      lo = quant_pack4_bf16(raw.x, raw.y, sc, rc);
      hi = quant_pack4_bf16(raw.z, raw.w, sc, rc);
    }
    uint32_t* ql = reinterpret_cast<uint32_t*>(q_lds + c8 * 8);
    ql[0] = lo;
    ql[1] = hi;
    if (tile == 0 && slot == 0) {
      uint32_t* o = reinterpret_cast<uint32_t*>(qx + c8 * 8);
      o[0] = lo;
      o[1] = hi;
    }
  }
  __syncthreads();
  // A operand of k chunk c: lanes of row 0 (j == 0) hold codes 64c + 16g ..
  // +15; the other rows are zero
  auto load_a = [&](int c) __attribute__((always_inline)) {
    return (j == 0 && c < nk) ? *reinterpret_cast<const v4i*>(q_lds + c * 64 + g * 16)
                              : v4i{0, 0, 0, 0};
  };

  v4i acc = {0, 0, 0, 0};
  for (int c0 = wv; c0 < nk; c0 += WAVES * U) {
    v4i bn[U];
    if (c0 + WAVES * U < nk) load_w(bn, c0 + WAVES * U);
    v4i a[U];
#pragma unroll
    for (int u = 0; u < U; u++) a[u] = load_a(c0 + u * WAVES);
#pragma unroll
    for (int u = 0; u < U; u++) acc = mfma_16x16x64_i8(a[u], bq[u], acc);
    if (c0 + WAVES * U < nk) {
#pragma unroll
      for (int u = 0; u < U; u++) bq[u] = bn[u];
    }
  }

  // wave 0 writes the tile
  red[wv][lane] = acc;
  __syncthreads();
  if (wv == 0) {
#pragma unroll
    for (int w2 = 1; w2 < WAVES; w2++) acc += red[w2][lane];
    keep_live(swc);
    // result lane l holds rows 4*(l/16)+v of column l%16: the token is row 0
    float h = (float)acc[0];
    h = h * sxv;
    h = h * swc;
    if (dbg_acc && g == 0) dbg_acc[(int64_t)slot * Nw + col] = acc[0];
    const float partner = __shfl_xor(h, 1, 64);
    float mag = 0.0f;
    if (g == 0 && (j & 1) == 0) {
      // SiLU(gate) * up; the gate is the even interleaved row
      const float sg = (float)((double)h / (1.0 + exp(-(double)h)));
      const float av = sg * partner;
      out[(int64_t)slot * ldo + (col >> 1)] = av;
      mag = fabsf(av);
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) mag = fmaxf(mag, __shfl_xor(mag, off, 64));
    if (lane == 0) amax_part[(int64_t)slot * ntiles + tile] = __float_as_uint(mag);
    if (tile == 0) {
      // the slot's segment for gemm2: expert e, pair `slot`
      if (lane == 0) {
        expert_list[slot] = e;
        seg_off[slot] = slot;
        sorted_pairs[slot] = slot;
      }
      if (slot == 0) {
        if (lane == 0) {
          n_active[0] = k;
          seg_off[k] = k;
          sx[0] = sxv;
        }
        if (lane < k) {
          topk_ids[lane] = sel_e;
          topk_w[lane] = sel_w;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// One routed token: requant, gemm2 and the weighted combine in one launch.
// Workgroup = 16 output columns; wave w takes slot w (and w + 8): it
// requantises the pair's activation row from the partial maxima gemm1 left,
// multiplies it with the 16 rows of its expert's w2 (all of K = I on the one
// wave), and puts the dequantised y2 values in LDS.  Wave 0 then forms
// out = bf16(sum over slots of w_s * y2_s) in fp32, slot order, no FMA --
// the combine of k_moe_combine -- without y2 going through memory.
// ---------------------------------------------------------------------------
template <bool PACKED>
__global__ __launch_bounds__(512) void k_moe_t1_gemm2(
    const float* __restrict__ act, const uint32_t* __restrict__ amax_part, int parts,
    const int32_t* __restrict__ ids, const float* __restrict__ wts, int k,
    const int8_t* __restrict__ W2, const float* __restrict__ s2, int H, int I,
    uint16_t* __restrict__ out, int8_t* __restrict__ dbg_qa, float* __restrict__ dbg_sa2,
    int32_t* __restrict__ dbg_acc) {
  constexpr int WAVES = 8, U = 8;
  __shared__ float ybuf[kMoeMaxTopk][16];
  __shared__ __attribute__((aligned(16))) int8_t qa_lds[WAVES][kMoeSkinnyMaxK2];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int j = lane & 15;
  const int g = lane >> 4;
  const int tile = blockIdx.x;
  const int nk = I >> 6;
  for (int sl = wv; sl < k; sl += WAVES) {
    const int e = __builtin_amdgcn_readfirstlane(ids[sl]);
    const int8_t* wbase = PACKED ? W2 + ((int64_t)e * (H >> 4) + tile) * nk * 1024 + lane * 16
                                 : W2 + ((int64_t)e * H + tile * 16 + j) * I + g * 16;
    constexpr int64_t wstep = PACKED ? 1024 : 64;
    const int col = tile * 16 + j;
    const float swc = s2[(int64_t)e * H + col];
    // the pair's |act| maximum from gemm1's partial maxima (non-negative
    // fp32 bit patterns), then its scale
    uint32_t mb = 0u;
    for (int i = lane; i < parts; i += 64) mb = max(mb, amax_part[(int64_t)sl * parts + i]);
    mb = wave_max_u32(mb);
    const float am = __uint_as_float(mb);
    const float sc = am != 0.0f ? am / 127.0f : 0.0f;
    // the row's codes, four per lane at a time, into this wave's LDS row
    int8_t* qrow = qa_lds[wv];
    for (int i = lane * 4; i < I; i += 256) {
      const v4f v = *reinterpret_cast<const v4f*>(act + (int64_t)sl * I + i);
      uint32_t wd = 0u;
      if (sc != 0.0f)
        wd = pack4_i8(quant_code(v.x, sc), quant_code(v.y, sc), quant_code(v.z, sc),
                      quant_code(v.w, sc));
      *reinterpret_cast<uint32_t*>(qrow + i) = wd;
      if (dbg_qa && tile == 0) *reinterpret_cast<uint32_t*>(dbg_qa + (int64_t)sl * I + i) = wd;
    }
    v4i acc = {0, 0, 0, 0};
    for (int c0 = 0; c0 < nk; c0 += U) {
      v4i b[U], a[U];
#pragma unroll
      for (int u = 0; u < U; u++) {
        const int c = c0 + u;
        b[u] = c < nk ? ld_stream(wbase + c * wstep) : v4i{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < U; u++) {
        // row 0 of the A operand (lanes j == 0): codes 64c + 16g .. +15; the
        // other rows are zero
        const int c = c0 + u;
        a[u] = (j == 0 && c < nk) ? *reinterpret_cast<const v4i*>(qrow + c * 64 + g * 16)
                                  : v4i{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < U; u++) acc = mfma_16x16x64_i8(a[u], b[u], acc);
    }
    // result row 0 (lanes g == 0) holds the token's sums for the 16 columns
    if (g == 0) {
      float y = (float)acc[0];
      y = y * sc;
      y = y * swc;
      ybuf[sl][j] = y;
      if (dbg_acc) dbg_acc[(int64_t)sl * H + col] = acc[0];
    }
    if (dbg_sa2 && tile == 0 && lane == 0) dbg_sa2[sl] = sc;
  }
  __syncthreads();
  if (wv == 0 && lane < 16) {
    float o = 0.0f;
    for (int sl = 0; sl < k; sl++) o = o + wts[sl] * ybuf[sl][lane];
    out[tile * 16 + lane] = (uint16_t)f32_to_bf16_bits(o);
  }
}

// ---------------------------------------------------------------------------
// Grouped GEMM for large batches.  Workgroup = (one m-block of up to kMoeBM
// sorted pairs of one expert, BN = 32 * WAVES weight rows of that expert);
// wave w owns weight rows n0 + 32w .. +31 and all the block's pair rows
// (v_mfma_i32_32x32x32_i8).  The kernel streams weights from HBM, so the
// weight operand goes straight from global memory into a ring of PF k steps
// of registers per wave (with 2 waves per SIMD that keeps ~128 KiB of weight
// loads in flight per CU; LDS could stage far less).  The gathered activation
// rows are shared by the waves and come from L2: each k step every wave
// loads two 16-row x 64-byte blocks into registers DA = 2 steps ahead and
// writes them to one of two LDS buffers (1 KiB blocks of 16 rows x 4
// k-slices, conflict-free), one barrier per step.  Loads never branch: rows
// past the segment end re-read its last row, and steps past K read step 0
// with the weight fragment zeroed.  32-row blocks past the segment end are
// not multiplied.
// MODE 1 = gemm1: A = qx rows of the pairs' tokens; epilogue dequantises and
//          writes SiLU(gate) * up (gate = even interleaved row) as fp32 rows.
// MODE 2 = gemm2: A = qa rows of the pairs; epilogue writes dequantised fp32.
// ---------------------------------------------------------------------------
template <int MODE, int WAVES, int PF, bool PACKED, int MINB = 2>
__global__ __launch_bounds__(WAVES * 64, MINB) void k_moe_tile(
    const int8_t* __restrict__ A, const float* __restrict__ sA, int a_div,
    const int8_t* __restrict__ W, const float* __restrict__ sW, int Nw, int K, int npw,
    const int32_t* __restrict__ expert_list, const int32_t* __restrict__ seg_off,
    const int32_t* __restrict__ blk_slot, const int32_t* __restrict__ blk_row0,
    const int32_t* __restrict__ n_blocks, const int32_t* __restrict__ sorted_pairs,
    float* __restrict__ out, int ldo, int32_t* __restrict__ dbg_acc) {
  constexpr int BM = kMoeBM;
  constexpr int BN = 32 * WAVES;
  constexpr int NA = BM / 16;  // activation blocks per k step
  constexpr int LA = NA / WAVES;
  constexpr int DA = 2;        // activation register ring depth (steps)
  static_assert(NA % WAVES == 0, "activation blocks must split evenly over waves");
  static_assert(PF % DA == 0, "ring depths must nest");
  // gemm2 walks npw weight blocks per workgroup with an epilogue after each;
  // gemm1 (heavier epilogue, longer k) takes one block (npw must be 1)
  constexpr bool kMulti = MODE == 2;
  __shared__ __attribute__((aligned(1024))) int8_t a_lds[2][NA * 1024];
  __shared__ int pair_lds[BM];
  __shared__ float sa_lds[BM];
  __shared__ float sw_lds[kMulti ? BN * kMoeMaxNpw : BN];

  // Workgroups go to the 8 XCDs round-robin.  All the workgroups of one
  // m-block run on the same XCD back to back, so its gathered activation rows
  // are fetched into that XCD's L2 once.  Workgroup = npw consecutive BN-row
  // weight blocks of the m-block's expert, streamed as one sequence of k steps.
  const int ngrp = Nw / (BN * npw);
  const int xcd = blockIdx.x & 7;
  const int t = blockIdx.x >> 3;
  const int mb = (t / ngrp) * 8 + xcd;
  if (mb >= n_blocks[0]) return;
  const int slot = blk_slot[mb];
  const int row0 = blk_row0[mb];
  const int e = expert_list[slot];
  const int rows = min(BM, seg_off[slot + 1] - row0);
  const int nfirst = (t % ngrp) * npw * BN;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int j = lane & 15;
  const int g = lane >> 4;
  const int nk = K >> 6;
  const int nsteps = (nk + PF - 1) / PF * PF;  // k steps per weight block, padded

  // weight fragment addresses: lane l feeds column c = n0 + 32 wv + l % 32,
  // k-slice 2h + l/32 of each 32-byte half h of a 64-byte k step.  Global
  // step s = (weight block s / nsteps, k step s % nsteps); padded steps read
  // k step 0 and are zeroed before use.
  const int c0 = nfirst + 32 * wv + (lane & 31);
  const int8_t* bsrc =
      PACKED ? W + ((int64_t)e * (Nw >> 4) + (c0 >> 4)) * nk * 1024 +
                   ((c0 & 15) + 16 * (lane >> 5)) * 16
             : W + ((int64_t)e * Nw + c0) * K + (lane >> 5) * 16;
  constexpr int BSTEP = PACKED ? 1024 : 64;
  constexpr int BHALF = PACKED ? 512 : 32;
  const int64_t bblock = PACKED ? (int64_t)(BN >> 4) * nk * 1024 : (int64_t)BN * K;
  const int send = npw * nsteps;
  auto load_b = [&](int sg, v4i* b) __attribute__((always_inline)) {
    const int sc = sg < send ? sg : 0;
    const int nb = sc / nsteps, kt = sc - nb * nsteps;
    const int8_t* q = bsrc + nb * bblock + (int64_t)(kt < nk ? kt : 0) * BSTEP;
    b[0] = ld_stream(q);
    b[1] = ld_stream(q + BHALF);
  };

  // the block's pair ids and activation scales, and the weight rows' scales,
  // read once into LDS (the gather addresses and the epilogue use them; the
  // epilogue then issues no global load)
  for (int r = threadIdx.x; r < rows; r += WAVES * 64) {
    const int p = sorted_pairs[row0 + r];
    pair_lds[r] = p;
    sa_lds[r] = sA[p / a_div];
  }
  for (int c = threadIdx.x; c < npw * BN; c += WAVES * 64)
    sw_lds[c] = sW[(int64_t)e * Nw + nfirst + c];
  // first weight loads go out before the wait for the pair table
  v4i bq[PF][2];
#pragma unroll
  for (int s = 0; s < PF; s++) load_b(s, bq[s]);
  lds_barrier();
  const int8_t* asrc[LA];
#pragma unroll
  for (int i = 0; i < LA; i++) {
    const int r = min((wv + i * WAVES) * 16 + j, rows - 1);
    asrc[i] = A + (int64_t)(pair_lds[r] / a_div) * K + g * 16;
  }
  auto load_a = [&](int sg, v4i* a) __attribute__((always_inline)) {
    const int kt = sg % nsteps;
    const int kc = kt < nk ? kt : 0;
#pragma unroll
    for (int i = 0; i < LA; i++) a[i] = *reinterpret_cast<const v4i*>(asrc[i] + kc * 64);
  };
  v4i aq[DA][LA];
#pragma unroll
  for (int s = 0; s < DA; s++) load_a(s, aq[s]);

  // 32x32x32 fragment of one 32-byte k half: lane l reads row (l % 32) of a
  // 32-row pair of blocks, k-slice 2h + l/32.
  const int frag_off = ((lane >> 4) & 1) * 1024 + ((lane & 15) + 16 * (lane >> 5)) * 16;
  v16i acc[BM / 32];
  const int odd = lane & 1;

  // epilogue of one weight block: lane holds weight row (product column)
  // n0 + 32 wv + lane % 32 and pair rows 8*(v/4) + 4*(lane/32) + v%4 of each
  // 32-row block.  Rows past the segment end hold the sums of its last row
  // (their activation loads re-read that row), so they are finished and
  // stored as that row: the duplicate stores write the same values to the
  // same places, and no store sits in a branch (a branch would make the
  // compiler wait for the stores before the next weight loads are used).
  auto epilogue = [&](int n0) __attribute__((always_inline)) {
    const int col = n0 + 32 * wv + (lane & 31);
    const float swc = sw_lds[col - nfirst];
    // opaque to the optimiser: otherwise the 128 row indices and their LDS
    // addresses are hoisted out of the main loop and spill
    int rlane = 4 * (lane >> 5);
    asm volatile("" : "+v"(rlane));
#pragma unroll
    for (int i = 0; i < BM / 32; i++) {
      if (32 * i >= rows) break;
      float h[16];
      int prow[MODE == 1 ? 16 : 1];  // gemm1 keeps the pair ids for the SiLU stores
#pragma unroll
      for (int v = 0; v < 16; v++) {
        const int r = min(32 * i + 8 * (v >> 2) + rlane + (v & 3), rows - 1);
        const int32_t av = acc[i][v];
        const int p = pair_lds[r];
        if (MODE == 1) prow[v] = p;
        if (dbg_acc) dbg_acc[(int64_t)p * Nw + col] = av;
        h[v] = (float)av;
        h[v] = h[v] * sa_lds[r];
        h[v] = h[v] * swc;
        if (MODE == 2) out[(int64_t)p * ldo + col] = h[v];
      }
      if (MODE == 1) {
        // gate = even interleaved row, up = the odd one in the neighbouring
        // lane.  The pair of lanes splits the 16 rows: the even lane finishes
        // rows v < 8, the odd lane rows v >= 8.
        float x[16];
#pragma unroll
        for (int v = 0; v < 16; v++) x[v] = __shfl_xor(h[v], 1, 64);
#pragma unroll
        for (int v = 0; v < 8; v++) {
          const float gate = odd ? x[v + 8] : h[v];
          const float up = odd ? h[v + 8] : x[v];
          const float sg = (float)((double)gate / (1.0 + exp(-(double)gate)));
          out[(int64_t)(odd ? prow[v + 8] : prow[v]) * ldo + (col >> 1)] = sg * up;
        }
      }
    }
  };

  auto mainloop = [&](auto tma_c) __attribute__((always_inline)) {
    constexpr int TMA = decltype(tma_c)::value;  // 32-row blocks holding pairs
#pragma unroll
    for (int i = 0; i < BM / 32; i++) acc[i] = v16i{0};
    for (int s0 = 0; s0 < send; s0 += PF) {
#pragma unroll
      for (int u = 0; u < PF; u++) {
        const int sg = s0 + u;
        int8_t* buf = a_lds[u & 1];
#pragma unroll
        for (int i = 0; i < LA; i++)
          *reinterpret_cast<v4i*>(buf + (wv + i * WAVES) * 1024 + lane * 16) = aq[u % DA][i];
        load_a(sg + DA, aq[u % DA]);
        lds_barrier();
        const int8_t* st = buf + frag_off;
        v4i fa[2][TMA];
#pragma unroll
        for (int h = 0; h < 2; h++)
#pragma unroll
          for (int i = 0; i < TMA; i++)
            fa[h][i] = *reinterpret_cast<const v4i*>(st + h * 512 + i * 2048);
        const bool kin = (sg % nsteps) < nk;
#pragma unroll
        for (int h = 0; h < 2; h++) {
          const v4i bf = kin ? bq[u][h] : v4i{0, 0, 0, 0};
#pragma unroll
          for (int i = 0; i < TMA; i++) acc[i] = mfma_32x32x32_i8(fa[h][i], bf, acc[i]);
        }
        load_b(sg + PF, bq[u]);
      }
      if (kMulti && (s0 + PF) % nsteps == 0) {  // a weight block is complete
        epilogue(nfirst + ((s0 + PF) / nsteps - 1) * BN);
#pragma unroll
        for (int i = 0; i < BM / 32; i++) acc[i] = v16i{0};
      }
    }
  };
  const int tma = (rows + 31) >> 5;
  if (tma >= 4)
    mainloop(std::integral_constant<int, 4>{});
  else if (tma == 3)
    mainloop(std::integral_constant<int, 3>{});
  else if (tma == 2)
    mainloop(std::integral_constant<int, 2>{});
  else
    mainloop(std::integral_constant<int, 1>{});
  if (!kMulti) epilogue(nfirst);
}

// Per-pair requant of the fp32 activation rows (one wave per pair row; the
// row maximum is found here).  I <= 4096: at most 64 values per lane.
template <int VPL>  // values per lane, I <= 64 * VPL
__global__ __launch_bounds__(256) void k_moe_requant(const float* __restrict__ act, int P,
                                                     int I, int8_t* __restrict__ qa,
                                                     float* __restrict__ sa2) {
  const int lane = threadIdx.x & 63;
  const int p = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (p >= P) return;
  const float* ar = act + (int64_t)p * I;
  v4f a[VPL / 4];
  float am = 0.0f;
#pragma unroll
  for (int u = 0; u < VPL / 4; u++) {
    const int c = (u * 64 + lane) * 4;
    a[u] = c < I ? *reinterpret_cast<const v4f*>(ar + c) : v4f{0.0f, 0.0f, 0.0f, 0.0f};
    am = fmaxf(am, fmaxf(fmaxf(fabsf(a[u].x), fabsf(a[u].y)), fmaxf(fabsf(a[u].z), fabsf(a[u].w))));
  }
  am = wave_max(am);
  const float sc = am / 127.0f;
  int8_t* qr = qa + (int64_t)p * I;
#pragma unroll
  for (int u = 0; u < VPL / 4; u++) {
    const int c = (u * 64 + lane) * 4;
    if (c >= I) break;
    uint32_t wd = 0;
    if (am != 0.0f)
      wd = pack4_i8(quant_code(a[u].x, sc), quant_code(a[u].y, sc), quant_code(a[u].z, sc),
                    quant_code(a[u].w, sc));
    *reinterpret_cast<uint32_t*>(qr + c) = wd;
  }
  if (lane == 0) sa2[p] = am != 0.0f ? sc : 0.0f;
}

// Weighted combine: out[t, c] = bf16( sum_j w[t,j] * y2[t*k + j, c] ), fp32,
// slot order, one product and one sum per slot (no fused multiply-add).
__global__ __launch_bounds__(256) void k_moe_combine(const float* __restrict__ y2,
                                                     const int32_t* __restrict__ ids,
                                                     const float* __restrict__ w, int T, int H,
                                                     int E, int k, uint16_t* __restrict__ out) {
  const int t = blockIdx.y;
  const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (c >= H) return;
  v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s = 0; s < k; s++) {
    const int64_t r = (int64_t)t * k + s;
    const int e = ids[r];
    if (e < 0 || e >= E) continue;
    const float ws = w[r];
    const v4f y = *reinterpret_cast<const v4f*>(y2 + r * H + c);
    acc.x = acc.x + ws * y.x;
    acc.y = acc.y + ws * y.y;
    acc.z = acc.z + ws * y.z;
    acc.w = acc.w + ws * y.w;
  }
  const uint32_t lo = f32_to_bf16_bits(acc.x) | (f32_to_bf16_bits(acc.y) << 16);
  const uint32_t hi = f32_to_bf16_bits(acc.z) | (f32_to_bf16_bits(acc.w) << 16);
  uint32_t* o = reinterpret_cast<uint32_t*>(out + (int64_t)t * H + c);
  o[0] = lo;
  o[1] = hi;
}

size_t moe_workspace_bytes(int64_t T, int64_t H, int64_t E, int64_t I, int k) {
  return carve(nullptr, T, H, E, I, k).bytes;
}

// Small batches (at most kMoeSmallPairs routed pairs) take the fused prep
// kernel and the skinny grouped GEMMs (gemm2 requantises in its prologue):
// four launches.  Larger batches: routing, sort and quant kernels, the
// 64-pair-block grouped GEMMs, a requant kernel and the combine.
constexpr int64_t kMoeSmallPairs = 2048;
// up to this many tokens the small path routes, quantises and sorts in one
// workgroup (16 waves); beyond, one wave per token and a separate sort

template <bool PACKED>
static hipError_t moe_forward_impl(const MoeArgs& a, hipStream_t stream) {
  const int64_t P = (int64_t)a.T * a.k;
  MoeWs ws = carve(a.ws, a.T, a.H, a.E, a.I, a.k);
  const int slots = (int)std::min<int64_t>(a.E, P);
  const int I2 = 2 * a.I;
  hipError_t err;
  const bool small = P <= kMoeSmallPairs && a.I <= kMoeSkinnyMaxK2;
  const bool t1 = small && a.T == 1 && a.logits;
  if (t1) {
    // one routed token: routing and quant fused into gemm1
    const int tiles1 = I2 / 16, tiles2 = a.H / 16;
    hipLaunchKernelGGL((k_moe_t1_gemm1<PACKED>), dim3(tiles1, a.k), dim3(512), 0, stream, a.x,
                       a.logits, a.H, a.E, a.k, a.topk_ids, a.topk_w, a.w13, a.s13, I2, ws.qx,
                       ws.sx, ws.expert_list, ws.seg_off, ws.n_active, ws.sorted_pairs, ws.act,
                       a.I, ws.amax_part, a.dbg_acc1);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL((k_moe_t1_gemm2<PACKED>), dim3(tiles2), dim3(512), 0, stream, ws.act,
                       ws.amax_part, tiles1, a.topk_ids, a.topk_w, a.k, a.w2, a.s2, a.H, a.I,
                       a.out, a.dbg_qa, a.dbg_sa2, a.dbg_acc2);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  } else if (small) {
    if (a.T <= kMoePrepTokens) {
      hipLaunchKernelGGL(k_moe_prep, dim3(1), dim3(1024), 0, stream, a.x, a.logits, a.T, a.H,
                         a.E, a.k, a.topk_ids, a.topk_w, ws.qx, ws.sx, ws.expert_list,
                         ws.seg_off, ws.n_active, ws.sorted_pairs, ws.amax);
    } else {
      hipLaunchKernelGGL(k_moe_route_quant, dim3((a.T + 3) / 4), dim3(512), 0, stream, a.x,
                         a.logits, a.T, a.H, a.E, a.k, a.topk_ids, a.topk_w, ws.qx, ws.sx);
      if ((err = hipGetLastError()) != hipSuccess) return err;
      hipLaunchKernelGGL(k_moe_sort, dim3(1), dim3(1024), 0, stream, a.topk_ids, (int)P, a.E,
                         ws.expert_list, ws.seg_off, ws.n_active, ws.sorted_pairs, ws.amax);
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
    // Workgroup shapes measured on MI355X at 256 experts, H=2048, I=512: up to
    // 64 pairs gemm1 takes one 16-row weight tile per 8-wave workgroup (most
    // parallelism) and gemm2 two tiles per 4-wave workgroup; larger batches
    // take two (gemm1) and four (gemm2) tiles per 4-wave workgroup.  H and I
    // are multiples of 64, so 2I/16 is even and H/16 a multiple of 4.
    const int tiles1 = I2 / 16, tiles2 = a.H / 16;
    if (P <= 64) {
      hipLaunchKernelGGL((k_moe_skinny<8, 1, 1, PACKED>), dim3(tiles1, slots), dim3(512), 0,
                         stream, ws.qx, ws.sx, nullptr, nullptr, a.k, a.w13, a.s13, I2, a.H,
                         ws.expert_list, ws.seg_off, ws.n_active, ws.sorted_pairs, ws.act, a.I,
                         ws.amax, nullptr, nullptr, a.dbg_acc1);
      if ((err = hipGetLastError()) != hipSuccess) return err;
      hipLaunchKernelGGL((k_moe_skinny<4, 2, 2, PACKED>), dim3(tiles2 / 2, slots), dim3(256), 16 * a.I,
                         stream, nullptr, nullptr, ws.act, ws.amax, a.k, a.w2, a.s2, a.H, a.I,
                         ws.expert_list, ws.seg_off, ws.n_active, ws.sorted_pairs, ws.y2, a.H,
                         nullptr, a.dbg_qa, a.dbg_sa2, a.dbg_acc2);
    } else {
      hipLaunchKernelGGL((k_moe_skinny<4, 2, 1, PACKED, 3>), dim3(tiles1 / 2, slots), dim3(256), 0,
                         stream, ws.qx, ws.sx, nullptr, nullptr, a.k, a.w13, a.s13, I2, a.H,
                         ws.expert_list, ws.seg_off, ws.n_active, ws.sorted_pairs, ws.act, a.I,
                         ws.amax, nullptr, nullptr, a.dbg_acc1);
      if ((err = hipGetLastError()) != hipSuccess) return err;
      hipLaunchKernelGGL((k_moe_skinny<4, 4, 2, PACKED>), dim3(tiles2 / 4, slots), dim3(256), 16 * a.I,
                         stream, nullptr, nullptr, ws.act, ws.amax, a.k, a.w2, a.s2, a.H, a.I,
                         ws.expert_list, ws.seg_off, ws.n_active, ws.sorted_pairs, ws.y2, a.H,
                         nullptr, a.dbg_qa, a.dbg_sa2, a.dbg_acc2);
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
  } else {
    // routing + per-token quant, then the sort by expert with the m-block
    // table (per-chunk counts, then the scatter)
    hipLaunchKernelGGL(k_moe_route_quant, dim3((a.T + 3) / 4), dim3(512), 0, stream, a.x,
                       a.logits, a.T, a.H, a.E, a.k, a.topk_ids, a.topk_w, ws.qx, ws.sx);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const int chunk = (int)std::max<int64_t>(1024, (P + kMoeSortChunks - 1) / kMoeSortChunks);
    const int nchunks = (int)((P + chunk - 1) / chunk);
    hipLaunchKernelGGL(k_moe_sort_hist, dim3(nchunks), dim3(1024), 0, stream, a.topk_ids,
                       (int)P, a.E, chunk, ws.hist, ws.rank);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(k_moe_sort_scatter, dim3(nchunks), dim3(1024), 0, stream, a.topk_ids,
                       (int)P, a.E, chunk, nchunks, ws.hist, ws.rank, ws.expert_list, ws.seg_off,
                       ws.n_active, ws.sorted_pairs, ws.blk_slot, ws.blk_row0, ws.n_blocks);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    // m-blocks: at most one partial block per expert that received pairs;
    // the grid covers that bound rounded up to the 8 XCDs.  Workgroups of 8
    // waves (256 weight rows, the gathered activation rows shared by twice
    // the weight rows of a 4-wave group) with a 2-step weight ring where the
    // weight rows allow it (measured on MI355X at 2048 tokens, 256 experts,
    // H=2048, I=512: gemm1 127-138 -> 113-121 us, gemm2 92-106 -> 82-90 us).
    const unsigned max_blocks = (unsigned)((P / kMoeBM + slots + 7) / 8 * 8);
    if (I2 % 256 == 0)
      hipLaunchKernelGGL((k_moe_tile<1, 8, 2, PACKED>), dim3(max_blocks * (I2 / 256)),
                         dim3(512), 0, stream, ws.qx, ws.sx, a.k, a.w13, a.s13, I2, a.H, 1,
                         ws.expert_list, ws.seg_off, ws.blk_slot, ws.blk_row0, ws.n_blocks,
                         ws.sorted_pairs, ws.act, a.I, a.dbg_acc1);
    else
      hipLaunchKernelGGL((k_moe_tile<1, 4, 4, PACKED>), dim3(max_blocks * (I2 / 128)),
                         dim3(256), 0, stream, ws.qx, ws.sx, a.k, a.w13, a.s13, I2, a.H, 1,
                         ws.expert_list, ws.seg_off, ws.blk_slot, ws.blk_row0, ws.n_blocks,
                         ws.sorted_pairs, ws.act, a.I, a.dbg_acc1);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (a.I <= 1024)
      hipLaunchKernelGGL(k_moe_requant<16>, dim3((unsigned)((P + 3) / 4)), dim3(256), 0, stream,
                         ws.act, (int)P, a.I, ws.qa, ws.sa2);
    else
      hipLaunchKernelGGL(k_moe_requant<64>, dim3((unsigned)((P + 3) / 4)), dim3(256), 0, stream,
                         ws.act, (int)P, a.I, ws.qa, ws.sa2);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (a.H % 256 == 0) {
      const int npw2 = (a.H / 256) % 2 == 0 ? 2 : 1;
      hipLaunchKernelGGL((k_moe_tile<2, 8, 2, PACKED>), dim3(max_blocks * (a.H / 256 / npw2)),
                         dim3(512), 0, stream, ws.qa, ws.sa2, 1, a.w2, a.s2, a.H, a.I, npw2,
                         ws.expert_list, ws.seg_off, ws.blk_slot, ws.blk_row0, ws.n_blocks,
                         ws.sorted_pairs, ws.y2, a.H, a.dbg_acc2);
    } else if (a.H % 128 == 0) {
      const int npw2 = (a.H / 128) % 8 == 0 ? 8 : (a.H / 128) % 4 == 0 ? 4 : 1;
      hipLaunchKernelGGL((k_moe_tile<2, 4, 4, PACKED>), dim3(max_blocks * (a.H / 128 / npw2)),
                         dim3(256), 0, stream, ws.qa, ws.sa2, 1, a.w2, a.s2, a.H, a.I, npw2,
                         ws.expert_list, ws.seg_off, ws.blk_slot, ws.blk_row0, ws.n_blocks,
                         ws.sorted_pairs, ws.y2, a.H, a.dbg_acc2);
    } else {
      hipLaunchKernelGGL((k_moe_tile<2, 2, 4, PACKED>), dim3(max_blocks * (a.H / 64)),
                         dim3(128), 0, stream, ws.qa, ws.sa2, 1, a.w2, a.s2, a.H, a.I, 1,
                         ws.expert_list, ws.seg_off, ws.blk_slot, ws.blk_row0, ws.n_blocks,
                         ws.sorted_pairs, ws.y2, a.H, a.dbg_acc2);
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (a.dbg_qa && (err = hipMemcpyAsync(a.dbg_qa, ws.qa, (size_t)P * a.I,
                                          hipMemcpyDeviceToDevice, stream)) != hipSuccess)
      return err;
    if (a.dbg_sa2 && (err = hipMemcpyAsync(a.dbg_sa2, ws.sa2, (size_t)P * 4,
                                           hipMemcpyDeviceToDevice, stream)) != hipSuccess)
      return err;
  }
  if (!t1) {  // the single-token path combined inside its gemm2
    hipLaunchKernelGGL(k_moe_combine, dim3((a.H / 4 + 255) / 256, a.T), dim3(256), 0, stream,
                       ws.y2, a.topk_ids, a.topk_w, a.T, a.H, a.E, a.k, a.out);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }

  // optional copies of the remaining intermediates, in pair order
  if (a.dbg_qx && (err = hipMemcpyAsync(a.dbg_qx, ws.qx, (size_t)a.T * a.H,
                                        hipMemcpyDeviceToDevice, stream)) != hipSuccess)
    return err;
  if (a.dbg_sx && (err = hipMemcpyAsync(a.dbg_sx, ws.sx, (size_t)a.T * 4,
                                        hipMemcpyDeviceToDevice, stream)) != hipSuccess)
    return err;
  if (a.dbg_act && (err = hipMemcpyAsync(a.dbg_act, ws.act, (size_t)P * a.I * 4,
                                         hipMemcpyDeviceToDevice, stream)) != hipSuccess)
    return err;
  return hipSuccess;
}

hipError_t launch_moe_forward(const MoeArgs& a, hipStream_t stream) {
  return a.packed ? moe_forward_impl<true>(a, stream) : moe_forward_impl<false>(a, stream);
}

}  // namespace w8a8
