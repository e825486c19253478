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

// The expert of one slot alone (E <= 256), from the lane's four logits
// (experts lane + 64 i): the rounds of route_select_sorted4 up to that slot,
// so the same selection.  A round whose maximum sits on one lane reads the
// expert there through a ballot; tied maxima take the second reduction.
// Lane s <= slot keeps round s's expert and logit in my_e, my_l, and mx gets
// the largest logit, so after k rounds route_slot_weight gives the weights.
__device__ __forceinline__ int route_slot_expert4(const float (&lv)[4], int E, int slot,
                                                  int lane, int& my_e, float& my_l,
                                                  double& mx) {
  uint32_t q[4];
  int ee[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    ee[i] = lane + 64 * i;
    q[i] = ee[i] < E ? float_key(lv[i]) : 0u;
  }
  order_pair(q[0], ee[0], q[1], ee[1]);
  order_pair(q[2], ee[2], q[3], ee[3]);
  order_pair(q[0], ee[0], q[2], ee[2]);
  order_pair(q[1], ee[1], q[3], ee[3]);
  order_pair(q[1], ee[1], q[2], ee[2]);
  int be = 0;
  my_e = 0;
  my_l = 0.0f;
  for (int s = 0; s <= slot; s++) {
    const uint32_t mh = wave_max_u32(q[0]);
    const uint64_t holders = __ballot(q[0] == mh);
    if (__popcll(holders) == 1)
      be = __builtin_amdgcn_readlane(ee[0], __ffsll((long long)holders) - 1);
    else
      be = (int)(0xffffffffu -
                 wave_max_u32(q[0] == mh ? 0xffffffffu - (uint32_t)ee[0] : 0u));
    if (s == 0) mx = (double)key_float(mh);
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
  return be;
}

// The renormalised weight of lane s's slot after k rounds of
// route_slot_expert4: the arithmetic of route_select_sorted4.
__device__ __forceinline__ float route_slot_weight(float my_l, double mx, int k) {
  const double myp = exp((double)my_l - mx);
  const uint64_t pb = (uint64_t)__double_as_longlong(myp);
  double kept = 0.0;
  for (int s = 0; s < k; s++) {
    const uint32_t plo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)pb, s);
    const uint32_t phi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(pb >> 32), s);
    kept += __longlong_as_double((long long)(((uint64_t)phi << 32) | plo));
  }
  return (float)(myp / kept);
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
  return sc < 0x1p-100f ? quant_code(x, sc) : quant_code_recip(x, sc, rc);
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
    const int8_t* ap = qx + (int64_t)(pair_lds[a_ok ? j : 0] / k) * K + g * 16;  // k = 1: qa rows
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
  // wave 0 finds this workgroup's expert (the selection is a chain of
  // wave-wide maximum rounds, slot + 1 of them up to 256 experts; on every
  // wave it would fill the SIMDs); the others wait at the barrier
  __shared__ int e_lds;
  int sel_e = 0;
  float sel_w = 0.0f;
  const bool few = E <= 256;
  float my_l = 0.0f;
  double mx = 0.0;
  if (wv == 0) {
    int es;
    if (few) {
      float lv[4];
#pragma unroll
      for (int i = 0; i < 4; i++) lv[i] = logits[min(lane + 64 * i, E - 1)];
      es = route_slot_expert4(lv, E, slot, lane, sel_e, my_l, mx);
    } else {
      route_select(logits, E, k, lane, sel_e, sel_w);
      es = __shfl(sel_e, slot, 64);
    }
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
  // the routing weights (workgroup (0, k - 1), which ran all k rounds), with
  // the weight loads already out
  if (few && wv == 0 && tile == 0 && slot == k - 1) sel_w = route_slot_weight(my_l, mx, k);

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
      if (slot == 0 && lane == 0) {
        n_active[0] = k;
        seg_off[k] = k;
        sx[0] = sxv;
      }
      if (slot == k - 1 && lane < k) {
        topk_ids[lane] = sel_e;
        topk_w[lane] = sel_w;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// One routed token: requant, gemm2 and the weighted combine in one launch.
// Workgroup = 16 output columns (HALF: 8 of them, two workgroups per 16-row
// weight tile); wave w takes slot w (and w + 8): it
// requantises the pair's activation row from the partial maxima gemm1 left,
// multiplies it with the 16 rows of its expert's w2 (all of K = I on the one
// wave), and puts the dequantised y2 values in LDS.  Wave 0 then forms
// out = bf16(sum over slots of w_s * y2_s) in fp32, slot order, no FMA --
// the combine of k_moe_combine -- without y2 going through memory.
// ---------------------------------------------------------------------------
template <bool PACKED, bool HALF>
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
  // HALF: the workgroup takes 8 of a 16-column weight tile's columns (twice
  // the workgroups); lanes of the other 8 columns load nothing
  const int tile = HALF ? (int)blockIdx.x >> 1 : (int)blockIdx.x;
  const bool mine = !HALF || (j >> 3) == (int)(blockIdx.x & 1);
  const int nk = I >> 6;
  for (int sl = wv; sl < k; sl += WAVES) {
    const int e = __builtin_amdgcn_readfirstlane(ids[sl]);
    const int8_t* wbase = PACKED ? W2 + ((int64_t)e * (H >> 4) + tile) * nk * 1024 + lane * 16
                                 : W2 + ((int64_t)e * H + tile * 16 + j) * I + g * 16;
    constexpr int64_t wstep = PACKED ? 1024 : 64;
    const int col = tile * 16 + j;
    const float swc = mine ? s2[(int64_t)e * H + col] : 0.0f;
    // the first U weight steps go out before the requantisation
    v4i b0[U];
#pragma unroll
    for (int u = 0; u < U; u++)
      b0[u] = (mine && u < nk) ? ld_stream(wbase + u * wstep) : v4i{0, 0, 0, 0};
    // the pair's |act| maximum from gemm1's partial maxima (non-negative
    // fp32 bit patterns), then its scale
    uint32_t mb = 0u;
    for (int i = lane; i < parts; i += 64) mb = max(mb, amax_part[(int64_t)sl * parts + i]);
    mb = wave_max_u32(mb);
    const float am = __uint_as_float(mb);
    const float sc = am != 0.0f ? am / 127.0f : 0.0f;
    // the row's codes, four per lane at a time, into this wave's LDS row
    // (after the previous slot's reads of that row)
    int8_t* qrow = qa_lds[wv];
    wave_lds_sync();
    for (int i = lane * 4; i < I; i += 256) {
      const v4f v = *reinterpret_cast<const v4f*>(act + (int64_t)sl * I + i);
      uint32_t wd = 0u;
      if (sc != 0.0f)
        wd = pack4_i8(quant_code(v.x, sc), quant_code(v.y, sc), quant_code(v.z, sc),
                      quant_code(v.w, sc));
      *reinterpret_cast<uint32_t*>(qrow + i) = wd;
      if (dbg_qa && blockIdx.x == 0)
        *reinterpret_cast<uint32_t*>(dbg_qa + (int64_t)sl * I + i) = wd;
    }
    wave_lds_sync();  // lanes j == 0 read codes other lanes stored
    v4i acc = {0, 0, 0, 0};
    for (int c0 = 0; c0 < nk; c0 += U) {
      v4i b[U], a[U];
#pragma unroll
      for (int u = 0; u < U; u++) {
        const int c = c0 + u;
        b[u] = c0 == 0 ? b0[u]
                       : ((mine && c < nk) ? ld_stream(wbase + c * wstep) : v4i{0, 0, 0, 0});
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
    if (g == 0 && mine) {
      float y = (float)acc[0];
      y = y * sc;
      y = y * swc;
      ybuf[sl][j] = y;
      if (dbg_acc) dbg_acc[(int64_t)sl * H + col] = acc[0];
    }
    if (dbg_sa2 && blockIdx.x == 0 && lane == 0) dbg_sa2[sl] = sc;
  }
  __syncthreads();
  if (wv == 0 && lane < 16 && mine) {
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
// Workgroup b covers token b / nbh, columns 1024 * (b % nbh) .. +1023 (the
// tokens sit on grid.x, whose range covers every accepted T).
__global__ __launch_bounds__(256) void k_moe_combine(const float* __restrict__ y2,
                                                     const int32_t* __restrict__ ids,
                                                     const float* __restrict__ w, int T, int H,
                                                     int E, int k, int nbh,
                                                     const float* __restrict__ shared,
                                                     uint16_t* __restrict__ out) {
  const int t = blockIdx.x / nbh;
  const int c = ((blockIdx.x - t * nbh) * 256 + threadIdx.x) * 4;
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
  if (shared) {  // the shared expert's output, after the routed sum
    const v4f y = *reinterpret_cast<const v4f*>(shared + (int64_t)t * H + c);
    acc.x = acc.x + y.x;
    acc.y = acc.y + y.y;
    acc.z = acc.z + y.z;
    acc.w = acc.w + y.w;
  }
  const uint32_t lo = f32_to_bf16_bits(acc.x) | (f32_to_bf16_bits(acc.y) << 16);
  const uint32_t hi = f32_to_bf16_bits(acc.z) | (f32_to_bf16_bits(acc.w) << 16);
  uint32_t* o = reinterpret_cast<uint32_t*>(out + (int64_t)t * H + c);
  o[0] = lo;
  o[1] = hi;
}

// ---------------------------------------------------------------------------
// Hadamard-domain routed experts and shared expert (the IQ8R container's
// format).  Source: "Qwen3.6-35B-A3B IQ8R - radiance container", Experts
// row (the routed experts int8 on the rotated grid with a bf16 scale per row
// and 128 of K; the shared expert likewise, its gate/up projection as the
// trunk's linears) and Activations row (int8 under the same rotation, the
// experts reading the codes the trunk's quantisers write); the routed order
// of the ATOM pull request's fused_moe_triton.py bullet.
//   - x is quantised under the fwht128 rotation, once per token;
//   - a g128 GEMM output is the sum over the 128-groups, in group order, of
//     the exact int32 group sum times the group's bf16 scale, in fp64, times
//     the row scale and 2^-7 (undoing <Hx, Hw> = 128 <x, w>), rounded to fp32;
//   - the gemm1 activation row is rotated by fwht128 before its per-row
//     requant (the down weights are rotated along their K);
//   - the combine adds the shared expert's fp32 output after the routed sum.
// ---------------------------------------------------------------------------

__device__ __forceinline__ void load8_f32(const uint16_t* __restrict__ p, float* v) {
  const v4u raw = *reinterpret_cast<const v4u*>(p);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    v[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
    v[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
  }
}

__device__ __forceinline__ void load8_f32(const float* __restrict__ p, float* v) {
  const v4f lo = *reinterpret_cast<const v4f*>(p);
  const v4f hi = *reinterpret_cast<const v4f*>(p + 4);
  v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
  v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
}

// One wave rotates a row of K values (K % 128 == 0, K <= 512 NR): round rd
// holds 128-blocks 4 rd .. 4 rd + 3, 16 lanes a block, 8 values a lane (the
// lane's values are k = 128 blk + 8 (lane % 16) + 0..7).  fp32 butterflies as
// k_fwht128_quant; returns the wave-wide maximum |value| of the rotated row.
template <int NR, typename TIn>
__device__ __forceinline__ float rot_row_wave(const TIn* __restrict__ x, int K, Block8 (&b)[NR],
                                              int lane) {
  const int l16 = lane & 15;
  const int nblk = K >> 7;
  float amax = 0.0f;
#pragma unroll
  for (int rd = 0; rd < NR; rd++) {
    const int blk = rd * 4 + (lane >> 4);
    if (blk < nblk) {
      load8_f32(x + blk * 128 + l16 * 8, b[rd].v);
    } else {
#pragma unroll
      for (int c = 0; c < 8; c++) b[rd].v[c] = 0.0f;
    }
    if (rd * 4 < nblk) {  // wave-uniform: every lane joins the butterflies
      fwht128_lanes(b[rd], l16);
#pragma unroll
      for (int c = 0; c < 8; c++) amax = fmaxf(amax, fabsf(b[rd].v[c]));
    }
  }
  return wave_max(amax);
}

// The int8 codes of one lane's 8 rotated values against s = amax / 127
// (all zero for a zero row), packed little-endian.
__device__ __forceinline__ uint2 rot_codes8(const Block8& b, float amax, float sc) {
  int cd[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (amax != 0.0f) {
#pragma unroll
    for (int c = 0; c < 8; c++) cd[c] = quant_code(b.v[c], sc);
  }
  return make_uint2(pack4_i8(cd[0], cd[1], cd[2], cd[3]), pack4_i8(cd[4], cd[5], cd[6], cd[7]));
}

// One wave rotates and quantises one row (bf16 or fp32) into row-major codes.
template <int NR, typename TIn>
__device__ __forceinline__ void rot_quant_row_wave(const TIn* __restrict__ x, int K,
                                                   int8_t* __restrict__ q,
                                                   float* __restrict__ s, int lane) {
  Block8 b[NR];
  const float amax = rot_row_wave<NR>(x, K, b, lane);
  const float sc = amax / 127.0f;
  const int nblk = K >> 7;
#pragma unroll
  for (int rd = 0; rd < NR; rd++) {
    const int blk = rd * 4 + (lane >> 4);
    if (blk < nblk)
      *reinterpret_cast<uint2*>(q + blk * 128 + (lane & 15) * 8) = rot_codes8(b[rd], amax, sc);
  }
  if (lane == 0) s[0] = amax != 0.0f ? sc : 0.0f;
}

// Routing and the rotated per-token quant of x (H <= 4096): workgroup b takes
// tokens 4b..4b+3; waves 0-3 route them (when logits are given) while waves
// 4-7 rotate and quantise them.
__global__ __launch_bounds__(512) void k_rot_route_quant(
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
    rot_quant_row_wave<8>(x + (int64_t)t * H, H, qx + (int64_t)t * H, sx + t, lane);
  }
}

// Rotated requant of fp32 activation rows (K <= 2048), one wave a row.
__global__ __launch_bounds__(512) void k_rot_requant(const float* __restrict__ act, int64_t P,
                                                     int K, int8_t* __restrict__ qa,
                                                     float* __restrict__ sa) {
  const int64_t r = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 6);
  if (r >= P) return;
  rot_quant_row_wave<4>(act + r * K, K, qa + r * K, sa + r, threadIdx.x & 63);
}

// The epilogues of the rotated-expert GEMMs.
enum { kRotSilu = 1, kRotActRot = 2, kRotG256Silu = 3, kRotCodes = 4, kRotG256SiluX = 5 };

// Which input rows a workgroup's pair block reads: expert slot grouping (the
// sorted pairs of one expert) or, in the dense form (expert_list == nullptr),
// rows [rows_per_y blockIdx.y, +rows_per_y) of a plain matrix (pair p = row p).
struct RotRows {
  int e, begin, end;
};

__device__ __forceinline__ bool rot_rows(const int32_t* __restrict__ expert_list,
                                         const int32_t* __restrict__ seg_off,
                                         const int32_t* __restrict__ n_active, int dense_rows,
                                         int rows_per_y, RotRows& rr) {
  if (expert_list == nullptr) {
    rr.e = 0;
    rr.begin = blockIdx.y * rows_per_y;
    rr.end = min(dense_rows, rr.begin + rows_per_y);
    return true;
  }
  const int slot = blockIdx.y;
  if (slot >= n_active[0]) return false;
  rr.e = expert_list[slot];
  rr.begin = seg_off[slot];
  rr.end = seg_off[slot + 1];
  return true;
}

// SiLU(gate) * up over the interleaved columns (even = gate, odd = up), the
// pair sharing lanes j and j ^ 1; every lane must call it (it shuffles).
__device__ __forceinline__ float rot_silu_pair(float h) {
  const float partner = __shfl_xor(h, 1, 64);
  const float sg = (float)((double)h / (1.0 + exp(-(double)h)));
  return sg * partner;
}

// Decodes a bf16 scale as m * 2^x with m a signed integer (|m| <= 255);
// returns false for Inf / NaN.
__device__ __forceinline__ bool bf16_int_exp(uint32_t bits, int& m, int& x) {
  const int ef = (bits >> 7) & 0xff;
  const int f = bits & 0x7f;
  if (ef == 0xff) return false;
  m = ef == 0 ? f : 128 + f;
  x = ef == 0 ? -133 : ef - 134;
  if (bits & 0x8000u) m = -m;
  return true;
}

// The exact integer form of one column's g128 fold.  The definition sums
// double(acc_g) * double(s_g) over the 128-groups in order, in fp64.  With
// s_g = m_g 2^x_g (m_g an integer, |m_g| <= 255) and xm the least x_g of the
// column's non-zero scales, every term is an integer multiple of 2^xm; if
// D = sum_g |m_g| 2^(x_g - xm) < 2^31, every partial sum is an integer of
// magnitude below 2^21 D < 2^52 times 2^xm (|acc_g| <= 128^3), so each fp64
// addition is exact and the sum equals S 2^xm with S = sum_g acc_g M_g,
// M_g = m_g 2^(x_g - xm), exact in int64 in any order.  Writes M_g and the
// fp32 scales of the column's G (<= MAXG) groups, 2^xm, and whether the
// integer form applies.  The scales come in with independent loads.
template <int MAXG>
__device__ __forceinline__ void rot_col_scales(const uint16_t* __restrict__ sp, int G,
                                               int32_t* m_out, float* s_out, float& cs,
                                               bool& ok) {
  uint32_t bits[MAXG];
#pragma unroll
  for (int gg = 0; gg < MAXG; gg++) bits[gg] = gg < G ? sp[gg] : 0u;
  int mm[MAXG], xx[MAXG];
  int xm = 1 << 20;
  ok = true;
#pragma unroll
  for (int gg = 0; gg < MAXG; gg++) {
    mm[gg] = 0;
    xx[gg] = 0;
    if (gg < G) {
      s_out[gg] = bf16_bits_to_f32(bits[gg]);
      if (!bf16_int_exp(bits[gg], mm[gg], xx[gg])) {
        ok = false;
        mm[gg] = 0;
      } else if (mm[gg] != 0) {
        xm = min(xm, xx[gg]);
      }
    }
  }
  if (xm == (1 << 20)) xm = 0;
  long long D = 0;
#pragma unroll
  for (int gg = 0; gg < MAXG; gg++) {
    if (gg < G) {
      int Mg = 0;
      if (mm[gg] != 0) {
        const int sh = xx[gg] - xm;
        if (sh > 23) {
          ok = false;
        } else {
          Mg = mm[gg] * (1 << sh);
          D += Mg < 0 ? -(long long)Mg : (long long)Mg;
        }
      }
      m_out[gg] = Mg;
    }
  }
  if (D >= (1LL << 31)) ok = false;
  cs = ldexpf(1.0f, xm);
}

// Grouped GEMM with per-group scales, split over K (small batches).  The
// workgroup takes one 16-column tile of one weight matrix (blockIdx.x) and
// its pair rows in blocks of 16; wave w takes the 128-groups w, w + WAVES, ...
// (two 16x16x64 MFMA steps each).  For g128 the waves leave every group's
// int32 sums in LDS and the fold walks the groups in order in fp64, as
// defined; for g256 each wave adds su8 * acc into int64 sums as its groups
// complete and the waves' sums are added through LDS (exact, so the order is
// free).  The epilogue runs on four waves, one output row of each lane's
// four a wave:
//   kRotSilu:     h = (float)(t sx 2^-7), t the fold; SiLU(gate) * up ->
//                 fp32 activation [pair, c / 2];
//   kRotActRot:   the prologue rotates each pair's fp32 activation row, takes
//                 its per-row scale and writes its codes into LDS in the
//                 packed operand layout; y = (float)(t sa 2^-7) -> fp32;
//   kRotCodes:    as kRotActRot with the rotated codes and scales given
//                 (qx = qa [P, K], sx = sa [P], k = 1);
//   kRotG256Silu: T = sum over 256-groups of su8 (acc_2g + acc_2g+1), exact
//                 in int64; h = (float)(T sx s2 2^-7); SiLU(gate) * up;
//   kRotG256SiluX: as kRotG256Silu with the prologue rotating and
//                 quantising the bf16 token rows (act = x, K <= 2048) itself.
// W is packed (16-row tiles of 1 KiB k-steps), as [E * Nw, K].  In the dense
// form (expert_list == nullptr) the rows are [16 blockIdx.y, +16) of a
// plain matrix (pair p = row p).
template <int MODE, int WAVES, int NT, int MAXG>
__global__ __launch_bounds__(WAVES * 64) void k_rot_gemm_splitk(
    const int8_t* __restrict__ qx, const float* __restrict__ sx, const float* __restrict__ act,
    int k, const int8_t* __restrict__ W, const uint16_t* __restrict__ sW,
    const uint8_t* __restrict__ su8, int Nw, int K, const int32_t* __restrict__ expert_list,
    const int32_t* __restrict__ seg_off, const int32_t* __restrict__ n_active,
    const int32_t* __restrict__ sorted_pairs, int dense_rows, float* __restrict__ out, int ldo,
    int8_t* __restrict__ qa_rec, float* __restrict__ sa_rec) {
  constexpr int GW = (MAXG + WAVES - 1) / WAVES;  // groups a wave takes
  constexpr bool G256 = MODE == kRotG256Silu || MODE == kRotG256SiluX;
  constexpr bool ROT_IN = MODE == kRotActRot || MODE == kRotG256SiluX;  // rows rotated here
  // a group's int32 sums, element v of lane l at [v][l] (the fold reads one
  // element of 64 consecutive lanes: no bank conflicts)
  __shared__ int32_t red[G256 ? 1 : NT][G256 ? 1 : MAXG][4][64];
  __shared__ long long sred[G256 ? WAVES : 1][4][64];
  __shared__ int32_t m_lds[G256 ? 16 : 1][MAXG + 1];
  __shared__ float s_lds[NT * 16][MAXG + 1];
  __shared__ float cs_lds[16];
  __shared__ __attribute__((aligned(16))) int8_t a_lds[ROT_IN ? 16 * 2048 : 16];
  __shared__ float sa_lds[16];
  __shared__ int pair_lds[16];
  static_assert(!G256 || NT == 1, "the g256 form takes one tile a workgroup");
  RotRows rr;
  if (!rot_rows(expert_list, seg_off, n_active, dense_rows, 16, rr)) return;
  const bool dense = expert_list == nullptr;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int j = lane & 15;
  const int g = lane >> 4;
  const int nk = K >> 6;
  const int G = K >> 7;
  const int tile0 = blockIdx.x * NT;
  const int8_t* wbase = W + ((int64_t)rr.e * (Nw >> 4) + tile0) * nk * 1024 + lane * 16;
  const int64_t tstride = (int64_t)nk * 1024;

  // all of the workgroup's weight bytes go out at once
  v4i bw[NT][GW][2];
#pragma unroll
  for (int t = 0; t < NT; t++)
#pragma unroll
    for (int i = 0; i < GW; i++) {
      const int gg = wv + i * WAVES;
#pragma unroll
      for (int h = 0; h < 2; h++)
        bw[t][i][h] = gg < G ? ld_stream(wbase + t * tstride + (int64_t)(2 * gg + h) * 1024)
                             : v4i{0, 0, 0, 0};
    }
  if (G256) {
    if (threadIdx.x < 16) {
      const int c = threadIdx.x;
      const int col = tile0 * 16 + c;
      const uint8_t* sp = su8 + (int64_t)col * (K >> 8);
      uint32_t u[MAXG / 2];
#pragma unroll
      for (int i = 0; i < MAXG / 2; i++) u[i] = 2 * i < G ? sp[i] : 0u;
#pragma unroll
      for (int gg = 0; gg < MAXG; gg++)
        if (gg < G) m_lds[c][gg] = (int32_t)u[gg >> 1];
      cs_lds[c] = bf16_bits_to_f32(sW[col]);
    }
  } else {
    // the tiles' scales are contiguous: NT * 16 rows of G
    const uint16_t* sp = sW + ((int64_t)rr.e * Nw + tile0 * 16) * G;
    for (int i = threadIdx.x; i < NT * 16 * G; i += WAVES * 64) {
      const int cc = i / G, gg = i - cc * G;
      s_lds[cc][gg] = bf16_bits_to_f32(sp[i]);
    }
  }

  // the first 16 threads hold their row's pair and token scale of the next
  // block: those loads are in flight while the current block computes (rows
  // past nrows are never read back: outputs use row min(r, nrows - 1))
  int pid = 0;
  float sxv = 0.0f;
  if (threadIdx.x < 16 && rr.begin + (int)threadIdx.x < rr.end) {
    pid = dense ? rr.begin + (int)threadIdx.x : sorted_pairs[rr.begin + threadIdx.x];
    if (!ROT_IN) sxv = sx[pid / k];
  }
  for (int pb = rr.begin; pb < rr.end; pb += 16) {
    const int nrows = min(16, rr.end - pb);
    __syncthreads();  // the previous block's LDS consumed
    if (threadIdx.x < 16) {
      pair_lds[threadIdx.x] = (int)threadIdx.x < nrows ? pid : 0;
      if (!ROT_IN) sa_lds[threadIdx.x] = sxv;
      const int nx = pb + 16 + (int)threadIdx.x;
      if (nx < rr.end) pid = dense ? nx : sorted_pairs[nx];
    }
    __syncthreads();
    if (ROT_IN) {
      for (int r = wv; r < nrows; r += WAVES) {
        Block8 bb[4];
        const float am =
            MODE == kRotG256SiluX
                ? rot_row_wave<4>(reinterpret_cast<const uint16_t*>(act) + (int64_t)pair_lds[r] * K,
                                  K, bb, lane)
                : rot_row_wave<4>(act + (int64_t)pair_lds[r] * K, K, bb, lane);
        const float sc = am / 127.0f;
#pragma unroll
        for (int rd = 0; rd < 4; rd++) {
          const int blk = rd * 4 + g;
          if (blk >= G) continue;
          const uint2 wd = rot_codes8(bb[rd], am, sc);
          const int kk = blk * 128 + j * 8;  // first of the lane's 8 values
          *reinterpret_cast<uint2*>(a_lds + (kk >> 6) * 1024 + (r + 16 * ((kk & 63) >> 4)) * 16 +
                                    (kk & 15)) = wd;
          if (MODE == kRotActRot && blockIdx.x == 0 && qa_rec)
            *reinterpret_cast<uint2*>(qa_rec + (int64_t)pair_lds[r] * K + kk) = wd;
        }
        if (lane == 0) {
          const float sv = am != 0.0f ? sc : 0.0f;
          sa_lds[r] = sv;
          if (MODE == kRotActRot && blockIdx.x == 0 && sa_rec) sa_rec[pair_lds[r]] = sv;
        }
      }
    }
    if (ROT_IN) __syncthreads();

    // this wave's groups: the activation slices once, every tile's MFMAs
    const bool a_ok = j < nrows;
    const int8_t* ap = qx + (int64_t)(pair_lds[a_ok ? j : 0] / k) * K + g * 16;
    long long S[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < GW; i++) {
      const int gg = wv + i * WAVES;
      if (gg < G) {
        v4i a[2];
#pragma unroll
        for (int h = 0; h < 2; h++) {
          const int c = 2 * gg + h;
          if (ROT_IN)
            a[h] = *reinterpret_cast<const v4i*>(&a_lds[c * 1024 + lane * 16]);
          else
            a[h] = a_ok ? *reinterpret_cast<const v4i*>(ap + (int64_t)c * 64) : v4i{0, 0, 0, 0};
        }
#pragma unroll
        for (int t = 0; t < NT; t++) {
          v4i acc = {0, 0, 0, 0};
#pragma unroll
          for (int h = 0; h < 2; h++) acc = mfma_16x16x64_i8(a[h], bw[t][i][h], acc);
          if (G256) {
            const long long M = m_lds[j][gg];
#pragma unroll
            for (int v = 0; v < 4; v++) S[v] += (long long)acc[v] * M;
          } else {
#pragma unroll
            for (int v = 0; v < 4; v++) red[t][gg][v][lane] = acc[v];
          }
        }
      }
    }
    if (G256) {
#pragma unroll
      for (int v = 0; v < 4; v++) sred[wv][v][lane] = S[v];
    }
    // the next block's token scales (its pairs have arrived by now)
    if (!ROT_IN && threadIdx.x < 16 && pb + 16 + (int)threadIdx.x < rr.end) sxv = sx[pid / k];
    __syncthreads();
    // (tile, element) units over the waves: element v of every lane is row
    // 4 (lane / 16) + v, column 16 (tile0 + t) + lane % 16
    for (int u = wv; u < NT * 4; u += WAVES) {
      const int t = u >> 2, v = u & 3;
      const int r = 4 * g + v;
      const int rc = min(r, nrows - 1);
      const int col = (tile0 + t) * 16 + j;
      double tt;
      if (G256) {
        long long tot = 0;
#pragma unroll
        for (int w = 0; w < WAVES; w++) tot += sred[w][v][lane];
        tt = (double)tot * (double)sa_lds[rc];
        tt = tt * (double)cs_lds[j];
      } else {
        tt = 0.0;
        for (int gg = 0; gg < G; gg++)
          tt = tt + (double)red[t][gg][v][lane] * (double)s_lds[t * 16 + j][gg];
        tt = tt * (double)sa_lds[rc];
      }
      tt = tt * 0.0078125;
      const float hv = (float)tt;
      const int p = pair_lds[rc];
      if (MODE == kRotActRot || MODE == kRotCodes) {
        if (r < nrows) out[(int64_t)p * ldo + col] = hv;
      } else {
        const float a = rot_silu_pair(hv);
        if ((j & 1) == 0 && r < nrows) out[(int64_t)p * ldo + (col >> 1)] = a;
      }
    }
  }
}

// Grouped g128 GEMM for large batches (gemm1 with the SiLU epilogue, or gemm2
// on given rotated codes), one wave per 16-row weight tile holding all of K
// of it in registers (NKMAX 1 KiB k steps), so the group sums never leave the
// wave: each 128-group's two MFMA steps are folded into fp64 sums right away,
// in group order, as defined.  Workgroup = four waves = four consecutive tiles
// of one expert; the expert's pair rows come in blocks of 16, each block's
// activation codes gathered straight into LDS (buffer loads to LDS, lane l =
// row l % 16, 16-byte k slice l / 16: the MFMA operand layout) one block
// ahead in two buffers, one barrier a block.  Every lane loads its row's pair
// id two blocks ahead and its token scale one block ahead; a block starts
// with a wait for every vector memory operation in flight (its copies, those
// loads, the stores of the block before last), so nothing that block uses
// waits again.
template <int MODE, int NKMAX, bool DENSE = false>
__global__ __launch_bounds__(256, 2) void k_rot_gemm_kw(
    const int8_t* __restrict__ qx, const float* __restrict__ sx, int k,
    const int8_t* __restrict__ W, const uint16_t* __restrict__ sW,
    const uint8_t* __restrict__ su8, int Nw, int K, int qx_rows,
    const int32_t* __restrict__ expert_list, const int32_t* __restrict__ seg_off,
    const int32_t* __restrict__ n_active, const int32_t* __restrict__ sorted_pairs,
    int rows_per_y, float* __restrict__ out, int ldo) {
  // g128 (kRotSilu, kRotCodes): the fold of the definition, fp64 in group
  // order; kRotG256Silu (the shared expert's gate/up): each 256-group's exact
  // int32 sum times its u8 scale into int64 sums, any order being exact
  constexpr bool G256 = MODE == kRotG256Silu;
  constexpr int GMAX = NKMAX / 2;
  __shared__ __attribute__((aligned(1024))) int8_t a_lds[2][NKMAX * 1024];
  RotRows rr;
  // DENSE: one plain matrix (expert_list null), rows_per_y token rows a
  // workgroup row; else one expert's segment of sorted pairs
  if (!rot_rows(DENSE ? nullptr : expert_list, seg_off, n_active, qx_rows,
                DENSE ? rows_per_y : 16, rr))
    return;
  const int nrows_all = rr.end - rr.begin;
  if (nrows_all <= 0) return;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int j = lane & 15;
  const int g = lane >> 4;
  const int nk = K >> 6;
  const int G = K >> 7;
  const int tile = blockIdx.x * 4 + wv;
  const int col = tile * 16 + j;

  // the wave's tile, all of K (streamed past the caches when one call reads
  // it once; a dense matrix is read again by every workgroup row), and the
  // lane's column scales (indices clamped, no branch between the loads)
  const int8_t* wb = W + ((int64_t)rr.e * (Nw >> 4) + tile) * nk * 1024 + lane * 16;
  v4i bw[NKMAX];
#pragma unroll
  for (int c = 0; c < NKMAX; c++) {
    const int8_t* pc = wb + (int64_t)min(c, nk - 1) * 1024;
    bw[c] = DENSE ? *reinterpret_cast<const v4i*>(pc) : ld_stream(pc);
  }
  float sv[GMAX];
  if constexpr (G256) {
    const uint8_t* up = su8 + (int64_t)col * (K >> 8);
#pragma unroll
    for (int gg = 0; gg < GMAX; gg++) sv[gg] = (float)up[min(gg, (K >> 8) - 1)];
  } else {
    const uint16_t* sp = sW + ((int64_t)rr.e * Nw + col) * G;
#pragma unroll
    for (int gg = 0; gg < GMAX; gg++) sv[gg] = bf16_bits_to_f32(sp[min(gg, G - 1)]);
  }
  const float s2c = G256 ? bf16_bits_to_f32(sW[col]) : 0.0f;

  const int nblk = (nrows_all + 15) >> 4;
  const __amdgpu_buffer_rsrc_t qrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)qx, 0, qx_rows * K, 0x00020000);
  // block b's pair of row j (rows past the segment end repeat its last pair)
  auto pair_of = [&](int b) __attribute__((always_inline)) {
    const int r = min(rr.begin + 16 * b + j, rr.end - 1);
    return DENSE ? r : sorted_pairs[r];
  };
  // block b's codes into buffer b & 1: wave w copies k steps w, w + 4, ...
  auto copy = [&](int b, int p) __attribute__((always_inline)) {
    int8_t* dst = a_lds[b & 1];
    const int voff = (p / k) * K + 16 * g;
    for (int c = wv; c < nk; c += 4)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          qrs, (__attribute__((address_space(3))) void*)(dst + c * 1024), 16, voff + c * 64, 0,
          0, 0);
  };
  auto store = [&](const float (&res)[4], int p_blk, int nrows) __attribute__((always_inline)) {
#pragma unroll
    for (int v = 0; v < 4; v++) {
      const int r = 4 * g + v;
      const int p = __shfl(p_blk, r, 64);
      if (r < nrows) {
        if (MODE != kRotCodes) {
          if ((j & 1) == 0) out[(int64_t)p * ldo + (col >> 1)] = res[v];
        } else {
          out[(int64_t)p * ldo + col] = res[v];
        }
      }
    }
  };
  int p_cur = pair_of(0), p_prev = 0;
  float s_cur = sx[p_cur / k];
  copy(0, p_cur);
  int p_nxt = pair_of(1);
  float res[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int b = 0; b < nblk; b++) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __builtin_amdgcn_s_barrier();
    if (b > 0) store(res, p_prev, min(16, nrows_all - 16 * (b - 1)));
    if (b + 1 < nblk) copy(b + 1, p_nxt);
    const int p_nn = pair_of(b + 2);
    const float s_nxt = sx[p_nxt / k];
    // block b: every group's two k steps, then the fold, in group order
    const int nrows = min(16, nrows_all - 16 * b);
    const int8_t* ab = a_lds[b & 1] + lane * 16;
    double tt[4] = {0.0, 0.0, 0.0, 0.0};
    if constexpr (G256) {
      long long S[4] = {0, 0, 0, 0};
#pragma unroll
      for (int gq = 0; gq < GMAX / 2; gq++) {
        if (4 * gq < nk) {
          v4i acc = {0, 0, 0, 0};
#pragma unroll
          for (int h = 0; h < 4; h++)
            acc = mfma_16x16x64_i8(*reinterpret_cast<const v4i*>(ab + (4 * gq + h) * 1024),
                                   bw[4 * gq + h], acc);
          // |acc| <= 256 * 127^2, so acc * u8 < 2^31 is exact in int32
          const int u8 = (int)sv[gq];
#pragma unroll
          for (int v = 0; v < 4; v++) S[v] += (long long)(acc[v] * u8);
        }
      }
#pragma unroll
      for (int v = 0; v < 4; v++) tt[v] = (double)S[v];
    } else {
#pragma unroll
      for (int gg = 0; gg < GMAX; gg++) {
        if (gg < G) {
          v4i acc = {0, 0, 0, 0};
          acc = mfma_16x16x64_i8(*reinterpret_cast<const v4i*>(ab + (2 * gg) * 1024),
                                 bw[2 * gg], acc);
          acc = mfma_16x16x64_i8(*reinterpret_cast<const v4i*>(ab + (2 * gg + 1) * 1024),
                                 bw[2 * gg + 1], acc);
#pragma unroll
          for (int v = 0; v < 4; v++) tt[v] = tt[v] + (double)acc[v] * (double)sv[gg];
        }
      }
    }
#pragma unroll
    for (int v = 0; v < 4; v++) {
      const float sa = __shfl(s_cur, min(4 * g + v, nrows - 1), 64);
      double t = tt[v] * (double)sa;
      if (G256) t = t * (double)s2c;
      t = t * 0.0078125;
      const float hv = (float)t;
      res[v] = MODE == kRotCodes ? hv : rot_silu_pair(hv);
    }
    p_prev = p_cur;
    p_cur = p_nxt;
    s_cur = s_nxt;
    p_nxt = p_nn;
  }
  store(res, p_prev, nrows_all - 16 * (nblk - 1));
}

// A single token in the Hadamard domain: two launches.  k_rot_t1_gemm1 fuses
// the routing and the rotated quant of x into gemm1 (every workgroup repeats
// them: wave 0 routes, wave 1 rotates and quantises the row into LDS; the
// first workgroup also writes the routing and the codes out), then folds
// its pair's 16 columns as k_rot_gemm_splitk.  k_rot_t1_gemm2 takes 16
// output columns for all k pairs: its prologue rotates and requantises the
// k activation rows into LDS, each (pair, group) unit runs the two MFMA
// steps of that pair's expert, the fold gives y2 for every pair, and the
// epilogue combines them in slot order (plus the shared term) into bf16 out.
// SH: with the shared expert's gate/up tiles as workgroup row k; the
// register budget then allows six waves a SIMD (three workgroups a CU: the
// shared tiles come on top of the routed ones)
template <bool SH>
__global__ __launch_bounds__(512, SH ? 6 : 1) void k_rot_t1_gemm1(
    const uint16_t* __restrict__ x, const float* __restrict__ logits, int H, int E, int k,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_w, const int8_t* __restrict__ W,
    const uint16_t* __restrict__ sW, int Nw, int8_t* __restrict__ qx_rec,
    float* __restrict__ sx_rec, float* __restrict__ act, int I,
    const int8_t* __restrict__ Wsh, const uint8_t* __restrict__ su8sh,
    const uint16_t* __restrict__ s2sh, int Nsh, float* __restrict__ act_sh) {
  constexpr int WAVES = 8, MAXG = 32, GW = MAXG / WAVES;
  __shared__ v4i red[MAXG][64];
  __shared__ float s_lds[16][MAXG];
  __shared__ __attribute__((aligned(16))) int8_t q_lds[4096];
  __shared__ float sx_lds;
  __shared__ int e_lds;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int j = lane & 15;
  const int g = lane >> 4;
  const int tile = blockIdx.x, slot = blockIdx.y;
  const int nk = H >> 6;
  const int G = H >> 7;
  const bool first = tile == 0 && slot == 0;
  // workgroup row k (with Wsh): the shared expert's gate/up (g256), one
  // 16-row tile a workgroup, beside the routed pairs' tiles
  const bool sh = SH && slot == k;
  if (tile >= (sh ? Nsh : Nw) >> 4) return;  // the wider of the two sets the grid
  // up to 256 experts each workgroup finds its slot's expert alone; workgroup
  // (0, k - 1), which ran all k rounds, writes the selection
  const bool few = logits && E <= 256;
  int sel_e = 0;
  float my_l = 0.0f;
  double mx = 0.0;
  if (wv == 0 && !sh) {
    float sel_w = 0.0f;
    int es;
    if (few) {
      float lv[4];
#pragma unroll
      for (int i = 0; i < 4; i++) lv[i] = logits[min(lane + 64 * i, E - 1)];
      es = route_slot_expert4(lv, E, slot, lane, sel_e, my_l, mx);
    } else {
      if (logits) {
        route_select(logits, E, k, lane, sel_e, sel_w);
        if (first && lane < k) {
          topk_ids[lane] = sel_e;
          topk_w[lane] = sel_w;
        }
      } else {
        sel_e = lane < k ? topk_ids[lane] : 0;
      }
      es = __shfl(sel_e, slot, 64);
    }
    if (lane == 0) e_lds = es;
  } else if (wv == 1) {
    rot_quant_row_wave<8>(x, H, q_lds, &sx_lds, lane);
  }
  __syncthreads();
  const int e = sh ? 0 : __builtin_amdgcn_readfirstlane(e_lds);
  const int8_t* wbase = sh ? Wsh + (int64_t)tile * nk * 1024 + lane * 16
                           : W + ((int64_t)e * (Nw >> 4) + tile) * nk * 1024 + lane * 16;
  v4i bw[GW][2];
#pragma unroll
  for (int i = 0; i < GW; i++) {
    const int gg = wv + i * WAVES;
#pragma unroll
    for (int h = 0; h < 2; h++)
      bw[i][h] = gg < G ? ld_stream(wbase + (int64_t)(2 * gg + h) * 1024) : v4i{0, 0, 0, 0};
  }
  if (sh) {
    // the tile's u8 scales per 256-group (exact as floats) and row scales
    const int G2 = H >> 8;
    for (int i = threadIdx.x; i < 16 * G2; i += WAVES * 64) {
      const int cc = i / G2, gg = i - cc * G2;
      s_lds[cc][gg] = (float)su8sh[(int64_t)(tile * 16 + cc) * G2 + gg];
    }
    if (threadIdx.x < 16) s_lds[threadIdx.x][MAXG - 1] = bf16_bits_to_f32(s2sh[tile * 16 + threadIdx.x]);
  } else {
    for (int i = threadIdx.x; i < 16 * G; i += WAVES * 64) {
      const int cc = i / G, gg = i - cc * G;
      s_lds[cc][gg] = bf16_bits_to_f32(sW[((int64_t)e * Nw + tile * 16 + cc) * G + gg]);
    }
  }
  if (few && tile == 0 && slot == k - 1 && wv == 0) {
    const float sel_w = route_slot_weight(my_l, mx, k);
    if (lane < k) {
      topk_ids[lane] = sel_e;
      topk_w[lane] = sel_w;
    }
  }
  if (first && qx_rec) {
    for (int i = threadIdx.x; i < (H >> 4); i += WAVES * 64)
      *reinterpret_cast<v4i*>(qx_rec + i * 16) = *reinterpret_cast<const v4i*>(q_lds + i * 16);
    if (threadIdx.x == 0) sx_rec[0] = sx_lds;
  }
  // the token is row 0 of the A tile (lanes with j == 0 feed it)
#pragma unroll
  for (int i = 0; i < GW; i++) {
    const int gg = wv + i * WAVES;
    if (gg < G) {
      v4i acc = {0, 0, 0, 0};
#pragma unroll
      for (int h = 0; h < 2; h++) {
        const int c = 2 * gg + h;
        const v4i a = j == 0 ? *reinterpret_cast<const v4i*>(q_lds + c * 64 + g * 16)
                             : v4i{0, 0, 0, 0};
        acc = mfma_16x16x64_i8(a, bw[i][h], acc);
      }
      red[gg][lane] = acc;
    }
  }
  __syncthreads();
  if (wv != 0) return;
  // row 0 of column tile * 16 + j sits in element 0 of lane j (g == 0)
  double t = 0.0;
  if (sh) {
    // g256: each 128-group's exact sum times its 256-group's u8, in int64
    // (exact, so in any order), then * sx * s2 * 2^-7 in fp64
    long long tot = 0;
    for (int gg = 0; gg < G; gg++)
      tot += (long long)red[gg][j][0] * (long long)s_lds[j][gg >> 1];
    t = (double)tot * (double)sx_lds;
    t = t * (double)s_lds[j][MAXG - 1];
  } else {
    for (int gg = 0; gg < G; gg++) t = t + (double)red[gg][j][0] * (double)s_lds[j][gg];
    t = t * (double)sx_lds;
  }
  t = t * 0.0078125;
  const float a = rot_silu_pair((float)t);
  if (g == 0 && (j & 1) == 0) {
    if (sh)
      act_sh[(tile * 16 + j) >> 1] = a;
    else
      act[(int64_t)slot * I + ((tile * 16 + j) >> 1)] = a;
  }
}

// k * (I / 128) <= kRotT1MaxUnits (pair, group) units; I <= 1024
constexpr int kRotT1MaxUnits = 64;

template <bool SH>
__global__ __launch_bounds__(512) void k_rot_t1_gemm2(
    const float* __restrict__ act, int I, int k, const int32_t* __restrict__ topk_ids,
    const float* __restrict__ topk_w, const int8_t* __restrict__ W,
    const uint16_t* __restrict__ sW, int H, const float* __restrict__ shared,
    uint16_t* __restrict__ out, int8_t* __restrict__ qa_rec, float* __restrict__ sa_rec,
    const float* __restrict__ act_sh, int Is, const int8_t* __restrict__ Wdsh,
    const uint16_t* __restrict__ sdsh) {
  constexpr int WAVES = 8, UW = kRotT1MaxUnits / WAVES;
  __shared__ v4i red[kRotT1MaxUnits][64];
  __shared__ __attribute__((aligned(16))) int8_t a_lds[16 * 1024];
  __shared__ float s_lds[kRotT1MaxUnits][16];
  __shared__ float sa_lds[16], w_lds[16], y_lds[16][16];
  __shared__ int e_lds[16];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int j = lane & 15;
  const int g = lane >> 4;
  const int tile = blockIdx.x;
  const int nk = I >> 6;
  const int G = I >> 7;
  // with act_sh: the shared expert's down projection as pair k (its own
  // weights, scales and row length), its y added after the slot-order sum
  constexpr bool has_sh = SH;
  const int Gs = has_sh ? Is >> 7 : 0;
  const int U0 = k * G;     // the routed pairs' (pair, group) units
  const int U = U0 + Gs;    // then the shared pair's
  const int rows = k + (has_sh ? 1 : 0);
  if (threadIdx.x < k) {
    e_lds[threadIdx.x] = topk_ids[threadIdx.x];
    w_lds[threadIdx.x] = topk_w[threadIdx.x];
  }
  __syncthreads();
  // the weight fragments of this wave's (pair, group) units
  v4i bw[UW][2];
#pragma unroll
  for (int i = 0; i < UW; i++) {
    const int u = wv + i * WAVES;
    const bool routed = u < U0;
    const int pr = routed ? u / G : 0;
    const int gg = routed ? u - pr * G : u - U0;
    const int8_t* wb =
        routed ? W + ((int64_t)e_lds[pr] * (H >> 4) + tile) * nk * 1024 + lane * 16 +
                     (int64_t)(2 * gg) * 1024
               : Wdsh + (int64_t)tile * (Is >> 6) * 1024 + lane * 16 + (int64_t)(2 * gg) * 1024;
#pragma unroll
    for (int h = 0; h < 2; h++)
      bw[i][h] = u < U ? ld_stream(wb + h * 1024) : v4i{0, 0, 0, 0};
  }
  for (int i = threadIdx.x; i < U * 16; i += WAVES * 64) {
    const int u = i >> 4, c = i & 15;
    if (u < U0) {
      const int pr = u / G, gg = u - pr * G;
      s_lds[u][c] = bf16_bits_to_f32(sW[((int64_t)e_lds[pr] * H + tile * 16 + c) * G + gg]);
    } else {
      s_lds[u][c] = bf16_bits_to_f32(sdsh[(int64_t)(tile * 16 + c) * Gs + (u - U0)]);
    }
  }
  // rotated requant of the k activation rows (and the shared row, row k)
  // into LDS (packed operand rows)
  for (int r = wv; r < rows; r += WAVES) {
    const bool rsh = r == k;
    const int len = rsh ? Is : I;
    const int gr = len >> 7;
    Block8 bb[2];
    const float am = rot_row_wave<2>(rsh ? act_sh : act + (int64_t)r * I, len, bb, lane);
    const float sc = am / 127.0f;
#pragma unroll
    for (int rd = 0; rd < 2; rd++) {
      const int blk = rd * 4 + g;
      if (blk >= gr) continue;
      const uint2 wd = rot_codes8(bb[rd], am, sc);
      const int kk = blk * 128 + j * 8;
      *reinterpret_cast<uint2*>(a_lds + (kk >> 6) * 1024 + (r + 16 * ((kk & 63) >> 4)) * 16 +
                                (kk & 15)) = wd;
      if (!rsh && tile == 0 && qa_rec)
        *reinterpret_cast<uint2*>(qa_rec + (int64_t)r * I + kk) = wd;
    }
    if (lane == 0) {
      const float sv = am != 0.0f ? sc : 0.0f;
      sa_lds[r] = sv;
      if (!rsh && tile == 0 && sa_rec) sa_rec[r] = sv;
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < UW; i++) {
    const int u = wv + i * WAVES;
    if (u < U) {
      const int gg = u < U0 ? u % G : u - U0;
      v4i acc = {0, 0, 0, 0};
#pragma unroll
      for (int h = 0; h < 2; h++)
        acc = mfma_16x16x64_i8(*reinterpret_cast<const v4i*>(&a_lds[(2 * gg + h) * 1024 +
                                                                       lane * 16]),
                               bw[i][h], acc);
      red[u][lane] = acc;
    }
  }
  __syncthreads();
  // y2 of pair pr, column c: row pr of the pair's own units (lane 16 (pr / 4)
  // + c, element pr % 4), folded in group order
  if (threadIdx.x < rows * 16) {
    const int pr = threadIdx.x >> 4, c = threadIdx.x & 15;
    const int L = (pr >> 2) * 16 + c;
    const int u0 = pr < k ? pr * G : U0, ng = pr < k ? G : Gs;
    double t = 0.0;
    for (int gg = 0; gg < ng; gg++)
      t = t + (double)red[u0 + gg][L][pr & 3] * (double)s_lds[u0 + gg][c];
    t = t * (double)sa_lds[pr];
    t = t * 0.0078125;
    y_lds[pr][c] = (float)t;
  }
  __syncthreads();
  if (threadIdx.x < 16) {
    const int c = threadIdx.x;
    float acc = 0.0f;
    for (int pr = 0; pr < k; pr++) {
      const float term = w_lds[pr] * y_lds[pr][c];
      acc = acc + term;
    }
    if (shared) acc = acc + shared[tile * 16 + c];
    else if (has_sh) acc = acc + y_lds[k][c];
    out[tile * 16 + c] = (uint16_t)f32_to_bf16_bits(acc);
  }
}

// The shared expert's GEMMs for large batches, LDS-tiled.  Workgroup = 64
// token rows (rows [128 mb + 64 half, +64)) x 128 weight rows; wave w takes
// weight rows 32 w .. 32 w + 31 (two 16-row tiles) of all 64 token rows
// (four 16-row blocks, 16x16x64 MFMA).
//
// The fold after every 128-group: a wave whose 32 columns all have the
// integer form of the fold (rot_col_scales) adds acc_g M_g into int64 sums;
// any other wave folds in fp64 in group order, as defined.  kRotG256Silu
// folds su8 * acc in int64 (exact, as its definition).
template <int MODE>
__global__ __launch_bounds__(256, 2) void k_rot_tile(const int8_t* __restrict__ A,
                                                     const float* __restrict__ sA,
                                                     const int8_t* __restrict__ W,
                                                     const uint16_t* __restrict__ sW,
                                                     const uint8_t* __restrict__ su8, int Nw,
                                                     int K, int dense_rows,
                                                     float* __restrict__ out, int ldo) {
  constexpr int BM = 64, BN = 128, MAXG = 32, CH = 4;
  constexpr bool G256 = MODE == kRotG256Silu;
  __shared__ __attribute__((aligned(1024))) int8_t a_lds[2][CH][4 * 1024];
  __shared__ int pair_lds[BM];
  __shared__ float sa_lds[BM];
  __shared__ int32_t m_lds[BN][MAXG + 1];  // rows padded: lanes read 16 rows at once
  __shared__ float s_lds[G256 ? 1 : BN][MAXG + 1];
  __shared__ float cs_lds[BN];  // 2^xm (g128) or the bf16 row scale (g256)
  __shared__ int ok_lds[BN];

  const int ngrp = Nw / BN;  // workgroups across the weight rows
  const int xcd = blockIdx.x & 7;
  const int tq = blockIdx.x >> 3;
  const int nper = 2 * ngrp;
  const int mb = (tq / nper) * 8 + xcd;
  const int rem = tq - (tq / nper) * nper;
  const int half = rem & 1;
  const int nfirst = (rem >> 1) * BN;
  const int row0 = mb * 128 + half * 64;
  const int rows = min(BM, dense_rows - row0);
  if (rows <= 0) return;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int j = lane & 15;
  const int g = lane >> 4;
  const int nk = K >> 6;
  const int G = K >> 7;
  const int nsteps = (nk + 2 * CH - 1) / (2 * CH) * (2 * CH);

  if (threadIdx.x < BM) {
    const int p = row0 + min((int)threadIdx.x, rows - 1);
    pair_lds[threadIdx.x] = p;
    sa_lds[threadIdx.x] = sA[p];
  }

  // weight fragments: tiles nfirst / 16 + 2 wv + cb
  const int8_t* bsrc = W + ((int64_t)(nfirst >> 4) + 2 * wv) * nk * 1024 +
                       lane * 16;
  const int64_t tstride = (int64_t)nk * 1024;
  // plain loads: the two 64-row halves of an m-block read the same weight
  // rows back to back on one XCD, the second from L2
  auto load_b = [&](int st, v4i* b) __attribute__((always_inline)) {
    const int c = st < nk ? st : 0;
    b[0] = *reinterpret_cast<const v4i*>(bsrc + (int64_t)c * 1024);
    b[1] = *reinterpret_cast<const v4i*>(bsrc + tstride + (int64_t)c * 1024);
  };
  if (G256) {
    if (threadIdx.x < BN) {
      const int c = threadIdx.x;
      const int col = nfirst + c;
      const uint8_t* sp = su8 + (int64_t)col * (K >> 8);
      uint32_t u[MAXG / 2];
#pragma unroll
      for (int i = 0; i < MAXG / 2; i++) u[i] = 2 * i < G ? sp[i] : 0u;
#pragma unroll
      for (int gg = 0; gg < MAXG; gg++)
        if (gg < G) m_lds[c][gg] = (int32_t)u[gg >> 1];
      cs_lds[c] = bf16_bits_to_f32(sW[col]);
      ok_lds[c] = 1;
    }
  } else {
    // the tile's BN x G scales (contiguous) decoded element-wise, the
    // exponents held in the activation buffer until the main loop
    int* x_tmp = reinterpret_cast<int*>(&a_lds[0][0][0]);  // [BN][MAXG + 1]
    const uint16_t* sp = sW + (int64_t)nfirst * G;
    const int n = BN * G;
#pragma unroll 8
    for (int i = threadIdx.x; i < n; i += 256) {
      const uint32_t bits = sp[i];
      const int c = i / G, gg = i - c * G;
      int m = 0, x = 0;
      const bool fin = bf16_int_exp(bits, m, x);
      s_lds[c][gg] = bf16_bits_to_f32(bits);
      m_lds[c][gg] = fin ? m : 0;
      x_tmp[c * (MAXG + 1) + gg] = fin ? x : (1 << 20);  // 1 << 20 marks Inf / NaN
    }
    lds_barrier();
    // two threads a column, alternate groups: least exponent, multipliers,
    // the bound D and the check, combined across the pair
    const int c = threadIdx.x >> 1, h = threadIdx.x & 1;
    int xm = 1 << 20;
    bool ok = true;
    for (int gg = h; gg < G; gg += 2) {
      const int x = x_tmp[c * (MAXG + 1) + gg];
      if (x == (1 << 20)) ok = false;
      else if (m_lds[c][gg] != 0) xm = min(xm, x);
    }
    xm = min(xm, __shfl_xor(xm, 1, 64));
    if (xm == (1 << 20)) xm = 0;
    long long D = 0;
    for (int gg = h; gg < G; gg += 2) {
      const int m = m_lds[c][gg];
      int Mg = 0;
      if (m != 0) {
        const int sh = x_tmp[c * (MAXG + 1) + gg] - xm;
        if (sh > 23 || sh < 0) {
          ok = false;
        } else {
          Mg = m * (1 << sh);
          D += Mg < 0 ? -(long long)Mg : (long long)Mg;
        }
      }
      m_lds[c][gg] = Mg;
    }
    // both shuffles run on every lane (a shuffle inside a short-circuited
    // expression would read an inactive partner)
    D += __shfl_xor(D, 1, 64);
    const int ok_pair = __shfl_xor(ok ? 1 : 0, 1, 64);
    ok = ok && ok_pair != 0 && D < (1LL << 31);
    if (h == 0) {
      cs_lds[c] = ldexpf(1.0f, xm);
      ok_lds[c] = ok ? 1 : 0;
    }
  }
  lds_barrier();

  // activation rows: wave wv gathers 16-row block wv of each k step
  const int8_t* asrc = A + (int64_t)pair_lds[16 * wv + j] * K + g * 16;
  auto load_a = [&](int st) __attribute__((always_inline)) {
    const int c = st < nk ? st : 0;
    return *reinterpret_cast<const v4i*>(asrc + (int64_t)c * 64);
  };
  // this wave folds with integers when all of its 32 columns allow it
  const bool fast = __all(ok_lds[32 * wv + (lane & 31)] != 0);

  long long acc64[4][2][4];
#pragma unroll
  for (int rb = 0; rb < 4; rb++)
#pragma unroll
    for (int cb = 0; cb < 2; cb++)
#pragma unroll
      for (int v = 0; v < 4; v++) acc64[rb][cb][v] = 0;
  v4i acc[4][2];

  // The k steps go in chunks of CH, double-buffered: while a chunk is
  // multiplied (its weights in one register set, its activation rows in one
  // LDS buffer), the next chunk's loads are in flight (weights into the other
  // register set, activation rows into staging registers).  The only waits
  // are where the staged rows are stored into LDS, once per chunk: by then
  // the whole chunk's compute has covered the loads' latency.  (A ring
  // carried in registers from step to step makes the compiler wait for
  // nearly every load at the loop head instead.)
  v4i b0[CH][2], b1[CH][2];
  v4i at[CH];
  auto issue = [&](int c0, v4i (*bq)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < CH; u++) load_b(c0 + u, bq[u]);
#pragma unroll
    for (int u = 0; u < CH; u++) at[u] = load_a(c0 + u);  // last: their wait covers all
  };
  auto stage = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < CH; u++)
      *reinterpret_cast<v4i*>(&a_lds[buf][u][wv * 1024 + lane * 16]) = at[u];
  };
  auto compute = [&](int c0, int buf, v4i (*bq)[2], auto fast_c) __attribute__((always_inline)) {
    constexpr bool FAST = decltype(fast_c)::value;
#pragma unroll
    for (int u = 0; u < CH; u++) {
      const int st = c0 + u;
      v4i fa[4];
#pragma unroll
      for (int rb = 0; rb < 4; rb++)
        fa[rb] = *reinterpret_cast<const v4i*>(&a_lds[buf][u][rb * 1024 + lane * 16]);
      const bool kin = st < nk;
#pragma unroll
      for (int cb = 0; cb < 2; cb++) {
        const v4i bf = kin ? bq[u][cb] : v4i{0, 0, 0, 0};
#pragma unroll
        for (int rb = 0; rb < 4; rb++)
          acc[rb][cb] = mfma_16x16x64_i8(fa[rb], bf, (u & 1) ? acc[rb][cb] : v4i{0, 0, 0, 0});
      }
      if ((u & 1) && kin) {  // a 128-group is complete: fold it
        const int gg = st >> 1;
#pragma unroll
        for (int cb = 0; cb < 2; cb++) {
          const int c = 32 * wv + 16 * cb + j;
          if (FAST) {
            const long long M = m_lds[c][gg];
#pragma unroll
            for (int rb = 0; rb < 4; rb++)
#pragma unroll
              for (int v = 0; v < 4; v++) acc64[rb][cb][v] += (long long)acc[rb][cb][v] * M;
          } else {
            const double sv = (double)s_lds[G256 ? 0 : c][gg];
#pragma unroll
            for (int rb = 0; rb < 4; rb++)
#pragma unroll
              for (int v = 0; v < 4; v++) {
                double t = __longlong_as_double(acc64[rb][cb][v]);
                t = t + (double)acc[rb][cb][v] * sv;
                acc64[rb][cb][v] = __double_as_longlong(t);
              }
          }
        }
      }
    }
  };

  // the empty asm statements keep the compiler from moving a chunk's loads
  // across the compute or the staging (scheduling barriers)
  // the fold's form is fixed per wave before the loop, so each loop carries
  // one form only (a branch inside it gets if-converted into both)
  auto mainloop = [&](auto fast_c) __attribute__((always_inline)) {
    issue(0, b0);
    asm volatile("" ::: "memory");
    stage(0);
    lds_barrier();
    for (int c0 = 0; c0 < nsteps; c0 += 2 * CH) {
      issue(c0 + CH, b1);
      asm volatile("" ::: "memory");
      compute(c0, 0, b0, fast_c);
      asm volatile("" ::: "memory");
      stage(1);
      lds_barrier();
      issue(c0 + 2 * CH, b0);
      asm volatile("" ::: "memory");
      compute(c0 + CH, 1, b1, fast_c);
      asm volatile("" ::: "memory");
      stage(0);
      lds_barrier();
    }
  };
  if (G256 || fast)
    mainloop(std::true_type{});
  else
    mainloop(std::false_type{});

  // epilogue: lane holds rows 16 rb + 4 g + v of columns nfirst + 32 wv + 16 cb + j
#pragma unroll
  for (int cb = 0; cb < 2; cb++) {
    const int c = 32 * wv + 16 * cb + j;
    const int col = nfirst + c;
    const double cs = (double)cs_lds[c];
#pragma unroll
    for (int rb = 0; rb < 4; rb++) {
      float hv[4];
#pragma unroll
      for (int v = 0; v < 4; v++) {
        const int r = 16 * rb + 4 * g + v;
        double t;
        if (G256) {
          t = (double)acc64[rb][cb][v] * (double)sa_lds[r];
          t = t * cs;
        } else {
          t = fast ? (double)acc64[rb][cb][v] * cs : __longlong_as_double(acc64[rb][cb][v]);
          t = t * (double)sa_lds[r];
        }
        t = t * 0.0078125;
        hv[v] = (float)t;
        if (MODE == kRotCodes && r < rows) out[(int64_t)pair_lds[r] * ldo + col] = hv[v];
      }
      if (MODE != kRotCodes) {
        // gate = even column, up = the odd one in the neighbouring lane; the
        // lane pair splits the rows: the even lane finishes v = 0, 1, the
        // odd lane v = 2, 3 (one exp per output, not two)
        float xv[4];
#pragma unroll
        for (int v = 0; v < 4; v++) xv[v] = __shfl_xor(hv[v], 1, 64);
        const bool odd = j & 1;
#pragma unroll
        for (int q = 0; q < 2; q++) {
          const int v = odd ? q + 2 : q;
          const float gate = odd ? xv[q + 2] : hv[q];
          const float up = odd ? hv[q + 2] : xv[q];
          const float sg = (float)((double)gate / (1.0 + exp(-(double)gate)));
          const int r = 16 * rb + 4 * g + v;
          if (r < rows) out[(int64_t)pair_lds[r] * ldo + (col >> 1)] = sg * up;
        }
      }
    }
  }
}

// pair counts up to kRotSplitMaxPairs take the split-K GEMMs with the rotated
// requant fused into gemm2's prologue; beyond, the split-K GEMMs around
// k_rot_requant (measured on MI355X at 2048 tokens, 256 experts, H=2048,
// I=512: gemm1 / gemm2 259 / 121 us, against 303 / 205 us for the LDS-tiled
// kernel, which the shared expert's large batches use)
constexpr int64_t kRotSplitMaxPairs = 256;

// the one-workgroup sort up to 2048 pairs, as the routed int8 layer; beyond,
// the two-launch chunked sort (measured on MI355X at 2048 tokens, 16384 pairs:
// the Hadamard-domain routed layer 384 -> 374 us)
constexpr int64_t kRotSortOneWgPairs = 2048;
hipError_t launch_rot_sort(const MoeArgs& a, const MoeWs& ws, int64_t P, hipStream_t stream) {
  if (P <= kRotSortOneWgPairs) {
    hipLaunchKernelGGL(k_moe_sort, dim3(1), dim3(1024), 0, stream, a.topk_ids, (int)P, a.E,
                       ws.expert_list, ws.seg_off, ws.n_active, ws.sorted_pairs, ws.amax);
    return hipGetLastError();
  }
  const int chunk = (int)std::max<int64_t>(1024, (P + kMoeSortChunks - 1) / kMoeSortChunks);
  const int nchunks = (int)((P + chunk - 1) / chunk);
  hipLaunchKernelGGL(k_moe_sort_hist, dim3(nchunks), dim3(1024), 0, stream, a.topk_ids, (int)P,
                     a.E, chunk, ws.hist, ws.rank);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_moe_sort_scatter, dim3(nchunks), dim3(1024), 0, stream, a.topk_ids,
                     (int)P, a.E, chunk, nchunks, ws.hist, ws.rank, ws.expert_list, ws.seg_off,
                     ws.n_active, ws.sorted_pairs, ws.blk_slot, ws.blk_row0, ws.n_blocks);
  return hipGetLastError();
}

// One token in two launches.  With sh: the shared expert rides along (its
// gate/up tiles as workgroup row k of gemm1, its down projection as pair k
// of gemm2, its y added after the slot-order sum), act_sh holding its
// activation row.
static bool rot_t1_fits(const MoeArgs& a, int64_t Is) {
  if (!(a.T == 1 && a.k <= 16 && a.I <= 1024 && a.k * (a.I / 128) <= kRotT1MaxUnits))
    return false;
  return Is == 0 || (a.k <= 15 && Is <= 1024 && a.k * (a.I / 128) + Is / 128 <= kRotT1MaxUnits);
}

static hipError_t launch_rot_t1(const MoeArgs& a, const MoeWs& ws, const uint16_t* s13,
                                const uint16_t* s2, const float* shared, const RotSharedW* sh,
                                float* act_sh, hipStream_t stream) {
  const int I2 = 2 * a.I;
  const int Nsh = sh ? (int)(2 * sh->Is) : 0;
  hipError_t err;
  // with the shared expert: three workgroups a CU (80 VGPRs), since its
  // gate/up tiles come on top of the k * 2I / 16 routed ones (measured on
  // MI355X at one token, 256 experts, top-8, H=2048, I=Is=512: the layer
  // after the router 23.3 -> 18.8 us; the routed-only kernels keep the wider
  // budget, 17.3 against 17.9 us with the narrower one)
  if (sh)
    hipLaunchKernelGGL(k_rot_t1_gemm1<true>, dim3((unsigned)(std::max(I2, Nsh) / 16), a.k + 1),
                       dim3(512), 0, stream, a.x, a.logits, a.H, a.E, a.k, a.topk_ids, a.topk_w,
                       a.w13, s13, I2, a.dbg_qx, a.dbg_sx, ws.act, a.I, sh->wgu, sh->su8,
                       sh->sgu, Nsh, act_sh);
  else
    hipLaunchKernelGGL(k_rot_t1_gemm1<false>, dim3((unsigned)(I2 / 16), a.k), dim3(512), 0, stream,
                       a.x, a.logits, a.H, a.E, a.k, a.topk_ids, a.topk_w, a.w13, s13, I2,
                       a.dbg_qx, a.dbg_sx, ws.act, a.I, nullptr, nullptr, nullptr, 0, nullptr);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (sh)
    hipLaunchKernelGGL(k_rot_t1_gemm2<true>, dim3(a.H / 16), dim3(512), 0, stream, ws.act, a.I,
                       a.k, a.topk_ids, a.topk_w, a.w2, s2, a.H, shared, a.out, a.dbg_qa,
                       a.dbg_sa2, act_sh, (int)sh->Is, sh->wd, sh->sd);
  else
    hipLaunchKernelGGL(k_rot_t1_gemm2<false>, dim3(a.H / 16), dim3(512), 0, stream, ws.act, a.I,
                       a.k, a.topk_ids, a.topk_w, a.w2, s2, a.H, shared, a.out, a.dbg_qa,
                       a.dbg_sa2, nullptr, 0, nullptr, nullptr);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const int64_t P = (int64_t)a.T * a.k;
  if (a.dbg_act && (err = hipMemcpyAsync(a.dbg_act, ws.act, (size_t)P * a.I * 4,
                                         hipMemcpyDeviceToDevice, stream)) != hipSuccess)
    return err;
  return hipSuccess;
}

// The K-per-wave grouped GEMM: K <= 2048 (a wave holds its tile's K in
// registers), the activation buffer addressable with 32-bit offsets, and at
// least 512 pairs (measured on MI355X, routed layer E=256 H=2048 I=512 k=8,
// against the split-K kernels: 64 tokens 152 -> 146 us, 256 tokens 189 ->
// 178 us, 2048 tokens 407 -> 372 us; from 4096 pairs only, 64 and 256 tokens
// unchanged).
constexpr int64_t kRotKwMinPairs = 512;
static bool rot_kw_fits(int64_t P, int64_t rows, int64_t K) {
  return P >= kRotKwMinPairs && K <= 2048 && rows * K < ((int64_t)1 << 31);
}

template <int MODE, bool DENSE = false>
static hipError_t launch_rot_kw(const int8_t* qx, const float* sx, int k, const int8_t* W,
                                const uint16_t* sW, const uint8_t* su8, int64_t Nw, int64_t K,
                                int64_t rows, const MoeWs* ws, unsigned grid_y,
                                int rows_per_y, float* out, int64_t ldo, hipStream_t stream) {
  const dim3 grid((unsigned)(Nw / 64), grid_y), block(256);
  const int32_t* el = ws ? ws->expert_list : nullptr;
  const int32_t* so = ws ? ws->seg_off : nullptr;
  const int32_t* na = ws ? ws->n_active : nullptr;
  const int32_t* sp = ws ? ws->sorted_pairs : nullptr;
#define W8A8_KW(n)                                                                          \
  hipLaunchKernelGGL((k_rot_gemm_kw<MODE, n, DENSE>), grid, block, 0, stream, qx, sx, k, W, \
                     sW, su8, (int)Nw, (int)K, (int)rows, el, so, na, sp, rows_per_y, out,  \
                     (int)ldo)
  if (K <= 512)
    W8A8_KW(8);
  else if (K <= 1024)
    W8A8_KW(16);
  else
    W8A8_KW(32);
#undef W8A8_KW
  return hipGetLastError();
}

hipError_t launch_moe_rot_forward(const MoeArgs& a, const uint16_t* s13, const uint16_t* s2,
                                  const float* shared, hipStream_t stream) {
  const int64_t P = (int64_t)a.T * a.k;
  MoeWs ws = carve(a.ws, a.T, a.H, a.E, a.I, a.k);
  const unsigned slots = (unsigned)std::min<int64_t>(a.E, P);
  const int I2 = 2 * a.I;
  hipError_t err;
  if (rot_t1_fits(a, 0)) return launch_rot_t1(a, ws, s13, s2, shared, nullptr, nullptr, stream);
  hipLaunchKernelGGL(k_rot_route_quant, dim3((a.T + 3) / 4), dim3(512), 0, stream, a.x, a.logits,
                     a.T, a.H, a.E, a.k, a.topk_ids, a.topk_w, ws.qx, ws.sx);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if ((err = launch_rot_sort(a, ws, P, stream)) != hipSuccess) return err;
  // four (H <= 2048) or two 16-row weight tiles a workgroup: the activation
  // slices loaded once for all, more weight bytes in flight; LDS sized for H
  if (rot_kw_fits(P, a.T, a.H)) {
    if ((err = launch_rot_kw<kRotSilu>(ws.qx, ws.sx, a.k, a.w13, s13, nullptr, I2, a.H, a.T,
                                       &ws, slots, 0, ws.act, a.I, stream)) != hipSuccess)
      return err;
  } else {
    auto g1 = a.H <= 2048 ? k_rot_gemm_splitk<kRotSilu, 8, 4, 16>
                          : k_rot_gemm_splitk<kRotSilu, 8, 2, 32>;
    const unsigned t1 = a.H <= 2048 ? I2 / 64 : I2 / 32;
    hipLaunchKernelGGL(g1, dim3(t1, slots), dim3(512), 0, stream, ws.qx, ws.sx, nullptr, a.k,
                       a.w13, s13, nullptr, I2, a.H, ws.expert_list, ws.seg_off, ws.n_active,
                       ws.sorted_pairs, 0, ws.act, a.I, nullptr, nullptr);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (P <= kRotSplitMaxPairs) {
    hipLaunchKernelGGL((k_rot_gemm_splitk<kRotActRot, 4, 1, 16>), dim3(a.H / 16, slots),
                       dim3(256), 0, stream, nullptr, nullptr, ws.act, a.k, a.w2, s2, nullptr,
                       a.H, a.I, ws.expert_list, ws.seg_off, ws.n_active, ws.sorted_pairs, 0,
                       ws.y2, a.H, a.dbg_qa, a.dbg_sa2);
  } else {
    hipLaunchKernelGGL(k_rot_requant, dim3((unsigned)((P + 7) / 8)), dim3(512), 0, stream,
                       ws.act, P, a.I, ws.qa, ws.sa2);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (rot_kw_fits(P, P, a.I)) {
      if ((err = launch_rot_kw<kRotCodes>(ws.qa, ws.sa2, 1, a.w2, s2, nullptr, a.H, a.I, P,
                                          &ws, slots, 0, ws.y2, a.H, stream)) != hipSuccess)
        return err;
    } else {
      // four 16-row weight tiles a workgroup; LDS sized for I
      auto g2 = a.I <= 512    ? k_rot_gemm_splitk<kRotCodes, 4, 4, 4>
                : a.I <= 1024 ? k_rot_gemm_splitk<kRotCodes, 4, 4, 8>
                              : k_rot_gemm_splitk<kRotCodes, 4, 4, 16>;
      hipLaunchKernelGGL(g2, dim3(a.H / 64, slots), dim3(256), 0, stream, ws.qa, ws.sa2,
                         nullptr, 1, a.w2, s2, nullptr, a.H, a.I, ws.expert_list, ws.seg_off,
                         ws.n_active, ws.sorted_pairs, 0, ws.y2, a.H, nullptr, nullptr);
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if (a.dbg_qa && (err = hipMemcpyAsync(a.dbg_qa, ws.qa, (size_t)(P * a.I),
                                          hipMemcpyDeviceToDevice, stream)) != hipSuccess)
      return err;
    if (a.dbg_sa2 && (err = hipMemcpyAsync(a.dbg_sa2, ws.sa2, (size_t)P * 4,
                                           hipMemcpyDeviceToDevice, stream)) != hipSuccess)
      return err;
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const int nbh = (a.H / 4 + 255) / 256;
  hipLaunchKernelGGL(k_moe_combine, dim3((unsigned)((int64_t)nbh * a.T)), dim3(256), 0, stream,
                     ws.y2, a.topk_ids, a.topk_w, a.T, a.H, a.E, a.k, nbh, shared, a.out);
  if ((err = hipGetLastError()) != hipSuccess) return err;
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

// The routed layer with its shared expert.  Workspace: the routed layer's,
// the shared expert's, the shared output [T, H] fp32 and one activation row.
size_t moe_rot_shared_workspace_bytes(int64_t T, int64_t H, int64_t E, int64_t I, int k,
                                      int64_t Is) {
  return align_up(moe_workspace_bytes(T, H, E, I, k)) +
         align_up(shared_expert_workspace_bytes(T, H, Is)) + align_up((size_t)(4 * T * H)) +
         align_up((size_t)(4 * Is));
}

hipError_t launch_moe_rot_shared_forward(const MoeArgs& a, const uint16_t* s13,
                                         const uint16_t* s2, const RotSharedW& sh,
                                         hipStream_t stream) {
  char* b = static_cast<char*>(a.ws);
  const size_t o1 = align_up(moe_workspace_bytes(a.T, a.H, a.E, a.I, a.k));
  const size_t o2 = o1 + align_up(shared_expert_workspace_bytes(a.T, a.H, sh.Is));
  const size_t o3 = o2 + align_up((size_t)(4 * (int64_t)a.T * a.H));
  float* y_sh = reinterpret_cast<float*>(b + o2);
  float* act_sh = reinterpret_cast<float*>(b + o3);
  if (rot_t1_fits(a, sh.Is)) {
    const MoeWs ws = carve(a.ws, a.T, a.H, a.E, a.I, a.k);
    return launch_rot_t1(a, ws, s13, s2, nullptr, &sh, act_sh, stream);
  }
  SharedArgs sa{};
  sa.x = a.x;
  sa.T = a.T;
  sa.H = a.H;
  sa.Is = sh.Is;
  sa.wgu = sh.wgu;
  sa.su8 = sh.su8;
  sa.s2 = sh.sgu;
  sa.wd = sh.wd;
  sa.sd = sh.sd;
  sa.y = y_sh;
  sa.ws = b + o1;
  hipError_t err = launch_shared_expert(sa, stream);
  if (err != hipSuccess) return err;
  return launch_moe_rot_forward(a, s13, s2, y_sh, stream);
}

// The shared expert: rotated codes of x, the g256 gate/up GEMM with the SiLU
// epilogue, then the rotated requant and the g128 down GEMM (dense forms).
namespace {
struct SharedWs {
  int8_t* qx;
  float* sx;
  float* act;
  int8_t* qa;
  float* sa;
  size_t bytes;
};

SharedWs carve_shared(void* base, int64_t T, int64_t H, int64_t Is) {
  SharedWs w;
  size_t off = 0;
  char* b = static_cast<char*>(base);
  auto take = [&](size_t bytes) {
    char* p = b ? b + off : nullptr;
    off += align_up(bytes);
    return p;
  };
  w.qx = reinterpret_cast<int8_t*>(take(T * H));
  w.sx = reinterpret_cast<float*>(take(T * 4));
  w.act = reinterpret_cast<float*>(take(T * Is * 4));
  w.qa = reinterpret_cast<int8_t*>(take(T * Is));
  w.sa = reinterpret_cast<float*>(take(T * 4));
  w.bytes = off;
  return w;
}
}  // namespace

size_t shared_expert_workspace_bytes(int64_t T, int64_t H, int64_t Is) {
  return carve_shared(nullptr, T, H, Is).bytes;
}

hipError_t launch_shared_expert(const SharedArgs& a, hipStream_t stream) {
  const SharedWs ws = carve_shared(a.ws, a.T, a.H, a.Is);
  const int T = (int)a.T, H = (int)a.H, Is = (int)a.Is;
  hipError_t err;
  // up to 8 tokens with H <= 2048 the gate/up GEMM rotates and quantises its
  // token rows itself (one launch less)
  const bool fused = a.T <= 8 && a.H <= 2048;
  if (!fused) {
    hipLaunchKernelGGL(k_rot_route_quant, dim3((unsigned)((T + 3) / 4)), dim3(512), 0, stream,
                       a.x, nullptr, T, H, 1, 1, nullptr, nullptr, ws.qx, ws.sx);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (a.T <= 64) {
    // one 16-row block of tokens a workgroup row (grid.y)
    const unsigned rb = (unsigned)((a.T + 15) / 16);
    if (fused)  // x passed as the rows to rotate (bf16; the mode reads them as such)
      hipLaunchKernelGGL((k_rot_gemm_splitk<kRotG256SiluX, 8, 1, 16>), dim3(2 * Is / 16, rb),
                         dim3(512), 0, stream, nullptr, nullptr,
                         reinterpret_cast<const float*>(a.x), 1, a.wgu, a.s2, a.su8, 2 * Is, H,
                         nullptr, nullptr, nullptr, nullptr, T, ws.act, Is, nullptr, nullptr);
    else
      hipLaunchKernelGGL((k_rot_gemm_splitk<kRotG256Silu, 8, 1, 32>), dim3(2 * Is / 16, rb),
                         dim3(512), 0, stream, ws.qx, ws.sx, nullptr, 1, a.wgu, a.s2, a.su8,
                         2 * Is, H, nullptr, nullptr, nullptr, nullptr, T, ws.act, Is, nullptr,
                         nullptr);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL((k_rot_gemm_splitk<kRotActRot, 4, 1, 16>), dim3(H / 16, rb), dim3(256), 0,
                       stream, nullptr, nullptr, ws.act, 1, a.wd, a.sd, nullptr, H, Is, nullptr,
                       nullptr, nullptr, nullptr, T, a.y, H, a.dbg_qa, a.dbg_sa);
  } else {
    const unsigned mbs = (unsigned)((a.T + 1023) / 1024 * 8);  // 128-row blocks, x 8 XCDs
    // one wave per weight tile holding all of K where K fits (H, Is <= 2048),
    // 32 token rows a workgroup row up to 1024 tokens, 64 beyond (measured on
    // MI355X, H=2048, Is=512, against the tiled GEMMs: 128 tokens 34.5 ->
    // 20.2 us, 512 tokens 36.2 -> 23.4 us, 2048 tokens 44.6 -> 43.9 us)
    const bool kw = a.H <= 2048 && a.Is <= 2048 && a.T * a.H < ((int64_t)1 << 31);
    const int kw_rows = a.T <= 1024 ? 32 : 64;
    const unsigned ry = (unsigned)((a.T + kw_rows - 1) / kw_rows);
    if (kw)
      err = launch_rot_kw<kRotG256Silu, true>(ws.qx, ws.sx, 1, a.wgu, a.s2, a.su8, 2 * Is, H, T,
                                              nullptr, ry, kw_rows, ws.act, Is, stream);
    else {
      hipLaunchKernelGGL(k_rot_tile<kRotG256Silu>, dim3(mbs * 2 * (2 * Is / 128)), dim3(256), 0,
                         stream, ws.qx, ws.sx, a.wgu, a.s2, a.su8, 2 * Is, H, T, ws.act, Is);
      err = hipGetLastError();
    }
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k_rot_requant, dim3((unsigned)((a.T + 7) / 8)), dim3(512), 0, stream,
                       ws.act, a.T, Is, ws.qa, ws.sa);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (kw)
      err = launch_rot_kw<kRotCodes, true>(ws.qa, ws.sa, 1, a.wd, a.sd, nullptr, H, Is, T,
                                           nullptr, ry, kw_rows, a.y, H, stream);
    else {
      hipLaunchKernelGGL(k_rot_tile<kRotCodes>, dim3(mbs * 2 * (H / 128)), dim3(256), 0, stream,
                         ws.qa, ws.sa, a.wd, a.sd, nullptr, H, Is, T, a.y, H);
      err = hipGetLastError();
    }
    if (err != hipSuccess) return err;
    if (a.dbg_qa && (err = hipMemcpyAsync(a.dbg_qa, ws.qa, (size_t)(a.T * a.Is),
                                          hipMemcpyDeviceToDevice, stream)) != hipSuccess)
      return err;
    if (a.dbg_sa && (err = hipMemcpyAsync(a.dbg_sa, ws.sa, (size_t)a.T * 4,
                                          hipMemcpyDeviceToDevice, stream)) != hipSuccess)
      return err;
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (a.dbg_act && (err = hipMemcpyAsync(a.dbg_act, ws.act, (size_t)(a.T * a.Is) * 4,
                                         hipMemcpyDeviceToDevice, stream)) != hipSuccess)
    return err;
  return hipSuccess;
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
    // two workgroups per 16-column tile: 2 H / 16 of them, so every CU
    // streams weights (measured on MI355X: 12.64 -> 12.37 us for the layer)
    hipLaunchKernelGGL((k_moe_t1_gemm2<PACKED, true>), dim3(2 * tiles2), dim3(512), 0, stream, ws.act,
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
    const int nbh = (a.H / 4 + 255) / 256;
    hipLaunchKernelGGL(k_moe_combine, dim3((unsigned)((int64_t)nbh * a.T)), dim3(256), 0, stream,
                       ws.y2, a.topk_ids, a.topk_w, a.T, a.H, a.E, a.k, nbh, nullptr, a.out);
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
