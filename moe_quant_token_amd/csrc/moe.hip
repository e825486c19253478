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
// count that depends on the routing stays on the device):
//   k_moe_route    softmax top-k over the logits, one wave per token
//   k_moe_sort     one workgroup: per-expert counts, the list of experts that
//                  received pairs, segment offsets, pairs grouped by expert
//   k_quant_rows   per-token int8 codes of x (quant.hip)
//   k_moe_gemm<1>  grouped gemm1: one grid row per active expert, each wave
//                  owns 16 interleaved w13 rows (8 gate/up column pairs) and
//                  walks every pair routed to that expert, 64 at a time, so a
//                  weight byte is fetched from HBM once per 64 pairs; epilogue
//                  dequantises, applies SiLU(gate)*up and records the per-pair
//                  |act| maximum with an integer atomic max (exact, order-free)
//   k_moe_requant  per-pair int8 codes of the activation, one wave per pair
//   k_moe_gemm<2>  grouped gemm2, epilogue writes dequantised fp32 rows
//   k_moe_combine  out[t] = sum over the k slots, in slot order, one bf16
//                  rounding; deterministic (no floating-point atomics)
#include <algorithm>

#include "kernels.h"

namespace w8a8 {

namespace {

constexpr size_t kAlign = 256;
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
  w.bytes = off;
  return w;
}

}  // namespace

// ---------------------------------------------------------------------------
// Routing: softmax over E, top-k, renormalise.  Selection compares the fp32
// logits (softmax is monotonic): slot s gets the s-th largest, equal logits
// go to the lower expert index.  Probabilities are formed in fp64 and the
// renormalised weight is rounded once to fp32.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_moe_route(const float* __restrict__ logits, int T,
                                                   int E, int k, int32_t* __restrict__ ids,
                                                   float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* lt = logits + (int64_t)t * E;
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; i++) {
    const int e = lane + 64 * i;
    v[i] = e < E ? lt[e] : -INFINITY;
  }
  uint32_t taken = 0;
  float selv[16];
  for (int s = 0; s < k; s++) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const int e = lane + 64 * i;
      // ascending e within a lane, strict '>' keeps the lower index on ties
      if (e < E && !(taken & (1u << i)) && (be == 0x7fffffff || v[i] > bv)) {
        bv = v[i];
        be = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oe = __shfl_xor(be, off, 64);
      if (ov > bv || (ov == bv && oe < be)) {
        bv = ov;
        be = oe;
      }
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    selv[s & 15] = bv;
    if (lane == 0) ids[(int64_t)t * k + s] = be;
  }
  // softmax denominator over all experts (fp64); the maximum is slot 0
  const double mx = (double)selv[0];
  double z = 0.0;
#pragma unroll
  for (int i = 0; i < 16; i++) {
    const int e = lane + 64 * i;
    if (e < E) z += exp((double)v[i] - mx);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) z += __shfl_xor(z, off, 64);
  double p[16];
  double kept = 0.0;
  for (int s = 0; s < k; s++) {
    p[s] = exp((double)selv[s] - mx) / z;
    kept += p[s];
  }
  if (lane < k) {
    double ps = 0.0;
    for (int s = 0; s < k; s++)
      if (s == lane) ps = p[s];
    w[(int64_t)t * k + lane] = (float)(ps / kept);
  }
}

// ---------------------------------------------------------------------------
// Sort / align by expert (one workgroup of 1024 threads).  Pairs with an id
// outside [0, E) are dropped.  Also clears the per-pair |act| maxima.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_moe_sort(const int32_t* __restrict__ ids, int P,
                                                   int E, int32_t* __restrict__ expert_list,
                                                   int32_t* __restrict__ seg_off,
                                                   int32_t* __restrict__ n_active,
                                                   int32_t* __restrict__ sorted_pairs,
                                                   uint32_t* __restrict__ amax) {
  __shared__ int cnt[1024];
  __shared__ int cursor[1024];
  __shared__ int wsum_c[16], wsum_f[16];
  const int tid = threadIdx.x;
  cnt[tid] = 0;
  __syncthreads();
  for (int r = tid; r < P; r += 1024) {
    const int e = ids[r];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    amax[r] = 0u;
  }
  __syncthreads();
  // exclusive scans of the counts and of the "expert is active" flags
  const int c = tid < E ? cnt[tid] : 0;
  const int f = c > 0 ? 1 : 0;
  const int lane = tid & 63, wv = tid >> 6;
  int ic = c, iflag = f;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int oc = __shfl_up(ic, off, 64);
    const int of = __shfl_up(iflag, off, 64);
    if (lane >= off) {
      ic += oc;
      iflag += of;
    }
  }
  if (lane == 63) {
    wsum_c[wv] = ic;
    wsum_f[wv] = iflag;
  }
  __syncthreads();
  int base_c = 0, base_f = 0, tot_c = 0, tot_f = 0;
  for (int i = 0; i < 16; i++) {
    if (i < wv) {
      base_c += wsum_c[i];
      base_f += wsum_f[i];
    }
    tot_c += wsum_c[i];
    tot_f += wsum_f[i];
  }
  const int off_c = base_c + ic - c;
  const int slot = base_f + iflag - f;
  if (f) {
    expert_list[slot] = tid;
    seg_off[slot] = off_c;
  }
  if (tid < E) cursor[tid] = off_c;
  if (tid == 0) {
    n_active[0] = tot_f;
    seg_off[tot_f] = tot_c;
  }
  __syncthreads();
  for (int r = tid; r < P; r += 1024) {
    const int e = ids[r];
    if (e >= 0 && e < E) {
      const int pos = atomicAdd(&cursor[e], 1);
      sorted_pairs[pos] = r;
    }
  }
}

// ---------------------------------------------------------------------------
// Grouped GEMM over the pairs of one expert.  MODE 1 = gemm1 (A = qx rows of
// the pairs' tokens, epilogue SiLU(gate)*up), MODE 2 = gemm2 (A = qa rows of
// the pairs, epilogue dequantised fp32 rows).  Wave tile: 16 pairs x 16
// weight rows; up to 4 pair blocks share each weight load.  Operand mapping as
// in gemm_skinny.hip.
// ---------------------------------------------------------------------------
template <int WAVES, int MODE>
__global__ __launch_bounds__(WAVES * 64) void k_moe_gemm(
    const int8_t* __restrict__ A, const float* __restrict__ sA, int a_div,
    const int8_t* __restrict__ W, const float* __restrict__ sW, int Nw, int K,
    const int32_t* __restrict__ expert_list, const int32_t* __restrict__ seg_off,
    const int32_t* __restrict__ n_active, const int32_t* __restrict__ sorted_pairs,
    float* __restrict__ out, int ldo, uint32_t* __restrict__ amax,
    int32_t* __restrict__ dbg_acc) {
  constexpr int U = 4;
  const int slot = blockIdx.x;
  if (slot >= n_active[0]) return;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int j = lane & 15;
  const int g = lane >> 4;
  const int e = expert_list[slot];
  const int seg_begin = seg_off[slot];
  const int seg_end = seg_off[slot + 1];
  const int n0 = (blockIdx.y * WAVES + wv) * 16;
  if (n0 >= Nw) return;
  const int8_t* wp = W + ((int64_t)e * Nw + n0 + j) * K + g * 16;
  const int nk = K >> 6;

  for (int pb = seg_begin; pb < seg_end; pb += 64) {
    const int nb = min(4, (seg_end - pb + 15) >> 4);  // wave-uniform
    const int8_t* ap[4];
    bool aok[4];
#pragma unroll
    for (int b = 0; b < 4; b++) {
      const int idx = pb + b * 16 + j;
      aok[b] = idx < seg_end;
      const int p = aok[b] ? sorted_pairs[idx] : 0;
      ap[b] = A + (int64_t)(p / a_div) * K + g * 16;
    }
    v4i acc[4];
#pragma unroll
    for (int b = 0; b < 4; b++) acc[b] = v4i{0, 0, 0, 0};

    for (int c = 0; c < nk; c += U) {
      v4i wb[U];
      v4i a[4][U];
#pragma unroll
      for (int u = 0; u < U; u++) {
        const bool in = c + u < nk;
        wb[u] = in ? *reinterpret_cast<const v4i*>(wp + (int64_t)(c + u) * 64) : v4i{0, 0, 0, 0};
#pragma unroll
        for (int b = 0; b < 4; b++)
          a[b][u] = (in && b < nb && aok[b])
                        ? *reinterpret_cast<const v4i*>(ap[b] + (int64_t)(c + u) * 64)
                        : v4i{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < U; u++)
#pragma unroll
        for (int b = 0; b < 4; b++)
          if (b < nb) acc[b] = mfma_16x16x64_i8(a[b][u], wb[u], acc[b]);
    }

    // epilogue: lane holds pair rows 4g+v of weight row n0 + j, per block b
    const int col = n0 + j;
    const float swc = sW[(int64_t)e * Nw + col];
#pragma unroll
    for (int b = 0; b < 4; b++) {
      if (b >= nb) break;
#pragma unroll
      for (int v = 0; v < 4; v++) {
        const int idx = pb + b * 16 + 4 * g + v;
        const bool valid = idx < seg_end;
        const int p = valid ? sorted_pairs[idx] : 0;
        const int32_t av = acc[b][v];
        if (dbg_acc && valid) dbg_acc[(int64_t)p * Nw + col] = av;
        float h = 0.0f;
        if (valid) {
          h = (float)av;
          h = h * sA[p / a_div];
          h = h * swc;
        }
        if (MODE == 1) {
          const float partner = __shfl_xor(h, 1, 64);
          float mag = 0.0f;
          if ((j & 1) == 0 && valid) {
            // SiLU(gate) * up; the gate is the even interleaved row
            const float sg = (float)((double)h / (1.0 + exp(-(double)h)));
            const float act = sg * partner;
            out[(int64_t)p * ldo + (col >> 1)] = act;
            mag = fabsf(act);
          }
#pragma unroll
          for (int off = 1; off < 16; off <<= 1) mag = fmaxf(mag, __shfl_xor(mag, off, 64));
          if (j == 0 && valid) atomicMax(&amax[p], __float_as_uint(mag));
        } else {
          if (valid) out[(int64_t)p * ldo + col] = h;
        }
      }
    }
  }
}

// Per-pair requant of the fp32 activation rows (one wave per pair).
__global__ __launch_bounds__(256) void k_moe_requant(const float* __restrict__ act,
                                                     const uint32_t* __restrict__ amax, int P,
                                                     int I, int8_t* __restrict__ qa,
                                                     float* __restrict__ sa2) {
  const int lane = threadIdx.x & 63;
  const int p = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (p >= P) return;
  const float am = __uint_as_float(amax[p]);
  const float sc = am / 127.0f;
  const float* ar = act + (int64_t)p * I;
  int8_t* qr = qa + (int64_t)p * I;
  for (int c = lane * 4; c < I; c += 256) {
    const v4f a = *reinterpret_cast<const v4f*>(ar + c);
    uint32_t wd = 0;
    if (am != 0.0f)
      wd = pack4_i8(quant_code(a.x, sc), quant_code(a.y, sc), quant_code(a.z, sc),
                    quant_code(a.w, sc));
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

hipError_t launch_moe_forward(const MoeArgs& a, hipStream_t stream) {
  const int64_t P = (int64_t)a.T * a.k;
  MoeWs ws = carve(a.ws, a.T, a.H, a.E, a.I, a.k);
  hipError_t err;
  if (a.logits) {
    hipLaunchKernelGGL(k_moe_route, dim3((a.T + 3) / 4), dim3(256), 0, stream, a.logits, a.T,
                       a.E, a.k, a.topk_ids, a.topk_w);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  hipLaunchKernelGGL(k_moe_sort, dim3(1), dim3(1024), 0, stream, a.topk_ids, (int)P, a.E,
                     ws.expert_list, ws.seg_off, ws.n_active, ws.sorted_pairs, ws.amax);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if ((err = launch_quant_rows(a.x, 0, a.T, a.H, a.H, ws.qx, a.H, ws.sx, stream)) != hipSuccess)
    return err;

  const int slots = (int)std::min<int64_t>(a.E, P);
  const int I2 = 2 * a.I;
  // Few pairs: one wave per workgroup spreads the weight stream over more CUs.
  if (P <= 256) {
    hipLaunchKernelGGL((k_moe_gemm<1, 1>), dim3(slots, I2 / 16), dim3(64), 0, stream, ws.qx,
                       ws.sx, a.k, a.w13, a.s13, I2, a.H, ws.expert_list, ws.seg_off,
                       ws.n_active, ws.sorted_pairs, ws.act, a.I, ws.amax, a.dbg_acc1);
  } else {
    hipLaunchKernelGGL((k_moe_gemm<4, 1>), dim3(slots, (I2 / 16 + 3) / 4), dim3(256), 0, stream,
                       ws.qx, ws.sx, a.k, a.w13, a.s13, I2, a.H, ws.expert_list, ws.seg_off,
                       ws.n_active, ws.sorted_pairs, ws.act, a.I, ws.amax, a.dbg_acc1);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(k_moe_requant, dim3((unsigned)((P + 3) / 4)), dim3(256), 0, stream, ws.act,
                     ws.amax, (int)P, a.I, ws.qa, ws.sa2);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (P <= 256) {
    hipLaunchKernelGGL((k_moe_gemm<1, 2>), dim3(slots, a.H / 16), dim3(64), 0, stream, ws.qa,
                       ws.sa2, 1, a.w2, a.s2, a.H, a.I, ws.expert_list, ws.seg_off, ws.n_active,
                       ws.sorted_pairs, ws.y2, a.H, nullptr, a.dbg_acc2);
  } else {
    hipLaunchKernelGGL((k_moe_gemm<4, 2>), dim3(slots, (a.H / 16 + 3) / 4), dim3(256), 0,
                       stream, ws.qa, ws.sa2, 1, a.w2, a.s2, a.H, a.I, ws.expert_list,
                       ws.seg_off, ws.n_active, ws.sorted_pairs, ws.y2, a.H, nullptr,
                       a.dbg_acc2);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(k_moe_combine, dim3((a.H / 4 + 255) / 256, a.T), dim3(256), 0, stream,
                     ws.y2, a.topk_ids, a.topk_w, a.T, a.H, a.E, a.k, a.out);
  if ((err = hipGetLastError()) != hipSuccess) return err;

  // optional copies of the intermediates, in pair order
  if (a.dbg_qx && (err = hipMemcpyAsync(a.dbg_qx, ws.qx, (size_t)a.T * a.H,
                                        hipMemcpyDeviceToDevice, stream)) != hipSuccess)
    return err;
  if (a.dbg_sx && (err = hipMemcpyAsync(a.dbg_sx, ws.sx, (size_t)a.T * 4,
                                        hipMemcpyDeviceToDevice, stream)) != hipSuccess)
    return err;
  if (a.dbg_act && (err = hipMemcpyAsync(a.dbg_act, ws.act, (size_t)P * a.I * 4,
                                         hipMemcpyDeviceToDevice, stream)) != hipSuccess)
    return err;
  if (a.dbg_qa && (err = hipMemcpyAsync(a.dbg_qa, ws.qa, (size_t)P * a.I,
                                        hipMemcpyDeviceToDevice, stream)) != hipSuccess)
    return err;
  if (a.dbg_sa2 && (err = hipMemcpyAsync(a.dbg_sa2, ws.sa2, (size_t)P * 4,
                                         hipMemcpyDeviceToDevice, stream)) != hipSuccess)
    return err;
  return hipSuccess;
}

}  // namespace w8a8
