// Dense W8A8 MLP block: gate_up -> SiLU(gate) * up -> per-token requant ->
// down.
//
// Source: "[gfx1151] Online INT8 W8A8 for Qwen3.6 27B / 35B-A3B on RDNA3.5,
// with working MTP" (ATOM pull request): A8W8 for all dense GEMMs (intro;
// the 27B dense model of its "Performance" section), with the order of its
// "Changes", fused_moe_triton.py bullet -- gemm1 with the gated SiLU over
// interleaved gate/up rows, per-token int8 requant, gemm2 -- applied to the
// dense gate_up and down linears.
//
// Four launches on the caller's stream (three for one token, whose requant
// runs inside the down GEMM's launch as in the decode linear):
//   1. per-token int8 codes of x (row-major for decode, tile layout for the
//      tiled GEMM);
//   2. the gate_up GEMM whose epilogue pairs the interleaved gate and up
//      columns (adjacent lanes of the MFMA result) and writes the fp32
//      activation row: the decode weight-streaming kernel up to 16 tokens,
//      the tiled MFMA kernel beyond;
//   3. per-token int8 requant of the fp32 activation rows (the row quantiser
//      on fp32 rows: amax / 127 and the IEEE quotient);
//   4. the down GEMM with the bf16 epilogue.
// The activation's per-token scale needs the maximum over the whole
// intermediate row, which many gate_up workgroups produce, so the requant is
// a launch of its own.
#include "kernels.h"

namespace w8a8 {

namespace {

constexpr size_t kAlign = 256;
size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct MlpWs {
  int8_t* qx;
  float* sx;
  float* act;
  int8_t* qa;
  float* sa;
  size_t bytes;
};

// codes for rows rounded up to whole 16-row tiles (the tile layout)
MlpWs carve(void* base, int64_t M, int64_t K, int64_t I) {
  MlpWs w{};
  char* p = static_cast<char*>(base);
  size_t off = 0;
  const size_t rows16 = (size_t)((M + 15) / 16 * 16);
  auto take = [&](size_t n) {
    char* r = p ? p + off : nullptr;
    off += up(n);
    return r;
  };
  w.qx = reinterpret_cast<int8_t*>(take(rows16 * (size_t)K));
  w.sx = reinterpret_cast<float*>(take((size_t)M * 4));
  w.act = reinterpret_cast<float*>(take((size_t)M * (size_t)I * 4));
  w.qa = reinterpret_cast<int8_t*>(take(rows16 * (size_t)I));
  w.sa = reinterpret_cast<float*>(take((size_t)M * 4));
  w.bytes = off;
  return w;
}

}  // namespace

size_t mlp_workspace_bytes(int64_t M, int64_t K, int64_t I) {
  return carve(nullptr, M, K, I).bytes;
}

hipError_t launch_mlp(const MlpArgs& a, hipStream_t stream) {
  const MlpWs w = carve(a.ws, a.M, a.K, a.I);
  const int64_t I2 = 2 * a.I;
  hipError_t e;
  const bool tiled = a.M > 16;
  if (!tiled) {
    if ((e = launch_quant_rows(a.x, 0, a.M, a.K, a.ldx, w.qx, a.K, w.sx, stream)) != hipSuccess)
      return e;
    if ((e = launch_gemm_skinny_silu(w.qx, w.sx, a.M, a.K, a.K, a.wgu, a.sgu, I2, w.act, a.I,
                                     stream)) != hipSuccess)
      return e;
    if (a.M == 1 && linear_fused_fits(a.M, a.N, a.I)) {
      // one token: requant and down GEMM in one launch (its first workgroup
      // also leaves the codes and scales in the workspace).  Measured on
      // MI355X at K=5120, I=8704, N=5120: the block 33.0 -> 31.0 us; at two
      // tokens (fp32 rows, 70 KiB a workgroup) 33.7 -> 34.9 us, so not there
      if ((e = launch_linear_skinny_fused_f32(w.act, a.I, a.M, a.I, a.wd, a.sd, a.N, a.y, a.ldy,
                                              w.qa, w.sa, stream)) != hipSuccess)
        return e;
    } else {
      if ((e = launch_quant_rows_f32(w.act, a.M, a.I, a.I, w.qa, a.I, w.sa, false, stream)) !=
          hipSuccess)
        return e;
      if ((e = launch_gemm_skinny(w.qa, w.sa, a.M, a.I, a.I, a.wd, a.sd, a.N, a.I, true, a.y,
                                  a.ldy, stream)) != hipSuccess)
        return e;
    }
  } else {
    if ((e = launch_quant_rows_packed(a.x, a.M, a.K, a.ldx, w.qx, w.sx, stream)) != hipSuccess)
      return e;
    if ((e = launch_gemm_tile_apacked_silu(w.qx, w.sx, a.M, a.K, a.wgu, a.sgu, I2, w.act, a.I,
                                           stream)) != hipSuccess)
      return e;
    if ((e = launch_quant_rows_f32(w.act, a.M, a.I, a.I, w.qa, 0, w.sa, true, stream)) !=
        hipSuccess)
      return e;
    if ((e = launch_gemm_tile_apacked(w.qa, w.sa, a.M, a.I, a.wd, a.sd, a.N, a.y, a.ldy,
                                      stream)) != hipSuccess)
      return e;
  }
  // optional copies of the intermediates (row-major)
  if (a.dbg_act && (e = hipMemcpyAsync(a.dbg_act, w.act, (size_t)a.M * a.I * 4,
                                       hipMemcpyDeviceToDevice, stream)) != hipSuccess)
    return e;
  if (a.dbg_qa) {
    if (!tiled) {
      if ((e = hipMemcpyAsync(a.dbg_qa, w.qa, (size_t)a.M * a.I, hipMemcpyDeviceToDevice,
                              stream)) != hipSuccess)
        return e;
    } else {
      // the tiled path keeps its codes in the tile layout: the same quantiser
      // writes a row-major copy (and the same scales again)
      if ((e = launch_quant_rows_f32(w.act, a.M, a.I, a.I, a.dbg_qa, a.I,
                                     a.dbg_sa ? a.dbg_sa : w.sa, false, stream)) != hipSuccess)
        return e;
    }
  }
  if (a.dbg_sa && !(tiled && a.dbg_qa) &&
      (e = hipMemcpyAsync(a.dbg_sa, w.sa, (size_t)a.M * 4, hipMemcpyDeviceToDevice, stream)) !=
          hipSuccess)
    return e;
  return hipSuccess;
}

}  // namespace w8a8
