// Launch helpers of the gfx950 kernels (internal to libw8a8).  Each enqueues
// on `stream` and returns hipGetLastError(); shapes are validated by the
// caller (abi.hip) before any of these runs.
#pragma once

#include "common.h"

namespace w8a8 {

// Compute units of the current device, cached when the entry point checked
// the device (256 on MI355X).
int device_cus();

hipError_t launch_quant_rows(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                             int8_t* q, int64_t ldq, float* s, hipStream_t stream);

// Codes written in the packed tile layout of pack.hip (K % 64 == 0; rows up
// to the next multiple of 16 are left unwritten).
hipError_t launch_quant_rows_packed(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                    int8_t* q, float* s, hipStream_t stream);

// fp32 rows (the dense MLP's activation requant): codes row-major (ldq) or,
// with `packed`, in the tile layout.
hipError_t launch_quant_rows_f32(const float* x, int64_t M, int64_t K, int64_t ldx, int8_t* q,
                                 int64_t ldq, float* s, bool packed, hipStream_t stream);

// `packed`: weights in the MFMA tile layout of pack.hip instead of row-major.
hipError_t launch_pack_weights(const int8_t* qw, int64_t N, int64_t K, int64_t ldw,
                               int8_t* out, hipStream_t stream);
// Activation codes [M, K] (row stride ld) into the same tile layout, rows past
// M in the last tile as zeros; out holds ceil(M / 16) * 16 * K bytes.
hipError_t launch_pack_rows(const int8_t* q, int64_t M, int64_t K, int64_t ld, int8_t* out,
                            hipStream_t stream);

hipError_t launch_gemm_skinny(const int8_t* qa, const float* sa, int64_t M, int64_t K,
                              int64_t lda, const int8_t* qw, const float* sw, int64_t N,
                              int64_t ldw, bool packed, uint16_t* y, int64_t ldy,
                              hipStream_t stream);
// Gated SiLU epilogue over an interleaved gate/up weight of 2I = N packed rows:
// act [M, N/2] fp32 (row stride ldact).
hipError_t launch_gemm_skinny_silu(const int8_t* qa, const float* sa, int64_t M, int64_t K,
                                   int64_t lda, const int8_t* qw_packed, const float* sw,
                                   int64_t N, float* act, int64_t ldact, hipStream_t stream);
hipError_t launch_gemm_skinny_i32(const int8_t* qa, int64_t M, int64_t K, int64_t lda,
                                  const int8_t* qw, int64_t N, int64_t ldw, bool packed,
                                  int32_t* acc, int64_t ldacc, hipStream_t stream);
// The whole linear (bf16 rows -> codes -> GEMM -> bf16) in one launch, for
// the shapes linear_fused_fits accepts (one or two rows, packed weights).
bool linear_fused_fits(int64_t M, int64_t N, int64_t K);
hipError_t launch_linear_skinny_fused(const uint16_t* x, int64_t ldx, int64_t M, int64_t K,
                                      const int8_t* qw_packed, const float* sw, int64_t N,
                                      uint16_t* y, int64_t ldy, hipStream_t stream);
// The same for fp32 rows (quantised as k_quant_rows<float>); q_out / s_out
// (nullable) receive the codes (row-major, stride K) and the scales.
hipError_t launch_linear_skinny_fused_f32(const float* x, int64_t ldx, int64_t M, int64_t K,
                                          const int8_t* qw_packed, const float* sw, int64_t N,
                                          uint16_t* y, int64_t ldy, int8_t* q_out, float* s_out,
                                          hipStream_t stream);

hipError_t launch_gemm_tile(const int8_t* qa, const float* sa, int64_t M, int64_t K,
                            int64_t lda, const int8_t* qw, const float* sw, int64_t N,
                            int64_t ldw, bool packed, uint16_t* y, int64_t ldy,
                            hipStream_t stream);
hipError_t launch_gemm_tile_i32(const int8_t* qa, int64_t M, int64_t K, int64_t lda,
                                const int8_t* qw, int64_t N, int64_t ldw, bool packed,
                                int32_t* acc, int64_t ldacc, hipStream_t stream);
// Both operands packed (activations from launch_quant_rows_packed).
hipError_t launch_gemm_tile_apacked(const int8_t* qa_packed, const float* sa, int64_t M,
                                    int64_t K, const int8_t* qw_packed, const float* sw,
                                    int64_t N, uint16_t* y, int64_t ldy, hipStream_t stream);
hipError_t launch_gemm_tile_apacked_silu(const int8_t* qa_packed, const float* sa, int64_t M,
                                         int64_t K, const int8_t* qw_packed, const float* sw,
                                         int64_t N, float* act, int64_t ldact,
                                         hipStream_t stream);
hipError_t launch_gemm_tile_apacked_i32(const int8_t* qa_packed, int64_t M, int64_t K,
                                        const int8_t* qw_packed, int64_t N, int32_t* acc,
                                        int64_t ldacc, hipStream_t stream);

// Routed MoE.  Workspace layout is owned by moe.hip.
struct MoeArgs {
  const uint16_t* x;
  const float* logits;
  int T, H, E, I, k;
  const int8_t* w13;
  const float* s13;
  const int8_t* w2;
  const float* s2;
  int32_t* topk_ids;
  float* topk_w;
  uint16_t* out;
  void* ws;
  int8_t* dbg_qx;
  float* dbg_sx;
  int32_t* dbg_acc1;
  float* dbg_act;
  int8_t* dbg_qa;
  float* dbg_sa2;
  int32_t* dbg_acc2;
  bool packed;  // w13 / w2 in the packed tile layout (per expert, as [E*rows, cols])
};
size_t moe_workspace_bytes(int64_t T, int64_t H, int64_t E, int64_t I, int k);
hipError_t launch_moe_forward(const MoeArgs& a, hipStream_t stream);
// Hadamard-domain routed experts: w13 / w2 packed, s13 bf16 [E, 2I, H/128],
// s2 bf16 [E, H, I/128]; shared fp32 [T, H] or nullptr.  Same workspace as
// launch_moe_forward.
hipError_t launch_moe_rot_forward(const MoeArgs& a, const uint16_t* s13, const uint16_t* s2,
                                  const float* shared, hipStream_t stream);

// The shared expert in the Hadamard domain (dense: every token).
struct SharedArgs {
  const uint16_t* x;  // bf16 [T, H], rows contiguous
  int64_t T, H, Is;
  const int8_t* wgu;  // packed [2Is, H], rows 2i = gate_i, 2i+1 = up_i (rotated codes)
  const uint8_t* su8;  // [2Is, H/256]
  const uint16_t* s2;  // bf16 [2Is]
  const int8_t* wd;   // packed [H, Is] (rotated codes)
  const uint16_t* sd;  // bf16 [H, Is/128]
  float* y;           // fp32 [T, H]
  void* ws;
  float* dbg_act;     // optional [T, Is]
  int8_t* dbg_qa;     // optional [T, Is]
  float* dbg_sa;      // optional [T]
};
size_t shared_expert_workspace_bytes(int64_t T, int64_t H, int64_t Is);
hipError_t launch_shared_expert(const SharedArgs& a, hipStream_t stream);

// The Hadamard-domain routed layer with its shared expert in one call: one
// token in two launches (the shared expert inside them), else the shared
// expert, then the routed layer with its output as the shared term.
struct RotSharedW {
  int64_t Is;
  const int8_t* wgu;   // packed [2Is, H] (g256 codes)
  const uint8_t* su8;  // [2Is, H/256]
  const uint16_t* sgu;  // bf16 [2Is]
  const int8_t* wd;    // packed [H, Is] (g128 codes)
  const uint16_t* sd;  // bf16 [H, Is/128]
};
size_t moe_rot_shared_workspace_bytes(int64_t T, int64_t H, int64_t E, int64_t I, int k,
                                      int64_t Is);
hipError_t launch_moe_rot_shared_forward(const MoeArgs& a, const uint16_t* s13,
                                         const uint16_t* s2, const RotSharedW& sh,
                                         hipStream_t stream);

// Dense MLP block.  Workspace layout is owned by mlp.hip.
struct MlpArgs {
  const uint16_t* x;
  int64_t M, K, ldx, I, N, ldy;
  const int8_t* wgu;  // packed [2I, K], rows 2i = gate_i, 2i+1 = up_i
  const float* sgu;
  const int8_t* wd;   // packed [N, I]
  const float* sd;
  uint16_t* y;
  void* ws;
  float* dbg_act;
  int8_t* dbg_qa;
  float* dbg_sa;
};
size_t mlp_workspace_bytes(int64_t M, int64_t K, int64_t I);
hipError_t launch_mlp(const MlpArgs& a, hipStream_t stream);

// int8 KV-cache quantisation (f16 scale per token and head), D <= 4096.
hipError_t launch_kv_quant_i8(const uint16_t* x, int64_t T, int64_t Hk, int64_t D, int64_t ldx,
                              const int32_t* slots, int64_t cache_rows, int8_t* q, int64_t ldq,
                              uint16_t* s, int64_t lds, hipStream_t stream);

// Hadamard-domain variant.
hipError_t launch_fwht128_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int8_t* q,
                                int64_t ldq, float* s, hipStream_t stream);
hipError_t launch_fwht128_weight_prep(const float* W, int64_t N, int64_t K, int8_t* qw,
                                      uint8_t* su8, uint16_t* s2, hipStream_t stream);
hipError_t launch_fwht128_weight_prep_g128(const float* W, int64_t N, int64_t K, int8_t* qw,
                                           uint16_t* s, hipStream_t stream);
hipError_t launch_router_gate_bf16(const uint16_t* x, int64_t T, int64_t H, int64_t ldx,
                                   const uint16_t* wg, int64_t E, float* logits, int64_t ldl,
                                   hipStream_t stream);
size_t g256_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_fwht128_quant_packed(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                       int8_t* q, float* s, hipStream_t stream);
hipError_t launch_linear_g256(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                              const int8_t* qw_packed, const uint8_t* su8, const uint16_t* s2,
                              int64_t N, uint16_t* y, int64_t ldy, int8_t* q, float* s,
                              hipStream_t stream);
hipError_t launch_gemm_g256(const int8_t* qa, const float* sa, int64_t M, int64_t K,
                            const int8_t* qw, const uint8_t* su8, const uint16_t* s2, int64_t N,
                            bool packed, uint16_t* y, int64_t ldy, void* ws, hipStream_t stream);

// Measurement only: reads bytes / chunk contiguous chunks of buf once.
hipError_t launch_stream_read(const int8_t* buf, int64_t bytes, int64_t chunk, int32_t* sink,
                              hipStream_t stream);

}  // namespace w8a8
