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
hipError_t launch_gemm_skinny_i32(const int8_t* qa, int64_t M, int64_t K, int64_t lda,
                                  const int8_t* qw, int64_t N, int64_t ldw, bool packed,
                                  int32_t* acc, int64_t ldacc, hipStream_t stream);
// The whole linear (bf16 rows -> codes -> GEMM -> bf16) in one launch, for
// the shapes linear_fused_fits accepts (one or two rows, packed weights).
bool linear_fused_fits(int64_t M, int64_t N, int64_t K);
hipError_t launch_linear_skinny_fused(const uint16_t* x, int64_t ldx, int64_t M, int64_t K,
                                      const int8_t* qw_packed, const float* sw, int64_t N,
                                      uint16_t* y, int64_t ldy, hipStream_t stream);

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

// Hadamard-domain variant.
hipError_t launch_fwht128_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int8_t* q,
                                int64_t ldq, float* s, hipStream_t stream);
hipError_t launch_fwht128_weight_prep(const float* W, int64_t N, int64_t K, int8_t* qw,
                                      uint8_t* su8, uint16_t* s2, hipStream_t stream);
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

}  // namespace w8a8
