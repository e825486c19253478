// Weight packing into MFMA operand tiles (done once, at load, like the weight
// quantisation itself).
//
// Packed layout of an int8 [N, K] weight (N % 16 == 0, K % 64 == 0): tile t
// holds rows 16t..16t+15; its 64-byte k step c is one contiguous 1 KiB block
// at byte offset (t * K/64 + c) * 1024, and inside the block the 16 bytes at
// offset 16*l are row 16t + (l % 16), columns 64c + 16*(l / 16) .. +15 -- the
// exact bytes lane l of a wave feeds to v_mfma_i32_16x16x64_i8 as its
// operand.  A wave therefore fetches a whole operand tile with one fully
// contiguous 1 KiB load, and an LDS copy of it needs no swizzle.  The layout
// is a pure permutation of bytes: values, scales and results are unchanged.
#include "kernels.h"

namespace w8a8 {

__global__ __launch_bounds__(256) void k_pack_weights(const int8_t* __restrict__ qw,
                                                      int64_t ldw, int64_t nchunk,
                                                      int64_t total16,
                                                      int8_t* __restrict__ out) {
  const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;  // 16-byte unit index
  if (o >= total16) return;
  const int64_t t = o / (nchunk * 64);
  const int64_t rem = o - t * nchunk * 64;
  const int64_t c = rem >> 6;
  const int l = (int)(rem & 63);
  const int8_t* src = qw + (t * 16 + (l & 15)) * ldw + c * 64 + (l >> 4) * 16;
  *reinterpret_cast<v4i*>(out + o * 16) = *reinterpret_cast<const v4i*>(src);
}

hipError_t launch_pack_weights(const int8_t* qw, int64_t N, int64_t K, int64_t ldw,
                               int8_t* out, hipStream_t stream) {
  const int64_t total16 = N * K / 16;
  const int64_t blocks = (total16 + 255) / 256;
  hipLaunchKernelGGL(k_pack_weights, dim3((unsigned)blocks), dim3(256), 0, stream, qw, ldw,
                     K / 64, total16, out);
  return hipGetLastError();
}

}  // namespace w8a8
