// Packing into MFMA operand tiles: the weights once, at load (like the weight
// quantisation itself), and the activation codes of the packed-weight GEMM
// entry point for more than 16 rows.
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

// Rows into the layout (weights at load; activation codes for the tiled GEMM):
// workgroup (tile t, group g) moves rows 16t..16t+15, k bytes 256g..256g+255 (four 1 KiB
// blocks).  Rows are read as contiguous 256-byte stretches into LDS (a 16-byte
// pad per row puts the 16 rows of one 16-byte slice in 16 different 4-bank
// groups), then the four blocks go out as 4 KiB of consecutive 16-byte
// stores.  Rows past `rows` in the last tile are written as zeros (the GEMM
// never stores their results).
__global__ __launch_bounds__(256) void k_pack_rows(const int8_t* __restrict__ q, int64_t ld,
                                                   int64_t rows, int nchunk, int groups,
                                                   int64_t n_work, int8_t* __restrict__ out) {
  constexpr int kStride = 256 + 16;
  __shared__ __attribute__((aligned(16))) int8_t tl[16 * kStride];
  const int i = threadIdx.x;
  for (int64_t w = blockIdx.x; w < n_work; w += gridDim.x) {
    const int64_t t = w / groups;
    const int g = (int)(w - t * groups);
    const int nb = min(4, nchunk - 4 * g);  // 1 KiB blocks in this group
    {
      const int r = i >> 4, c16 = i & 15;  // row, 16-byte column of the stretch
      const int64_t row = t * 16 + r;
      v4i v = {0, 0, 0, 0};
      if (row < rows && c16 < nb * 4)
        v = *reinterpret_cast<const v4i*>(q + row * ld + (int64_t)g * 256 + c16 * 16);
      *reinterpret_cast<v4i*>(tl + r * kStride + c16 * 16) = v;
    }
    __syncthreads();
    const int b = i >> 6, slot = i & 63;  // block of the group, 16-byte slot in it
    if (b < nb) {
      const v4i v = *reinterpret_cast<const v4i*>(tl + (slot & 15) * kStride + b * 64 +
                                                  (slot >> 4) * 16);
      *reinterpret_cast<v4i*>(out + ((t * nchunk + 4 * g + b) * 1024) + slot * 16) = v;
    }
    __syncthreads();  // the next item overwrites tl
  }
}

hipError_t launch_pack_rows(const int8_t* q, int64_t M, int64_t K, int64_t ld, int8_t* out,
                            hipStream_t stream) {
  const int nchunk = (int)(K / 64);
  const int groups = (nchunk + 3) / 4;
  const int64_t n_work = (M + 15) / 16 * groups;
  const int64_t grid = n_work < ((int64_t)1 << 24) ? n_work : ((int64_t)1 << 24);
  hipLaunchKernelGGL(k_pack_rows, dim3((unsigned)grid), dim3(256), 0, stream, q, ld, M, nchunk,
                     groups, n_work, out);
  return hipGetLastError();
}

hipError_t launch_pack_weights(const int8_t* qw, int64_t N, int64_t K, int64_t ldw,
                               int8_t* out, hipStream_t stream) {
  return launch_pack_rows(qw, N, K, ldw, out, stream);  // N % 16 == 0: no padded rows
}

}  // namespace w8a8
