// C-ABI entry points of libw8a8 (declared in include/w8a8.h): argument
// validation, device check, workspace carving and kernel dispatch.  Nothing
// here allocates, synchronises or reads device memory on the host.
#include <atomic>
#include <cstring>

#include "../../include/w8a8.h"
#include "kernels.h"

using namespace w8a8;

namespace {

thread_local int g_last_hip_error = 0;

int hip_fail(hipError_t e) {
  g_last_hip_error = (int)e;
  return W8A8_HIP_ERROR;
}

// Device check, cached per device id (gfx950 only), with the CU count the
// launch plans use.
constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_ok[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other
std::atomic<int> g_dev_cus[kMaxDevices];

int check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return W8A8_UNSUPPORTED_DEVICE;
  int st = g_dev_ok[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e);
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_dev_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
    g_dev_ok[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? W8A8_OK : W8A8_UNSUPPORTED_DEVICE;
}

// Scratch of linear_w8a8_packed_noalloc: device memory of the library itself,
// one copy per GPU (each at its own address), held until the process ends.
// Host code never passes the array's name to a kernel (on the host it only
// names the symbol): the per-device address comes from hipGetSymbolAddress,
// taken once per device on the first call with that device current.
constexpr size_t kNoallocScratchBytes = W8A8_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) int8_t scratch[kNoallocScratchBytes];
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// The current device's copy of `scratch` (check_device() ran before).
int noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e);
    if (p == nullptr) return W8A8_HIP_ERROR;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return W8A8_OK;
}

}  // namespace

int w8a8::device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  const int n = g_dev_cus[dev].load(std::memory_order_relaxed);
  return n > 0 ? n : 256;
}

namespace {

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool al4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// activation codes in the workspace: rows rounded up to whole 16-row tiles
size_t act_codes_bytes(int64_t M, int64_t K) {
  return align_up((size_t)((M + 15) / 16 * 16) * (size_t)K);
}

// Shape rules shared by gemm_w8a8, gemm_w8a8_i32acc and linear_w8a8.
int check_gemm_shape(int64_t M, int64_t K, int64_t lda, int64_t N, int64_t ldw, int64_t ldo) {
  if (M < 0 || K <= 0 || N <= 0) return W8A8_INVALID_ARG;
  if (lda < K || ldw < K || ldo < N) return W8A8_INVALID_ARG;
  if (K % 64 != 0 || K > 131072 || N % 16 != 0 || N > (int64_t)1 << 30 ||
      M > (int64_t)1 << 30)
    return W8A8_UNSUPPORTED_SHAPE;
  if (lda % 16 != 0 || ldw % 16 != 0) return W8A8_MISALIGNED;
  return W8A8_OK;
}

int dispatch_gemm(const int8_t* qa, const float* sa, int64_t M, int64_t K, int64_t lda,
                  const int8_t* qw, const float* sw, int64_t N, int64_t ldw, bool packed,
                  uint16_t* y, int64_t ldy, hipStream_t st) {
  hipError_t e =
      (M <= 16) ? launch_gemm_skinny(qa, sa, M, K, lda, qw, sw, N, ldw, packed, y, ldy, st)
                : launch_gemm_tile(qa, sa, M, K, lda, qw, sw, N, ldw, packed, y, ldy, st);
  return e == hipSuccess ? W8A8_OK : hip_fail(e);
}

int dispatch_gemm_i32(const int8_t* qa, int64_t M, int64_t K, int64_t lda, const int8_t* qw,
                      int64_t N, int64_t ldw, bool packed, int32_t* acc, int64_t ldacc,
                      hipStream_t st) {
  hipError_t e =
      (M <= 16) ? launch_gemm_skinny_i32(qa, M, K, lda, qw, N, ldw, packed, acc, ldacc, st)
                : launch_gemm_tile_i32(qa, M, K, lda, qw, N, ldw, packed, acc, ldacc, st);
  return e == hipSuccess ? W8A8_OK : hip_fail(e);
}

int gemm_common(const int8_t* qa, const float* sa, int64_t M, int64_t K, int64_t lda,
                const int8_t* qw, const float* sw, int64_t N, int64_t ldw, bool packed,
                uint16_t* y, int64_t ldy, void* ws, size_t ws_bytes, void* stream) {
  int r = check_gemm_shape(M, K, lda, N, ldw, ldy);
  if (r != W8A8_OK) return r;
  if (M == 0) return W8A8_OK;
  if (!qa || !sa || !qw || !sw || !y) return W8A8_INVALID_ARG;
  if (!al16(qa) || !al16(qw) || !al4(sa) || !al4(sw) || !al4(y) || ldy % 2 != 0)
    return W8A8_MISALIGNED;
  // only the packed-weight path uses the workspace
  if (packed && ws_bytes < gemm_w8a8_workspace_bytes(M, N, K)) return W8A8_WORKSPACE_TOO_SMALL;
  if (packed && M > 16 && (!ws || !al16(ws))) return ws ? W8A8_MISALIGNED : W8A8_INVALID_ARG;
  if ((r = check_device()) != W8A8_OK) return r;
  hipStream_t st = as_stream(stream);
  if (packed && M > 16) {
    // the tiled GEMM reads its activation operand as contiguous 1 KiB tiles:
    // the row-major codes are repacked into the workspace first (row-major
    // operand loads fetch 16 half-line pieces per 1 KiB)
    int8_t* qp = static_cast<int8_t*>(ws);
    hipError_t e = launch_pack_rows(qa, M, K, lda, qp, st);
    if (e != hipSuccess) return hip_fail(e);
    e = launch_gemm_tile_apacked(qp, sa, M, K, qw, sw, N, y, ldy, st);
    return e == hipSuccess ? W8A8_OK : hip_fail(e);
  }
  return dispatch_gemm(qa, sa, M, K, lda, qw, sw, N, ldw, packed, y, ldy, st);
}

int gemm_i32_common(const int8_t* qa, int64_t M, int64_t K, int64_t lda, const int8_t* qw,
                    int64_t N, int64_t ldw, bool packed, int32_t* acc, int64_t ldacc,
                    void* ws, size_t ws_bytes, void* stream) {
  int r = check_gemm_shape(M, K, lda, N, ldw, ldacc);
  if (r != W8A8_OK) return r;
  if (M == 0) return W8A8_OK;
  if (!qa || !qw || !acc) return W8A8_INVALID_ARG;
  if (!al16(qa) || !al16(qw) || !al4(acc)) return W8A8_MISALIGNED;
  if (packed && ws_bytes < gemm_w8a8_workspace_bytes(M, N, K)) return W8A8_WORKSPACE_TOO_SMALL;
  if (packed && M > 16 && (!ws || !al16(ws))) return ws ? W8A8_MISALIGNED : W8A8_INVALID_ARG;
  if ((r = check_device()) != W8A8_OK) return r;
  hipStream_t st = as_stream(stream);
  if (packed && M > 16) {
    // as gemm_common: repacked activation codes, the same tiled kernel
    int8_t* qp = static_cast<int8_t*>(ws);
    hipError_t e = launch_pack_rows(qa, M, K, lda, qp, st);
    if (e != hipSuccess) return hip_fail(e);
    e = launch_gemm_tile_apacked_i32(qp, M, K, qw, N, acc, ldacc, st);
    return e == hipSuccess ? W8A8_OK : hip_fail(e);
  }
  return dispatch_gemm_i32(qa, M, K, lda, qw, N, ldw, packed, acc, ldacc, st);
}

int linear_common(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const int8_t* qw,
                  const float* sw, int64_t N, int64_t ldw, bool packed, uint16_t* y,
                  int64_t ldy, void* ws, size_t ws_bytes, void* stream) {
  int r = check_gemm_shape(M, K, ldx, N, ldw, ldy);
  if (r != W8A8_OK) return r;
  if (M == 0) return W8A8_OK;
  if (!x || !qw || !sw || !y) return W8A8_INVALID_ARG;
  if (!al16(x) || !al16(qw) || !al4(sw) || !al4(y) || ldy % 2 != 0 || ldx % 16 != 0)
    return W8A8_MISALIGNED;
  if (ws_bytes < linear_w8a8_workspace_bytes(M, N, K)) return W8A8_WORKSPACE_TOO_SMALL;
  if (!ws || !al16(ws)) return ws ? W8A8_MISALIGNED : W8A8_INVALID_ARG;
  if ((r = check_device()) != W8A8_OK) return r;
  hipStream_t st = as_stream(stream);
  int8_t* q = static_cast<int8_t*>(ws);
  float* s = reinterpret_cast<float*>(static_cast<char*>(ws) + act_codes_bytes(M, K));
  if (packed && M > 16) {
    // prefill: activation codes in the packed tile layout too, so both
    // operands stream as contiguous 1 KiB blocks
    hipError_t e = launch_quant_rows_packed(x, M, K, ldx, q, s, st);
    if (e != hipSuccess) return hip_fail(e);
    e = launch_gemm_tile_apacked(q, s, M, K, qw, sw, N, y, ldy, st);
    return e == hipSuccess ? W8A8_OK : hip_fail(e);
  }
  if (packed && linear_fused_fits(M, N, K)) {
    // one or two tokens: the quantisation inside the GEMM launch
    hipError_t e = launch_linear_skinny_fused(x, ldx, M, K, qw, sw, N, y, ldy, st);
    return e == hipSuccess ? W8A8_OK : hip_fail(e);
  }
  hipError_t e = launch_quant_rows(x, 0, M, K, ldx, q, K, s, st);
  if (e != hipSuccess) return hip_fail(e);
  return dispatch_gemm(q, s, M, K, K, qw, sw, N, ldw, packed, y, ldy, st);
}

}  // namespace

extern "C" {

const char* w8a8_status_string(int status) {
  switch (status) {
    case W8A8_OK: return "ok";
    case W8A8_INVALID_ARG: return "invalid argument";
    case W8A8_UNSUPPORTED_SHAPE: return "unsupported shape";
    case W8A8_MISALIGNED: return "misaligned pointer or row stride";
    case W8A8_WORKSPACE_TOO_SMALL: return "workspace too small";
    case W8A8_HIP_ERROR: return "HIP error";
    case W8A8_UNSUPPORTED_DEVICE: return "unsupported device (gfx950 required)";
    default: return "unknown status";
  }
}

int w8a8_last_hip_error(void) { return g_last_hip_error; }

int w8a8_version(void) { return 100; }

int quant_per_token_i8(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx, int8_t* q,
                       int64_t ldq, float* s, void* stream) {
  if (M < 0 || K <= 0 || ldx < K || ldq < K) return W8A8_INVALID_ARG;
  if (x_dtype != 0 && x_dtype != 1) return W8A8_INVALID_ARG;
  if (K % 16 != 0 || K > 65536 || M > INT32_MAX) return W8A8_UNSUPPORTED_SHAPE;
  if (M == 0) return W8A8_OK;
  if (!x || !q || !s) return W8A8_INVALID_ARG;
  if (!al16(x) || !al16(q) || !al4(s) || ldx % 16 != 0 || ldq % 16 != 0) return W8A8_MISALIGNED;
  int r = check_device();
  if (r != W8A8_OK) return r;
  hipError_t e = launch_quant_rows(x, x_dtype, M, K, ldx, q, ldq, s, as_stream(stream));
  return e == hipSuccess ? W8A8_OK : hip_fail(e);
}

size_t gemm_w8a8_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  // the tile-layout copy of the activation codes for the tiled GEMM (packed
  // weights; the row-major-weight calls use none)
  if (M <= 16 || N <= 0 || K <= 0) return 0;
  return act_codes_bytes(M, K);
}

int gemm_w8a8(const int8_t* qa, const float* sa, int64_t M, int64_t K, int64_t lda,
              const int8_t* qw, const float* sw, int64_t N, int64_t ldw, uint16_t* y,
              int64_t ldy, void* ws, size_t ws_bytes, void* stream) {
  return gemm_common(qa, sa, M, K, lda, qw, sw, N, ldw, false, y, ldy, ws, ws_bytes, stream);
}

int gemm_w8a8_i32acc(const int8_t* qa, int64_t M, int64_t K, int64_t lda, const int8_t* qw,
                     int64_t N, int64_t ldw, int32_t* acc, int64_t ldacc, void* ws,
                     size_t ws_bytes, void* stream) {
  return gemm_i32_common(qa, M, K, lda, qw, N, ldw, false, acc, ldacc, ws, ws_bytes, stream);
}

size_t linear_w8a8_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || K <= 0) return 0;
  (void)N;
  return act_codes_bytes(M, K) + align_up((size_t)M * 4);
}

int linear_w8a8(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const int8_t* qw,
                const float* sw, int64_t N, int64_t ldw, uint16_t* y, int64_t ldy, void* ws,
                size_t ws_bytes, void* stream) {
  return linear_common(x, M, K, ldx, qw, sw, N, ldw, false, y, ldy, ws, ws_bytes, stream);
}

int w8a8_pack_weights(const int8_t* qw, int64_t N, int64_t K, int64_t ldw, int8_t* qw_packed,
                      void* stream) {
  if (N < 0 || K <= 0 || ldw < K) return W8A8_INVALID_ARG;
  if (N % 16 != 0 || K % 64 != 0 || K > 131072 || N > (int64_t)1 << 30)
    return W8A8_UNSUPPORTED_SHAPE;
  if (N == 0) return W8A8_OK;
  if (!qw || !qw_packed) return W8A8_INVALID_ARG;
  if (!al16(qw) || !al16(qw_packed) || ldw % 16 != 0) return W8A8_MISALIGNED;
  int r = check_device();
  if (r != W8A8_OK) return r;
  hipError_t e = launch_pack_weights(qw, N, K, ldw, qw_packed, as_stream(stream));
  return e == hipSuccess ? W8A8_OK : hip_fail(e);
}

int gemm_w8a8_packed(const int8_t* qa, const float* sa, int64_t M, int64_t K, int64_t lda,
                     const int8_t* qw_packed, const float* sw, int64_t N, uint16_t* y,
                     int64_t ldy, void* ws, size_t ws_bytes, void* stream) {
  return gemm_common(qa, sa, M, K, lda, qw_packed, sw, N, K, true, y, ldy, ws, ws_bytes,
                     stream);
}

int gemm_w8a8_packed_i32acc(const int8_t* qa, int64_t M, int64_t K, int64_t lda,
                            const int8_t* qw_packed, int64_t N, int32_t* acc, int64_t ldacc,
                            void* ws, size_t ws_bytes, void* stream) {
  return gemm_i32_common(qa, M, K, lda, qw_packed, N, K, true, acc, ldacc, ws, ws_bytes,
                         stream);
}

int linear_w8a8_packed(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                       const int8_t* qw_packed, const float* sw, int64_t N, uint16_t* y,
                       int64_t ldy, void* ws, size_t ws_bytes, void* stream) {
  return linear_common(x, M, K, ldx, qw_packed, sw, N, K, true, y, ldy, ws, ws_bytes, stream);
}

int linear_w8a8_packed_noalloc(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                               const int8_t* qw_packed, const float* sw, int64_t N, uint16_t* y,
                               int64_t ldy, void* stream) {
  int r = check_gemm_shape(M, K, ldx, N, K, ldy);
  if (r != W8A8_OK) return r;
  if (M == 0) return W8A8_OK;
  // the codes and scales linear_w8a8_packed keeps in its workspace must fit
  // the static scratch
  if (linear_w8a8_workspace_bytes(M, N, K) > kNoallocScratchBytes) return W8A8_UNSUPPORTED_SHAPE;
  if ((r = check_device()) != W8A8_OK) return r;
  void* ws = nullptr;
  if ((r = noalloc_scratch(&ws)) != W8A8_OK) return r;
  return linear_common(x, M, K, ldx, qw_packed, sw, N, K, true, y, ldy, ws,
                       kNoallocScratchBytes, stream);
}

size_t mlp_w8a8_workspace_bytes(int64_t M, int64_t K, int64_t I, int64_t N) {
  if (M <= 0 || K <= 0 || I <= 0 || N <= 0) return 0;
  return mlp_workspace_bytes(M, K, I);
}

int mlp_w8a8_packed(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                    const int8_t* wgu_packed, const float* sgu, int64_t I,
                    const int8_t* wd_packed, const float* sd, int64_t N, uint16_t* y, int64_t ldy,
                    void* ws, size_t ws_bytes, const mlp_w8a8_debug* dbg, void* stream) {
  if (M < 0 || K <= 0 || I <= 0 || N <= 0 || ldx < K || ldy < N) return W8A8_INVALID_ARG;
  if (K % 64 != 0 || K > 131072 || I % 64 != 0 || I > 65536 || N % 16 != 0 ||
      N > (int64_t)1 << 30 || M > (int64_t)1 << 30)
    return W8A8_UNSUPPORTED_SHAPE;
  if (M == 0) return W8A8_OK;
  if (!x || !wgu_packed || !sgu || !wd_packed || !sd || !y) return W8A8_INVALID_ARG;
  if (!al16(x) || ldx % 16 != 0 || !al16(wgu_packed) || !al16(wd_packed) || !al4(sgu) ||
      !al4(sd) || !al4(y) || ldy % 2 != 0)
    return W8A8_MISALIGNED;
  if (dbg && ((dbg->act && !al16(dbg->act)) || (dbg->qa && !al16(dbg->qa)) ||
              (dbg->sa && !al4(dbg->sa))))
    return W8A8_MISALIGNED;
  if (ws_bytes < mlp_w8a8_workspace_bytes(M, K, I, N)) return W8A8_WORKSPACE_TOO_SMALL;
  if (!ws) return W8A8_INVALID_ARG;
  if (!al16(ws)) return W8A8_MISALIGNED;
  int r = check_device();
  if (r != W8A8_OK) return r;
  MlpArgs a{};
  a.x = x;
  a.M = M;
  a.K = K;
  a.ldx = ldx;
  a.I = I;
  a.N = N;
  a.ldy = ldy;
  a.wgu = wgu_packed;
  a.sgu = sgu;
  a.wd = wd_packed;
  a.sd = sd;
  a.y = y;
  a.ws = ws;
  if (dbg) {
    a.dbg_act = dbg->act;
    a.dbg_qa = dbg->qa;
    a.dbg_sa = dbg->sa;
  }
  hipError_t e = launch_mlp(a, as_stream(stream));
  return e == hipSuccess ? W8A8_OK : hip_fail(e);
}

int kv_quant_i8(const uint16_t* x, int64_t T, int64_t Hk, int64_t D, int64_t ldx,
                const int32_t* slots, int64_t cache_rows, int8_t* q_cache, int64_t ldq,
                uint16_t* s_cache, int64_t lds, void* stream) {
  if (T < 0 || Hk <= 0 || D <= 0 || cache_rows < 0 || ldx < Hk * D || ldq < Hk * D ||
      lds < Hk)
    return W8A8_INVALID_ARG;
  if (D % 8 != 0 || D > 4096 || Hk > 65536 || T > INT32_MAX || T * Hk > ((int64_t)1 << 32))
    return W8A8_UNSUPPORTED_SHAPE;
  if (!slots && cache_rows < T) return W8A8_INVALID_ARG;
  if (T == 0 || cache_rows == 0) return W8A8_OK;
  if (!x || !q_cache || !s_cache) return W8A8_INVALID_ARG;
  if (!al16(x) || ldx % 8 != 0 || (reinterpret_cast<uintptr_t>(q_cache) & 7u) != 0 ||
      ldq % 8 != 0 || (reinterpret_cast<uintptr_t>(s_cache) & 1u) != 0 ||
      (slots && !al4(slots)))
    return W8A8_MISALIGNED;
  int r = check_device();
  if (r != W8A8_OK) return r;
  hipError_t e = launch_kv_quant_i8(x, T, Hk, D, ldx, slots, cache_rows, q_cache, ldq, s_cache,
                                    lds, as_stream(stream));
  return e == hipSuccess ? W8A8_OK : hip_fail(e);
}

int w8a8_stream_read(const void* buf, int64_t bytes, int64_t chunk, int32_t* sink,
                     void* stream) {
  if (bytes <= 0 || chunk <= 0 || chunk % 1024 != 0 || bytes % chunk != 0 ||
      bytes / chunk > INT32_MAX)
    return W8A8_INVALID_ARG;
  if (!buf || !sink) return W8A8_INVALID_ARG;
  if (!al16(buf) || !al4(sink)) return W8A8_MISALIGNED;
  int r = check_device();
  if (r != W8A8_OK) return r;
  hipError_t e = launch_stream_read(static_cast<const int8_t*>(buf), bytes, chunk, sink,
                                    as_stream(stream));
  return e == hipSuccess ? W8A8_OK : hip_fail(e);
}

size_t moe_w8a8_workspace_bytes(int64_t T, int64_t H, int64_t E, int64_t I, int topk) {
  if (T <= 0 || H <= 0 || E <= 0 || I <= 0 || topk <= 0) return 0;
  return moe_workspace_bytes(T, H, E, I, topk);
}

static int moe_common(const uint16_t* x, const float* logits, int64_t T, int64_t H, int64_t E,
                      int64_t I, int topk, const int8_t* w13, const float* s13, const int8_t* w2,
                      const float* s2, int32_t* topk_ids, float* topk_w, uint16_t* out,
                      void* ws, size_t ws_bytes, const moe_w8a8_debug* dbg, bool packed,
                      void* stream) {
  if (T < 0 || H <= 0 || E <= 0 || I <= 0 || topk <= 0) return W8A8_INVALID_ARG;
  if (H % 64 != 0 || I % 64 != 0 || H > 16384 || I > 4096 || topk > 16 || topk > E ||
      E > 1024 || T * topk > ((int64_t)1 << 24))
    return W8A8_UNSUPPORTED_SHAPE;
  if (T == 0) return W8A8_OK;
  if (!x || !w13 || !s13 || !w2 || !s2 || !topk_ids || !topk_w || !out)
    return W8A8_INVALID_ARG;
  if (!al16(x) || !al16(w13) || !al16(w2) || !al4(s13) || !al4(s2) || !al4(topk_ids) ||
      !al4(topk_w) || !al16(out) || (logits && !al4(logits)))
    return W8A8_MISALIGNED;
  if (ws_bytes < moe_w8a8_workspace_bytes(T, H, E, I, topk)) return W8A8_WORKSPACE_TOO_SMALL;
  if (!ws) return W8A8_INVALID_ARG;
  if (!al16(ws)) return W8A8_MISALIGNED;
  int r = check_device();
  if (r != W8A8_OK) return r;
  MoeArgs a{};
  a.x = x;
  a.logits = logits;
  a.T = (int)T;
  a.H = (int)H;
  a.E = (int)E;
  a.I = (int)I;
  a.k = topk;
  a.w13 = w13;
  a.s13 = s13;
  a.w2 = w2;
  a.s2 = s2;
  a.topk_ids = topk_ids;
  a.topk_w = topk_w;
  a.out = out;
  a.ws = ws;
  a.packed = packed;
  if (dbg) {
    a.dbg_qx = dbg->qx;
    a.dbg_sx = dbg->sx;
    a.dbg_acc1 = dbg->acc1;
    a.dbg_act = dbg->act;
    a.dbg_qa = dbg->qa;
    a.dbg_sa2 = dbg->sa2;
    a.dbg_acc2 = dbg->acc2;
  }
  hipError_t e = launch_moe_forward(a, as_stream(stream));
  return e == hipSuccess ? W8A8_OK : hip_fail(e);
}

int moe_w8a8_forward(const uint16_t* x, const float* logits, int64_t T, int64_t H, int64_t E,
                     int64_t I, int topk, const int8_t* w13, const float* s13, const int8_t* w2,
                     const float* s2, int32_t* topk_ids, float* topk_w, uint16_t* out, void* ws,
                     size_t ws_bytes, const moe_w8a8_debug* dbg, void* stream) {
  return moe_common(x, logits, T, H, E, I, topk, w13, s13, w2, s2, topk_ids, topk_w, out, ws,
                    ws_bytes, dbg, false, stream);
}

int moe_w8a8_forward_packed(const uint16_t* x, const float* logits, int64_t T, int64_t H,
                            int64_t E, int64_t I, int topk, const int8_t* w13_packed,
                            const float* s13, const int8_t* w2_packed, const float* s2,
                            int32_t* topk_ids, float* topk_w, uint16_t* out, void* ws,
                            size_t ws_bytes, const moe_w8a8_debug* dbg, void* stream) {
  return moe_common(x, logits, T, H, E, I, topk, w13_packed, s13, w2_packed, s2, topk_ids,
                    topk_w, out, ws, ws_bytes, dbg, true, stream);
}

int fwht128_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int8_t* q, int64_t ldq,
                  float* s, void* stream) {
  if (M < 0 || K <= 0 || ldx < K || ldq < K) return W8A8_INVALID_ARG;
  if (K % 128 != 0 || K > 16384 || M > INT32_MAX) return W8A8_UNSUPPORTED_SHAPE;
  if (M == 0) return W8A8_OK;
  if (!x || !q || !s) return W8A8_INVALID_ARG;
  if (!al16(x) || !al16(q) || !al4(s) || ldx % 16 != 0 || ldq % 16 != 0) return W8A8_MISALIGNED;
  int r = check_device();
  if (r != W8A8_OK) return r;
  hipError_t e = launch_fwht128_quant(x, M, K, ldx, q, ldq, s, as_stream(stream));
  return e == hipSuccess ? W8A8_OK : hip_fail(e);
}

int fwht128_weight_prep_g256(const float* W, int64_t N, int64_t K, int8_t* qw, uint8_t* su8,
                             uint16_t* s2, void* stream) {
  if (N < 0 || K <= 0) return W8A8_INVALID_ARG;
  if (K % 256 != 0 || K > 16384 || N > INT32_MAX) return W8A8_UNSUPPORTED_SHAPE;
  if (N == 0) return W8A8_OK;
  if (!W || !qw || !su8 || !s2) return W8A8_INVALID_ARG;
  if (!al16(W) || !al16(qw)) return W8A8_MISALIGNED;
  int r = check_device();
  if (r != W8A8_OK) return r;
  hipError_t e = launch_fwht128_weight_prep(W, N, K, qw, su8, s2, as_stream(stream));
  return e == hipSuccess ? W8A8_OK : hip_fail(e);
}

int fwht128_weight_prep_g128(const float* W, int64_t N, int64_t K, int8_t* qw, uint16_t* s,
                             void* stream) {
  if (N < 0 || K <= 0) return W8A8_INVALID_ARG;
  if (K % 128 != 0 || K > 16384 || N > INT32_MAX) return W8A8_UNSUPPORTED_SHAPE;
  if (N == 0) return W8A8_OK;
  if (!W || !qw || !s) return W8A8_INVALID_ARG;
  if (!al16(W) || !al16(qw) || !al4(s)) return W8A8_MISALIGNED;
  int r = check_device();
  if (r != W8A8_OK) return r;
  hipError_t e = launch_fwht128_weight_prep_g128(W, N, K, qw, s, as_stream(stream));
  return e == hipSuccess ? W8A8_OK : hip_fail(e);
}

int router_gate_bf16(const uint16_t* x, int64_t T, int64_t H, int64_t ldx, const uint16_t* wg,
                     int64_t E, float* logits, int64_t ldl, void* stream) {
  if (T < 0 || H <= 0 || E <= 0 || ldx < H || ldl < E) return W8A8_INVALID_ARG;
  if (H % 32 != 0 || H > 16384 || E % 16 != 0 || E > 4096 || T > ((int64_t)1 << 22))
    return W8A8_UNSUPPORTED_SHAPE;
  if (T == 0) return W8A8_OK;
  if (!x || !wg || !logits) return W8A8_INVALID_ARG;
  if (!al16(x) || !al16(wg) || !al4(logits) || ldx % 8 != 0) return W8A8_MISALIGNED;
  int r = check_device();
  if (r != W8A8_OK) return r;
  hipError_t e = launch_router_gate_bf16(x, T, H, ldx, wg, E, logits, ldl, as_stream(stream));
  return e == hipSuccess ? W8A8_OK : hip_fail(e);
}

int moe_w8a8_rot_forward_packed(const uint16_t* x, const float* logits, int64_t T, int64_t H,
                                int64_t E, int64_t I, int topk, const int8_t* w13_packed,
                                const uint16_t* s13, const int8_t* w2_packed,
                                const uint16_t* s2, const float* shared, int32_t* topk_ids,
                                float* topk_w, uint16_t* out, void* ws, size_t ws_bytes,
                                const moe_w8a8_debug* dbg, void* stream) {
  if (T < 0 || H <= 0 || E <= 0 || I <= 0 || topk <= 0) return W8A8_INVALID_ARG;
  if (H % 256 != 0 || I % 128 != 0 || H > 4096 || I > 2048 || topk > 16 || topk > E ||
      E > 1024 || T * topk > ((int64_t)1 << 24))
    return W8A8_UNSUPPORTED_SHAPE;
  if (T == 0) return W8A8_OK;
  if (!x || !w13_packed || !s13 || !w2_packed || !s2 || !topk_ids || !topk_w || !out)
    return W8A8_INVALID_ARG;
  if (!al16(x) || !al16(w13_packed) || !al16(w2_packed) || !al4(s13) || !al4(s2) ||
      !al4(topk_ids) || !al4(topk_w) || !al16(out) || (logits && !al4(logits)) ||
      (shared && !al16(shared)))
    return W8A8_MISALIGNED;
  if (ws_bytes < moe_w8a8_workspace_bytes(T, H, E, I, topk)) return W8A8_WORKSPACE_TOO_SMALL;
  if (!ws) return W8A8_INVALID_ARG;
  if (!al16(ws)) return W8A8_MISALIGNED;
  int r = check_device();
  if (r != W8A8_OK) return r;
  MoeArgs a{};
  a.x = x;
  a.logits = logits;
  a.T = (int)T;
  a.H = (int)H;
  a.E = (int)E;
  a.I = (int)I;
  a.k = topk;
  a.w13 = w13_packed;
  a.w2 = w2_packed;
  a.topk_ids = topk_ids;
  a.topk_w = topk_w;
  a.out = out;
  a.ws = ws;
  a.packed = true;
  if (dbg) {
    a.dbg_qx = dbg->qx;
    a.dbg_sx = dbg->sx;
    a.dbg_act = dbg->act;
    a.dbg_qa = dbg->qa;
    a.dbg_sa2 = dbg->sa2;
  }
  hipError_t e = launch_moe_rot_forward(a, s13, s2, shared, as_stream(stream));
  return e == hipSuccess ? W8A8_OK : hip_fail(e);
}

size_t moe_w8a8_rot_shared_workspace_bytes(int64_t T, int64_t H, int64_t E, int64_t I,
                                           int topk, int64_t Is) {
  if (T <= 0 || H <= 0 || E <= 0 || I <= 0 || topk <= 0 || Is <= 0) return 0;
  return moe_rot_shared_workspace_bytes(T, H, E, I, topk, Is);
}

int moe_w8a8_rot_shared_forward_packed(
    const uint16_t* x, const float* logits, int64_t T, int64_t H, int64_t E, int64_t I,
    int topk, const int8_t* w13_packed, const uint16_t* s13, const int8_t* w2_packed,
    const uint16_t* s2, int64_t Is, const int8_t* wgu_packed, const uint8_t* su8,
    const uint16_t* sgu, const int8_t* wd_packed, const uint16_t* sd, int32_t* topk_ids,
    float* topk_w, uint16_t* out, void* ws, size_t ws_bytes, const moe_w8a8_debug* dbg,
    void* stream) {
  if (T < 0 || H <= 0 || E <= 0 || I <= 0 || topk <= 0 || Is <= 0) return W8A8_INVALID_ARG;
  if (H % 256 != 0 || I % 128 != 0 || Is % 128 != 0 || H > 4096 || I > 2048 || Is > 2048 ||
      topk > 16 || topk > E || E > 1024 || T * topk > ((int64_t)1 << 24))
    return W8A8_UNSUPPORTED_SHAPE;
  if (T == 0) return W8A8_OK;
  if (!x || !w13_packed || !s13 || !w2_packed || !s2 || !wgu_packed || !su8 || !sgu ||
      !wd_packed || !sd || !topk_ids || !topk_w || !out)
    return W8A8_INVALID_ARG;
  if (!al16(x) || !al16(w13_packed) || !al16(w2_packed) || !al4(s13) || !al4(s2) ||
      !al16(wgu_packed) || !al16(wd_packed) || !al4(sd) || !al4(topk_ids) || !al4(topk_w) ||
      !al16(out) || (logits && !al4(logits)))
    return W8A8_MISALIGNED;
  if (ws_bytes < moe_w8a8_rot_shared_workspace_bytes(T, H, E, I, topk, Is))
    return W8A8_WORKSPACE_TOO_SMALL;
  if (!ws) return W8A8_INVALID_ARG;
  if (!al16(ws)) return W8A8_MISALIGNED;
  int r = check_device();
  if (r != W8A8_OK) return r;
  MoeArgs a{};
  a.x = x;
  a.logits = logits;
  a.T = (int)T;
  a.H = (int)H;
  a.E = (int)E;
  a.I = (int)I;
  a.k = topk;
  a.w13 = w13_packed;
  a.w2 = w2_packed;
  a.topk_ids = topk_ids;
  a.topk_w = topk_w;
  a.out = out;
  a.ws = ws;
  a.packed = true;
  if (dbg) {
    a.dbg_qx = dbg->qx;
    a.dbg_sx = dbg->sx;
    a.dbg_act = dbg->act;
    a.dbg_qa = dbg->qa;
    a.dbg_sa2 = dbg->sa2;
  }
  RotSharedW sh{Is, wgu_packed, su8, sgu, wd_packed, sd};
  hipError_t e = launch_moe_rot_shared_forward(a, s13, s2, sh, as_stream(stream));
  return e == hipSuccess ? W8A8_OK : hip_fail(e);
}

size_t shared_expert_w8a8_rot_workspace_bytes(int64_t T, int64_t H, int64_t Is) {
  if (T <= 0 || H <= 0 || Is <= 0) return 0;
  return shared_expert_workspace_bytes(T, H, Is);
}

int shared_expert_w8a8_rot_packed(const uint16_t* x, int64_t T, int64_t H, int64_t Is,
                                  const int8_t* wgu_packed, const uint8_t* su8,
                                  const uint16_t* s2, const int8_t* wd_packed,
                                  const uint16_t* sd, float* y, void* ws, size_t ws_bytes,
                                  const shared_expert_debug* dbg, void* stream) {
  if (T < 0 || H <= 0 || Is <= 0) return W8A8_INVALID_ARG;
  if (H % 256 != 0 || Is % 128 != 0 || H > 4096 || Is > 2048 || T > ((int64_t)1 << 24))
    return W8A8_UNSUPPORTED_SHAPE;
  if (T == 0) return W8A8_OK;
  if (!x || !wgu_packed || !su8 || !s2 || !wd_packed || !sd || !y) return W8A8_INVALID_ARG;
  if (!al16(x) || !al16(wgu_packed) || !al16(wd_packed) || !al4(sd) || !al16(y))
    return W8A8_MISALIGNED;
  if (ws_bytes < shared_expert_w8a8_rot_workspace_bytes(T, H, Is))
    return W8A8_WORKSPACE_TOO_SMALL;
  if (!ws) return W8A8_INVALID_ARG;
  if (!al16(ws)) return W8A8_MISALIGNED;
  int r = check_device();
  if (r != W8A8_OK) return r;
  SharedArgs a{};
  a.x = x;
  a.T = T;
  a.H = H;
  a.Is = Is;
  a.wgu = wgu_packed;
  a.su8 = su8;
  a.s2 = s2;
  a.wd = wd_packed;
  a.sd = sd;
  a.y = y;
  a.ws = ws;
  if (dbg) {
    a.dbg_act = dbg->act;
    a.dbg_qa = dbg->qa;
    a.dbg_sa = dbg->sa;
  }
  hipError_t e = launch_shared_expert(a, as_stream(stream));
  return e == hipSuccess ? W8A8_OK : hip_fail(e);
}

size_t gemm_w8a8_g256_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  return g256_workspace_bytes(M, N, K);
}

static int g256_common(const int8_t* qa, const float* sa, int64_t M, int64_t K,
                       const int8_t* qw, const uint8_t* su8, const uint16_t* s2, int64_t N,
                       bool packed, uint16_t* y, int64_t ldy, void* ws, size_t ws_bytes,
                       void* stream) {
  if (M < 0 || K <= 0 || N <= 0 || ldy < N) return W8A8_INVALID_ARG;
  if (K % 256 != 0 || K > 16384 || N % 16 != 0 || N > (int64_t)1 << 30 || M > (int64_t)1 << 30)
    return W8A8_UNSUPPORTED_SHAPE;
  if (M == 0) return W8A8_OK;
  if (!qa || !sa || !qw || !su8 || !s2 || !y) return W8A8_INVALID_ARG;
  if (!al16(qa) || !al16(qw) || !al4(sa) || !al4(y) || ldy % 2 != 0) return W8A8_MISALIGNED;
  if (ws_bytes < gemm_w8a8_g256_workspace_bytes(M, N, K)) return W8A8_WORKSPACE_TOO_SMALL;
  int r = check_device();
  if (r != W8A8_OK) return r;
  hipError_t e =
      launch_gemm_g256(qa, sa, M, K, qw, su8, s2, N, packed, y, ldy, ws, as_stream(stream));
  return e == hipSuccess ? W8A8_OK : hip_fail(e);
}

size_t linear_w8a8_g256_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || K <= 0) return 0;
  return act_codes_bytes(M, K) + align_up((size_t)M * 4);
}

int linear_w8a8_g256_packed(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                            const int8_t* qw_packed, const uint8_t* su8, const uint16_t* s2,
                            int64_t N, uint16_t* y, int64_t ldy, void* ws, size_t ws_bytes,
                            void* stream) {
  if (M < 0 || K <= 0 || N <= 0 || ldx < K || ldy < N) return W8A8_INVALID_ARG;
  if (K % 256 != 0 || K > 16384 || N % 16 != 0 || N > (int64_t)1 << 30 || M > (int64_t)1 << 30)
    return W8A8_UNSUPPORTED_SHAPE;
  if (M == 0) return W8A8_OK;
  if (!x || !qw_packed || !su8 || !s2 || !y) return W8A8_INVALID_ARG;
  if (!al16(x) || !al16(qw_packed) || !al4(y) || ldy % 2 != 0 || ldx % 16 != 0)
    return W8A8_MISALIGNED;
  if (ws_bytes < linear_w8a8_g256_workspace_bytes(M, N, K)) return W8A8_WORKSPACE_TOO_SMALL;
  if (!ws || !al16(ws)) return ws ? W8A8_MISALIGNED : W8A8_INVALID_ARG;
  int r = check_device();
  if (r != W8A8_OK) return r;
  int8_t* q = static_cast<int8_t*>(ws);
  float* s = reinterpret_cast<float*>(static_cast<char*>(ws) + act_codes_bytes(M, K));
  hipError_t e =
      launch_linear_g256(x, M, K, ldx, qw_packed, su8, s2, N, y, ldy, q, s, as_stream(stream));
  return e == hipSuccess ? W8A8_OK : hip_fail(e);
}

int gemm_w8a8_g256(const int8_t* qa, const float* sa, int64_t M, int64_t K, const int8_t* qw,
                   const uint8_t* su8, const uint16_t* s2, int64_t N, uint16_t* y, int64_t ldy,
                   void* ws, size_t ws_bytes, void* stream) {
  return g256_common(qa, sa, M, K, qw, su8, s2, N, false, y, ldy, ws, ws_bytes, stream);
}

int gemm_w8a8_g256_packed(const int8_t* qa, const float* sa, int64_t M, int64_t K,
                          const int8_t* qw_packed, const uint8_t* su8, const uint16_t* s2,
                          int64_t N, uint16_t* y, int64_t ldy, void* ws, size_t ws_bytes,
                          void* stream) {
  return g256_common(qa, sa, M, K, qw_packed, su8, s2, N, true, y, ldy, ws, ws_bytes, stream);
}

}  // extern "C"
