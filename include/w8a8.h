/*
 * libw8a8 - online INT8 W8A8 linear layers, the routed int8 MoE layer and the
 * Hadamard-domain (fwht128, g256) variant, as hand-written HIP kernels for
 * AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages; titles abbreviated):
 *   [ATOM]  "[gfx1151] Online INT8 W8A8 for Qwen3.6 27B / 35B-A3B on RDNA3.5,
 *            with working MTP" (ATOM pull request), "Changes" section.
 *   [QUARK] "Qwen3.6-27B-Quark-W8A8-INT8" model card, "Quantization Scheme".
 *   [IQ8R]  "Qwen3.6-35B-A3B IQ8R - radiance container", file table and the
 *            recipe under "How this file was made".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *    library keeps no reference after a call returns, never allocates device
 *    memory and never synchronises: work is enqueued on `stream` (a
 *    hipStream_t passed as void*; NULL = the legacy default stream) and the
 *    call returns at once, so the calls can be captured into a HIP graph.
 *  - Matrices are row-major with the last dimension contiguous; ld* is the
 *    row stride in elements.  Weights are [N, K]: one row per output channel.
 *    bf16 values are passed as uint16_t bit patterns.
 *  - Scratch memory comes from a caller-provided workspace `ws` of
 *    `ws_bytes` bytes, sized by the matching *_workspace_bytes() function.
 *    Its contents need no initialisation and are undefined after the call.
 *  - A size of zero (M == 0 or T == 0) is a no-op that returns W8A8_OK.
 *  - Arguments are validated before anything is enqueued: a rejected call
 *    launches nothing and leaves every output untouched.
 *  - Return value: W8A8_OK (0) or a negative w8a8_status.  Launch failures
 *    return W8A8_HIP_ERROR; the HIP error code is kept per thread and read
 *    with w8a8_last_hip_error().  Faults inside a kernel surface at the
 *    caller's next synchronisation, as in any HIP program.
 *  - Calls are re-entrant and thread-safe.  Calls that share a workspace
 *    must be ordered on one stream.
 */
#ifndef W8A8_H
#define W8A8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum w8a8_status {
    W8A8_OK = 0,
    W8A8_INVALID_ARG = -1,         /* null pointer, negative size, ld < row length */
    W8A8_UNSUPPORTED_SHAPE = -2,   /* a size the kernels do not handle (see each call) */
    W8A8_MISALIGNED = -3,          /* pointer or row stride not 16-byte aligned */
    W8A8_WORKSPACE_TOO_SMALL = -4, /* ws_bytes below the *_workspace_bytes() value */
    W8A8_HIP_ERROR = -5,           /* a HIP call or kernel launch failed */
    W8A8_UNSUPPORTED_DEVICE = -6   /* the current device is not gfx950 */
} w8a8_status;

/* Human-readable name of a status code (static string, never NULL). */
const char *w8a8_status_string(int status);

/* The hipError_t of the last W8A8_HIP_ERROR returned on this thread (0 if none). */
int w8a8_last_hip_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int w8a8_version(void);

/* ------------------------------------------------------------------------ */
/* Per-row dynamic int8 quantisation.                                        */
/* [QUARK] Quantization Scheme: activations INT8 per token (ch_axis=1) and   */
/* weights INT8 per channel (ch_axis=0), both symmetric.  [IQ8R] Trunk row:  */
/* codes -127..127, round to nearest.                                        */
/*   s[m] = max_k |x[m,k]| / 127            (fp32, IEEE division)            */
/*   q[m,k] = clamp(round_half_even(x[m,k] / s[m]), -127, 127)               */
/* An all-zero row gets s = 0 and q = 0.  Inputs must be finite.             */
/* x: [M, K], x_dtype 0 = bf16 (uint16 bits), 1 = fp32 (weight preparation  */
/*    uses the same arithmetic on fp32 rows); row stride ldx elements.       */
/* q: int8 [M, K], row stride ldq; s: fp32 [M].                              */
/* Requires K % 16 == 0 and 1 <= K <= 65536; x, q 16-byte aligned and ldx,   */
/* ldq multiples of 16 elements.                                             */
/* ------------------------------------------------------------------------ */
int quant_per_token_i8(const void *x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                       int8_t *q, int64_t ldq, float *s, void *stream);

/* ------------------------------------------------------------------------ */
/* W8A8 GEMM with the per-token x per-channel epilogue.                      */
/* [ATOM] Changes, linear.py bullet: int8 activations (per token) times int8 */
/* weights (per channel, fp32 scales), bf16 out.                             */
/*   acc[m,n] = sum_k qa[m,k] * qw[n,k]                     (exact int32)    */
/*   y[m,n]   = bf16_rne( (float(acc[m,n]) * sa[m]) * sw[n] )  (fp32)        */
/* qa: int8 [M, K] (lda), sa: fp32 [M]; qw: int8 [N, K] (ldw), sw: fp32 [N]; */
/* y: bf16 [M, N] (ldy).  M <= 16 runs the weight-streaming decode kernel,   */
/* larger M the LDS-tiled MFMA kernel.  gemm_w8a8 and gemm_w8a8_i32acc use  */
/* no workspace (ws may be NULL).  The packed-weight variants below need     */
/* gemm_w8a8_workspace_bytes(M, N, K): none for M <= 16, else                */
/* ceil(M/16)*16*K bytes, where they repack the activation codes into the    */
/* tile layout described at w8a8_pack_weights.                               */
/* Requires K % 64 == 0, K <= 131072, N % 16 == 0; qa, qw 16-byte aligned;   */
/* lda, ldw multiples of 16; y 4-byte aligned and ldy even.                  */
/* ------------------------------------------------------------------------ */
size_t gemm_w8a8_workspace_bytes(int64_t M, int64_t N, int64_t K);
int gemm_w8a8(const int8_t *qa, const float *sa, int64_t M, int64_t K, int64_t lda,
              const int8_t *qw, const float *sw, int64_t N, int64_t ldw, uint16_t *y,
              int64_t ldy, void *ws, size_t ws_bytes, void *stream);

/* The same kernels as gemm_w8a8 with the epilogue replaced by a store of the */
/* exact int32 sums acc[m,n] (int32 [M, N], row stride ldacc).  For tests.   */
int gemm_w8a8_i32acc(const int8_t *qa, int64_t M, int64_t K, int64_t lda, const int8_t *qw,
                     int64_t N, int64_t ldw, int32_t *acc, int64_t ldacc, void *ws,
                     size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------ */
/* The whole online W8A8 linear: bf16 x -> per-token int8 (as               */
/* quant_per_token_i8) -> GEMM and epilogue (as gemm_w8a8) -> bf16 y.        */
/* The codes and scales go to the workspace, except where the quantisation   */
/* runs inside the GEMM launch (one or two tokens, packed weights, few       */
/* output tiles a CU).  Same shape rules as gemm_w8a8; x 16-byte aligned     */
/* with ldx a multiple of 16.                                                */
/* ------------------------------------------------------------------------ */
size_t linear_w8a8_workspace_bytes(int64_t M, int64_t N, int64_t K);
int linear_w8a8(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, const int8_t *qw,
                const float *sw, int64_t N, int64_t ldw, uint16_t *y, int64_t ldy, void *ws,
                size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------ */
/* Packed weight layout (done once, at load, like the weight quantisation).  */
/* A pure byte permutation of an int8 [N, K] weight into MFMA operand tiles: */
/* tile t = rows 16t..16t+15; its 64-byte k step c is the contiguous 1 KiB   */
/* block at offset (t * K/64 + c) * 1024; inside it the 16 bytes at offset   */
/* 16*l are row 16t + (l % 16), columns 64c + 16*(l / 16) .. +15.  Every     */
/* wave-wide weight load then reads 1 KiB of consecutive bytes.              */
/* qw: int8 [N, K] row-major (ldw); qw_packed: int8, N*K bytes, must not     */
/* overlap qw.  Requires N % 16 == 0, K % 64 == 0, K <= 131072.              */
/* ------------------------------------------------------------------------ */
int w8a8_pack_weights(const int8_t *qw, int64_t N, int64_t K, int64_t ldw, int8_t *qw_packed,
                      void *stream);

/* gemm_w8a8 / gemm_w8a8_i32acc / linear_w8a8 with packed weights: same      */
/* arithmetic, same results, same shape rules (weight row stride is implied). */
int gemm_w8a8_packed(const int8_t *qa, const float *sa, int64_t M, int64_t K, int64_t lda,
                     const int8_t *qw_packed, const float *sw, int64_t N, uint16_t *y,
                     int64_t ldy, void *ws, size_t ws_bytes, void *stream);
int gemm_w8a8_packed_i32acc(const int8_t *qa, int64_t M, int64_t K, int64_t lda,
                            const int8_t *qw_packed, int64_t N, int32_t *acc, int64_t ldacc,
                            void *ws, size_t ws_bytes, void *stream);
int linear_w8a8_packed(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                       const int8_t *qw_packed, const float *sw, int64_t N, uint16_t *y,
                       int64_t ldy, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------ */
/* linear_w8a8_packed for callers that cannot allocate device memory (code   */
/* under HIP-graph capture, tight serving loops, harnesses that forbid       */
/* allocation): the same kernels and results, but the activation codes and  */
/* scales go to scratch memory the library itself holds -- a static device  */
/* array of W8A8_NOALLOC_SCRATCH_BYTES (32 MiB) on every GPU it runs on,     */
/* kept until the process ends -- instead of a caller workspace.  No         */
/* allocation happens in the call.  Shapes whose                             */
/* linear_w8a8_workspace_bytes(M, N, K) exceeds that size (e.g. 4096 tokens  */
/* at K = 5120 fit, 4096 at K = 8704 do not) return W8A8_UNSUPPORTED_SHAPE   */
/* and launch nothing.  Every call on one GPU shares that GPU's scratch: two */
/* calls that can overlap on one GPU (different streams without ordering,   */
/* different threads) race and give undefined results; calls ordered on one */
/* stream are safe.  Other arguments and rules as linear_w8a8_packed.        */
/* ------------------------------------------------------------------------ */
#define W8A8_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int linear_w8a8_packed_noalloc(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                               const int8_t *qw_packed, const float *sw, int64_t N,
                               uint16_t *y, int64_t ldy, void *stream);

/* ------------------------------------------------------------------------ */
/* Dense W8A8 MLP block.  [ATOM] intro: A8W8 for all dense GEMMs (the 27B    */
/* dense model of its "Performance" section); the order of its "Changes",    */
/* fused_moe_triton.py bullet (gemm1 with the gated SiLU over interleaved    */
/* gate/up rows, per-token int8 requant, gemm2) on the dense gate_up and     */
/* down linears:                                                             */
/*   qx, sx = per-token quant of x (as quant_per_token_i8)                    */
/*   h[m,c]   = (float(sum_k qx[m,k] wgu[c,k]) * sx[m]) * sgu[c],  c < 2I     */
/*   act[m,i] = silu(h[m,2i]) * h[m,2i+1]   (row 2i = gate_i, 2i+1 = up_i;   */
/*              silu(g) = g / (1 + exp(-g)) in fp64, rounded to fp32)       */
/*   qa, sa   = per-token quant of the fp32 act rows                         */
/*   y[m,n]   = bf16_rne((float(sum_i qa[m,i] wd[n,i]) * sa[m]) * sd[n])      */
/* x: bf16 [M, K] (ldx); wgu_packed: int8 [2I, K] in the packed tile layout  */
/* (w8a8_pack_weights), sgu fp32 [2I]; wd_packed: int8 [N, I] packed, sd     */
/* fp32 [N]; y: bf16 [M, N] (ldy).  A checkpoint with concatenated [gate;    */
/* up] rows is permuted to the interleaved order at load.                    */
/* Workspace: mlp_w8a8_workspace_bytes(M, K, I, N) (codes, scales and the    */
/* fp32 activation rows).  Requires K % 64 == 0, K <= 131072, I % 64 == 0,   */
/* I <= 65536, N % 16 == 0; x, weights, ws 16-byte aligned, ldx a multiple  */
/* of 16, y 4-byte aligned with even ldy.                                    */
/* dbg (nullable; each member nullable, 16-byte aligned): row-major copies   */
/* of the intermediates act fp32 [M, I], qa int8 [M, I], sa fp32 [M].        */
/* ------------------------------------------------------------------------ */
typedef struct mlp_w8a8_debug {
    float *act;  /* [M, I] */
    int8_t *qa;  /* [M, I] */
    float *sa;   /* [M] */
} mlp_w8a8_debug;

size_t mlp_w8a8_workspace_bytes(int64_t M, int64_t K, int64_t I, int64_t N);
int mlp_w8a8_packed(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                    const int8_t *wgu_packed, const float *sgu, int64_t I,
                    const int8_t *wd_packed, const float *sd, int64_t N, uint16_t *y,
                    int64_t ldy, void *ws, size_t ws_bytes, const mlp_w8a8_debug *dbg,
                    void *stream);

/* ------------------------------------------------------------------------ */
/* int8 KV-cache quantisation.  [IQ8R] Serve: kv-cache-dtype i8 stores the   */
/* attention cache as int8 with an f16 scale per token and head.  For every  */
/* token t and head h, the D values x[t, h, :] (bf16):                       */
/*   s = f16_rne(max_d |x| / 127)        (fp32 quotient, then binary16)      */
/*   q = clamp(round_half_even(x / float(s)), -127, 127); q = 0 if s == 0     */
/* (codes against the stored f16 scale: code * s is the cached value).      */
/* Token t is written to cache row slots[t] (slots NULL: row t); a slot      */
/* outside [0, cache_rows) skips the token.  Precondition: max |x| / 127     */
/* below 65520 (a finite f16 scale; an infinite one gives zero codes).      */
/* x: bf16 [T, Hk, D], token stride ldx >= Hk*D elements (heads contiguous); */
/* q_cache: int8 [cache_rows, Hk, D], row stride ldq >= Hk*D;                */
/* s_cache: f16 bits [cache_rows, Hk], row stride lds >= Hk.  No workspace.  */
/* Requires D % 8 == 0, D <= 4096; x 16-byte aligned with ldx % 8 == 0,      */
/* q_cache 8-byte aligned with ldq % 8 == 0, s_cache 2-byte aligned; without */
/* slots cache_rows >= T.                                                    */
/* ------------------------------------------------------------------------ */
int kv_quant_i8(const uint16_t *x, int64_t T, int64_t Hk, int64_t D, int64_t ldx,
                const int32_t *slots, int64_t cache_rows, int8_t *q_cache, int64_t ldq,
                uint16_t *s_cache, int64_t lds, void *stream);

/* ------------------------------------------------------------------------ */
/* Measurement helper, not part of the method: reads `bytes` of `buf` once, */
/* one 512-thread workgroup per `chunk` contiguous bytes, each wave keeping */
/* ten 1 KiB loads in flight (the access pattern of the decode GEMM).  The  */
/* time of such a read is the streaming ceiling the GEMM's HBM fraction is  */
/* compared with.  sink: int32 [1], written only for one bit pattern of the */
/* data (never for a buffer of zeros).  Requires chunk a positive multiple  */
/* of 1024, bytes a positive multiple of chunk with bytes / chunk < 2^31;   */
/* buf 16-byte aligned.  No workspace; buf is not modified.                  */
/* ------------------------------------------------------------------------ */
int w8a8_stream_read(const void *buf, int64_t bytes, int64_t chunk, int32_t *sink, void *stream);

/* ------------------------------------------------------------------------ */
/* Routed int8 MoE layer.                                                    */
/* [ATOM] Changes, fused_moe_triton.py bullet: routing -> per-token int8     */
/* quant -> gemm1 with fused gated SiLU over interleaved w13 -> per-token    */
/* int8 quant -> gemm2 with scatter/combine; moe.py bullet: int8 w13/w2 with */
/* per-channel fp32 scales.                                                  */
/*   routing (if logits != NULL): softmax over E, keep the top-k (slot j =   */
/*     j-th largest logit, ties to the lower expert index), renormalise the  */
/*     kept probabilities; ids/weights are written to topk_ids/topk_w.       */
/*     If logits == NULL, topk_ids/topk_w are inputs (ids in [0, E)).        */
/*   qx, sx = per-token quant of x (once per token, shared by its k pairs)   */
/*   for pair r = t*k + j, e = topk_ids[t,j]:                                */
/*     h[c]   = (float(sum_h qx[t,h] w13[e,c,h]) * sx[t]) * s13[e,c], c<2I   */
/*     act[i] = silu(h[2i]) * h[2i+1]     (row 2i = gate, 2i+1 = up)         */
/*     qa, sa2 = per-row quant of act (one scale per pair)                   */
/*     y2[c]  = (float(sum_i qa[i] w2[e,c,i]) * sa2) * s2[e,c], c<H          */
/*   out[t,c] = bf16_rne( sum_j topk_w[t,j] * y2[(t,j), c] )   (fp32)        */
/* x: bf16 [T, H]; logits: fp32 [T, E]; w13: int8 [E, 2I, H], s13: fp32      */
/* [E, 2I]; w2: int8 [E, H, I], s2: fp32 [E, H]; topk_ids: int32 [T, k];     */
/* topk_w: fp32 [T, k]; out: bf16 [T, H].  All contiguous.                   */
/* Requires H % 64 == 0, I % 64 == 0, H <= 16384, I <= 4096, 1 <= k <= 16,   */
/* k <= E <= 1024, T*k <= 2^24; pointers 16-byte aligned.                    */
/* dbg (nullable; each member nullable): extra copies of the intermediates,  */
/* in pair order r = t*k + j.                                                */
/* ------------------------------------------------------------------------ */
typedef struct moe_w8a8_debug {
    int8_t *qx;    /* [T, H] */
    float *sx;     /* [T] */
    int32_t *acc1; /* [T*k, 2I] */
    float *act;    /* [T*k, I] */
    int8_t *qa;    /* [T*k, I] */
    float *sa2;    /* [T*k] */
    int32_t *acc2; /* [T*k, H] */
} moe_w8a8_debug;

size_t moe_w8a8_workspace_bytes(int64_t T, int64_t H, int64_t E, int64_t I, int topk);
/* Same call with the expert weights in the packed tile layout: w13 packed  */
/* as one [E*2I, H] matrix and w2 as one [E*H, I] matrix (w8a8_pack_weights). */
/* Results are identical to moe_w8a8_forward on the unpacked weights.       */
int moe_w8a8_forward_packed(const uint16_t *x, const float *logits, int64_t T, int64_t H,
                            int64_t E, int64_t I, int topk, const int8_t *w13_packed,
                            const float *s13, const int8_t *w2_packed, const float *s2,
                            int32_t *topk_ids, float *topk_w, uint16_t *out, void *ws,
                            size_t ws_bytes, const moe_w8a8_debug *dbg, void *stream);
int moe_w8a8_forward(const uint16_t *x, const float *logits, int64_t T, int64_t H, int64_t E,
                     int64_t I, int topk, const int8_t *w13, const float *s13,
                     const int8_t *w2, const float *s2, int32_t *topk_ids, float *topk_w,
                     uint16_t *out, void *ws, size_t ws_bytes, const moe_w8a8_debug *dbg,
                     void *stream);

/* ------------------------------------------------------------------------ */
/* Hadamard-domain activations.  [IQ8R] Trunk and Activations rows: each 128 */
/* of K rotated by the unnormalised Hadamard, int8 activations under the     */
/* same rotation.  Per row: every 128-block goes through the fp32 fast       */
/* Walsh-Hadamard butterfly in natural (Sylvester) order, stages h = 1, 2,   */
/* ..., 64, pair (i, i+h) -> (a + b, a - b); then the whole rotated row is   */
/* quantised as in quant_per_token_i8.                                       */
/* x: bf16 [M, K] (ldx); q: int8 [M, K] (ldq); s: fp32 [M].                  */
/* Requires K % 128 == 0, K <= 16384; 16-byte alignment as above.            */
/* ------------------------------------------------------------------------ */
int fwht128_quant(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int8_t *q,
                  int64_t ldq, float *s, void *stream);

/* ------------------------------------------------------------------------ */
/* Hadamard-domain weight preparation (done once, at load).  [IQ8R] Trunk    */
/* row and recipe "rtn codes=i8 group=256 scale=u8 scale2=bf16 block2=1x*    */
/* transform=fwht128 clamp=sym".  Per row n of W (fp32 [N, K], contiguous):  */
/*   w' = fwht128 of each 128-block (as above);                              */
/*   a_g = max |w'| over group g of 256, s_g = a_g / 127;                    */
/*   s2[n] = bf16_rne(max_g s_g / 255);                                      */
/*   su8[n,g] = a_g == 0 ? 0 : clamp(round_half_even(s_g / s2[n]), 1, 255);  */
/*   qw[n,k] = clamp(round_half_even(w' / (s2[n] * su8[n,g])), -127, 127)    */
/*   (codes 0 where the effective scale is 0).                               */
/* qw: int8 [N, K]; su8: uint8 [N, K/256]; s2: bf16 [N].                     */
/* Requires K % 256 == 0, K <= 16384.                                        */
/* ------------------------------------------------------------------------ */
int fwht128_weight_prep_g256(const float *W, int64_t N, int64_t K, int8_t *qw, uint8_t *su8,
                             uint16_t *s2, void *stream);

/* ------------------------------------------------------------------------ */
/* Hadamard-domain GEMM with u8 group scales.  [IQ8R] Trunk row.             */
/*   acc_g[m,n] = sum over the 256 k of group g of qa[m,k] * qw[n,k]         */
/*   T[m,n]     = sum_g su8[n,g] * acc_g[m,n]                 (exact int64)  */
/*   y[m,n]     = bf16_rne( float( T * sa[m] * s2[n] * 2^-7 ) )  (fp64)      */
/* The 2^-7 undoes <Hx, Hw> = 128 <x, w> of the unnormalised transform.      */
/* qa: int8 [M, K] contiguous, sa: fp32 [M]; qw: int8 [N, K] contiguous;     */
/* su8: uint8 [N, K/256]; s2: bf16 [N]; y: bf16 [M, N] (ldy).                */
/* Requires K % 256 == 0, K <= 16384, N % 16 == 0.                           */
/* ------------------------------------------------------------------------ */
size_t gemm_w8a8_g256_workspace_bytes(int64_t M, int64_t N, int64_t K);
int gemm_w8a8_g256(const int8_t *qa, const float *sa, int64_t M, int64_t K, const int8_t *qw,
                   const uint8_t *su8, const uint16_t *s2, int64_t N, uint16_t *y, int64_t ldy,
                   void *ws, size_t ws_bytes, void *stream);

/* gemm_w8a8_g256 with the codes in the packed tile layout of                */
/* w8a8_pack_weights (applied to the prepared qw once, at load): same        */
/* arithmetic, same results, same shape rules and workspace.                 */
int gemm_w8a8_g256_packed(const int8_t *qa, const float *sa, int64_t M, int64_t K,
                          const int8_t *qw_packed, const uint8_t *su8, const uint16_t *s2,
                          int64_t N, uint16_t *y, int64_t ldy, void *ws, size_t ws_bytes,
                          void *stream);

/* ------------------------------------------------------------------------ */
/* The whole Hadamard-domain linear: bf16 x -> fwht128 + per-token quant    */
/* (as fwht128_quant) -> g256 GEMM (as gemm_w8a8_g256) on packed codes ->    */
/* bf16 y.  [IQ8R] Trunk and Activations rows.  The activation codes and     */
/* scales live in the workspace (linear_w8a8_g256_workspace_bytes).          */
/* x: bf16 [M, K] (ldx, multiple of 16, 16-byte aligned); other operands as  */
/* gemm_w8a8_g256_packed.  Requires K % 256 == 0, K <= 16384, N % 16 == 0.   */
/* ------------------------------------------------------------------------ */
size_t linear_w8a8_g256_workspace_bytes(int64_t M, int64_t N, int64_t K);
int linear_w8a8_g256_packed(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                            const int8_t *qw_packed, const uint8_t *su8, const uint16_t *s2,
                            int64_t N, uint16_t *y, int64_t ldy, void *ws, size_t ws_bytes,
                            void *stream);

/* ------------------------------------------------------------------------ */
/* Rotated weight preparation with a bf16 scale per row per 128 of K (done   */
/* once, at load; the routed experts and the shared expert's down            */
/* projection).  [IQ8R] Experts row and the recipe lines for the expert      */
/* gate/up, expert down and shared down tensors (i8 codes, group 128, bf16   */
/* scale, fwht128, symmetric clamp).  Per row n of W (fp32 [N, K],           */
/* contiguous), per 128-block g (one group):                                 */
/*   w' = fwht128 of the block (as fwht128_quant);                           */
/*   s[n,g] = bf16_rne(max |w'| / 127);                                      */
/*   qw[n,k] = clamp(round_half_even(w' / float(s[n,g])), -127, 127), and 0  */
/*   where s[n,g] is 0 (the codes are taken against the stored bf16 scale).  */
/* qw: int8 [N, K] row-major (pack it with w8a8_pack_weights for the GEMMs); */
/* s: bf16 [N, K/128].  Requires K % 128 == 0, K <= 16384.                   */
/* ------------------------------------------------------------------------ */
int fwht128_weight_prep_g128(const float *W, int64_t N, int64_t K, int8_t *qw, uint16_t *s,
                             void *stream);

/* ------------------------------------------------------------------------ */
/* The MoE router gate in bf16.  [ATOM] intro: the precision split keeps the */
/* router gate in BF16 (the experts run A8W8).                               */
/*   logits[t,e] = sum_h x[t,h] * wg[e,h]  (bf16 operands, fp32 accumulate,  */
/*   fixed order: repeated calls give identical bits).                       */
/* x: bf16 [T, H] (ldx, multiple of 8, 16-byte aligned rows); wg: bf16       */
/* [E, H] contiguous; logits: fp32 [T, E] (ldl >= E).  Requires H % 32 == 0, */
/* H <= 16384, E % 16 == 0, E <= 4096, T <= 2^22.  The result differs from   */
/* the exact sum by at most the fp32 summation bound.                        */
/* ------------------------------------------------------------------------ */
int router_gate_bf16(const uint16_t *x, int64_t T, int64_t H, int64_t ldx, const uint16_t *wg,
                     int64_t E, float *logits, int64_t ldl, void *stream);

/* ------------------------------------------------------------------------ */
/* Routed MoE layer in the Hadamard domain.  [IQ8R] Experts row (the routed  */
/* experts int8 on the rotated grid with a bf16 scale per row and 128 of K)  */
/* and Activations row (the experts read the rotated codes the trunk's       */
/* quantisers write); the routed order of [ATOM] Changes, fused_moe_triton.py */
/* bullet.  Routing as moe_w8a8_forward (logits NULL: topk_ids/topk_w are    */
/* inputs).  Then, with g128(a, w, s, sa) = float( (sum over 128-groups g,   */
/* in order, of double(acc_g) * double(s_g)) * sa * 2^-7 ) in fp64 (acc_g    */
/* the exact int32 group sum; 2^-7 undoes <Hx, Hw> = 128 <x, w>):            */
/*   qx, sx = fwht128 + per-token quant of x (as fwht128_quant);             */
/*   per pair r = t*k + j, e = topk_ids[t,j]:                                */
/*     h[c]   = g128(qx[t], w13[e,c], s13[e,c], sx[t]),  c < 2I              */
/*     act[i] = silu(h[2i]) * h[2i+1]    (silu in fp64, rounded to fp32)     */
/*     qa, sa2 = fwht128 of each 128-block of act, then per-row quant        */
/*     y2[c]  = g128(qa, w2[e,c], s2[e,c], sa2),  c < H                      */
/*   out[t,c] = bf16_rne( (sum_j topk_w[t,j] * y2[(t,j),c], fp32, j order)    */
/*                        + shared[t,c] )    (no shared term when NULL)      */
/* x: bf16 [T, H] contiguous; w13_packed: the prepared codes (as             */
/* fwht128_weight_prep_g128) of [E, 2I, H] packed as one [E*2I, H] matrix;   */
/* s13: bf16 [E, 2I, H/128]; w2_packed: [E, H, I] packed as [E*H, I]; s2:    */
/* bf16 [E, H, I/128]; shared: fp32 [T, H] or NULL (the shared expert's      */
/* output, shared_expert_w8a8_rot_packed); out: bf16 [T, H].  Workspace:     */
/* moe_w8a8_workspace_bytes(T, H, E, I, topk).  dbg: qx, sx, act, qa, sa2    */
/* are written (acc1, acc2 are not).  Requires H % 256 == 0, H <= 4096,      */
/* I % 128 == 0, I <= 2048, 1 <= k <= 16, k <= E <= 1024, T*k <= 2^24.        */
/* ------------------------------------------------------------------------ */
int moe_w8a8_rot_forward_packed(const uint16_t *x, const float *logits, int64_t T, int64_t H,
                                int64_t E, int64_t I, int topk, const int8_t *w13_packed,
                                const uint16_t *s13, const int8_t *w2_packed,
                                const uint16_t *s2, const float *shared, int32_t *topk_ids,
                                float *topk_w, uint16_t *out, void *ws, size_t ws_bytes,
                                const moe_w8a8_debug *dbg, void *stream);

/* ------------------------------------------------------------------------ */
/* The shared expert in the Hadamard domain.  [IQ8R] Experts row: the shared */
/* expert like the routed ones, its gate/up projection as the trunk's        */
/* linears (g256 u8 under a bf16 row scale) and its down projection g128.    */
/*   qx, sx = fwht128 + per-token quant of x;                                */
/*   h[c] = float( (sum_g su8[c,g] * acc_g, exact) * sx * s2[c] * 2^-7 )     */
/*          (fp64; 256-groups), c < 2Is, rows 2i = gate_i, 2i+1 = up_i;      */
/*   act_i = silu(h[2i]) * h[2i+1]; qa, sa = fwht128 + per-row quant of act; */
/*   y[t,n] = g128(qa, wd[n], sd[n], sa)   (fp32, as above).                 */
/* x: bf16 [T, H] contiguous; wgu_packed: prepared codes (as                 */
/* fwht128_weight_prep_g256) of [2Is, H], packed; su8: uint8 [2Is, H/256];   */
/* s2: bf16 [2Is]; wd_packed: prepared codes (as fwht128_weight_prep_g128)   */
/* of [H, Is], packed; sd: bf16 [H, Is/128]; y: fp32 [T, H].  Requires       */
/* H % 256 == 0, H <= 4096, Is % 128 == 0, Is <= 2048, T <= 2^24.            */
/* dbg (nullable; each member nullable): act fp32 [T, Is], qa int8 [T, Is],  */
/* sa fp32 [T].                                                              */
/* ------------------------------------------------------------------------ */
typedef struct shared_expert_debug {
    float *act;  /* [T, Is] */
    int8_t *qa;  /* [T, Is] */
    float *sa;   /* [T] */
} shared_expert_debug;

size_t shared_expert_w8a8_rot_workspace_bytes(int64_t T, int64_t H, int64_t Is);
int shared_expert_w8a8_rot_packed(const uint16_t *x, int64_t T, int64_t H, int64_t Is,
                                  const int8_t *wgu_packed, const uint8_t *su8,
                                  const uint16_t *s2, const int8_t *wd_packed,
                                  const uint16_t *sd, float *y, void *ws, size_t ws_bytes,
                                  const shared_expert_debug *dbg, void *stream);

/* ------------------------------------------------------------------------ */
/* The Hadamard-domain MoE layer with its shared expert in one call.  [IQ8R] */
/* Experts row: routed and shared experts of one layer; [ATOM] Changes,      */
/* fused_moe_triton.py bullet (the routed order).  The result is exactly     */
/*   moe_w8a8_rot_forward_packed(..., shared = y) with                        */
/*   y = shared_expert_w8a8_rot_packed(x, Is, wgu_packed, su8, sgu,          */
/*                                     wd_packed, sd),                        */
/* computed together: for one token (k <= 15, I <= 1024, Is <= 1024,         */
/* k*I/128 + Is/128 <= 64) in two launches, the shared gate/up tiles beside */
/* the routed gemm1 and the shared down projection as one more pair of      */
/* gemm2; otherwise the shared expert first, then the routed layer.          */
/* Arguments as in those two calls (sgu is the shared gate/up's bf16 row     */
/* scale, there named s2).  Workspace:                                       */
/* moe_w8a8_rot_shared_workspace_bytes(T, H, E, I, topk, Is).  dbg as in     */
/* moe_w8a8_rot_forward_packed (the routed pairs' intermediates).  Requires  */
/* the conditions of both calls.                                             */
/* ------------------------------------------------------------------------ */
size_t moe_w8a8_rot_shared_workspace_bytes(int64_t T, int64_t H, int64_t E, int64_t I,
                                           int topk, int64_t Is);
int moe_w8a8_rot_shared_forward_packed(
    const uint16_t *x, const float *logits, int64_t T, int64_t H, int64_t E, int64_t I,
    int topk, const int8_t *w13_packed, const uint16_t *s13, const int8_t *w2_packed,
    const uint16_t *s2, int64_t Is, const int8_t *wgu_packed, const uint8_t *su8,
    const uint16_t *sgu, const int8_t *wd_packed, const uint16_t *sd, int32_t *topk_ids,
    float *topk_w, uint16_t *out, void *ws, size_t ws_bytes, const moe_w8a8_debug *dbg,
    void *stream);

#ifdef __cplusplus
}
#endif

#endif /* W8A8_H */
