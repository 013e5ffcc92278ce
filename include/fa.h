/*
 * libfa -- exact, tiled, fused scaled-dot-product attention for AMD MI355X (gfx950).
 *
 * What is computed (per batch entry b and head h, N queries, N keys, head dim d):
 *   S = scale * Q K^T, masked to -inf where a key is not allowed for a query;
 *   P = softmax(S) along keys;  O = P V;  LSE_i = ln sum_j exp(S_ij).
 * This is standard attention as described on the page "FlashAttention学习笔记"
 * (amentiraz.github.io), section Forward运作流程 / 标准attention计算 and 标准Safe softmax;
 * the method returns exactly that output while never writing S or P to HBM
 * ("高效注意力算法实现 (FlashAttention)", apxml.com, section FlashAttention：融合算子与分块
 * 处理, and 优势与影响). The backward pass recomputes P from the saved per-row statistic
 * instead of storing it (report on "FlashAttention：一种基于I/O感知的快速且内存高效的自注意力
 * 算法", fmread.com, section 算法设计); here that statistic is LSE in natural log.
 *
 * Masks (any combination; a key is allowed iff every active mask allows it):
 *   causal     key j allowed for query i iff j <= i;
 *   window     (window_left, window_right), fa_fwd_window / fa_bwd_window only: key j allowed
 *              for query i iff i - window_left <= j <= i + window_right; a negative bound means
 *              no limit on that side. This is the sliding-window (local) attention the page
 *              "IO感知计算如何重塑Transformer内存优化技术格局" (bxzpzcl.cn) lists among the
 *              supported options (section 高级功能配置); (-1, 0) equals the causal mask;
 *   blockmask  uint8 table [nb][nb], nb = ceil(N/128): entry [i/128][j/128] != 0 keeps the
 *              128x128 block (block-sparse attention: the report's 研究亮点 item 3 and the
 *              abstract of "FlashAttention: Fast and Memory-Efficient Exact Attention with
 *              IO-Awareness"), the same table for every (b, h);
 *   kv_len     int32 [B]: keys j >= kv_len[b] are masked (key padding). Values must lie in
 *              [0, N]; they are read on the device and not validated on the host.
 * A query row with no allowed key gets O = 0, LSE = -inf, and contributes no gradient.
 *
 * Element types: every entry point without a suffix takes bfloat16 tensors; the *_f16 entry
 * points take fp16 (the deployment page lists fp16 and bf16 among the ROCm data types:
 * "IO感知计算如何重塑Transformer内存优化技术格局", bxzpzcl.cn, section AMD ROCm生态支持). Both
 * feed the matrix units in that type and accumulate in fp32; P and dS are rounded to the
 * same type before the second product of each pair, outputs to nearest even.
 *
 * Data layout and ownership:
 *   q, k, v, o, dO, dq, dk, dv: contiguous [B][H][N][d] bfloat16 or fp16 (raw bits,
 *     uint16), DEVICE pointers, 16-byte aligned.
 *   lse, delta: contiguous [B][H][N] float32, DEVICE pointers, 4-byte aligned.
 *   blockmask, kv_len: DEVICE pointers or NULL (NULL = mask not used); blockmask at any
 *     byte alignment, kv_len 4-byte aligned.
 *   workspace: DEVICE pointer, 256-byte aligned, at least fa_bwd_workspace_bytes() bytes.
 *   The caller allocates and frees everything; the library allocates nothing and keeps no
 *   global mutable state (except the scratch array of fa_bwd_noalloc, described there).
 *   Outputs must not alias inputs or each other.
 *   stream: a hipStream_t (NULL = the default stream). All work is enqueued asynchronously
 *   on it; inputs must stay valid and unmodified until the stream has run the work.
 *   Supported head dims: d a multiple of 8 from 8 to 256 (the FP8 forward: 64 and 128).
 *   The kernels' tiles are 64, 128 or 256 columns wide (256: four waves of 32 queries per
 *   workgroup, one per SIMD, for the register budget). d = 32 and 96 run on the 64 / 128
 *   tiles but compute only their own width. Any other d runs on the next tile width up
 *   with the extra columns zero-padded: zero columns add nothing to Q K^T, and the padded
 *   output columns are never written. That costs the padded matrix work.
 *   scale must be finite and nonzero (negative values are allowed).
 *   Sizes: B, H, N >= 1 with B*H*N <= 2^31 - 1 rows and N*d <= 2^31 - 1 elements per
 *   head; anything larger returns FA_ERR_SHAPE. Every shape within these limits runs: a
 *   grid holding more work-items than one dispatch counts (2^32 - 1) is enqueued as
 *   several launches over consecutive heads (the preprocess: over consecutive rows), all
 *   on the caller's stream.
 *
 * Errors: every entry point validates its arguments on the host before any HIP call and
 * returns a nonzero fa_status without launching anything when they are invalid. A failed
 * kernel launch returns FA_ERR_LAUNCH. Faults during execution surface at the caller's
 * next synchronisation of the stream.
 */
#ifndef LIBFA_FA_H
#define LIBFA_FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t fa_bf16; /* raw bfloat16 bits */
typedef uint16_t fa_f16;  /* raw IEEE binary16 (fp16) bits */

enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL = 1,           /* a required pointer is NULL                          */
  FA_ERR_SHAPE = 2,          /* B, H or N < 1, or the problem is too large          */
  FA_ERR_UNSUPPORTED_D = 3,  /* d not a multiple of 8 in [8, 256] (see above)       */
  FA_ERR_ALIGN = 4,          /* a pointer does not have the alignment stated above  */
  FA_ERR_SCALE = 5,          /* scale is zero, NaN or infinite (or an FP8 descale <= 0) */
  FA_ERR_LAUNCH = 6,         /* the HIP runtime rejected a kernel launch            */
  FA_ERR_ALIAS = 7,          /* an output buffer overlaps an input or another output */
  FA_ERR_DROPOUT = 8,        /* dropout probability not in [0, 1)                    */
  FA_ERR_DTYPE = 9,          /* element type other than 0 (bfloat16) or 1 (fp16)     */
  FA_ERR_SCRATCH = 10        /* fa_bwd_noalloc: B * H * N above its static scratch     */
};

/* Forward. Writes O [B][H][N][d] (bf16) and LSE [B][H][N] (fp32, natural log).
 * causal: 0 or 1. blockmask: NULL or device uint8 [ceil(N/128)][ceil(N/128)]. */
int fa_fwd(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, fa_bf16* o, float* lse,
           int B, int H, int N, int d, float scale, int causal, const uint8_t* blockmask,
           void* stream);

/* Forward with key padding: as fa_fwd, plus kv_len (NULL or device int32 [B]). */
int fa_fwd_ex(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, fa_bf16* o, float* lse,
              int B, int H, int N, int d, float scale, int causal, const uint8_t* blockmask,
              const int32_t* kv_len, void* stream);

/* Forward with every mask: as fa_fwd_ex, plus a sliding window (window_left, window_right),
 * negative = no limit on that side; any value is accepted (bounds of N or more allow every key
 * on that side). Key tiles outside every query's window are never read. */
int fa_fwd_window(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, fa_bf16* o,
                  float* lse, int B, int H, int N, int d, float scale, int causal,
                  const uint8_t* blockmask, const int32_t* kv_len, int window_left,
                  int window_right, void* stream);

/* Backward preprocess: delta[b][h][i] = sum_c dO[b][h][i][c] * O[b][h][i][c], summed in
 * fp32 over the given bf16 O and dO. This is the row statistic D of the softmax gradient
 * dS = P * (dP - D). fa_bwd forms D itself, at the start of its dQ pass; this entry point
 * is exported for callers that want D on its own. */
int fa_bwd_preprocess(const fa_bf16* o, const fa_bf16* dO, float* delta, int B, int H, int N,
                      int d, void* stream);

/* Bytes of device workspace fa_bwd needs: delta and a log2-scaled copy of LSE (fp32
 * [B][H][N] each, each padded to 256 bytes). Linear in N. Returns 0 for invalid shapes. */
size_t fa_bwd_workspace_bytes(int B, int H, int N, int d);

/* Backward. Inputs: q, k, v, the forward's o and lse, and dO = dL/dO. Outputs dq, dk, dv
 * (bf16). Recomputes P from lse; no N x N matrix is stored. The workspace contents on
 * entry are ignored. Every output is bitwise reproducible from run to run. */
int fa_bwd(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, const fa_bf16* o,
           const float* lse, const fa_bf16* dO, fa_bf16* dq, fa_bf16* dk, fa_bf16* dv, int B,
           int H, int N, int d, float scale, int causal, const uint8_t* blockmask,
           void* workspace, void* stream);

/* Backward with key padding (kv_len: NULL or device int32 [B]). */
int fa_bwd_ex(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, const fa_bf16* o,
              const float* lse, const fa_bf16* dO, fa_bf16* dq, fa_bf16* dk, fa_bf16* dv,
              int B, int H, int N, int d, float scale, int causal, const uint8_t* blockmask,
              const int32_t* kv_len, void* workspace, void* stream);

/* Backward with every mask (key padding and sliding window, as fa_fwd_window). */
int fa_bwd_window(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, const fa_bf16* o,
                  const float* lse, const fa_bf16* dO, fa_bf16* dq, fa_bf16* dk, fa_bf16* dv,
                  int B, int H, int N, int d, float scale, int causal,
                  const uint8_t* blockmask, const int32_t* kv_len, int window_left,
                  int window_right, void* workspace, void* stream);

/* fp16 versions, each with every mask (causal, block table, key padding, sliding window):
 * arguments, layout, ownership and errors as fa_fwd_window, fa_bwd_preprocess and
 * fa_bwd_window, with fp16 tensors. */
int fa_fwd_f16(const fa_f16* q, const fa_f16* k, const fa_f16* v, fa_f16* o, float* lse, int B,
               int H, int N, int d, float scale, int causal, const uint8_t* blockmask,
               const int32_t* kv_len, int window_left, int window_right, void* stream);
int fa_bwd_preprocess_f16(const fa_f16* o, const fa_f16* dO, float* delta, int B, int H, int N,
                          int d, void* stream);
int fa_bwd_f16(const fa_f16* q, const fa_f16* k, const fa_f16* v, const fa_f16* o,
               const float* lse, const fa_f16* dO, fa_f16* dq, fa_f16* dk, fa_f16* dv, int B,
               int H, int N, int d, float scale, int causal, const uint8_t* blockmask,
               const int32_t* kv_len, int window_left, int window_right, void* workspace,
               void* stream);

/* Dropout on the attention probabilities, fused into the kernels and regenerated in the
 * backward pass (nothing of size N x N is stored): "FlashAttention学习笔记"
 * (amentiraz.github.io), section Kernel融合, lists dropout among the operations fused into
 * one kernel, and its section 分块计算整体流程(Tiling) applies it to each block's scores on
 * the way to P̂; the fmread.com report's 算法设计 section says backward recomputes instead
 * of storing.
 * O = (P * keep / (1 - dropout_p)) V, with LSE the statistic of the undropped softmax.
 * keep for element (query i, key j) of head (b, h): Philox4x32-10 (Salmon et al., SC 2011)
 * with key = seed (low word first) and counter (j >> 2, i >> 1, b*H + h, offset); output
 * word j & 3, its low 16 bits for even i and its high 16 bits for odd i, is the element's
 * draw r, and the element is kept iff r >= floor(dropout_p * 2^16) (dropout_p is resolved
 * to 2^-16; the scale stays 1 / (1 - dropout_p)). The backward must get the same dropout_p,
 * seed and offset as the forward. dtype: 0 = bfloat16, 1 = fp16 (q, k, v, o, dO, dq, dk, dv
 * in that type). Every mask as in fa_fwd_window. dropout_p = 0 runs the kernels without
 * dropout; any dropout_p > 0 runs the dropout kernels, even where floor(dropout_p * 2^16)
 * is 0 (then every element is kept and scaled by 1 / (1 - dropout_p)). Errors: FA_ERR_DROPOUT for dropout_p outside [0, 1) or NaN, FA_ERR_DTYPE for an
 * unknown dtype, otherwise as fa_fwd_window / fa_bwd_window. */
int fa_fwd_dropout(int dtype, const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int N, int d, float scale, int causal,
                   const uint8_t* blockmask, const int32_t* kv_len, int window_left,
                   int window_right, float dropout_p, uint64_t seed, uint32_t offset,
                   void* stream);
int fa_bwd_dropout(int dtype, const void* q, const void* k, const void* v, const void* o,
                   const float* lse, const void* dO, void* dq, void* dk, void* dv, int B, int H,
                   int N, int d, float scale, int causal, const uint8_t* blockmask,
                   const int32_t* kv_len, int window_left, int window_right, float dropout_p,
                   uint64_t seed, uint32_t offset, void* workspace, void* stream);

/* FP8 forward (E4M3 inputs). FlashAttention-3 brought FP8 to the forward pass
 * ("IO感知计算如何重塑Transformer内存优化技术格局", bxzpzcl.cn, section 技术演进时间线); the
 * pages give no quantisation policy. This one is used:
 *   q, k, v: DEVICE, OCP E4M3 codes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits;
 *     subnormals; S.1111.111 is NaN; largest finite 448), [B][H][N][d] row-major, one
 *     byte per element; the values are descale_q * q, descale_k * k, descale_v * v.
 *   S = scale * (descale_q q)(descale_k k)^T, masked as in fa_fwd_window. In log2 units the
 *     scaled probabilities are P = 2^(S log2(e) - m + 6) for an integer reference m of the
 *     row. Each P is rounded to E4M3 (nearest, ties to even) for the product with V, and
 *     the normaliser is the sum of the unrounded P. m is a running maximum rounded up (an
 *     integer at most 3 below ceil(row max), so P <= 2^8.8 < 448), and the rounded P equal,
 *     up to a power of two, those of the reference m = ceil(row max) wherever both lie in
 *     the E4M3 normal range, which holds for every P down to 2^-12 of the row's largest.
 *     Keys masked by kv_len contribute nothing, whatever bytes k and v hold there.
 *   o: DEVICE bf16 [B][H][N][d] = descale_v * (rounded P) v / normaliser; lse: DEVICE fp32
 *     [B][H][N], the natural-log logsumexp of the scores (-inf for a row with no allowed
 *     key, whose o is 0).
 *   workspace: DEVICE, 256-byte aligned, fa_fwd_fp8_workspace_bytes(B, H, N, d) bytes:
 *     receives v transposed to [B][H][d][N rounded up to 128] (zero past N and past the
 *     batch entry's kv_len).
 *   d must be 64 or 128; scale finite and nonzero; each descale finite and > 0.
 * Errors: FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED_D, FA_ERR_SCALE, FA_ERR_ALIGN
 * (q, k, v, o 16 bytes, lse and kv_len 4, workspace 256), FA_ERR_ALIAS (o, lse, workspace
 * overlapping each other or q, k, v), FA_ERR_LAUNCH. */
size_t fa_fwd_fp8_workspace_bytes(int B, int H, int N, int d);
int fa_fwd_fp8(const uint8_t* q, const uint8_t* k, const uint8_t* v, fa_bf16* o, float* lse,
               int B, int H, int N, int d, float scale, float descale_q, float descale_k,
               float descale_v, int causal, const uint8_t* blockmask, const int32_t* kv_len,
               int window_left, int window_right, void* workspace, void* stream);

/* Backward without a workspace argument, for callers that cannot allocate device memory
 * around the call (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation). Arguments, layout, semantics and results as fa_bwd_dropout (dtype, every
 * mask, dropout_p = 0 for none), bitwise; it allocates nothing and calls no allocating
 * routine. Its workspace is a static device array of 32 MiB in the library, one copy per
 * GPU, held until the process ends: B * H * N must be at most 4,194,304 (2^22) rows, else
 * FA_ERR_SCRATCH and nothing is launched. It uses the copy of the current device (the
 * stream must belong to it); the first call on a device looks the copy up. Calls on one GPU
 * share the array, so calls that overlap on one GPU (different streams or threads) race;
 * calls on one stream are ordered and safe. Errors as fa_bwd_dropout, plus FA_ERR_SCRATCH,
 * and FA_ERR_LAUNCH if the device or its copy of the array cannot be found. */
int fa_bwd_noalloc(int dtype, const void* q, const void* k, const void* v, const void* o,
                   const float* lse, const void* dO, void* dq, void* dk, void* dv, int B, int H,
                   int N, int d, float scale, int causal, const uint8_t* blockmask,
                   const int32_t* kv_len, int window_left, int window_right, float dropout_p,
                   uint64_t seed, uint32_t offset, void* stream);

/* Static description of a status code. */
const char* fa_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* LIBFA_FA_H */
