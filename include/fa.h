/*
 * fa.h -- C ABI of the MI355X (gfx950) exact-attention library, libfa.so.
 *
 * The operation is exact attention, O = softmax(scale * Q K^T) V, computed
 * tile by tile on chip with an online softmax so that the N x N score matrix
 * never reaches HBM ("FlashAttention." plate, opening section and "Never
 * write the scores"; "FlashAttention: Fast and Memory-Efficient Exact
 * Attention with IO-Awareness", Abstract).  The result is the standard
 * attention result up to floating-point rounding (same plate, "Never write
 * the scores").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  Layout     Q, K, V, O, dO, dQ, dK, dV are dense, contiguous [B][H][N][d]
 *             tensors (row-major, d fastest); the _gqa entry points take K,
 *             V, dK, dV as [B][Hkv][N][d].  LSE is [B][H][N] fp32, the
 *             natural-log log-sum-exp of row i of the scaled, masked scores.
 *  Memory     every tensor pointer is a DEVICE pointer on the current HIP
 *             device; `block_mask` is a device pointer too.  The caller owns
 *             every buffer (inputs, outputs, workspace); the library never
 *             allocates or frees memory, so it is re-entrant.  Buffers must
 *             not overlap.  The one exception is fa_backward_noalloc, which
 *             uses a fixed scratch array the library holds on each device
 *             (see there).
 *  Streams    `stream` is a hipStream_t passed as void* (NULL = the null
 *             stream).  Calls are asynchronous: they enqueue kernels on the
 *             stream and return; buffers must stay alive until it syncs.
 *  Alignment  tensor pointers must be 16-byte aligned; LSE and the workspace
 *             4-byte aligned.
 *  Sizes      B, H, N >= 0; d in {64, 128}.  If B*H*N == 0 the call does
 *             nothing and returns FA_OK (pointers may then be NULL).
 *  scale      finite and > 0 (1/sqrt(d) is the usual choice).
 *  causal     nonzero: key j is visible to query i only if j <= i.
 *  Masks      a fully masked row yields O = 0 and LSE = -infinity.
 *  Errors     status codes only; nothing is thrown across the ABI.  Argument
 *             errors are detected before anything is enqueued.
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1, /* NULL pointer, negative size, bad scale, misalignment */
  FA_ERR_UNSUPPORTED = 2, /* valid request outside what is built (d, mask block) */
  FA_ERR_HIP = 3,         /* the HIP runtime reported an error at launch */
  FA_ERR_TOO_LARGE = 4    /* the problem needs more than the fixed no-allocation scratch */
} fa_status;

/* Bytes of the fixed per-device scratch array of fa_backward_noalloc. */
#define FA_NOALLOC_SCRATCH_BYTES (8u << 20)

/*
 * Forward pass, bf16 storage, fp32 accumulation.
 *   q, k, v  in : bf16 [B][H][N][d]
 *   o        out: bf16 [B][H][N][d]
 *   lse      out: fp32 [B][H][N]   (saved for fa_backward)
 * The scores are tiled through LDS and registers and never written to HBM
 * ("FlashAttention." plate, opening section).
 */
int fa_forward(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
               int N, int d, float scale, int causal, void* stream);

/*
 * Forward pass with fp32 inputs, arithmetic and outputs (q, k, v, o fp32),
 * for small problems that need fp32 accuracy.  Same arguments as fa_forward.
 */
int fa_forward_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B,
                   int H, int N, int d, float scale, int causal, void* stream);

/*
 * Bytes of device workspace fa_backward needs for this shape: two fp32
 * [B][H][N] arrays, the per-row -D_i = -(dO_i . O_i) and LSE_i * log2(e), which
 * the first launch writes and the other two read.  Returns 0 for empty or
 * invalid shapes.
 */
size_t fa_backward_workspace_size(int B, int H, int N, int d);

/*
 * Backward pass: bf16 inputs, fp32 accumulation and fp32 gradients.  The
 * probabilities are recomputed tile by tile from Q, K and the saved LSE
 * instead of being stored ("FlashAttention." plate, "Never write the scores":
 * the backward recomputes the scores).  Gradients by the chain rule through
 * P = softmax(S):
 *   dV = P^T dO,  dP = dO V^T,  D_i = dO_i . O_i,  dS = P * (dP - D),
 *   dQ = scale dS K,  dK = scale dS^T Q.
 *   q, k, v, o, dout in : bf16 [B][H][N][d]  (o and lse from fa_forward with
 *                         the same q, k, v, scale and causal flag)
 *   lse              in : fp32 [B][H][N]
 *   dq, dk, dv       out: fp32 [B][H][N][d] (fp32 so that output rounding does
 *                         not eat the accuracy of the fp32 accumulation)
 *   workspace        scratch device memory of at least
 *                    fa_backward_workspace_size(B, H, N, d) bytes, owned by
 *                    the caller; its contents on entry do not matter.
 * Deterministic: no atomics; the same inputs give bitwise the same outputs.
 */
int fa_backward(const void* q, const void* k, const void* v, const void* o, const void* dout,
                const float* lse, float* dq, float* dk, float* dv, void* workspace,
                size_t workspace_bytes, int B, int H, int N, int d, float scale, int causal,
                void* stream);

/*
 * fa_backward for callers that cannot allocate memory (code under HIP graph
 * capture, serving loops or harnesses that forbid allocation): the same
 * kernels and results as fa_backward, but the workspace (D and LSE * log2(e),
 * two fp32 per row) lives in a fixed device array of
 * FA_NOALLOC_SCRATCH_BYTES bytes that the library holds on each GPU it runs
 * on until the process ends.  The call itself allocates nothing.
 *   Arguments as fa_backward without workspace / workspace_bytes.
 *   Limit: fa_backward_workspace_size(B, H, N, d) <= FA_NOALLOC_SCRATCH_BYTES,
 *          i.e. B * H * N <= 1048576 rows; larger problems return
 *          FA_ERR_TOO_LARGE before anything is enqueued.
 *   Device: the scratch of the device `stream` belongs to (the current device
 *          for the null stream) is used; its address is looked up on the
 *          first call on that device.
 *   Races: every call on one GPU shares that GPU's scratch, so calls whose
 *          kernels can overlap on one GPU (different streams without
 *          ordering between them) race and must not be issued.  Each call
 *          writes the scratch before reading it; nothing has to be cleared.
 */
int fa_backward_noalloc(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, float* dq, float* dk, float* dv,
                        int B, int H, int N, int d, float scale, int causal, void* stream);

/*
 * Block-sparse forward: like fa_forward, but scores in tiles whose mask entry
 * is 0 are -infinity, and such tiles are skipped entirely (no loads, no
 * matrix work): "Flash Attention: IO-Aware Attention Computation", paragraph
 * on block-sparse attention; "FlashAttention: Fast and Memory-Efficient Exact
 * Attention with IO-Awareness", Abstract.
 *   block_mask  in: uint8 device array [nb][nb], nb = ceil(N / mask_block);
 *               entry [qb][kb] != 0 means query tile qb attends to key tile
 *               kb.  One mask is shared by every batch and head.
 *   mask_block  tile edge in tokens; must be 128 (FA_ERR_UNSUPPORTED
 *               otherwise).
 * causal may be combined with the mask (both apply).
 */
int fa_forward_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int N, int d, float scale, int causal,
                           const uint8_t* block_mask, int mask_block, void* stream);

/*
 * Block-sparse backward: the gradients of fa_forward_blocksparse with the same
 * mask.  Tiles whose mask entry is 0 are skipped in both gradient passes (the
 * dQ pass walks each mask row, the dK/dV pass each mask column), so masked
 * tiles cost no loads and no matrix work here either ("Flash Attention:
 * IO-Aware Attention Computation", paragraph on block-sparse attention).
 * Arguments as fa_backward, plus block_mask / mask_block as
 * fa_forward_blocksparse; o and lse must come from fa_forward_blocksparse
 * with the same mask.  Rows whose mask row is all zero get dQ = 0, and keys
 * whose mask column is all zero get dK = dV = 0.
 */
int fa_backward_blocksparse(const void* q, const void* k, const void* v, const void* o,
                            const void* dout, const float* lse, float* dq, float* dk, float* dv,
                            void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                            float scale, int causal, const uint8_t* block_mask, int mask_block,
                            void* stream);

/*
 * Grouped K/V heads (multi-query attention for Hkv = 1, grouped-query
 * attention for 1 < Hkv < H): "Flash Attention: IO-Aware Attention
 * Computation", closing paragraph on future directions, names these variants
 * as a way to shrink the key/value memory.  Query head h of batch b attends
 * to K/V head h / (H / Hkv) of batch b; everything else is fa_forward.
 *   q, o      bf16 [B][H][N][d]      lse fp32 [B][H][N]
 *   k, v      bf16 [B][Hkv][N][d]    (1 <= Hkv <= H, H % Hkv == 0, else
 *                                     FA_ERR_INVALID_ARG)
 * fa_forward_gqa with Hkv == H is fa_forward.
 */
int fa_forward_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                   int Hkv, int N, int d, float scale, int causal, void* stream);

/*
 * Backward of fa_forward_gqa.  dq is fp32 [B][H][N][d]; dk and dv are fp32
 * [B][Hkv][N][d]: the gradient of a shared K/V head is the sum, over the
 * H / Hkv query heads that read it, of each head's gradient.  The sum is
 * taken in a fixed order (no atomics): deterministic.
 * workspace: at least fa_backward_workspace_size(B, H, N, d) bytes
 * (H = query heads).  With fa_backward_gqa_workspace_size(B, H, Hkv, N, d)
 * bytes or more, each group's query heads are split over several dK/dV
 * workgroups whose fp32 partial sums are added in a fixed order afterwards
 * (needed to fill the chip when B * Hkv is small, e.g. MQA); with less, one
 * workgroup sums the whole group (same result up to rounding order).
 */
int fa_backward_gqa(const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, float* dq, float* dk, float* dv, void* workspace,
                    size_t workspace_bytes, int B, int H, int Hkv, int N, int d, float scale,
                    int causal, void* stream);

/*
 * Workspace bytes with which fa_backward_gqa splits each group's query heads
 * over several dK/dV workgroups: fa_backward_workspace_size(B, H, N, d) plus
 * room for the partial sums (2 * S * B * Hkv * N * d fp32, S = the number of
 * slices, a divisor of H / Hkv).  Equal to fa_backward_workspace_size when no
 * split is needed; 0 for invalid shapes or groupings.
 */
size_t fa_backward_gqa_workspace_size(int B, int H, int Hkv, int N, int d);

/*
 * Forward pass with fp8 inputs: q, k, v hold OCP e4m3 codes (1 sign, 4
 * exponent bits with bias 7, 3 mantissa bits; largest finite value 448) in
 * the fa_forward layout, one byte per element, and the real value of an
 * element is code * descale (one fp32 descale per tensor, finite and > 0,
 * else FA_ERR_INVALID_ARG).  Both products run on the 8-bit matrix cores
 * with fp32 accumulation; the attention weights are rounded to e4m3 for the
 * second product.  Lower-precision matrix inputs are the direction the
 * "FlashAttention." plate's "Never write the scores" section gives for the
 * H100 generation of the method.
 *   o    out: bf16 [B][H][N][d]
 *   lse  out: fp32 [B][H][N], of scale * (q_descale q)(k_descale k)^T
 * d in {64, 128}; causal as fa_forward.
 */
int fa_forward_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                   int N, int d, float scale, float q_descale, float k_descale, float v_descale,
                   int causal, void* stream);

/* Static text for a status code (never NULL). */
const char* fa_error_string(int status);

/* Library version, major*10000 + minor*100 + patch. */
int fa_version(void);

/* hipRuntimeGetVersion() of the HIP runtime the library is running on, or -1. */
int fa_runtime_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
