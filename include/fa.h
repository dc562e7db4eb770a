/*
 * fa.h -- C ABI of the MI355X (gfx950) exact-attention library (libfa355.so).
 *
 * The library computes exact scaled-dot-product attention
 *
 *     O = softmax(scale * Q K^T [+ mask]) V
 *
 * in one fused forward kernel that streams K/V tiles through LDS and keeps a running
 * row maximum and row sum (online softmax), so the N x N score matrix never reaches
 * HBM; the backward pass recomputes the probabilities on chip from the saved per-row
 * log-sum-exp instead of storing them.  Sources: "FlashAttention" concept wiki page
 * (notes.yuuk.io), section 定義 -- tiling with online softmax (1) and recomputation in
 * the backward (2), exact result, O(N) extra memory; singularity-lens FA1 explainer,
 * paragraphs on tiling, on the online softmax and on recomputation.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors q, k, v, o, dout, dq, dk, dv are DEVICE pointers to contiguous row-major
 *    [B][H][N][d] arrays of bfloat16 (IEEE binary32 upper halves, stored as uint16).
 *    Rows must be 16-byte aligned (true for any hipMalloc'd base since d*2 is a
 *    multiple of 16).
 *  - lse is a DEVICE pointer to a contiguous [B][H][N] float32 array holding, per query
 *    row, the natural-log log-sum-exp of that row's scaled, masked scores
 *    (-inf for a row with no admissible key).
 *  - kv_len (the *_kvlen variants) is a DEVICE pointer to int32[B]; for batch b only
 *    keys j < kv_len[b] are attended (values are clamped to [0, N]).  NULL = no padding.
 *  - causal != 0: query i attends keys j <= i (square problem, the same N for queries
 *    and keys).  Both masks may be combined.
 *  - scale is any finite float (it multiplies Q K^T before the softmax; the definition
 *    on the pages puts no sign on it).  scale = 0 gives uniform weights over the
 *    admissible keys (LSE = ln of their count, dQ = dK = 0); a negative scale favours
 *    the smallest scores.  NaN and +-inf are rejected with FA_ERR_SCALE.
 *  - Supported head dims: d = 64 and d = 128.  Any N >= 1, B >= 1, H >= 1 with
 *    B*H*N*d < 2^62 and N*d*2 < 2^32 (one head's matrix below 4 GiB).
 *  - The caller owns every buffer.  The library never allocates, frees or
 *    synchronises; it only enqueues kernels on `stream` (0 = the null stream) and
 *    returns.  Execution faults surface at the caller's next synchronisation.
 *  - Arguments are validated on the host before any HIP call; an invalid call
 *    returns a negative fa_status and enqueues nothing.  A failed launch returns
 *    FA_ERR_LAUNCH.  There is no global mutable state: calls on different streams
 *    may run concurrently.
 */
#ifndef FA355_FA_H
#define FA355_FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* fa_stream_t; /* identical to hipStream_t */

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = -1,      /* a required pointer is NULL                          */
  FA_ERR_SHAPE = -2,     /* B, H or N < 1, or the element count overflows        */
  FA_ERR_HEADDIM = -3,   /* d is not 64 or 128                                   */
  FA_ERR_SCALE = -4,     /* scale is NaN or infinite (fp8 post_scale: also <= 0)  */
  FA_ERR_WORKSPACE = -5, /* backward workspace NULL or smaller than required     */
  FA_ERR_LAUNCH = -6,    /* a kernel launch failed (hipGetLastError)             */
  FA_ERR_ALIGN = -7,     /* a tensor pointer is not 16-byte aligned              */
  FA_ERR_KVHEADS = -8    /* H_kv < 1 or H_kv does not divide H (grouped heads)   */
} fa_status;

/*
 * Forward pass.  Writes o [B][H][N][d] (bf16) and lse [B][H][N] (fp32).
 * Operation: exact attention with online softmax over K/V tiles ("FlashAttention"
 * wiki page, 定義 (1); FA1 explainer, tiling and online-softmax paragraphs).
 * Inputs q, k, v are read only; o and lse are overwritten entirely (every row < N).
 */
int fa_forward(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
               float scale, int causal, fa_stream_t stream);

/* Forward pass with per-batch key padding (kv_len, device int32[B]); otherwise as fa_forward. */
int fa_forward_kvlen(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                     float scale, int causal, const int32_t* kv_len, fa_stream_t stream);

/*
 * Forward pass for a block of Nq queries against Nk keys: query row i of q sits at
 * position q_offset + i of the key sequence.  q, o: [B][H][Nq][d]; k, v: [B][H][Nk][d];
 * lse: [B][H][Nq].  causal != 0: key j is admissible for query row i iff
 * j <= q_offset + i; kv_len (device int32[B] or NULL) as in fa_forward_kvlen, clamped to
 * [0, Nk].  With Nq = Nk and q_offset = 0 it is fa_forward_kvlen.  This is one GPU's share
 * of a forward whose query rows are split over several GPUs that each hold all keys and
 * values (or their admissible prefix): rows [q_offset, q_offset + Nq) of the whole
 * problem's O and LSE, from the same definition ("FlashAttention" wiki page, 定義 (1)).
 * Errors: as fa_forward; FA_ERR_SHAPE also for Nk < 1, q_offset < 0 or
 * q_offset + Nq + 256 > 2^31 - 1.
 */
int fa_forward_offset(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq,
                      int Nk, int d, float scale, int causal, int q_offset, const int32_t* kv_len,
                      fa_stream_t stream);

/*
 * Size in bytes of the device workspace fa_backward needs: two fp32 per query row,
 * -D_i (D_i = sum_k dO_ik O_ik) and LSE_i * log2(e), for N rounded up to a multiple of 256
 * rows per head: 8 * B * H * (256 * ceil(N / 256)) bytes.  dQ needs no accumulator: it
 * is produced by a query-outer pass that keeps its rows in registers.  Returns 0 for
 * invalid sizes.
 */
size_t fa_backward_workspace_size(int B, int H, int N, int d);

/*
 * Backward pass: gradients of L = sum(O * dout) with respect to q, k and v.
 * P is recomputed on chip from q, k and the forward's lse (no N x N matrix is stored:
 * "FlashAttention" wiki page, 定義 (2); FA1 explainer, recomputation paragraph).
 * o and lse must be the outputs of fa_forward on the same q, k, v, scale and masks.
 * Writes dq, dk, dv [B][H][N][d] (bf16) entirely; keys masked out for every query
 * (padding) get exact zeros in dk and dv.  No atomics are used: the results are
 * bitwise reproducible run to run.  workspace: device buffer of at least
 * fa_backward_workspace_size(B,H,N,d) bytes, 256-byte aligned, owned by the caller;
 * its contents on entry are ignored and on return are unspecified.
 */
int fa_backward(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal, void* workspace,
                size_t workspace_bytes, fa_stream_t stream);

/* Backward pass with per-batch key padding (kv_len, device int32[B]); otherwise as fa_backward. */
int fa_backward_kvlen(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                      void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal,
                      const int32_t* kv_len, void* workspace, size_t workspace_bytes, fa_stream_t stream);

/*
 * The two passes of the backward, for callers that schedule them separately and for
 * per-kernel timing: fa_backward_kvlen(args) is exactly fa_backward_dq_pass(args)
 * followed by fa_backward_dkdv_pass(args) on the same stream.  Arguments, validation
 * and error codes are those of fa_backward_kvlen (kv_len: device int32[B] or NULL for
 * no padding).
 *   fa_backward_dq_pass:   writes dq and the row statistics -D_i and LSE_i * log2(e)
 *                          into the workspace (dk, dv are not touched);
 *   fa_backward_dkdv_pass: reads those statistics and writes dk and dv (dq is not
 *                          touched); it must follow a dQ pass on the same inputs and
 *                          workspace, in stream order.
 */
int fa_backward_dq_pass(const void* q, const void* k, const void* v, const void* o, const void* dout,
                        const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                        int causal, const int32_t* kv_len, void* workspace, size_t workspace_bytes,
                        fa_stream_t stream);
int fa_backward_dkdv_pass(const void* q, const void* k, const void* v, const void* o, const void* dout,
                          const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                          int causal, const int32_t* kv_len, void* workspace, size_t workspace_bytes,
                          fa_stream_t stream);

/*
 * Allocation-free backward, for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, results (bit for bit) and errors as fa_backward_kvlen (kv_len: device
 * int32[B] or NULL), without the workspace: the row statistics the two passes exchange
 * live in a device array owned by the library, FA_NOALLOC_SCRATCH_BYTES per GPU, held
 * from the first call on that GPU until the process ends.  The call allocates and frees
 * nothing.
 *   - A problem whose statistics exceed the array (fa_backward_workspace_size(B, H, N, d)
 *     > FA_NOALLOC_SCRATCH_BYTES, i.e. more than 2^21 padded rows B * H * ceil(N/256) *
 *     256) returns FA_ERR_WORKSPACE before any HIP call.
 *   - Every call on one GPU uses that GPU's one array: calls that overlap on one GPU (on
 *     different streams, or from several threads) race and may return wrong gradients.
 *     Serialise them (one stream, or events).  Nothing in the array needs clearing
 *     between calls: the dQ pass writes every entry the dK/dV pass reads.
 *   - The first call on a GPU looks up the array's device address (hipGetSymbolAddress,
 *     with that GPU current); a failure there returns FA_ERR_LAUNCH.
 */
#define FA_NOALLOC_SCRATCH_BYTES (16u << 20)
int fa_backward_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                        const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                        int causal, const int32_t* kv_len, fa_stream_t stream);

/*
 * Grouped-query and multi-query attention (GQA, MQA): H query heads share H_kv K/V
 * heads, query head h using K/V head h / (H / H_kv) (groups of consecutive query
 * heads); H_kv = H is ordinary multi-head attention and H_kv = 1 is MQA.  The
 * "FlashAttention" concept wiki page lists GQA/MQA among its open questions (section
 * 未解決の問い) without defining it; the result here is that of ordinary attention
 * with every K/V head repeated for the query heads of its group, so dk and dv are the
 * sums over the group of the per-query-head gradients.
 *   q, o, dout, dq: [B][H][N][d];  k, v, dk, dv: [B][H_kv][N][d];  lse: [B][H][N].
 * kv_len: device int32[B] or NULL for no padding.  Everything else (masks, scale,
 * alignment, ownership and errors) is as in fa_forward_kvlen / fa_backward_kvlen, except
 * that the backward's workspace must hold fa_backward_gqa_workspace_size(B, H, H_kv, N,
 * d) bytes; H_kv < 1 or H % H_kv != 0 returns FA_ERR_KVHEADS.  The backward is
 * deterministic: each K/V head's dk and dv accumulate its group's query heads in a
 * fixed order (in registers, and across workgroups through fp32 partials summed in
 * split order).
 */
int fa_forward_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int H_kv, int N,
                   int d, float scale, int causal, const int32_t* kv_len, fa_stream_t stream);
/*
 * Workspace bytes fa_backward_gqa needs: the row statistics of fa_backward_workspace_size
 * (B, H, N, d), plus, when the B * H_kv * ceil(N / 128) (key block, K/V head) pairs are
 * too few to fill the GPU, fp32 partial dK and dV for each of the S workgroups that split
 * a group's query heads (2 * S * B * H_kv * N * d * 4 bytes, S <= H / H_kv); the partials
 * are summed in a fixed order, so results stay deterministic.  Equals
 * fa_backward_workspace_size(B, H, N, d) when H_kv = H.  Returns 0 for invalid sizes.
 */
size_t fa_backward_gqa_workspace_size(int B, int H, int H_kv, int N, int d);
int fa_backward_gqa(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                    void* dq, void* dk, void* dv, int B, int H, int H_kv, int N, int d, float scale, int causal,
                    const int32_t* kv_len, void* workspace, size_t workspace_bytes, fa_stream_t stream);

/*
 * FP8 forward with block quantisation and incoherent processing.  The
 * "FlashAttention" concept wiki page (section FA3 (3), and the cross-cutting insight on
 * FP8 stability) names the method -- FP8 inputs with FP32 accumulation, block
 * quantisation, incoherent processing -- and nothing more; the format, block size and
 * transform below are this library's readings.  Format: OCP E4M3 (1-4-3, bias 7,
 * subnormals, largest finite 448, 0x7F/0xFF NaN); every conversion rounds to nearest
 * even after clamping to +-448.  Three steps, each one call:
 *
 * fa_fp8_quantize_qk -- block quantisation of Q or K.  x: bf16 [B][H][N][d] (read only);
 *   x8: E4M3 codes [B][H][N][d] (written); scales: fp32 [B][H][ceil(N/64)] (written),
 *   one per block of 64 rows of a head.  For each row y = x, or, when signs != NULL
 *   (device fp32[d] of +-1), y = (x * signs) H_d with H_d the unnormalised d x d
 *   Sylvester-Hadamard matrix (fast Walsh-Hadamard butterflies in fp32, fixed order:
 *   stage h = 1, 2, ..., d/2, pairs (i, i+h) -> (a+b, a-b)).  Per block: amax = max |y|,
 *   code = e4m3(y * (448 / amax)), scale = (amax / 448) * post_scale (all fp32); a block
 *   of zeros has scale 0 and codes 0.  Incoherent processing rotates Q and K with the
 *   same signs, which multiplies Q K^T by d: pass post_scale = 1/d for Q (1 for K) so
 *   that (codes * scales) of Q and K reproduce Q K^T.
 * fa_fp8_quantize_v -- column quantisation of V.  v: bf16 [B][H][N][d] (read only);
 *   v8t: E4M3 codes in the layout the forward consumes, [B][H][ceil(N/64)][d][64]
 *   (written; byte 32*g + p of row c of tile t is the code of V[64 t + key(g, p)][c],
 *   key(g, p) = 32*(p/16) + 8*((p%16)/4) + 4*g + p%4, g in {0,1}, p in 0..31; keys past N
 *   hold code 0); scales: fp32 [B][H][d] (written), one per column of a head over all N
 *   rows, with the formulas above (post_scale 1).  Four kernel launches on `stream`.
 * fa_forward_fp8 -- O = softmax(scale * Qd Kd^T [+ masks]) Vd for the dequantised
 *   inputs Qd = q8 * q_scale (per 64-row block), Kd = k8 * k_scale, Vd = v8t * v_scale
 *   (per column), computed with E4M3 x E4M3 products and fp32 accumulation; P is rounded
 *   to E4M3 before P V.  o: bf16 [B][H][N][d], lse: fp32 [B][H][N] (natural log, of the
 *   dequantised scores), both overwritten.  Masks, scale, kv_len and the rules on
 *   ownership, streams and errors are those of fa_forward_kvlen.
 *
 * All pointers are device pointers; x8, q8, k8 and v8t must be 16-byte aligned, scale
 * arrays 4-byte aligned.  d must be 64 or 128.
 */
int fa_fp8_quantize_qk(const void* x, uint8_t* x8, float* scales, const float* signs, float post_scale, int B, int H,
                       int N, int d, fa_stream_t stream);
int fa_fp8_quantize_v(const void* v, uint8_t* v8t, float* scales, int B, int H, int N, int d, fa_stream_t stream);
int fa_forward_fp8(const uint8_t* q8, const float* q_scale, const uint8_t* k8, const float* k_scale,
                   const uint8_t* v8t, const float* v_scale, void* o, float* lse, int B, int H, int N, int d,
                   float scale, int causal, const int32_t* kv_len, fa_stream_t stream);

/* Human-readable name of a status code (static string, never NULL). */
const char* fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA355_FA_H */
