/*
 * attn.h — C ABI of the MI355X (gfx950) exact tiled attention forward pass.
 *
 * Operation (standard attention of the zsdodo.com page "AI训练的最大障碍不是算力,
 * 而是“内存墙”", code block of standard PyTorch attention; softmax with the row
 * max subtracted, unite.ai page "闪电注意力：革命性地提高Transformer效率", section
 * "闪电注意力的数学原理", formula 1; tiled with a running max m and running sum ℓ as
 * in the ``safe_softmax_block`` code block of the zsdodo.com page): for batch b,
 * query head h, query row i, with kv head g = h / (H / Hkv) and admissible keys
 *     A(b,i) = { j in [0, N) : j < key_len_b  and  (causal == 0 or j <= i) },
 *     s_ij   = scale * <q[b,h,i,:], k[b,g,j,:]>,
 *     m_i    = max_{j in A} s_ij,   ℓ_i = sum_{j in A} exp(s_ij - m_i),
 *     o[b,h,i,:] = sum_{j in A} exp(s_ij - m_i) * v[b,g,j,:] / ℓ_i,
 *     lse[b,h,i] = m_i + ln ℓ_i   (natural log).
 * A row with no admissible key (key_len_b == 0) gets o = 0 and lse = -inf.
 * The N x N score matrix is never written to memory; the library allocates
 * nothing (only the split-KV forward takes a caller-owned workspace).
 *
 * Layouts (all contiguous, row-major, element strides implied by the sizes):
 *     q, o : [B][H][N][d]      k, v : [B][Hkv][N][d]      lse : [B][H][N] fp32
 *     key_lens : NULL (every sequence has N keys) or int32 [B] in DEVICE memory;
 *                each value is clamped to [0, N] on the device.
 * All pointers except key_lens are DEVICE pointers owned by the caller; every
 * non-NULL pointer must be 16-byte aligned.  o must not overlap q, k or v
 * (undefined result otherwise).
 *
 * Execution: the kernel is enqueued on `stream` (a hipStream_t; NULL = the
 * null stream) and the call returns without waiting.  Arguments are validated
 * on the host before any HIP call, so an invalid call touches no device
 * state.  Calls keep no state and are thread-safe.  No C++ exception crosses
 * this interface.
 *
 * Sizes: B >= 0, N >= 0 (B == 0 or N == 0 is a no-op returning ATTN_OK, and
 * the data pointers may then be NULL), H >= 1, Hkv >= 1, H % Hkv == 0,
 * d in {64, 128}, causal in {0, 1}, scale finite; B*H*ceil(N/128) work tiles
 * must not exceed 16,777,215, N*d*4 must stay below 2^31 (one head's slice is
 * addressed with 32-bit byte offsets: N <= 4,194,303 at d = 128) and B*H*N*d
 * below 2^62.  Checks run in this order: shape, head dim, scale, size limits,
 * empty problem (returns ATTN_OK), NULL pointers, alignment.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_NULL = 1,      /* a required pointer is NULL                         */
    ATTN_ERR_SHAPE = 2,     /* B, H, Hkv, N or causal out of range, or too large  */
    ATTN_ERR_HEAD_DIM = 3,  /* d is not 64 or 128                                 */
    ATTN_ERR_ALIGN = 4,     /* a pointer is not 16-byte aligned                   */
    ATTN_ERR_SCALE = 5,     /* scale is NaN or infinite                           */
    ATTN_ERR_HIP = 6,       /* the kernel launch failed (hipGetLastError)         */
    ATTN_ERR_WORKSPACE = 7, /* split-KV workspace NULL or too small               */
    ATTN_ERR_SCRATCH = 8    /* larger than the built-in scratch of a no-alloc call */
} attn_status;

/* Floats of the built-in device scratch of attn_bwd_bf16_noalloc (16 MiB). */
#define ATTN_NOALLOC_SCRATCH_FLOATS (4 * 1024 * 1024)

/* Most key ranges one split-KV call may use. */
#define ATTN_MAX_SPLITS 64

/* bf16 q, k, v, o (raw 16-bit bfloat16 storage); fp32 lse.  QKᵀ and P·V run on
 * bf16 matrix cores with fp32 accumulation; the softmax runs in fp32; P is
 * rounded to bf16 before P·V and o is rounded to bf16 (nearest even). */
int attn_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int H, int Hkv, int N, int d, float scale, int causal,
                  const int32_t* key_lens, void* stream);

/* fp32 q, k, v, o and lse; every product and sum in fp32 (fp32 matrix cores). */
int attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                 int B, int H, int Hkv, int N, int d, float scale, int causal,
                 const int32_t* key_lens, void* stream);

/* Packed variable-length sequences, bf16 (the padding handling of the aifi
 * page, production tips, dynamic sequences: padded positions must not take
 * part; here the sequences are packed end to end so that no padding exists).
 * Sequence b (0 <= b < B) is tokens s_b .. e_b − 1 with s_b = cu_seqlens[b],
 * e_b = cu_seqlens[b + 1]; within it the operation above applies with
 * N = key_len = e_b − s_b and query row i = token s_b + i:
 *     q, o : [total][H][d]     k, v : [total][Hkv][d]     lse : [H][total] fp32
 * (token-major, heads interleaved: the `b n (h d)` activations of the aifi
 * page's PyTorch example with the sequences laid end to end).  Every token of
 * a sequence is a query and a key of that sequence only; causal == 1 admits
 * keys j <= i of the same sequence.  cu_seqlens is int32 [B + 1] in DEVICE
 * memory (4-byte aligned) and must satisfy 0 = cu[0] <= cu[1] <= ... <=
 * cu[B] = total and e_b − s_b <= max_seqlen; the device clamps offsets into
 * [0, total] and lengths to max_seqlen, so bad offsets cannot make it read or
 * write out of bounds, but tokens they leave out are not written.  Sizes:
 * B >= 0, total >= 0, max_seqlen >= 0 (B, total or max_seqlen == 0: no-op),
 * the limits of attn_fwd_bf16 with N = max_seqlen, and (max_seqlen + 128)·H·d·2
 * below 2^31.  Same status codes and check order as attn_fwd_bf16; the other
 * pointers must be 16-byte aligned.  Enqueued on `stream`, not waited on. */
int attn_fwd_varlen_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                         const int32_t* cu_seqlens, int B, int H, int Hkv, int total, int max_seqlen,
                         int d, float scale, int causal, void* stream);

/* FP8 forward (the low-precision step of the unite.ai page, section
 * "闪电注意力-3"): the operation above on fp8 operands.  q [B][H][N][d],
 * k [B][Hkv][N][d] and vt [B][Hkv][d][N16] (V TRANSPOSED: its rows are the d
 * features, each over the keys; N16 = N rounded up to a multiple of 16, and
 * the columns N .. N16 - 1 of a row are never used) hold OCP fp8 e4m3 bytes;
 * the values they stand for are q_descale·q, k_descale·k, v_descale·v.
 * Outputs o bf16 [B][H][N][d] and lse fp32 [B][H][N] as for attn_fwd_bf16,
 * for those values.  Both products run on fp8 matrix cores with fp32
 * accumulation; the softmax runs in fp32 and its weights are rounded to fp8
 * e4m3 (relative error at most 2^-4 each, after scaling by 2^7 relative to a
 * running reference that is at most 2x below the true max, so they stay in
 * range) before P·V; the row sums use the fp32 weights.  Any N >= 0;
 * descale factors finite; scale·q_descale·k_descale finite.  Other limits,
 * checks and status codes as attn_fwd_bf16 (vt is checked as its v).  Padded
 * keys (past key_lens[b]) never reach the output, NaN included.  The inputs
 * can be made on the GPU with attn_fp8_amax, attn_fp8_quantize (queries and
 * keys, optionally rotated: incoherent processing) and attn_fp8_quantize_vt. */
int attn_fwd_fp8(const void* q, const void* k, const void* vt, void* o, float* lse,
                 float q_descale, float k_descale, float v_descale,
                 int B, int H, int Hkv, int N, int d, float scale, int causal,
                 const int32_t* key_lens, void* stream);

/* Incoherent processing and fp8 quantisation (unite.ai page, section
 * "闪电注意力-3": FlashAttention-3 uses incoherent processing to lower the
 * quantisation error of its FP8 step).  The rotation R = H_d · diag(signs)
 * / sqrt(d) (H_d the Sylvester-Hadamard matrix, H[i][j] =
 * (-1)^popcount(i & j); signs a caller-drawn fp32 vector of d values +1 or
 * -1) multiplies every row of q and of k: applied to both with the same
 * signs it leaves every score q·k, and so O and LSE, unchanged, while an
 * outlier feature is spread over all d features before the per-tensor scale
 * is chosen.  V is not rotated.
 *
 * attn_fp8_amax: *amax = the largest |R x| over the `rows` rows of d bf16
 * values of x ([rows][d], contiguous); signs == NULL: the largest |x| (no
 * rotation).  NaN entries take no part.  amax is a DEVICE float, first set
 * to 0 and then raised with atomic maxima (two kernels on `stream`).
 *
 * attn_fp8_quantize: x8[r][:] = e4m3(R x[r] / descale) (or x[r] / descale
 * when signs is NULL), e4m3 meaning OCP fp8 E4M3FN, nearest value, ties to
 * even, after clamping to +-448 (NaN stays NaN), with descale = *amax / 448
 * in fp32 (1 when *amax is 0); the kernel also writes that descale into the
 * DEVICE float *descale, the value attn_fwd_fp8 needs for this tensor.  x8
 * is [rows][d] bytes.
 *
 * attn_fp8_quantize_vt: V [heads][N][d] bf16 (heads = B·Hkv) to its
 * transposed fp8 form vt8 [heads][d][N16] (N16 = N rounded up to a multiple
 * of 16, columns N .. N16 - 1 written as 0), e4m3(v / descale) with descale
 * from *amax as above (use attn_fp8_amax with signs == NULL on v first),
 * also written to *descale.
 *
 * All pointers are DEVICE pointers: x, x8, v, vt8 and signs 16-byte aligned,
 * amax and descale 4-byte aligned; outputs must not overlap inputs.  rows >=
 * 0 (at most 2^46), heads >= 0, N >= 0 (N·d·2 below 2^31), d in {64, 128}.
 * Status codes: ATTN_ERR_SHAPE, ATTN_ERR_HEAD_DIM, ATTN_ERR_NULL,
 * ATTN_ERR_ALIGN (checked in that order, before any HIP call), ATTN_ERR_HIP.
 * Enqueued on `stream`, not waited on.  These kernels are bound by HBM (2
 * bytes read and 1 written per element). */
int attn_fp8_amax(const void* x, const float* signs, int64_t rows, int d, float* amax, void* stream);
int attn_fp8_quantize(const void* x, const float* signs, int64_t rows, int d, const float* amax, void* x8,
                      float* descale, void* stream);
int attn_fp8_quantize_vt(const void* v, int64_t heads, int N, int d, const float* amax, void* vt8, float* descale,
                         void* stream);

/* Split-KV (the key range of every query cut into pieces whose partial
 * results are combined afterwards: the softmax-merge rule of the unite.ai
 * page, section "闪电注意力的数学原理", formula 2, read as LSE = ln Σ_s e^{LSE_s},
 * O = Σ_s e^{LSE_s − LSE}·O_s; the same page's FlashAttention-2 section counts
 * parallelism over the sequence among its improvements).
 *
 * attn_fwd_partial_bf16: attention of Nq queries over ONE block of Nk keys.
 * q [B][H][Nq][d] and k, v [B][Hkv][Nk][d] bf16; query i sits at position
 * q_offset + i and key j at k_offset + j of the whole sequence, and under a
 * causal mask key j is admissible for query i iff k_offset + j <= q_offset + i
 * (no mask: every key of the block).  Writes the block's own normalised
 * result: o_part [B][H][Nq][d] fp32 (o = Σ_j P_ij v_j / Σ_j P_ij over the
 * block's admissible keys) and lse_part [B][H][Nq] fp32; a row with no
 * admissible key in the block gets o_part = 0 and lse_part = -inf.  Nk == 0
 * is allowed (every row empty; k and v may then be NULL).  Other checks,
 * limits (with N = Nq, and Nk·d·4 below 2^31) and status codes as
 * attn_fwd_bf16.  Enqueued on `stream`, not waited on. */
int attn_fwd_partial_bf16(const void* q, const void* k, const void* v, float* o_part, float* lse_part,
                          int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                          int q_offset, int k_offset, void* stream);

/* attn_merge: combines S partial results over disjoint key sets of the same
 * queries.  o_parts fp32 [S][B][H][N][d] and lse_parts fp32 [S][B][H][N]
 * (as written by attn_fwd_partial_bf16); o is [B][H][N][d], bf16 when
 * o_bf16 == 1 and fp32 when 0 (so that merges can be chained), lse fp32
 * [B][H][N].  Parts with lse = -inf take no part; a row empty in every part
 * gets o = 0, lse = -inf.  S >= 1, B >= 0, H >= 1, N >= 0, d in {64, 128};
 * all pointers device, 16-byte aligned; o must not overlap the inputs.
 * Enqueued on `stream`, not waited on. */
int attn_merge(const float* o_parts, const float* lse_parts, int S, int B, int H, int N, int d,
               void* o, int o_bf16, float* lse, void* stream);

/* attn_fwd_splitkv_bf16: attention of Nq queries over Nk keys, the keys cut
 * into num_splits (1 .. ATTN_MAX_SPLITS) ranges of ceil(Nk / num_splits) keys
 * rounded up to a multiple of 128 (so fewer ranges may result), one partial
 * result per range (O in bf16, LSE in fp32, in the workspace), merged as in
 * attn_merge: two kernels on
 * `stream`.  q, o [B][H][Nq][d] and k, v [B][Hkv][Nk][d] bf16, lse
 * [B][H][Nq] fp32; positions and the causal rule as attn_fwd_partial_bf16
 * (self-attention: Nq = Nk = N, q_offset = k_offset = 0, which is
 * attn_fwd_bf16's operation); key_lens as in attn_fwd_bf16, cutting the Nk
 * keys.  It fills the GPU when B·H·ceil(Nq/128) is small (few queries over
 * many keys).  workspace: caller-owned device memory of at least
 * attn_splitkv_workspace_bytes(B, H, Nq, d, num_splits) bytes, 16-byte
 * aligned, overwritten (ATTN_ERR_WORKSPACE if NULL or too small; unused, and
 * may be NULL, when a single range results).  Checks and limits as
 * attn_fwd_partial_bf16, then num_splits, then the workspace. */
int attn_fwd_splitkv_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                          int q_offset, int k_offset, const int32_t* key_lens, int num_splits,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes attn_fwd_splitkv_bf16 needs for Nq queries (0 for invalid sizes). */
size_t attn_splitkv_workspace_bytes(int B, int H, int Nq, int d, int num_splits);

/* Backward pass, bf16 (gradients of L = Σ O ∘ dout through the operation
 * above; the attention weights are recomputed from q, k and the forward's lse
 * rather than stored: unite.ai page "闪电注意力：革命性地提高Transformer效率",
 * section "闪电注意力的到来", key idea 2):
 *     P = exp(scale·q kᵀ − lse) on the admissible keys, D_i = Σ_d dout_i,d o_i,d,
 *     dS = P ∘ (dout vᵀ − D),  dq = scale·dS k,  dk = scale·dSᵀ q,  dv = Pᵀ dout,
 * with the grouped query heads of a kv head adding into its dk and dv.
 * Inputs q, k, v, o, dout (bf16) and lse (fp32) in the layouts above; o and lse
 * must be this library's forward results for the same arguments.  Outputs
 * dq [B][H][N][d], dk, dv [B][Hkv][N][d] (bf16, every element written; padded
 * keys get 0).  delta: caller-owned fp32 [2][B][H][N] scratch, overwritten
 * with D and with lse·log2(e).
 * Products on bf16 matrix cores with fp32 accumulation; P and dS are rounded
 * to bf16 as operands.  Any finite scale.  Two kernels are enqueued on
 * `stream` in order; same validation and status codes as attn_fwd_bf16 (q, k,
 * v, dq and lse are checked as its q, k, v, o and lse; then o, dout, dk, dv,
 * delta for NULL and alignment).  Outputs must not overlap the inputs. */
int attn_bwd_bf16(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                  void* dq, void* dk, void* dv, float* delta,
                  int B, int H, int Hkv, int N, int d, float scale, int causal,
                  const int32_t* key_lens, void* stream);

/* attn_bwd_bf16 for callers that cannot allocate device memory (code under
 * HIP graph capture, tight training loops, harnesses that forbid hipMalloc):
 * the same arguments without `delta`, the same kernels and results.  The D /
 * base-2 LSE scratch (2·B·H·N floats) lives in a device array built into the
 * library, ATTN_NOALLOC_SCRATCH_FLOATS floats (16 MiB) on each GPU the
 * library runs on, held until the process ends; a problem with 2·B·H·N above
 * that limit returns ATTN_ERR_SCRATCH (checked on the host after the checks
 * of attn_bwd_bf16, before any HIP call).  The call allocates nothing: no
 * hipMalloc, no hipFree, no allocating library routine.  The first call on a
 * device looks up the array's address there (hipGetSymbolAddress).  Every
 * call on one GPU shares that GPU's array, so calls that overlap on one GPU
 * (concurrent streams, or threads on one stream) race and give undefined
 * results; calls in stream order do not.  Nothing needs clearing between
 * calls: the first kernel writes every scratch value the second reads. */
int attn_bwd_bf16_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                          const float* lse, void* dq, void* dk, void* dv,
                          int B, int H, int Hkv, int N, int d, float scale, int causal,
                          const int32_t* key_lens, void* stream);

/* The hot path: identical to attn_fwd_bf16. */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int Hkv, int N, int d, float scale, int causal,
             const int32_t* key_lens, void* stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* attn_status_str(int status);

/* Name, code and text of the HIP error behind the calling thread's most recent
 * ATTN_ERR_HIP ("none" if it has had none).  The pointer is owned by the
 * library and stays valid until the thread's next call of this function. */
const char* attn_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
