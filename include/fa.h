/*
 * fa.h - C ABI of the exact tiled attention forward pass on AMD Instinct MI355X (gfx950).
 *
 * The operation ("vectorized-flash-attention-kernel", Core algorithm; Constructor
 * options; Key design decisions 1, 3 and 4): for every batch b, head h and query
 * row i,
 *
 *     J_i   = { j : j < kv_len[b]  and  (causal == 0  or  j <= i) }
 *     s_j   = scale * sum_d Q[b,h,i,d] * K[b,h,j,d]                  (j in J_i)
 *     O_i   = sum_j exp(s_j - m) V[b,h,j,:] / l,  m = max_j s_j,  l = sum_j exp(s_j - m)
 *     LSE_i = m + ln l                                               (natural log)
 *
 * computed tile by tile with the online-softmax recurrence (running row max and
 * denominator, accumulator rescaled by exp(m_old - m_new)), so the N x N score
 * matrix never reaches device memory. A row with no valid key (J_i empty) yields
 * O_i = 0 exactly and LSE_i = -inf, never NaN
 * ("js-flash-attention-tiled-online-softmax-exactness", Root causes addressed 2).
 * Key padding follows "Paper: FlashAttention", Objectives, Code (hardened masking:
 * padding, empty rows): keys at or past kv_len[b] are masked; query rows never are.
 * The causal mask is top-left aligned: key j is visible to query i iff j <= i.
 *
 * Arithmetic: Q.K^T and P.V run on the matrix cores with float32 accumulation;
 * softmax statistics are float32. For bf16/f16 inputs the probabilities P are
 * rounded to the input type (round to nearest even) before P.V, and O is
 * rounded to the input type on store. The float32 path keeps P in float32.
 */
#ifndef FA_H
#define FA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of Q, K, V and O. */
typedef enum { FA_F32 = 0, FA_BF16 = 1, FA_F16 = 2 } fa_dtype;

/* Return codes: 0 on success, negative on error. */
enum {
  FA_OK = 0,
  FA_ERR_NULL = -1,        /* a required pointer is NULL                                   */
  FA_ERR_SHAPE = -2,       /* a negative size, or sizes whose products overflow            */
  FA_ERR_UNSUPPORTED = -3, /* head dimension or dtype not built                            */
  FA_ERR_ALIGN = -4,       /* Q, K, V, O or a stride not 16-byte aligned; LSE/kv_len 4-byte */
  FA_ERR_ARG = -5,         /* scale not finite, causal not 0/1, bad strides, O aliases */
  FA_ERR_HIP = -6,         /* the kernel launch was rejected by the HIP runtime            */
  FA_ERR_TOO_LARGE = -7    /* fa_bwd_noalloc: the problem needs more than its static scratch */
};

/*
 * fa_fwd - attention forward, asynchronous on `stream`.
 *
 * Q, K, V : device pointers, contiguous [B][H][N][D] of `dtype` (read only).
 * O       : device pointer, contiguous [B][H][N][D] of `dtype` (fully overwritten).
 *           Must not be any of Q, K, V.
 * LSE     : device pointer, contiguous [B][H][N] float32 (fully overwritten):
 *           ln of the softmax denominator in units of scaled logits; -inf for a
 *           fully masked row.
 * B, H, N, D : sizes. D must be 32, 64, 96 or 128 (or 256 for bf16/f16). If any of B, H,
 *           N is 0 the call does nothing and returns FA_OK (pointers are then not inspected).
 * scale   : softmax scale applied to Q.K^T; any finite value, of either sign or zero
 *           (1/sqrt(D) is usual).
 * causal  : 1 for the causal mask, 0 for none.
 * kv_len  : device pointer to int32[B], valid key count per batch, or NULL for
 *           N everywhere. Values outside [0, N] are clamped to it by the kernel.
 * dtype   : an fa_dtype value.
 * stream  : a hipStream_t, or NULL for the default stream.
 *
 * Ownership: the caller owns every buffer. The library allocates nothing, frees
 * nothing and does not synchronise; it launches one kernel on `stream`. Every
 * argument is validated before any HIP call. No global state: thread-safe.
 * Device faults (for example an out-of-range pointer) surface at the caller's
 * next synchronisation, not here.
 */
int fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE,
           int64_t B, int64_t H, int64_t N, int64_t D, float scale, int causal,
           const int32_t* kv_len, int dtype, void* stream);

/*
 * fa_fwd_strided - fa_fwd over strided Q, K, V and O. The pages' forward takes flat
 * contiguous arrays ("vectorized-flash-attention-kernel", Core algorithm); this entry point
 * accepts the strided views callers usually hold (for example [B][N][H][D] storage seen as
 * [B][H][N][D]) without a copy. The arithmetic is that of fa_fwd.
 *
 * strides : host pointer to 12 int64 element strides, or NULL for contiguous [B][H][N][D]:
 *           { q_b, q_h, q_n,  k_b, k_h, k_n,  v_b, v_h, v_n,  o_b, o_h, o_n }.
 *           Element (b, h, n, d) of X lives at X + b*x_b + h*x_h + n*x_n + d: the head
 *           dimension is contiguous. Every stride must be >= 0 and a multiple of 16 bytes.
 *           Q, K and V may overlap themselves (a stride of 0 shares one K/V head among all
 *           query heads); O must not (no two (b, h, n, d) may name the same element).
 *           K and V token strides may not exceed 16 MiB. LSE stays contiguous [B][H][N].
 * D       : 32, 64, 96 or 128 for every dtype; 256 for FA_BF16 and FA_F16.
 * q_len   : device pointer to int32[B], the number of query rows present in each batch
 *           element, or NULL for N everywhere (values outside [0, N] are clamped by the
 *           kernel). Query-side padding, the pages' hardened masking for padding applied to
 *           queries: a row at or past q_len[b] attends to nothing, its Q row is not read
 *           (it may hold anything), and it is written as O = 0, LSE = -inf. The causal mask is
 *           unchanged (row i sees keys j <= i). 4-byte aligned.
 * Other arguments, ownership and errors as fa_fwd; a negative stride or an overlapping O
 * gives FA_ERR_ARG, a misaligned stride FA_ERR_ALIGN.
 */
int fa_fwd_strided(const void* Q, const void* K, const void* V, void* O, float* LSE,
                   int64_t B, int64_t H, int64_t N, int64_t D, const int64_t* strides,
                   float scale, int causal, const int32_t* q_len, const int32_t* kv_len,
                   int dtype, void* stream);

/*
 * fa_fwd_split_workspace_bytes - device workspace that fa_fwd_split needs for these sizes
 * and n_splits: S*B*H*N*D float32 of partial O, padded to 256 bytes, then S*B*H*N float32
 * of partial LSE. Returns 0 when n_splits == 1 or any size is 0, and -1 for a negative size,
 * n_splits outside [1, 256], or sizes whose byte count overflows. Pure host arithmetic.
 */
int64_t fa_fwd_split_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D, int n_splits);

/*
 * fa_fwd_split - fa_fwd_strided with the key axis of every query tile cut into n_splits
 * parts that separate workgroups process, followed by a merge of the partial states.
 * Partial softmax states over disjoint key sets combine associatively, with the empty set
 * (O = 0, LSE = -inf) as identity ("Paper: FlashAttention", Objectives, Math & data
 * structures), so the result is the same attention up to rounding. It raises the number of
 * workgroups when B*H*ceil(N/128) alone does not fill the GPU (short batches, few heads).
 *
 * A query tile that sees T key tiles gives part s the tiles [s*c, min(T, (s+1)*c)),
 * c = ceil(T / n_splits); a part with no key writes the identity state. The partial O is
 * kept in float32 and normalised per part; the merge (fa_merge_states) rounds O once.
 *
 * n_splits        : 1..256. 1 is exactly fa_fwd_strided (the workspace is then unused).
 * workspace       : device pointer, 256-byte aligned, at least
 *                   fa_fwd_split_workspace_bytes(B, H, N, D, n_splits) bytes, not overlapping
 *                   Q, K, V, O or LSE. Its contents on entry do not matter; on return it holds
 *                   the partial states (part_o then part_lse, as fa_merge_states takes them).
 * workspace_bytes : its size in bytes.
 * Other arguments as fa_fwd_strided. Two kernels are launched on `stream`, nothing is
 * allocated. Errors: n_splits out of range or a workspace that is too small gives
 * FA_ERR_ARG, a NULL workspace FA_ERR_NULL, a misaligned one FA_ERR_ALIGN; otherwise as
 * fa_fwd_strided. Calls that share one workspace on different streams race.
 */
int fa_fwd_split(const void* Q, const void* K, const void* V, void* O, float* LSE,
                 int64_t B, int64_t H, int64_t N, int64_t D, const int64_t* strides,
                 float scale, int causal, const int32_t* q_len, const int32_t* kv_len,
                 int dtype, int n_splits, void* workspace, int64_t workspace_bytes,
                 void* stream);

/*
 * fa_fwd_split_count - a suggested n_splits for fa_fwd_split on the current HIP device.
 * Picks the smallest count whose work units (B*H*query tiles*parts) fill every workgroup
 * slot of the device once (twice when causal, whose query tiles differ in length), capped at
 * 16 and so that every part keeps at least 4 key tiles; 1 when B*H*query tiles alone already
 * do. The slot count comes from the device's compute-unit count and the kernel's occupancy.
 * Writes the count (>= 1) to *n_splits and returns FA_OK; errors as fa_fwd for bad sizes,
 * dtype, D or causal, FA_ERR_NULL for a NULL n_splits, FA_ERR_HIP if the device query fails.
 * If any of B, H, N is 0 it writes 1 without a HIP call.
 */
int fa_fwd_split_count(int64_t B, int64_t H, int64_t N, int64_t D, int causal, int dtype,
                       int* n_splits);

/*
 * fa_merge_states - merge S partial attention states per row ("Paper: FlashAttention",
 * Objectives, Math & data structures: the associative merge of partial softmax states).
 * For row (b, h, n), with m = max_s LSE_s and w_s = exp(LSE_s - m):
 *     LSE = m + ln(sum_s w_s),   O = sum_s w_s O_s / sum_s w_s;
 * states with LSE_s = -inf are the identity and are skipped; a row whose every state is the
 * identity gets O = 0 and LSE = -inf.
 *
 * part_o   : device pointer, contiguous float32 [S][B][H][N][D], each O_s normalised over
 *            its own key set (16-byte aligned). Read only.
 * part_lse : device pointer, contiguous float32 [S][B][H][N], natural-log LSE_s. Read only.
 * n_states : S, 1..256.
 * O        : device pointer of `dtype`, strided as o_strides (3 int64 element strides
 *            {b, h, n} on the host, or NULL for contiguous [B][H][N][D]); fully overwritten.
 * LSE      : device pointer, contiguous float32 [B][H][N]; fully overwritten.
 * D        : 32, 64, 96, 128 or 256 for every dtype.
 * One kernel on `stream`; nothing is allocated. Errors as fa_fwd_strided, FA_ERR_ARG for
 * n_states out of range.
 */
int fa_merge_states(const float* part_o, const float* part_lse, int n_states,
                    int64_t B, int64_t H, int64_t N, int64_t D, void* O,
                    const int64_t* o_strides, float* LSE, int dtype, void* stream);

/*
 * fa_bwd_workspace_bytes - device workspace fa_bwd needs: B*H*ceil(N/64)*128 float32 (per
 * 64-row block of each (b, h): the rows' exponent offsets, then their negated Delta values). 0 when any
 * size is 0, -1 for a negative size or a byte count that overflows. Pure host arithmetic.
 */
int64_t fa_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D);

/*
 * fa_bwd - gradients of the forward above by recomputation, asynchronous on `stream`
 * ("vectorized-flash-attention-kernel", Key design decision 4: the forward's per-row
 * statistics let every block of S and P be rebuilt for dQ, dK, dV; "Paper: FlashAttention",
 * Objectives, Math & data structures: the backward by recomputation and the identity
 * rowsum(dP o P) = rowsum(dO o O)). For the loss gradient dO = dL/dO:
 *
 *     P_ij  = exp(scale <q_i, k_j> - LSE_i)   (0 for masked pairs; J_i as for fa_fwd)
 *     Delta_i = sum_d dO_id O_id
 *     dV_j  = sum_i P_ij dO_i
 *     dS_ij = P_ij (<dO_i, v_j> - Delta_i)
 *     dQ_i  = scale sum_j dS_ij k_j,     dK_j = scale sum_i dS_ij q_i
 *
 * Keys at or past kv_len[b] get dK = dV = 0; rows with no valid key get dQ = 0.
 *
 * Q, K, V, O, dO : device pointers, contiguous [B][H][N][D] of `dtype` (read only). O and LSE
 *           are the outputs of fa_fwd (or fa_fwd_strided / fa_fwd_split) for the same Q, K, V,
 *           scale, causal and kv_len.
 * LSE     : device pointer, contiguous [B][H][N] float32 (read only).
 * dQ, dK, dV : device pointers, contiguous [B][H][N][D] of `dtype` (fully overwritten); they may
 *           not overlap each other, any input, or the workspace.
 * D       : 32, 64, 96 or 128. dtype: FA_BF16 or FA_F16 (FA_F32 gives FA_ERR_UNSUPPORTED).
 * workspace, workspace_bytes : device memory of at least fa_bwd_workspace_bytes(B, H, N, D)
 *           bytes, 256-byte aligned; its contents on entry do not matter.
 * Arithmetic: the products run on the matrix cores with float32 accumulation; P and dS are
 * rounded to `dtype` before the products that take them; dQ, dK, dV are rounded on store.
 * Two kernels run on `stream` (the second reads what the first writes to the workspace);
 * dQ and dK/dV each have a single writer, so results are identical run to run.
 * Errors as fa_fwd; a workspace that is too small, or overlapping outputs, give FA_ERR_ARG.
 */
int fa_bwd(const void* Q, const void* K, const void* V, const void* O, const float* LSE,
           const void* dO, void* dQ, void* dK, void* dV,
           int64_t B, int64_t H, int64_t N, int64_t D, float scale, int causal,
           const int32_t* kv_len, int dtype, void* workspace, int64_t workspace_bytes,
           void* stream);

/*
 * fa_bwd_strided - fa_bwd over strided tensors: the views callers usually hold (for example
 * [B][N][H][D] storage seen as [B][H][N][D]) without a copy. The arithmetic is that of fa_bwd.
 *
 * strides : host pointer to 24 int64 element strides, or NULL for contiguous [B][H][N][D]
 *           (then exactly fa_bwd): { q_b, q_h, q_n,  k_b, k_h, k_n,  v_b, v_h, v_n,
 *           o_b, o_h, o_n,  do_b, do_h, do_n,  dq_b, dq_h, dq_n,  dk_b, dk_h, dk_n,
 *           dv_b, dv_h, dv_n }. Element (b, h, n, d) of X lives at X + b*x_b + h*x_h + n*x_n + d.
 *           Every stride must be >= 0 and a multiple of 16 bytes; the token strides of Q, K, V
 *           and dO may not exceed 16 MiB. Inputs may overlap themselves (a zero head stride on K
 *           and V shares one K/V head among all query heads; dK and dV are then the gradients
 *           per query head, which the caller sums over the heads that share one). dQ, dK and dV
 *           must not overlap themselves (FA_ERR_ARG), nor each other or any input; only an
 *           output starting at an input, another output or the workspace is detected.
 * q_len   : device pointer to int32[B] or NULL, as for fa_fwd_strided (pass the forward's
 *           q_len). Rows at or past q_len[b] are not part of the batch element: their rows of
 *           Q, O and dO are not read (they may hold anything, NaN included), their dQ rows are
 *           written as 0, and they add nothing to dK or dV. 4-byte aligned.
 * LSE and the workspace stay contiguous. Other arguments and errors as fa_bwd.
 */
int fa_bwd_strided(const void* Q, const void* K, const void* V, const void* O, const float* LSE,
                   const void* dO, void* dQ, void* dK, void* dV,
                   int64_t B, int64_t H, int64_t N, int64_t D, const int64_t* strides,
                   float scale, int causal, const int32_t* q_len, const int32_t* kv_len,
                   int dtype, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * fa_bwd_noalloc - fa_bwd for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving or training loops, harnesses that forbid hipMalloc): the same
 * arguments, arithmetic, outputs and errors as fa_bwd, without the workspace arguments. Its
 * workspace is a static device array of FA_NOALLOC_SCRATCH_BYTES bytes inside this library,
 * one copy per GPU, held until the process ends. The call allocates nothing and frees nothing.
 *
 * Limit: fa_bwd_workspace_bytes(B, H, N, D) <= FA_NOALLOC_SCRATCH_BYTES, i.e. B*H*ceil(N/64)
 * <= 65536 blocks of 64 rows (e.g. B*H = 64 heads of N = 65536); a larger problem returns
 * FA_ERR_TOO_LARGE before any HIP call.
 * Sharing: every call on one GPU uses that GPU's array, which keeps the last call's contents
 * (each call writes every entry it reads before reading it). Calls that overlap on one GPU
 * (on different streams, or from different threads without ordering) race on the array:
 * order them on one stream. The first call on a GPU looks up the array's device address
 * (hipGetSymbolAddress with that GPU current) and keeps it for later calls.
 * stream : as for fa_bwd; the array of the stream's device is used (the current device for
 *          the null stream).
 */
#define FA_NOALLOC_SCRATCH_BYTES (32LL << 20)
int fa_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O, const float* LSE,
                   const void* dO, void* dQ, void* dK, void* dV,
                   int64_t B, int64_t H, int64_t N, int64_t D, float scale, int causal,
                   const int32_t* kv_len, int dtype, void* stream);

/* Static, human-readable text for a return code of fa_fwd. Never NULL. */
const char* fa_strerror(int code);

/* Version of this ABI; bumped when a signature or a semantic changes. */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
