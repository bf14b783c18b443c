/*
 * tokengate.h -- C ABI of the TokenGate gated-prefill hot path on gfx950.
 *
 * The four calls implement, for one gated layer L of a decoder:
 *   tg_score        scoring network + per-sequence RMS normalisation
 *   tg_select_topk  top-K of the prunable tokens, prompt tokens always kept
 *   tg_gather       compaction of the kept rows
 *   tg_gated_attn   token-gated causal attention over the kept tokens
 * and, between the last two, tg_qkv_proj, the projections of the kept rows;
 * tg_gated_decode runs one decode step over the pruned caches afterwards;
 * tg_gated_attn_bwd and tg_score_bwd give the gradients for training.
 * Source: "TokenGate: Adapting LLMs for Fast and Memory-Efficient Prefill
 * with Learned Token Pruning", §4.1 (Eq. 3-4) and §4.2 (Eq. 5-8).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Pointers marked "dev" are device pointers (hipMalloc'd or any memory the
 *   GPU can read); "host" pointers are ordinary host memory read during the
 *   call.  The library never allocates, frees or synchronises: every call
 *   only validates its arguments on the host and enqueues kernels on
 *   `stream`, so it can be captured into a HIP graph.  Scratch memory is a
 *   caller-owned workspace sized by the matching *_workspace_size query; its
 *   contents need no initialisation and are overwritten by every call.
 * - Token layout: sequences are packed back to back; cu_seqlens[s] is the
 *   first token of sequence s, cu_seqlens[n_seq] the total.  Within a
 *   sequence, any token may be prunable (document) or not (prompt).
 * - Outputs must not alias inputs.  Calls that share a workspace must not
 *   overlap in time (same stream is fine).
 * - Errors: arguments are checked before anything is launched.  A bad
 *   argument returns TG_ERR_INVALID_ARG, a valid but unimplemented shape or
 *   dtype TG_ERR_UNSUPPORTED, a short workspace TG_ERR_WORKSPACE, a failed
 *   launch TG_ERR_HIP; tg_last_error() then gives a thread-local message.
 *   No call aborts the process.
 */
#ifndef TOKENGATE_H
#define TOKENGATE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tg_status {
  TG_OK = 0,
  TG_ERR_INVALID_ARG = 1,
  TG_ERR_UNSUPPORTED = 2,
  TG_ERR_WORKSPACE = 3,
  TG_ERR_HIP = 4
} tg_status;

typedef enum tg_dtype { TG_F32 = 0, TG_BF16 = 1 } tg_dtype;

/* An opaque HIP stream (hipStream_t); NULL is the default stream. */
typedef void* tg_stream;

/* Static text for a status code; never NULL. */
const char* tg_status_string(int status);
/* Detail of the last failing call on this thread ("" if none). */
const char* tg_last_error(void);
/* ABI version: major * 10000 + minor * 100 + patch. */
int tg_version(void);

/* ------------------------------------------------------------------------
 * tg_score -- the gate's scoring network and score normalisation, §4.1 Eq. 3.
 *
 *   b~_j = w2 . SiLU(W1 x_j + b1) + b2                  for every token j
 *   r_s  = sqrt(mean_{j in P_s} b~_j^2 + eps)            per sequence s
 *   b_j  = b~_j / r_s  if prunable[j],  b_j = 0 otherwise
 *
 * x        dev  [t_in rows, d] of `dt`, row r at x + r * x_row_stride elements.
 *                Rows are the scorer's input (the post-attention hidden state
 *                after the block's second norm), or the residual before that
 *                norm when norm_eps >= 0.
 * w1       dev  [h, d] of `dt`, row-major (row j = input weights of hidden unit j).
 * b1       dev  [h] f32, or NULL for zero.      w2  dev [h] f32.     b2  scalar.
 * prunable dev  [t_in] u8, nonzero = document token (may be pruned).
 * cu_seqlens dev [n_seq + 1] i32, non-decreasing, cu_seqlens[n_seq] == t_in.
 * eps      >= 0; the normaliser of a sequence without prunable tokens is 1.
 * norm_eps < 0: x rows are the scorer's input as they are.  norm_eps >= 0:
 *          x rows are the residual a^L and the scorer applies the block's
 *          second norm first (§3 Eq. 1, a~ = LN2(a), an RMSNorm):
 *          x_j / sqrt(mean_c x_jc^2 + norm_eps), with the norm's weight g
 *          folded into w1 by the caller (w1[j][c] * g[c]).  No extra pass
 *          over x: the row sums of squares are taken while x is staged.
 * b_raw    dev  [t_in] f32 out (b~), or NULL (then kept in the workspace).
 * b        dev  [t_in] f32 out (normalised; 0 on prompt tokens).
 * ws       dev  workspace of >= tg_score_workspace_size(t_in, n_seq) bytes.
 * Supported: dt = TG_BF16 with d % 64 == 0 and h % 32 == 0, h <= 256,
 * x_row_stride < 2^22; or dt = TG_F32 with h <= 1024.  x and w1 rows must
 * be 16-byte aligned.
 * Reduction order is fixed, so results are bitwise reproducible.
 * ---------------------------------------------------------------------- */
size_t tg_score_workspace_size(int64_t t_in, int32_t n_seq);
tg_status tg_score(const void* x, tg_dtype dt, int64_t x_row_stride, int64_t t_in,
                   int32_t d, int32_t h, const void* w1, const float* b1, const float* w2,
                   float b2, const uint8_t* prunable, const int32_t* cu_seqlens,
                   int32_t n_seq, float eps, float norm_eps, float* b_raw, float* b,
                   void* ws, size_t ws_bytes, tg_stream stream);

/* ------------------------------------------------------------------------
 * tg_kept_sizes -- host arithmetic for the output sizes of tg_select_topk,
 * §4.1 Eq. 4: |S_s| = min(K_s, |P_s|) + |N_s|.  Lets the caller size every
 * downstream buffer without reading anything back from the device.
 *
 * cu_seqlens_host [n_seq + 1], n_prunable_host [n_seq], k_host [n_seq]: host.
 * kept_cu_seqlens_host [n_seq + 1] host out; *t_kept host out (total).
 * K_s < 0 or n_prunable outside [0, len_s] is TG_ERR_INVALID_ARG.
 * ---------------------------------------------------------------------- */
tg_status tg_kept_sizes(const int32_t* cu_seqlens_host, const int32_t* n_prunable_host,
                        const int32_t* k_host, int32_t n_seq, int32_t* kept_cu_seqlens_host,
                        int64_t* t_kept);

/* ------------------------------------------------------------------------
 * tg_select_topk -- the top-K selector with forced keep of prompt tokens,
 * §4.1 Eq. 4:  S_s = top-K_{j in P_s}(b_j)  U  N_s.
 *
 * Order: b descending, lower index first on ties; -0.0 == +0.0; NaN ranks
 * below -inf.  K_s counts prunable tokens; K_s >= |P_s| keeps all of P_s;
 * K_s == 0 keeps only the prompt tokens.
 * b          dev [t_in] f32 scores (normally tg_score's output).
 * prunable   dev [t_in] u8.          cu_seqlens dev [n_seq + 1] i32.
 * k          dev [n_seq] i32 budgets, each >= 0 (negative budgets are read as 0).
 * Outputs, ascending original index within each sequence, sequences in order:
 *   kept_idx        dev [t_kept_capacity] i32, global token index
 *   kept_pos        dev [t_kept_capacity] i32 (or NULL), index within its sequence
 *   kept_b          dev [t_kept_capacity] f32 (or NULL), b at the kept token
 *   kept_cu_seqlens dev [n_seq + 1] i32, offsets of each sequence's kept tokens
 * t_kept_capacity: length of the three per-token outputs.  The exact count is
 * tg_kept_sizes()'s t_kept; entries beyond the capacity are not written.
 * ws dev workspace of >= tg_select_workspace_size(t_in, n_seq) bytes.
 * Integer work throughout: the result is exact and reproducible.
 * ---------------------------------------------------------------------- */
size_t tg_select_workspace_size(int64_t t_in, int32_t n_seq);
tg_status tg_select_topk(const float* b, const uint8_t* prunable, const int32_t* cu_seqlens,
                         const int32_t* k, int32_t n_seq, int64_t t_in,
                         int64_t t_kept_capacity, int32_t* kept_idx, int32_t* kept_pos,
                         float* kept_b, int32_t* kept_cu_seqlens, void* ws, size_t ws_bytes,
                         tg_stream stream);

/* ------------------------------------------------------------------------
 * tg_select_topk_noalloc -- tg_select_topk for callers that cannot allocate
 * device memory at all (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same selection, the same kernels
 * and the same arguments without ws / ws_bytes.  Its scratch memory is a
 * static device array of TG_SELECT_SCRATCH_BYTES bytes, one per GPU, held
 * by the library until the process ends; the call itself allocates nothing.
 *
 * Limit: tg_select_workspace_size(t_in, n_seq) must not exceed
 * TG_SELECT_SCRATCH_BYTES (8 MiB: e.g. one sequence of up to 3.2 million
 * tokens, or 64 sequences of 32k); larger calls return TG_ERR_WORKSPACE
 * before anything is launched.  The first call on a device looks up that
 * device's copy of the array (a failure there is TG_ERR_HIP).
 * Every call on one GPU shares that GPU's array, so calls that overlap in
 * time on one GPU (different streams, or other host threads) race and give
 * wrong results; calls in order on one stream are fine.  Nothing needs to
 * be cleared between calls: the selector zeroes what it counts into.
 * ---------------------------------------------------------------------- */
#define TG_SELECT_SCRATCH_BYTES ((size_t)8 << 20)
tg_status tg_select_topk_noalloc(const float* b, const uint8_t* prunable,
                                 const int32_t* cu_seqlens, const int32_t* k, int32_t n_seq,
                                 int64_t t_in, int64_t t_kept_capacity, int32_t* kept_idx,
                                 int32_t* kept_pos, float* kept_b, int32_t* kept_cu_seqlens,
                                 tg_stream stream);

/* ------------------------------------------------------------------------
 * tg_gather -- compaction of the kept rows (§4.1: the residual stream of a
 * pruned token stops at layer L; only kept rows go on to the layers above).
 *
 *   dst row r = src row idx[r],  r in [0, n_rows)   (bytes copied unchanged)
 * src dev, row i at src + i * src_row_stride_bytes; n_src_rows rows.
 * idx dev [n_rows] i32; an index outside [0, n_src_rows) writes a zero row.
 * dst dev, row r at dst + r * dst_row_stride_bytes.
 * row_bytes % 4 == 0 and 4-byte aligned rows are required; 16-byte multiples
 * with 16-byte aligned rows take the vector path.
 * ---------------------------------------------------------------------- */
tg_status tg_gather(const void* src, int64_t src_row_stride_bytes, int64_t n_src_rows,
                    int64_t row_bytes, const int32_t* idx, int64_t n_rows, void* dst,
                    int64_t dst_row_stride_bytes, tg_stream stream);

/* ------------------------------------------------------------------------
 * tg_gated_attn -- token-gated causal attention over the kept tokens,
 * §4.2 Eq. 8 with the head-wise gain of Eq. 6 and the temperature of Eq. 7:
 *
 *   alpha_ij^h = softmax_{j in S, j <= i}( tau_i^h * (s * q_i^h . k_j + gain_h * b_j) )
 *   tau_i^h    = temp_h * log(m_i) / log(max(2, p_i))
 *   O_i^h      = sum_j alpha_ij^h v_j
 *
 * m_i = kept keys visible to query i (itself included) = its index within the
 * sequence's kept tokens + 1; p_i = kept_pos[i] + 1, its original position.
 * Causality is by original position, i.e. by kept order.  Query head h reads
 * KV head h / (hq / hkv).  The gate g_j = softmax_S(gain_h * b_j) of Eq. 5-6
 * is never formed: its normaliser is constant in j and cancels.
 *
 * q   dev [t_kept, hq, dh] of `dt`.     k, v dev [t_kept, hkv, dh] of `dt`.
 * out dev [t_kept, hq, dh] of `dt` (accumulation in f32).
 * kept_b dev [t_kept] f32 scores of the kept tokens (0 on prompt tokens).
 * kept_pos dev [t_kept] i32 original index in the sequence, or NULL: then the
 *   length factor is 1 (tau = temp).
 * kept_cu_seqlens dev [n_seq + 1] i32; max_kept_seqlen = longest sequence
 *   (host value, used only to size the launch; a larger one is harmless).
 * gain, temp dev [hq] f32: positive post-softplus values of Eq. 6 and Eq. 7.
 * sm_scale: s; <= 0 selects 1/sqrt(dh).
 * lse2 dev [hq, t_kept] f32 out (head-major), or NULL (TG_BF16 only): each row's
 *   log2 sum_{j <= i} exp(l_ij), with l_ij the logit above, i.e. the softmax
 *   normaliser in base 2.  tg_gated_attn_bwd can take it with `out` instead
 *   of recomputing it.
 * Supported: dh in {64, 128}; hq % hkv == 0 with hq/hkv in {1, 2, 4} or a
 * multiple of 4; dt = TG_BF16 (matrix cores) or TG_F32 (vector ALU).
 * ---------------------------------------------------------------------- */
tg_status tg_gated_attn(const void* q, const void* k, const void* v, tg_dtype dt, void* out,
                        int64_t t_kept, const float* kept_b, const int32_t* kept_pos,
                        const int32_t* kept_cu_seqlens, int32_t n_seq,
                        int32_t max_kept_seqlen, int32_t hq, int32_t hkv, int32_t dh,
                        const float* gain, const float* temp, float sm_scale, float* lse2,
                        tg_stream stream);

/* ------------------------------------------------------------------------
 * tg_gated_attn_split -- the same attention (§4.2 Eq. 8, as tg_gated_attn,
 * same arguments and outputs, bf16 only), balanced for inputs whose query
 * blocks are few or uneven (short sequences, small budgets, ragged
 * batches).  A one-workgroup launch first plans the work on the GPU: query
 * blocks with more key tiles than a workgroup's share of the causal work
 * are split over the keys into chunks, and all items are sorted by size,
 * largest first, for the workgroups.  Each chunk leaves its unnormalised
 * output, running maximum and sum in the workspace, and a last launch merges
 * them (flash-decoding's split over the keys, applied to the prefill).
 * ws  dev workspace of >= tg_gated_attn_split_workspace_size(t_kept, n_seq,
 *     max_kept_seqlen, hq, hkv, dh) bytes (the same max_kept_seqlen as the
 *     call), 256-byte aligned: the plan (a few bytes per query block) and,
 *     when blocks are split, the partial results.  Calls that share a
 *     workspace must not overlap.
 * max_kept_seqlen steers the split (how long a chunk is, how many a block
 *     may have); with a wrong one the results are still the attention (a
 *     block longer than planned has its last chunk run to its end), only
 *     the balance suffers.
 * How blocks are split depends on the sizes alone (it is planned for a
 * 256-CU gfx950), so results are bitwise reproducible; rows of split blocks
 * differ from tg_gated_attn's in the last bits (the merge's order of
 * additions), the other rows are identical.
 * ---------------------------------------------------------------------- */
size_t tg_gated_attn_split_workspace_size(int64_t t_kept, int32_t n_seq, int32_t max_kept_seqlen,
                                          int32_t hq, int32_t hkv, int32_t dh);
tg_status tg_gated_attn_split(const void* q, const void* k, const void* v, tg_dtype dt, void* out,
                              int64_t t_kept, const float* kept_b, const int32_t* kept_pos,
                              const int32_t* kept_cu_seqlens, int32_t n_seq,
                              int32_t max_kept_seqlen, int32_t hq, int32_t hkv, int32_t dh,
                              const float* gain, const float* temp, float sm_scale, float* lse2,
                              void* ws, size_t ws_bytes, tg_stream stream);

/* ------------------------------------------------------------------------
 * tg_gated_attn_bwd -- gradients of tg_gated_attn: the path by which the
 * loss reaches the gate's scores (§4.3: token-gated attention gives top-K a
 * gradient), and the gradients of gain (Eq. 6) and temperature (Eq. 7).
 * With z_ij = s q_i.k_j + gain_h b_j, l_ij = tau_i z_ij (j <= i), P the
 * row softmax of l, dP_ij = dout_i . v_j, D_i = sum_j P_ij dP_ij and
 * dl_ij = P_ij (dP_ij - D_i):
 *
 *   dv_j = sum_i P_ij dout_i              dq_i = s tau_i sum_j dl_ij k_j
 *   dk_j = s sum_i tau_i dl_ij q_i        db_j = sum_{h,i} tau_i gain_h dl_ij
 *   dgain_h = sum_ij tau_i b_j dl_ij      dtemp_h = sum_ij lambda_i z_ij dl_ij
 *
 * (tau_i = temp_h lambda_i; KV gradients sum over the query heads sharing a
 * KV head.)  Arguments as for tg_gated_attn, plus:
 * dout dev [t_kept, hq, dh] of `dt`: the gradient of the loss w.r.t. out.
 * dq   dev [t_kept, hq, dh] f32 out;  dk, dv dev [t_kept, hkv, dh] f32 out.
 * db   dev [t_kept] f32 out (rows past kept_cu_seqlens[n_seq] get 0).
 * dgain, dtemp dev [hq] f32 out.
 * fwd_out, fwd_lse2: the forward's `out` and `lse2` for the same inputs, or
 *      both NULL.  Given (TG_BF16 only; 16- and 4-byte aligned), D_i is taken
 *      as dout_i . out_i (equal to sum_j P_ij dP_ij, since out_i =
 *      sum_j P_ij v_j) and fwd_lse2 as the softmax normaliser, so the pass
 *      that recomputes both from q, k, v and dout is skipped.  D then
 *      carries out's bf16 rounding.  NULL: the statistics are recomputed.
 * ws   dev workspace of >= tg_gated_attn_bwd_workspace_size(t_kept, n_seq,
 *      hq, hkv) bytes, 4-byte aligned.
 * TG_F32: fp32 arithmetic on the vector ALU.  TG_BF16: matrix cores
 * with fp32 accumulation; P and dS enter the dv, dk and dq products rounded
 * to bf16, while db, dgain and dtemp are formed from the fp32 values.
 * Results are bitwise reproducible.  Supported: dh in {64, 128},
 * hq % hkv == 0, 16-byte aligned tensors.
 * ---------------------------------------------------------------------- */
size_t tg_gated_attn_bwd_workspace_size(int64_t t_kept, int32_t n_seq, int32_t hq, int32_t hkv);
tg_status tg_gated_attn_bwd(const void* q, const void* k, const void* v, const void* dout,
                            tg_dtype dt, int64_t t_kept, const float* kept_b,
                            const int32_t* kept_pos, const int32_t* kept_cu_seqlens,
                            int32_t n_seq, int32_t hq, int32_t hkv, int32_t dh,
                            const float* gain, const float* temp, float sm_scale, float* dq,
                            float* dk, float* dv, float* db, float* dgain, float* dtemp,
                            const void* fwd_out, const float* fwd_lse2, void* ws,
                            size_t ws_bytes, tg_stream stream);

/* ------------------------------------------------------------------------
 * tg_score_bwd -- gradients of the gate's scorer (§4.1 Eq. 3) from the
 * gradient that reaches the kept scores through the attention (§4.3), for
 * L = sum_r db_kept[r] * b[kept_idx[r]] with the kept set held fixed (the
 * selection passes no gradient).  Per sequence, with P its prunable tokens,
 * r = sqrt(mean_P b~^2 + eps) and C = sum over kept prunable j of db_j b~_j:
 *
 *   db~_k = [k kept] db_k / r - b~_k C / (|P| r^3)  (k in P; 0 on prompt tokens)
 *   dz_k  = db~_k w2 * SiLU'(W1 x_k + b1)
 *   dW1 = sum_k dz_k x_k^T   db1 = sum_k dz_k   dw2 = sum_k db~_k SiLU(z_k)
 *   db2 = sum_k db~_k        dx_k = W1^T dz_k
 *
 * x, dt, x_row_stride, t_in, d, h, w1, b1, w2, prunable, cu_seqlens, n_seq,
 *   eps, norm_eps: as for tg_score, the same values as the forward call.
 * norm_eps >= 0 (the LN2-fused form, §3 Eq. 1 in front of Eq. 3): x rows
 *          are the residual a and w1 is W1' = W1 diag(g) with the norm's
 *          weight folded in.  With inv_k = 1 / sqrt(mean_c a_kc^2 + norm_eps)
 *          and z_k = inv_k W1' a_k + b1, the outputs are the gradients at a
 *          and at W1':
 *            dW1' = sum_k (inv_k dz_k) a_k^T
 *            dx_k = W1'^T (inv_k dz_k) - c_k a_k,  c_k = inv_k^3 / d * dz_k . (W1' a_k)
 *          (db1, dw2, db2 unchanged).  The caller unfolds the weight:
 *          dW1 = dW1' diag(g) and dg_c = sum_j W1[j][c] dW1'[j][c].
 * b_raw    dev [t_in] f32: b~ of the forward (tg_score's b_raw output).
 * kept_idx, kept_cu_seqlens dev: tg_select_topk's outputs; t_kept rows.
 * db_kept  dev [t_kept] f32: gradient w.r.t. the kept scores (the db of
 *          tg_gated_attn_bwd, or any other).
 * dx       dev [t_in, d] f32 out, or NULL to skip it.
 * dw1 dev [h, d] f32 out; db1, dw2 dev [h] f32 out; db2 dev [1] f32 out.
 * ws       dev workspace of >= tg_score_bwd_workspace_size(t_in, n_seq, d, h)
 *          bytes, 256-byte aligned (it holds dz and, on the matrix-core
 *          path, a transposed copy of w1).
 * f32 rows, and bf16 rows with h != 256 or d % 256 != 0: fp32 arithmetic on
 * the vector ALU.  bf16 rows with h == 256 and d % 256 == 0: dz is recomputed
 * on the matrix cores with the forward's tiling and rounded to bf16 for the
 * dW1 and dx products (fp32 accumulation); db1, dw2, db2 and the LN2 term
 * c_k a_k stay fp32.  Fixed reduction orders on both paths (bitwise
 * reproducible).  Supported: d % 64 == 0, h % 64 == 0, x_row_stride and
 * d < 2^22, x and w1 rows 16-byte aligned.
 * ---------------------------------------------------------------------- */
size_t tg_score_bwd_workspace_size(int64_t t_in, int32_t n_seq, int32_t d, int32_t h);
tg_status tg_score_bwd(const void* x, tg_dtype dt, int64_t x_row_stride, int64_t t_in, int32_t d,
                       int32_t h, const void* w1, const float* b1, const float* w2,
                       const uint8_t* prunable, const int32_t* cu_seqlens, int32_t n_seq,
                       float eps, float norm_eps, const float* b_raw, const int32_t* kept_idx,
                       const int32_t* kept_cu_seqlens, int64_t t_kept, const float* db_kept,
                       float* dx, float* dw1, float* db1, float* dw2, float* db2, void* ws,
                       size_t ws_bytes, tg_stream stream);

/* ------------------------------------------------------------------------
 * tg_qkv_proj -- query, key and value projections of the kept rows: the
 * step between tg_gather and tg_gated_attn (§4.1: the kept tokens continue
 * through the layers above the gate; §4.2 Eq. 8 reads q, k, v of the kept
 * tokens only).  One GEMM over the concatenated weight:
 *
 *   q[r, h, e] = sum_c x[r, c] * w[h * dh + e, c]                 (h < hq)
 *   k[r, h, e] = sum_c x[r, c] * w[(hq + h) * dh + e, c]          (h < hkv)
 *   v[r, h, e] = sum_c x[r, c] * w[(hq + hkv + h) * dh + e, c]    (h < hkv)
 *
 * with fp32 accumulation and the result rounded to bf16 (nearest even).
 * x  dev [t, d] bf16 (normally tg_gather's output), row r at
 *    x + r * x_row_stride elements.
 * w  dev [(hq + 2 hkv) * dh, d] bf16: the rows of Wq, then Wk, then Wv, one
 *    row per output feature (the nn.Linear weight layout).
 * q  dev [t, hq, dh] bf16 out;  k, v dev [t, hkv, dh] bf16 out.
 * Supported: dt = TG_BF16, d % 64 == 0, dh % 32 == 0,
 * (hq + 2 hkv) * dh % 256 == 0, x_row_stride % 8 == 0 and < 2^22,
 * 16-byte aligned x and w.  No rotary embedding or q/k norm is applied.
 * ---------------------------------------------------------------------- */
tg_status tg_qkv_proj(const void* x, tg_dtype dt, int64_t x_row_stride, int64_t t, int32_t d,
                      const void* w, int32_t hq, int32_t hkv, int32_t dh, void* q, void* k,
                      void* v, tg_stream stream);

/* ------------------------------------------------------------------------
 * tg_qkv_proj_rope -- tg_qkv_proj followed, in the same kernel, by the
 * per-head treatment of q and k in the Qwen3 family: an RMSNorm over each
 * head's dh values, then the rotary embedding at each kept token's original
 * position (the pages give neither; kept_pos from tg_select_topk holds the
 * positions, §4.1: pruned tokens leave gaps, kept ones keep their place):
 *
 *   q[r, h, :] <- q[r, h, :] / sqrt(mean_e q[r, h, e]^2 + norm_eps) * q_norm
 *   (k likewise with k_norm; skipped for a NULL weight), then for each pair
 *   e < dh/2 with a = pos[r] * rope_theta^(-2e/dh):
 *   (x[e], x[e + dh/2]) <- (x[e] cos a - x[e + dh/2] sin a,
 *                           x[e + dh/2] cos a + x[e] sin a)   for x in q, k.
 *
 * The norm and the rotation run in fp32 on the accumulators; the angle is
 * reduced to one turn in fp64.  v is as in tg_qkv_proj.
 * pos     dev [t] i32 positions (required when rope_theta > 0).
 * q_norm, k_norm dev [dh] f32 or NULL.  norm_eps >= 0.
 * rope_theta > 1 turns the rotation on, <= 0 off (values in (0, 1] are
 * rejected).
 * Supported: as tg_qkv_proj, with dh in {64, 128} and hq * dh, hkv * dh
 * multiples of 128.
 * ---------------------------------------------------------------------- */
tg_status tg_qkv_proj_rope(const void* x, tg_dtype dt, int64_t x_row_stride, int64_t t,
                           int32_t d, const void* w, int32_t hq, int32_t hkv, int32_t dh,
                           const int32_t* pos, const float* q_norm, const float* k_norm,
                           float norm_eps, float rope_theta, void* q, void* k, void* v,
                           tg_stream stream);

/* ------------------------------------------------------------------------
 * tg_gated_decode -- one decode step of token-gated attention over pruned KV
 * caches: a decode step attends to the cache and appends to it (§3, "Prefill,
 * decode, and the KV cache"); above the gate the cache holds only the kept
 * tokens (§4.1), and generated tokens are never pruned.  One new query token
 * per sequence, its own key and value already appended as the sequence's
 * last cache row:
 *
 *   logit_j^h = tau^h * (s * q^h . k_j + gain_h * b_j),   j over the cache
 *   tau^h     = temp_h * log(m) / log(max(2, p))           (Eq. 7)
 *   out^h     = sum_j softmax_j(logit^h) v_j               (Eq. 8)
 *
 * m = the sequence's cache length, p = q_pos + 1: the result equals the last
 * query row of tg_gated_attn over the same rows.  Pruning the cache of a
 * layer to the kept tokens is tg_gather over its [rows, hkv * dh] K and V.
 *
 * q        dev [n_seq, hq, dh] bf16, the new token of each sequence.
 * k_cache, v_cache dev [t_cache, hkv, dh] bf16, sequences back to back.
 * out      dev [n_seq, hq, dh] bf16 (accumulation in f32).
 * cache_b  dev [t_cache] f32 scores of the cached tokens (0 on prompt and
 *          generated tokens), or NULL for all zero.
 * q_pos    dev [n_seq] i32 original 0-based position of the new token in its
 *          sequence, or NULL: then the length factor is 1 (tau = temp).
 * cache_cu_seqlens dev [n_seq + 1] i32, non-decreasing, last <= t_cache.  An
 *          empty sequence gives zeros.
 * max_cache_len: host value that sizes the key split (and the workspace);
 *          any value is correct, the longest sequence's length is fastest.
 * gain, temp dev [hq] f32, as for tg_gated_attn.  sm_scale: s; <= 0 selects
 *          1/sqrt(dh).
 * ws       dev workspace of >= tg_gated_decode_workspace_size(n_seq, hq, hkv,
 *          dh, max_cache_len) bytes, 4-byte aligned.
 * Supported: dt = TG_BF16, dh in {64, 128}, hq/hkv in {1, 2, 4, 8},
 * t_cache < 2^31, n_seq <= 65535, 16-byte aligned q and caches.
 * ---------------------------------------------------------------------- */
size_t tg_gated_decode_workspace_size(int32_t n_seq, int32_t hq, int32_t hkv, int32_t dh,
                                      int64_t max_cache_len);
tg_status tg_gated_decode(const void* q, const void* k_cache, const void* v_cache, tg_dtype dt,
                          void* out, int64_t t_cache, const float* cache_b,
                          const int32_t* q_pos, const int32_t* cache_cu_seqlens, int32_t n_seq,
                          int64_t max_cache_len, int32_t hq, int32_t hkv, int32_t dh,
                          const float* gain, const float* temp, float sm_scale, void* ws,
                          size_t ws_bytes, tg_stream stream);

/* ------------------------------------------------------------------------
 * Device-side contract checks (debugging aid, off by default).
 *
 * Some preconditions depend on device data the host never reads.  When they
 * are broken the kernels still stay inside their buffers (offsets are
 * clamped, out-of-range gather indices give zero rows, selected tokens past
 * the capacity are dropped), but the results are meaningless.  With
 * tg_set_contract_checks(1), every later call on this process also enqueues
 * small check kernels on its stream that OR one bit per broken rule into a
 * per-GPU flag word:
 *   TG_CONTRACT_OFFSETS          cu_seqlens of tg_score, tg_select_topk(_noalloc),
 *                                tg_score_bwd: cu[0] < 0, decreasing, or past t_in
 *   TG_CONTRACT_NEGATIVE_BUDGET  a budget k[s] < 0 (tg_select_topk reads it as 0;
 *                                §4.1 Eq. 4 defines K >= 0)
 *   TG_CONTRACT_CAPACITY         t_kept_capacity below the kept count (tokens dropped)
 *   TG_CONTRACT_INDEX            tg_gather (or tg_score_bwd's kept_idx) index
 *                                outside [0, n_src)
 *   TG_CONTRACT_KEPT_OFFSETS     kept_cu_seqlens / cache_cu_seqlens of tg_gated_attn,
 *                                tg_gated_attn_bwd, tg_gated_decode, tg_score_bwd:
 *                                negative, decreasing, or past the row count
 *   TG_CONTRACT_POSITIONS        kept_pos negative or not strictly increasing within
 *                                a sequence (§4.2 Eq. 8: causality by original
 *                                position is then not the order of the rows)
 * The checks cost a few microseconds per call and are meant for debugging.
 * tg_contract_status waits for the work queued on `stream`, returns the
 * word in *flags (host) and clears it; unlike every other call it
 * synchronises the stream.  Checks of calls on other streams are ordered
 * only by the caller's own synchronisation.
 * ---------------------------------------------------------------------- */
#define TG_CONTRACT_OFFSETS 0x1u
#define TG_CONTRACT_NEGATIVE_BUDGET 0x2u
#define TG_CONTRACT_CAPACITY 0x4u
#define TG_CONTRACT_INDEX 0x8u
#define TG_CONTRACT_KEPT_OFFSETS 0x10u
#define TG_CONTRACT_POSITIONS 0x20u
tg_status tg_set_contract_checks(int32_t on);
tg_status tg_contract_status(uint32_t* flags, tg_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* TOKENGATE_H */
