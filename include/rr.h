/*
 * rr.h -- C ABI of librr, jagged candidate-isolated attention for MI355X (gfx950).
 *
 * The problem (Candidate isolation attention mask page, sections "为什么需要它",
 * "段 ID：掩码的表达方式" and "只更新候选的末尾层"; HSTU scaling notes, section
 * "手算 padding 的浪费与 offset"):
 *
 *   A batch holds B users.  Their rows are concatenated (jagged values) and user b
 *   owns rows [offsets[b], offsets[b+1]); offsets[0] = 0 and offsets[B] = T.  A
 *   user's rows are laid out [prefix | history | candidates]; cand_start[b] is
 *   the absolute row of its first candidate.  Each row gets a segment ID:
 *   1 = valid prefix/history, -1 = valid candidate, 0 = padding.  A query may
 *   read a key of its own user when the key is segment 1 and the query is not
 *   padding, or when both are candidates at the same row.  No row ever reads
 *   another user's rows.  Output rows of segment 0 are 0.
 *
 *   Candidate-only layers: candidate queries read a frozen history K/V (the
 *   user's prefix and history states) plus their own K/V.
 *
 * Attention is softmax(scale * q k^T) v per head over the admitted keys.
 *
 * Conventions shared by every entry point:
 *   - Tensors are token-major [rows][H][d], contiguous, in device memory.  Row r,
 *     head h, element e sits at index (r * H + h) * d + e.
 *   - Every pointer argument is DEVICE memory owned by the caller; the library
 *     keeps no pointer after the call returns and allocates nothing.  Scratch
 *     comes from the caller's `workspace` (size from the *_workspace_bytes query).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and the
 *     call returns without waiting for it.  Results are valid once the stream has
 *     reached that point.  No call synchronises the host with the device.
 *   - Argument errors are found on the host before anything is enqueued; the call
 *     then returns a negative rr_status and has no effect.  A failed kernel launch
 *     returns RR_EHIP.  B = 0 or T = 0 is a valid empty call that returns RR_OK.
 *   - Data contract, not checked on the hot path (rr_validate_jagged checks it):
 *     offsets non-decreasing with offsets[0] = 0 and offsets[B] = T, and
 *     offsets[b] <= cand_start[b] <= offsets[b+1].  Kernels clamp every row index
 *     into the user's own rows, so data that breaks the contract can give wrong
 *     numbers but never reads another user's rows or outside [0, T).
 *   - Supported: d in {16, 32, 64, 128}; H <= 1023; dtype RR_F32 or RR_BF16 (q, k, v
 *     and the output share it; accumulation is fp32).  scale <= 0 selects 1/sqrt(d).
 *   - Calls on the same stream are ordered; calls on different streams that share
 *     a workspace race.
 */
#ifndef RR_H_
#define RR_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RR_OK = 0,
  RR_EINVAL = -1,        /* NULL where not allowed, negative size, inconsistent sizes */
  RR_EDTYPE = -2,        /* dtype not RR_F32 / RR_BF16 */
  RR_EUNSUPPORTED = -3,  /* d not in {16, 32, 64, 128}, or sizes past the documented limits
                            (attention: H <= 1023 and fewer than 2^21 tiles of 64 query rows,
                            i.e. at most 2^27 - 64 query rows per call) */
  RR_EWORKSPACE = -4,    /* workspace NULL or smaller than the *_workspace_bytes query */
  RR_EHIP = -5           /* a kernel launch failed */
} rr_status;

typedef enum { RR_F32 = 0, RR_BF16 = 1 } rr_dtype;

/* Text for a status code (static storage). */
const char* rr_status_string(int status);

/* Library ABI version (increments when a signature changes). */
int rr_abi_version(void);

/* Digest of the forward attention kernels' gfx950 machine code in the loaded library: equal
 * digests mean equal forward kernels, so a profile taken with one library applies to another. */
const char* rr_forward_fingerprint(void);

/*
 * rr_segment_ids -- per-row segment IDs.
 * Candidate isolation attention mask page, section "段 ID：掩码的表达方式":
 *   is_candidate = row >= cand_start[b];  valid = valid_mask[row] (1 when valid == NULL);
 *   if attend_padded_history: valid = valid || !is_candidate;
 *   seg = valid ? (is_candidate ? -1 : 1) : 0.
 *
 * offsets    int32 [B+1]  device
 * cand_start int32 [B]    device, absolute rows
 * valid      uint8 [T]    device, nonzero = valid; NULL = every row valid
 * seg_out    int8  [T]    device, written
 */
int rr_segment_ids(const int32_t* offsets, const int32_t* cand_start, const uint8_t* valid,
                   int attend_padded_history, int32_t B, int32_t T, int8_t* seg_out,
                   hipStream_t stream);

/*
 * rr_bounds -- per-user history and candidate intervals from segment IDs.
 * Candidate isolation attention mask page, section "段 ID：掩码的表达方式" (the operator
 * derives [history_lower, history_upper) and [candidate_lower, candidate_upper)).
 * Reading: the tight hull of the user's segment-1 rows and of its segment -1 rows,
 * as absolute rows; an empty history hull is [offsets[b], offsets[b]) and an empty
 * candidate hull [offsets[b+1], offsets[b+1]).  Segment-0 rows inside a hull
 * (holes) stay excluded from attention by their segment ID.
 *
 * seg        int8  [T]    device (from rr_segment_ids)
 * bounds_out int32 [4][B] device, written: rows hist_lo, hist_hi, cand_lo, cand_hi
 */
int rr_bounds(const int32_t* offsets, const int8_t* seg, int32_t B, int32_t T, int32_t* bounds_out,
              hipStream_t stream);

/* Bytes of workspace rr_attn_fwd needs for these sizes (0 on invalid sizes). */
size_t rr_attn_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t d);

/*
 * rr_attn_fwd -- full-sequence candidate-isolated attention over a jagged batch.
 * Candidate isolation attention mask page, sections "段 ID：掩码的表达方式" (mask rule:
 * history_mask | candidate_self_mask) and "掩码长什么样" (the P/H/C table).
 *
 * q, k, v, o  [T][H][d] of `dtype`, device; o is written (segment-0 rows get 0)
 * offsets     int32 [B+1], cand_start int32 [B] (absolute rows), device
 * valid       uint8 [T] device or NULL; attend_padded_history as in rr_segment_ids
 * scale       softmax scale; <= 0 selects 1/sqrt(d)
 * workspace   device scratch of at least rr_attn_workspace_bytes(B, T, H, d) bytes
 *
 * A small unpadded bf16 batch (valid == NULL, at most 256 users, a grid of at most 1024
 * workgroups) is planned inside the attention kernel: one launch, and no plan is left in
 * the workspace.  Larger or padded batches run rr_attn_plan + rr_attn_run.  Both give the
 * same bits.
 */
int rr_attn_fwd(const void* q, const void* k, const void* v, void* o, const int32_t* offsets,
                const int32_t* cand_start, const uint8_t* valid, int attend_padded_history,
                int32_t B, int32_t T, int32_t H, int32_t d, int dtype, float scale,
                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * rr_attn_fwd_rope -- rr_attn_fwd with the queries' rotary encoding done inside the
 * attention kernel (candidate isolation attention mask page, section
 * "位置编码：候选共用一个位置": a history row sits at its place in the user's row, the
 * newest at history_end - 1, and every candidate at history_end).  q is NOT rotated: the
 * kernel rotates each query row in registers right after loading it, with the same angle
 * and rotation arithmetic as rr_rope_qk, so the result equals, bit for bit, rr_attn_fwd
 * on rr_rope_qk's rotated q.  k must already be rotated (rr_rope_qk with q = NULL), since
 * every query tile of a user reads it; v is never rotated.
 *   theta_base  rotary base (<= 0: 10000)
 *   no padding mask (every row valid); bf16 with d in {32, 64, 128} only (else
 *   RR_EUNSUPPORTED).  Other arguments, layouts, ownership, errors: as rr_attn_fwd.
 */
int rr_attn_fwd_rope(const void* q, const void* k, const void* v, void* o, const int32_t* offsets,
                     const int32_t* cand_start, int32_t B, int32_t T, int32_t H, int32_t d, int dtype,
                     float scale, float theta_base, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/*
 * rr_attn_fwd_noalloc -- rr_attn_fwd for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  It
 * takes no workspace and allocates nothing (no hipMalloc, hipFree or allocating library
 * call): what rr_attn_fwd keeps in its workspace (the plan, and the key-norm bounds of
 * wide-tile batches) lives in a static device array of rr_attn_fwd_noalloc_max_bytes()
 * bytes (16 MiB), one copy per GPU, held until the process ends.
 *   arguments, layouts, ownership, stream semantics: as rr_attn_fwd (the caller passes
 *     inputs and outputs; the current device must be the stream's device)
 *   errors: as rr_attn_fwd; RR_EUNSUPPORTED when rr_attn_workspace_bytes(B, T, H, d)
 *     exceeds rr_attn_fwd_noalloc_max_bytes(); RR_EHIP if the array's device address
 *     cannot be looked up
 *   concurrency: every call on a GPU shares that GPU's array; calls in stream order are
 *     independent (each rewrites the whole plan and the bounds it reads), calls that overlap
 *     on one GPU race.
 */
size_t rr_attn_fwd_noalloc_max_bytes(void);
int rr_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, const int32_t* offsets,
                        const int32_t* cand_start, const uint8_t* valid, int attend_padded_history,
                        int32_t B, int32_t T, int32_t H, int32_t d, int dtype, float scale,
                        hipStream_t stream);

/*
 * rr_attn_plan + rr_attn_run -- rr_attn_fwd in two steps.
 * The plan depends only on the batch's lengths (offsets, cand_start, valid, flag):
 * segment IDs and bounds per user, the compacted row lists when `valid` is given,
 * and the length-sorted list of work items.  It is written into `workspace`.
 * rr_attn_run then computes attention from q, k, v with the plan found in the
 * workspace, so a stack of layers over one batch can plan once and run per layer.
 * rr_attn_run must get the same B, T, H, d and dtype as the plan it uses; the
 * kernels check this against the plan and leave `o` unwritten if they differ.
 * A plan stays valid until the workspace is overwritten.  rr_attn_run leaves the plan
 * as it is but writes another area of the workspace: for batches of long users (the
 * 256-row query tile) a pass over k first stores, per 64 key rows and head, the largest
 * squared key norm, from which the attention kernel bounds every row's scores
 * (Cauchy-Schwarz) and skips forming tile maxima that cannot change its softmax
 * reference; the output bits are the same either way.  Runs over one workspace must
 * therefore be ordered on one stream: concurrent runs over a shared workspace race.
 */
int rr_attn_plan(const int32_t* offsets, const int32_t* cand_start, const uint8_t* valid,
                 int attend_padded_history, int32_t B, int32_t T, int32_t H, int32_t d, int dtype,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);
int rr_attn_run(const void* q, const void* k, const void* v, void* o, int32_t B, int32_t T, int32_t H,
                int32_t d, int dtype, float scale, void* workspace, size_t workspace_bytes,
                hipStream_t stream);

/*
 * rr_attn_run_lse -- rr_attn_run that also writes each row's log-sum-exp.
 * lse  float [T][H] device, written: the natural log of the sum of exp(scale * q.k)
 *      over the keys row r reads in head h (-inf for segment-0 rows).  The backward
 *      pass recomputes the softmax from it.  NULL = not written (then as rr_attn_run).
 */
int rr_attn_run_lse(const void* q, const void* k, const void* v, void* o, float* lse, int32_t B,
                    int32_t T, int32_t H, int32_t d, int dtype, float scale, void* workspace,
                    size_t workspace_bytes, hipStream_t stream);

/*
 * Backward pass of full-sequence candidate-isolated attention.
 * Candidate isolation attention mask page, section "训练时的序列打包" (training keeps the
 * same attention contract; the page prints no gradient formulas).  The gradients are
 * those of the forward's definition, with the softmax recomputed from the forward's
 * lse:  P = exp(scale q.k - lse),  dv = P^T dO,  dP = dO v^T,
 *       dS = P (dP - rowsum(dO * o)),  dq = scale dS k,  dk = scale dS^T q.
 * A history key's dk, dv sum over every valid query of its user; a candidate's own
 * key and value get gradients from that candidate alone; segment-0 rows get 0.  Every
 * output element is written by one workgroup without atomics: repeated calls give the
 * same bits.  Supported: dtype RR_BF16 and d in {64, 128} (other valid sizes return
 * RR_EUNSUPPORTED); accumulation is fp32.
 *
 * Two steps, as the forward's: rr_attn_plan into a workspace of
 * rr_attn_bwd_workspace_bytes (which also holds rowsum(dO * o) between the two kernels
 * of the backward), rr_attn_run_lse for o and lse, then rr_attn_bwd_run over the same
 * plan.  rr_attn_bwd plans and runs the backward in one call.
 *
 * q, k, v     [T][H][d] bf16 device, the forward's inputs
 * o           [T][H][d] bf16 device, the forward's output for these inputs and scale
 * dout        [T][H][d] bf16 device, gradient of the loss w.r.t. o
 * lse         float [T][H] device, from rr_attn_run_lse on these inputs and scale
 * dq, dk, dv  [T][H][d] bf16 device, written (every row, 0 for segment-0 rows); they
 *             must not alias any input
 * offsets, cand_start, valid, attend_padded_history, scale: as rr_attn_fwd
 */
size_t rr_attn_bwd_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t d);
int rr_attn_bwd_run(const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, void* dq, void* dk, void* dv, int32_t B, int32_t T, int32_t H,
                    int32_t d, int dtype, float scale, void* workspace, size_t workspace_bytes,
                    hipStream_t stream);
int rr_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                const float* lse, void* dq, void* dk, void* dv, const int32_t* offsets,
                const int32_t* cand_start, const uint8_t* valid, int attend_padded_history, int32_t B,
                int32_t T, int32_t H, int32_t d, int dtype, float scale, void* workspace,
                size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace rr_cand_only_attn_fwd needs for these sizes (0 on invalid sizes). */
size_t rr_cand_only_workspace_bytes(int32_t B, int32_t Th, int32_t Tc, int32_t H, int32_t d);

/*
 * rr_cand_only_attn_fwd -- attention of a candidate-only layer.
 * Candidate isolation attention mask page, section "只更新候选的末尾层": the candidate
 * query attends the frozen history K/V (prefix and history states) and its own K/V;
 * the result equals the candidate rows of the full layer over [history | candidates].
 *
 * q_cand, k_cand, v_cand, o_cand  [Tc][H][d] device; o_cand is written
 * k_hist, v_hist                  [Th][H][d] device (frozen)
 * hist_offsets int32 [B+1] into k_hist/v_hist; cand_offsets int32 [B+1] into the
 *   candidate tensors (hist_offsets[B] = Th, cand_offsets[B] = Tc), device
 * workspace    device scratch of at least rr_cand_only_workspace_bytes(...) bytes
 */
int rr_cand_only_attn_fwd(const void* q_cand, const void* k_hist, const void* v_hist,
                          const void* k_cand, const void* v_cand, void* o_cand,
                          const int32_t* hist_offsets, const int32_t* cand_offsets, int32_t B,
                          int32_t Th, int32_t Tc, int32_t H, int32_t d, int dtype, float scale,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * rr_cand_only_attn_fwd_rope -- rr_cand_only_attn_fwd with the candidates' rotary
 * encoding done inside the attention kernel: every candidate of user b sits at position
 * h_b = hist_offsets[b+1] - hist_offsets[b] (its frozen history's length, the history
 * end).  q_cand is NOT rotated; k_hist (at positions 0 .. h_b - 1) and k_cand (at h_b)
 * must already be rotated (rr_rope_qk).  Bit for bit equal to rr_cand_only_attn_fwd on
 * rr_rope_qk's rotated q_cand.  bf16 with d in {32, 64, 128} only.  theta_base as
 * rr_attn_fwd_rope; everything else as rr_cand_only_attn_fwd.
 */
int rr_cand_only_attn_fwd_rope(const void* q_cand, const void* k_hist, const void* v_hist,
                               const void* k_cand, const void* v_cand, void* o_cand,
                               const int32_t* hist_offsets, const int32_t* cand_offsets, int32_t B,
                               int32_t Th, int32_t Tc, int32_t H, int32_t d, int dtype, float scale,
                               float theta_base, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* rr_cand_only_attn_fwd in two steps, as rr_attn_plan / rr_attn_run (the frozen
 * history K/V of a user can be planned once and reused across candidate batches of
 * the same lengths). */
int rr_cand_only_plan(const int32_t* hist_offsets, const int32_t* cand_offsets, int32_t B, int32_t Th,
                      int32_t Tc, int32_t H, int32_t d, int dtype, void* workspace,
                      size_t workspace_bytes, hipStream_t stream);
int rr_cand_only_run(const void* q_cand, const void* k_hist, const void* v_hist, const void* k_cand,
                     const void* v_cand, void* o_cand, int32_t B, int32_t Th, int32_t Tc, int32_t H,
                     int32_t d, int dtype, float scale, const void* workspace,
                     size_t workspace_bytes, hipStream_t stream);

/*
 * Candidate-only layers: forward with log-sum-exp and backward (Candidate isolation
 * attention mask page, section "只更新候选的末尾层"; gradients as for rr_attn_bwd, of the
 * layer's fallback: the full layer over [frozen history | candidates] keeping the
 * candidate rows, i.e. with no output gradient on the history rows).
 *
 * rr_cand_only_run_lse: rr_cand_only_run that also writes lse float [Tc][H], each
 * candidate row's natural-log sum of exp(scale q.k) over the keys it reads.
 *
 * rr_cand_only_bwd_run: with the plan rr_cand_only_plan made in a workspace of
 * rr_cand_only_bwd_workspace_bytes (the same workspace rr_cand_only_run_lse ran with),
 * writes dq_cand [Tc][H][d], dk_hist, dv_hist [Th][H][d] (0 for the keys of users without
 * candidates) and dk_cand, dv_cand [Tc][H][d] (a candidate's own key and value, read by it
 * alone).  It builds a second plan whose items are key tiles of the frozen history.  bf16,
 * d in {64, 128}; no atomics, so repeated calls give the same bits.  Outputs must not alias
 * inputs.
 */
int rr_cand_only_run_lse(const void* q_cand, const void* k_hist, const void* v_hist, const void* k_cand,
                         const void* v_cand, void* o_cand, float* lse, int32_t B, int32_t Th, int32_t Tc, int32_t H,
                         int32_t d, int dtype, float scale, const void* workspace, size_t workspace_bytes,
                         hipStream_t stream);
size_t rr_cand_only_bwd_workspace_bytes(int32_t B, int32_t Th, int32_t Tc, int32_t H, int32_t d);
int rr_cand_only_bwd_run(const void* q_cand, const void* k_hist, const void* v_hist, const void* k_cand,
                         const void* v_cand, const void* o_cand, const void* dout, const float* lse, void* dq_cand,
                         void* dk_hist, void* dv_hist, void* dk_cand, void* dv_cand, const int32_t* hist_offsets,
                         const int32_t* cand_offsets, int32_t B, int32_t Th, int32_t Tc, int32_t H, int32_t d,
                         int dtype, float scale, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * rr_rope_positions -- right-anchored positions of every row.
 * Candidate isolation attention mask page, section "位置编码：候选共用一个位置": the
 * newest history row sits at history_end - 1 whatever the history length, and every
 * candidate takes the one position history_end.  Rows are numbered within the user's
 * row [prefix | (pad) | history | candidates] and history_end is the candidate start:
 *   pos[r] = pos_base[b] + min(r - offsets[b], cand_start[b] - offsets[b])  for r in user b.
 * pos_base (int32 [B], device, or NULL = all 0) shifts a user's positions: for the
 * candidate rows of a candidate-only layer pass offsets = cand_offsets,
 * cand_start = cand_offsets (each user's first candidate row) and pos_base = the frozen
 * history lengths, so every candidate sits at its user's history end; for the frozen
 * rows pass cand_start = hist_offsets + 1 (no candidates), so row i sits at i.
 *
 * offsets int32 [B+1], cand_start int32 [B], pos_out int32 [T]; all device.
 */
int rr_rope_positions(const int32_t* offsets, const int32_t* cand_start, const int32_t* pos_base,
                      int32_t B, int32_t T, int32_t* pos_out, hipStream_t stream);

/*
 * rr_rope_qk -- rotary encoding of q and k at right-anchored positions, one pass.
 * Positions as rr_rope_positions, computed on the fly from offsets / cand_start /
 * pos_base.  The rotation is the standard pairwise one (a reading: the page names the
 * rotary encoding without its formula): features (2i, 2i+1) of every head rotate by
 * pos * theta_base^(-2i/d); the angle is formed and reduced modulo 2 pi in double
 * precision, its sine and cosine taken in float,
 * the rotation in float, bf16 results rounded to nearest even.
 *
 * q, k         [T][H][d] device inputs; either may be NULL (not rotated)
 * q_out, k_out [T][H][d] device outputs (required when the input is given); an output
 *              may be its own input (in place)
 * d            even, 2 <= d <= 256;  dtype RR_F32 or RR_BF16
 * theta_base   <= 0 selects 10000
 */
int rr_rope_qk(const void* q, const void* k, void* q_out, void* k_out, const int32_t* offsets,
               const int32_t* cand_start, const int32_t* pos_base, int32_t B, int32_t T, int32_t H,
               int32_t d, int dtype, float theta_base, hipStream_t stream);

/*
 * The ranker's layer stack (Candidate isolation attention mask page, section
 * "只更新候选的末尾层"): the first n_layers - n_cand_only layers run over the whole
 * sequence under the isolation mask; then the hidden states split into history
 * (frozen from here on) and candidates, and the last n_cand_only layers update only
 * the candidates, whose queries read the frozen history's keys and values and their
 * own.  Rotary positions are right-anchored (section "位置编码：候选共用一个位置").
 *
 * The pages do not print the layer's inside.  Each layer is read as a pre-norm
 * attention block with the caller's weights:
 *   h = x / sqrt(mean(x^2) + 1e-6) * norm_gain;  [q | k | v] = h W_qkv^T (bf16);
 *   q, k rotated (base theta_base, <= 0 selects 10000);  x += attention(q, k, v) W_o^T.
 * A frozen history row gives a candidate-only layer its key and value through that
 * layer's norm and projections.  No feed-forward block or action head.
 *
 * x (the residual stream) is float32 [rows][D], D = H d, head h of a row at columns
 * h d .. h d + d - 1.  Supported: d in {32, 64, 128}, D a multiple of 128 (<= 16384);
 * the attention runs in bf16 with its default scale 1/sqrt(d).  Every kernel computes
 * a row from that row alone in a fixed order, so a candidate's result does not depend
 * on the other rows of the batch.
 */
typedef struct {
  const float* norm_gain;  /* float [D], device */
  const void* w_qkv;       /* bf16 [3D][D] (out x in), device: rows 0..D-1 give q, D..2D-1 k, 2D.. v */
  const void* w_o;         /* bf16 [D][D] (out x in), device */
} rr_layer;

/* out = bf16(x / sqrt(mean(x^2) + eps) * gain) per row; x float [M][D], D % 4 == 0; eps <= 0 -> 1e-6. */
int rr_rms_norm(const float* x, const float* gain, void* out, int32_t M, int32_t D, float eps,
                hipStream_t stream);

/*
 * rr_linear -- C = A W^T on the matrix cores: A bf16 [M][K], W bf16 [N][K]; exactly one of
 * out (bf16 [M][N], written) and residual (float [M][N], residual += C) is given.
 * N % 128 == 0 and K % 64 == 0 (else RR_EUNSUPPORTED); fp32 accumulation in a fixed order.
 */
int rr_linear(const void* a, const void* w, void* out, float* residual, int32_t M, int32_t N, int32_t K,
              hipStream_t stream);

/* Bytes of workspace rr_ranker_fwd needs (0 on unsupported sizes); Tp = 0 without user tokens. */
size_t rr_ranker_workspace_bytes(int32_t B, int32_t T, int32_t Tc, int32_t Tp, int32_t H, int32_t d);

/*
 * rr_ranker_fwd -- one request: the whole stack over a jagged batch (no padding mask).
 *
 * x           float [T][D] device: the input states; the full layers update it in place,
 *             so afterwards it holds the states after the last full layer
 * layers      HOST array of n_layers rr_layer (device pointers inside)
 * n_cand_only the last n_cand_only layers are candidate-only (0 <= n_cand_only <= n_layers)
 * offsets, cand_start  as rr_attn_fwd; Tc = total candidate rows (sum of offsets[b+1] -
 *             cand_start[b]), the caller's count; Th = T - Tc history rows
 * user_tokens int32 [B] device or NULL: candidate_only_layers_update_user_token (section
 *             "只更新候选的末尾层" names it, off by default, without defining it).  Reading:
 *             with it, the first user_tokens[b] rows of user b (its user tokens, clamped to
 *             its rows before cand_start) keep being updated in the candidate-only layers
 *             under their full-layer contract (they read the user's rows before cand_start,
 *             never candidates); only the other rows freeze.  Tp = sum of user_tokens (the
 *             caller's count); ignored when user_tokens is NULL
 * x_cand_out  float [Tc][D] device, written: the candidates' final states, users in order
 * x_hist_out  float [Th][D] device or NULL: the states of the rows before each user's
 *             candidate start, users in order (frozen; with user tokens, theirs updated)
 * kv_cache    bf16 [n_layers][2][Th][H][d] device or NULL: written with every layer's
 *             history keys (rotated) and values, for rr_ranker_cached_fwd
 * workspace   rr_ranker_workspace_bytes(B, T, Tc, Tp, H, d) bytes
 */
int rr_ranker_fwd(float* x, const rr_layer* layers, int32_t n_layers, int32_t n_cand_only,
                  const int32_t* offsets, const int32_t* cand_start, const int32_t* user_tokens, int32_t B,
                  int32_t T, int32_t Tc, int32_t Tp, int32_t H, int32_t d, float theta_base, float* x_cand_out,
                  float* x_hist_out, void* kv_cache, void* workspace, size_t workspace_bytes,
                  hipStream_t stream);

/*
 * rr_user_token_attn_plan / _run -- jagged attention with no self-term: every query row of
 * user b (rows query_offsets[b] .. query_offsets[b+1]) reads exactly the key rows of user b
 * (key_offsets[b] .. key_offsets[b+1]); a query whose user has no keys gets 0.  These are the
 * user tokens of candidate-only layers with candidate_only_layers_update_user_token (they
 * read the user's prefix and frozen history, as in the full layers, and no candidate).
 * q, o [Tq][H][d]; k, v [Tk][H][d]; dtype, scale and workspace as rr_cand_only_plan / _run
 * (workspace: rr_user_token_attn_workspace_bytes).
 */
size_t rr_user_token_attn_workspace_bytes(int32_t B, int32_t Tk, int32_t Tq, int32_t H, int32_t d);
int rr_user_token_attn_plan(const int32_t* key_offsets, const int32_t* query_offsets, int32_t B, int32_t Tk,
                            int32_t Tq, int32_t H, int32_t d, int dtype, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);
int rr_user_token_attn_run(const void* q, const void* k, const void* v, void* o, int32_t B, int32_t Tk,
                           int32_t Tq, int32_t H, int32_t d, int dtype, float scale, const void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace rr_ranker_cached_fwd needs (0 on unsupported sizes). */
size_t rr_ranker_cached_workspace_bytes(int32_t B, int32_t Th, int32_t Tc, int32_t H, int32_t d);

/*
 * rr_ranker_cached_fwd -- a later request for the same users with new candidates.  The
 * history never reads candidates (section "掩码长什么样"), so its keys and values of
 * every layer are those rr_ranker_fwd left in kv_cache, and every layer becomes a
 * candidate-only layer over them.  The candidates' final states equal, bit for bit, those
 * rr_ranker_fwd gives the same candidates with the same users.
 *
 * x_cand       float [Tc][D] device: the candidates' input states, updated in place to
 *              their final states
 * kv_cache     bf16 [n_layers][2][Th][H][d] device, from rr_ranker_fwd
 * hist_offsets int32 [B+1] into the cache's rows; cand_offsets int32 [B+1] into x_cand
 * workspace    rr_ranker_cached_workspace_bytes(B, Th, Tc, H, d) bytes
 */
int rr_ranker_cached_fwd(float* x_cand, const rr_layer* layers, int32_t n_layers, const void* kv_cache,
                         const int32_t* hist_offsets, const int32_t* cand_offsets, int32_t B, int32_t Th,
                         int32_t Tc, int32_t H, int32_t d, float theta_base, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/*
 * rr_validate_jagged -- debug check of the data contract (HSTU scaling notes, section
 * "手算 padding 的浪费与 offset": empty sequences, offset type and user boundaries need
 * checking).  ORs bits into *err_flags (device int32, caller zeroes it first):
 *   1 offsets[0] != 0, 2 offsets decrease somewhere, 4 offsets[B] != T,
 *   8 some cand_start outside [offsets[b], offsets[b+1]].
 */
int rr_validate_jagged(const int32_t* offsets, const int32_t* cand_start, int32_t B, int32_t T,
                       int32_t* err_flags, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RR_H_ */
