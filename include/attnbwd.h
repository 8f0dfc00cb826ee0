/*
 * attnbwd.h -- C ABI of the MI355X (gfx950) attention-backward library.
 *
 * Operation.  Backward pass of causal grouped-query multi-head attention with
 * a per-query document-start mask, as defined on the page
 * "llm.istanbul -- 10_backward_attention.wgsl" (header comment; kernel
 * attention_backward, Pass 0 / Pass A / Pass B / Final):
 *
 *   kv_h(h)  = h / (n_heads / n_kv_heads)            (contiguous head groups)
 *   visible  : key j is visible to query s  iff  seg[s] <= j <= s
 *   P[s,j]   = exp(scale * Q[s,h,:] . K[j,kv_h,:] - LSE[s,h])
 *   dP[s,j]  = dO[s,h,:] . V[j,kv_h,:]
 *   D[s,h]   = sum over visible j of P[s,j] * dP[s,j]
 *   dS[s,j]  = scale * P[s,j] * (dP[s,j] - D[s,h])
 *   dQ[s,h,:]    += sum_j dS[s,j] * K[j,kv_h,:]
 *   dK[j,kv,:]   += sum over s and the heads h of group kv of dS[s,j] * Q[s,h,:]
 *   dV[j,kv,:]   += sum over s and the heads h of group kv of P[s,j] * dO[s,h,:]
 *
 * Invisible (masked) pairs contribute exactly nothing for finite inputs: the
 * probability and score-gradient of an invisible pair are selected to zero
 * (never computed as a product with zero), so an overflowing exponential or a
 * -inf LSE there cannot reach a visible row.  Non-finite input values (Q, K,
 * V, dO, O) follow IEEE arithmetic (no NaN guards): they reach the outputs
 * that depend on them, and may also reach rows that share a row tile with
 * them (tiles are aligned blocks of at most 128 rows), since a masked entry
 * enters a tile product with weight zero and 0 * NaN is NaN.  Rows of a
 * document separated from the non-finite value by a boundary at a multiple
 * of 128 rows are unaffected, bit for bit.
 *
 * Layouts (all fp32 unless noted, contiguous, row-major, no batch dimension --
 * packed documents replace batching):
 *   Q, dO, dQ, O   [seq_len, n_heads,    head_dim]
 *   K, V, dK, dV   [seq_len, n_kv_heads, head_dim]
 *   LSE            [seq_len, n_heads]      natural log
 *   seg            [seq_len] uint32        start index of the query's document;
 *                                          NULL means all zeros (plain causal).
 *                                          Values must be < 2^31.  A row with
 *                                          seg[s] > s sees no key: it contributes
 *                                          nothing (and its forward LSE is -inf).
 *
 * Pointers.  Every tensor pointer is a device pointer on the current HIP
 * device, 16-byte aligned.  The caller owns every buffer; the library keeps
 * no pointer after a call returns.  dQ, dK, dV must not overlap each other
 * or any input; inputs are only read.
 *
 * Streams.  `stream` is a hipStream_t (NULL = the default stream).  Calls only
 * enqueue work and return; kernel-execution faults surface at the caller's
 * next synchronisation.  Launch-time errors return ATTN_ERR_HIP.
 *
 * Threads.  Reentrant.  Global state: the per-device memory pools (created
 * once, under a lock), the scratch limit (an atomic, set by
 * attn_set_scratch_limit) and, per thread, the text of the last error and the
 * event log of the measurement hooks.
 */
#ifndef ATTNBWD_H
#define ATTNBWD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  /* a required pointer is NULL (only seg and, for attn_fwd_lse, O may be);
     seq_len < 0; n_heads < 1; n_kv_heads < 1; n_heads % n_kv_heads != 0;
     scale not finite */
  ATTN_ERR_INVALID_ARG = 1,
  /* head_dim not a multiple of 16 in [16, 256]; a pointer not 16-byte
     aligned; seq_len * n_heads >= 2^31; n_heads * head_dim >= 2^23 */
  ATTN_ERR_UNSUPPORTED = 2,
  /* a HIP runtime call or kernel launch failed (text: attn_last_error) */
  ATTN_ERR_HIP = 3
} attn_status_t;

/*
 * attn_bwd -- the backward pass above.
 *
 * dQ, dK and dV are ACCUMULATED ("+=": the header comment of the wgsl page
 * gives dQ += semantics with the host zeroing before the first call, and dK,
 * dV accumulate likewise).  Zero them before the first accumulation.
 *
 * Workspace.  Each call takes one stream-ordered workspace from a private
 * per-device memory pool (hipMallocFromPoolAsync on `stream`, released with
 * hipFreeAsync on `stream` before returning).  The pool keeps freed memory
 * for later calls up to 4 GiB; whatever it holds above that goes back to the
 * device at the caller's next synchronisation.  The workspace holds the row
 * term D (seq_len * n_heads * 4 bytes), per-32-row block metadata, and a
 * scratch of the probabilities P and the products P*dP of every visible
 * (32-query block, 32-key block, head) tile, written by the first pass and
 * read by the key-major pass instead of recomputing the scores.  The scratch
 * is sized by the causal bound, 8 KiB per block pair and head: 2 GiB at
 * seq_len 4096 with 32 heads, 16 GiB at 16384 with 16.  Its limit is 32 GiB
 * (attn_set_scratch_limit changes it).  When the tiles of all heads exceed
 * the limit, the passes run in head chunks one after another, each on the
 * same scratch: as many whole KV groups as fit, or else the largest share of
 * one group's heads (a divisor of n_heads / n_kv_heads) that fits; each
 * chunk adds its part into dK, dV.  When not even one head's tiles fit, or
 * the pool cannot supply the workspace (out of device memory), the call
 * recomputes the scores in the key-major pass instead and the workspace is
 * only D and the metadata.  With the scratch, a call given a seg whose
 * key-major pass would have fewer than 2048 workgroups (64-key tiles x KV
 * heads of a chunk) splits each group's heads over 2^k workgroups (k as
 * large as that bound and the group size allow); the first adds into dK, dV,
 * and the workspace then also holds the others' partial dK and dV:
 * 2 * (2^k - 1) * seq_len * n_kv_heads * head_dim * 4 bytes (192 MiB at
 * seq_len 16384, 2 KV heads, head_dim 256, 4 splits).  attn_bwd_plan reports
 * the choice and the largest size for a problem.
 *
 * seq_len == 0 returns ATTN_OK and enqueues nothing.
 */
attn_status_t attn_bwd(const float* Q, const float* K, const float* V, const float* dO,
                       const float* LSE, const uint32_t* seg,
                       float* dQ, float* dK, float* dV,
                       int seq_len, int n_heads, int n_kv_heads, int head_dim, float scale,
                       void* stream);

/*
 * attn_bwd_o -- attn_bwd for callers that kept the forward output O [S, H, d]
 * (fp32, same layout as Q; attn_fwd_lse produces it).  The row term is read
 * off it, D[s,h] = dO[s,h,:] . O[s,h,:], which equals sum_j P*dP when O and
 * LSE come from the same forward: summing P_j (dO . v_j) over the visible
 * keys gives dO . (sum_j P_j v_j), and that sum is the forward's output (page
 * "tang 0.2.0 -- src/gpu/llm.rs", causal_attention_fused: the
 * probability-weighted sum of V).  With D known up front the first pass
 * forms dS directly; otherwise as attn_bwd (arguments, layouts, +=
 * semantics, errors, workspace).  O is read only; NULL O is
 * ATTN_ERR_INVALID_ARG.
 */
attn_status_t attn_bwd_o(const float* Q, const float* K, const float* V, const float* O,
                         const float* dO, const float* LSE, const uint32_t* seg,
                         float* dQ, float* dK, float* dV,
                         int seq_len, int n_heads, int n_kv_heads, int head_dim, float scale,
                         void* stream);

/*
 * attn_bwd_rope -- attn_bwd (O == NULL) or attn_bwd_o (O given) followed by
 * the RoPE backward of page "llm.istanbul -- 10_backward_attention.wgsl"
 * (kernels rope_q_backward, rope_k_backward) applied in place to dQ and dK,
 * fused into the kernels' write-back: for row s, head h and column pair
 * (2p, 2p+1), angle = (s + pos_offset) * rope_base^(-2p/head_dim) and
 * (g0, g1) -> (g0 cos + g1 sin, -g0 sin + g1 cos), the transpose of the
 * forward rotation (q0 cos - q1 sin, q0 sin + q1 cos).  So
 *   dQ <- R^T (dQ + attention gradient),  dK <- R^T (dK + attention gradient),
 *   dV <- dV + attention gradient,
 * exactly what the unfused sequence leaves.  Q and K are the rotated tensors
 * the forward used.  The angle is computed in double precision.
 * Errors as attn_bwd, plus ATTN_ERR_INVALID_ARG for rope_base <= 0 or not
 * finite, pos_offset < 0, or pos_offset + seq_len > 2^31.
 */
attn_status_t attn_bwd_rope(const float* Q, const float* K, const float* V, const float* O,
                            const float* dO, const float* LSE, const uint32_t* seg,
                            float* dQ, float* dK, float* dV,
                            int seq_len, int n_heads, int n_kv_heads, int head_dim, float scale,
                            float rope_base, int pos_offset, void* stream);

/*
 * attn_bwd_f16 -- the same gradients with 16-bit matrix-core operands.
 * Every operand of the page's products (Q, K, V, dO, and the probability and
 * score-gradient tiles P and scale*dS of kernel attention_backward) is rounded
 * to IEEE fp16 (round to nearest even) and every sum is accumulated in fp32;
 * inputs, outputs, LSE, the row term and the masks stay fp32.  The pages
 * compute in fp32 throughout: this is a reduced-precision variant of their
 * sums (it runs the products at the fp16 matrix rate), meant for activations
 * of ordinary magnitude -- inputs beyond the fp16 range (|x| > 65504)
 * overflow to infinity.  Measured against the fp64 definition it stays
 * within 1e-3 of the largest gradient on the workloads the tests cover.
 *
 * O is the forward output, as for attn_bwd_o, or NULL: the row term is then
 * computed by an extra pass over the scores.  Arguments, layouts, +=
 * semantics and errors as attn_bwd.  Workspace (same private pool): fp16
 * row-tile copies of Q, dO, K and V, (2 * n_heads + 2 * n_kv_heads) * Sp *
 * DP * 2 bytes, with Sp = seq_len rounded up to 128 and DP = head_dim rounded
 * up to 32, 64, 96, 128, 192 or 256 (the products that contract over rows
 * read these tiles through transposing LDS loads); the row term and the
 * rows' LSE * log2(e) (seq_len * n_heads * 4 bytes each) and block metadata;
 * and, when the key-major pass splits each KV group's heads over
 * `splits` workgroups (a power of two dividing n_heads / n_kv_heads, chosen
 * from the shape: one round of resident workgroups for plain causal calls,
 * about 1024 workgroups under a document mask), 2 * splits * seq_len * n_kv_heads *
 * head_dim * 4 bytes of partial dK, dV sums, added in split order (the result
 * does not depend on the schedule); and the score-gradient tiles scale*dS in
 * fp16 that the key-major pass stores for the dQ pass, 2 KiB per (32-query
 * block, 32-key block, head) slot of the causal bound, nblk * (nblk + 1) / 2
 * * n_heads * 2048 bytes with nblk = ceil(seq_len / 32), when that fits the
 * scratch limit (attn_set_scratch_limit) and the pool can supply it; else
 * the dQ pass forms dS again from the scores instead (the same sums, three
 * products per visible pair instead of one).  0.64 GiB at seq_len 4096, 32 heads, 8 KV heads,
 * head_dim 128, plain causal (2 splits, 0.50 GiB of dS tiles).
 */
attn_status_t attn_bwd_f16(const float* Q, const float* K, const float* V, const float* O,
                           const float* dO, const float* LSE, const uint32_t* seg,
                           float* dQ, float* dK, float* dV,
                           int seq_len, int n_heads, int n_kv_heads, int head_dim, float scale,
                           void* stream);

/*
 * attn_bwd_f16_rope -- attn_bwd_f16 followed by the RoPE backward of page
 * "llm.istanbul -- 10_backward_attention.wgsl" (kernels rope_q_backward,
 * rope_k_backward) on dQ and dK, fused into the write-back exactly as in
 * attn_bwd_rope: dQ <- R^T (dQ + attention gradient), dK <- R^T (dK +
 * attention gradient), dV <- dV + attention gradient, with angle = (s +
 * pos_offset) * rope_base^(-2p/head_dim) for column pair (2p, 2p+1) of row
 * s, taken in double precision.  Q and K are the rotated tensors the forward
 * used.  When the key-major pass splits a KV group's heads, the partial sums
 * are added and dK rotated in one pass after it.  Arguments, precision,
 * workspace and errors as attn_bwd_f16, plus ATTN_ERR_INVALID_ARG for
 * rope_base <= 0 or not finite, pos_offset < 0, or pos_offset + seq_len >
 * 2^31.
 */
attn_status_t attn_bwd_f16_rope(const float* Q, const float* K, const float* V, const float* O,
                                const float* dO, const float* LSE, const uint32_t* seg,
                                float* dQ, float* dK, float* dV,
                                int seq_len, int n_heads, int n_kv_heads, int head_dim, float scale,
                                float rope_base, int pos_offset, void* stream);

/*
 * attn_bwd_short -- the backward for short sequences (seq_len <= 1024): page
 * "llm.istanbul -- 10_backward_attention.wgsl", attention_backward_short and
 * attention_backward_short_dKdV, the page's variant for sequences of at most
 * 1024 positions.  The same sums, arguments, layouts, += semantics and mask
 * as attn_bwd; O is the forward output (as for attn_bwd_o: D = dO . O) or
 * NULL (D = sum_j P dP, computed by a first launch).  With O given the whole
 * backward is ONE kernel launch and needs no workspace: workgroups that own
 * 32 queries of one head (dQ) and workgroups that own 32 keys of one KV head
 * (dK, dV) run side by side, each splitting its visible blocks over its four
 * waves and adding the waves' partial sums in a fixed order (deterministic,
 * no atomics).  Without O, a workspace of seq_len * n_heads * 4 bytes (same
 * pool) holds D between a row-term launch and the backward.  When a KV
 * group's heads are many against the sequence (a key block at the start of
 * a long document would otherwise take one workgroup's whole time), the
 * key-side workgroups split the group's heads into `splits` shares (a power
 * of two dividing n_heads / n_kv_heads, chosen from the shape alone), write
 * partial dK, dV sums to a workspace of 2 * splits * seq_len * n_kv_heads *
 * head_dim * 4 bytes, and one more launch adds them in split order (still
 * deterministic).  Above 128 columns (up to the 256 of every entry) the
 * single-launch kernels do not fit a wave's registers, and the call runs
 * attn_bwd_o (O given) or attn_bwd instead: the same results, with their
 * launches and workspace.  Errors as attn_bwd, plus ATTN_ERR_UNSUPPORTED for
 * seq_len > 1024, or, up to 128 columns, seq_len * n_heads * head_dim * 4 >=
 * 2^31.
 */
attn_status_t attn_bwd_short(const float* Q, const float* K, const float* V, const float* O,
                             const float* dO, const float* LSE, const uint32_t* seg,
                             float* dQ, float* dK, float* dV,
                             int seq_len, int n_heads, int n_kv_heads, int head_dim, float scale,
                             void* stream);

/*
 * attn_bwd_decode -- the single-query backward over a KV history (one decode
 * step) with the forward's probabilities stored: page "rullama 0.5.0 --
 * src/backend/dispatch/training.rs", attention_backward_dq_chained and
 * attention_backward_dkv_chained (pass 1: score gradients and dq; pass 2:
 * key-major dK and dV).  The query of head h (kv_h = h / (n_heads /
 * n_kv_heads)) sees every one of the history_len keys:
 *   dP[h][j] = dO[h,:] . V[j,kv_h,:],  D[h] = sum_j P[h][j] dP[h][j],
 *   dS[h][j] = P[h][j] (dP[h][j] - D[h]),
 *   dq[h,:] += scale sum_j dS[h][j] K[j,kv_h,:],
 *   dK[j,kv,:] += scale sum_{h in kv's group} dS[h][j] q[h,:],
 *   dV[j,kv,:] += sum_{h in kv's group} P[h][j] dO[h,:].
 * Layouts (fp32, contiguous, device pointers): q, dO, dq [n_heads, head_dim];
 * P [n_heads, history_len]; K, V, dK, dV [history_len, n_kv_heads, head_dim]
 * (the history's positions in order, like K and V above).  dq, dK, dV are
 * ACCUMULATED.  scale multiplies the scores (the page's parameters carry
 * none; a caller passes 1/sqrt(head_dim) for the usual attention).
 * Deterministic (no atomics).  Workspace (same pool): (n_heads * history_len
 * + n_heads * ceil(history_len/128) * (head_dim + 1)) * 4 bytes.
 * Errors as attn_bwd (history_len in the place of seq_len).  history_len
 * == 0 returns ATTN_OK and does nothing (K, V, P, dK and dV may then be
 * NULL).
 */
attn_status_t attn_bwd_decode(const float* q, const float* K, const float* V, const float* P,
                              const float* dO, float* dq, float* dK, float* dV,
                              int history_len, int n_heads, int n_kv_heads, int head_dim,
                              float scale, void* stream);

/*
 * attn_bwd_noalloc -- attn_bwd for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Same arguments, layouts, += semantics, mask and
 * results as attn_bwd; it calls no hipMalloc, hipFree or pool allocation.
 * Its workspace is a fixed 32 MiB device array inside the library, one per
 * device (taken when the library's code loads on that device, held until the
 * process ends; its address is looked up on the first call on each device).
 * The workspace holds D and the block metadata and, when they fit beside
 * them, the stored probability tiles of as many heads as fit (run in head
 * chunks as above); otherwise the key-major pass recomputes the scores.
 * Limit: seq_len * n_heads * 4 bytes of row term plus about seq_len / 2
 * bytes of metadata must fit in 32 MiB (seq_len * n_heads up to about 8.3
 * million); larger problems return ATTN_ERR_UNSUPPORTED before any GPU work.
 * Every call on a device shares that device's array, and nothing in it needs
 * clearing between calls (each call writes what it reads): calls that may
 * overlap on one device -- on different streams, or from several threads --
 * race on it and must be serialised by the caller.  Errors as attn_bwd.
 */
attn_status_t attn_bwd_noalloc(const float* Q, const float* K, const float* V, const float* dO,
                               const float* LSE, const uint32_t* seg,
                               float* dQ, float* dK, float* dV,
                               int seq_len, int n_heads, int n_kv_heads, int head_dim,
                               float scale, void* stream);

/*
 * attn_bwd_plan -- host-side query (no GPU work): the most workspace bytes
 * one attn_bwd (or attn_bwd_o, attn_bwd_rope) call of this size takes under
 * the current scratch limit (that of a call with a seg, with head splits
 * where they apply; plain causal calls take no splits), and how its
 * key-major pass gets the probabilities: *stored_heads = the number of heads
 * whose tiles one chunk stores (n_heads when the call runs in one piece), or
 * 0 when the scores are recomputed.  Either output pointer may be NULL.
 * Same argument checks as attn_bwd.
 */
attn_status_t attn_bwd_plan(int seq_len, int n_heads, int n_kv_heads, int head_dim,
                            size_t* workspace_bytes, int* stored_heads);

/*
 * attn_set_scratch_limit -- the most bytes of stored probability tiles one
 * attn_bwd, attn_bwd_o or attn_bwd_rope call may take, and of stored fp16
 * score-gradient tiles one attn_bwd_f16 or attn_bwd_f16_rope call may take
 * (default 32 GiB, about 11% of the 288 GB of HBM3E); 0 turns the stored
 * tiles off (the key-major pass then recomputes the scores; the fp16 dQ pass
 * forms dS again).  Process-wide, read when a call is
 * planned; calls already enqueued keep their workspace.  The previous limit
 * goes to *previous when it is not NULL.  Always ATTN_OK.
 */
attn_status_t attn_set_scratch_limit(size_t bytes, size_t* previous);

/*
 * attn_fwd_lse -- the forward pass that produces the backward's inputs:
 *   LSE[s,h] = ln sum over visible j of exp(scale * Q[s,h,:] . K[j,kv_h,:])
 *   O[s,h,:] = sum over visible j of exp(scale * Q[s,h,:] . K[j,kv_h,:] - LSE[s,h]) * V[j,kv_h,:]
 * (page "tang 0.2.0 -- src/gpu/llm.rs", causal_attention_fused: row max,
 * exp-sum, weighted V; with the document mask above and the log-sum-exp
 * output the backward consumes).  O and LSE are OVERWRITTEN.  O may be NULL
 * (LSE only).  A row that sees no key gets LSE = -inf and O = 0.
 */
attn_status_t attn_fwd_lse(const float* Q, const float* K, const float* V, const uint32_t* seg,
                           float* O, float* LSE,
                           int seq_len, int n_heads, int n_kv_heads, int head_dim, float scale,
                           void* stream);

/*
 * Measurement hooks (benchmarks only; normal callers never need them).
 *
 * attn_profile_begin: from now on, on the calling thread, every attn_bwd call
 *   records HIP events on its stream before, between and after its passes:
 *   the query-major pass (row term D, and dQ or the stored tiles), the
 *   key-major pass (dK, dV), and -- with stored tiles -- the dQ pass.  An
 *   attn_bwd_f16 call records its three: the fp16 copies and the row term,
 *   the key-major pass, the dQ pass; an attn_bwd_decode call its three:
 *   the score-gradient pass, the dK/dV pass, the dq pass; an attn_bwd_short
 *   call its one (the whole backward, with the split sums when the heads are
 *   split; with O NULL two: the row term, then the backward).
 * attn_profile_end: waits for those events, writes into ms[0], ms[1], ms[2]
 *   the summed device time in milliseconds of each of the three passes over
 *   the recorded calls (ms[2] = 0 for calls without the dQ pass), into
 *   *n_calls their number, releases the events and stops recording.  ms
 *   (room for 3 doubles) and n_calls may be NULL.
 */
attn_status_t attn_profile_begin(void);
attn_status_t attn_profile_end(double* ms, int* n_calls);

/* Text describing the last non-OK status returned on the calling thread
   ("" if none).  The pointer stays valid until the thread's next call. */
const char* attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTNBWD_H */
