/*
 * tokengate.h -- C ABI of the TokenGate gated-prefill hot path on MI355X (gfx950).
 *
 * The path has four steps, one entry point each:
 *   tg_gate_score       a small MLP scores every token's post-attention residual
 *   tg_select_topk      keeps every question token and the K best document tokens
 *   tg_gather_kept      compacts the kept rows (and their scores) in position order
 *   tg_gated_attention  attention over the kept tokens with the score as a key bias
 * plus tg_select_topk_multi (several budgets in one launch), tg_select_random (the
 * random-K selector), tg_gated_attention_backward (the gradient of the gated attention)
 * and tg_qkv_rope (kept-row projection, rotary embedding and KV emission).
 *
 * Sources, cited by page title and section:
 *   aiproducthub.cn "斯坦福伯克利TokenGate 预填充提速11.3倍", section 事件详情
 *     (three-phase forward, MLP gate on the post-attention residual, top-K, only the
 *     document is prunable, score as attention-logit bias with per-head gain and
 *     temperature);
 *   aisight.pl "TokenGate: Stanford i Berkeley ucza model, ktore tokeny pominac ...",
 *     sections "Jak to dziala" (same mechanism) and "Wdrozenie i zastrzezenia"
 *     (the {state} document placeholder and the max_kept_prefill_tokens budget);
 *   news.chathome.org TokenGate article, sections
 *     "TokenGate の学習可能なトークンプルーニングの仕組み" and
 *     "トークンゲート付きアテンションとは".
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless marked (host).  The caller owns every
 *     buffer, including workspaces; the library allocates and frees nothing.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the null
 *     stream).  The library never synchronises the stream.
 *   - All arguments are validated on the host before anything is enqueued; on a
 *     non-zero status nothing was enqueued and no output was touched.
 *   - Return values are tg_status codes (int32).  TG_ERR_HIP means a launch failed
 *     (hipGetLastError); the stream state is then undefined.
 *   - Calls that share a workspace must not run concurrently.
 */
#ifndef TOKENGATE_H
#define TOKENGATE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TG_ABI_VERSION 1

/* element types of hidden states, weights, Q/K/V and outputs */
#define TG_F32  0   /* IEEE float32 */
#define TG_BF16 1   /* bfloat16 storage, float32 accumulation */

/* status codes */
#define TG_OK              0
#define TG_ERR_INVALID_ARG 1   /* null pointer, negative size, bad span, bad stride ... */
#define TG_ERR_UNSUPPORTED 2   /* a shape or alignment this library has no kernel for */
#define TG_ERR_WORKSPACE   3   /* workspace too small */
#define TG_ERR_HIP         4   /* the HIP runtime reported an error at launch */
#define TG_ERR_INCOMPLETE  5   /* tg_select_check: a selection gave up waiting (see there) */

typedef int32_t tg_status;

/* Version of this ABI (TG_ABI_VERSION of the built library). Host only. */
int32_t tg_abi_version(void);

/* Static, human-readable text for a status code. Host only; never NULL. */
const char* tg_status_string(tg_status status);

/*
 * tg_gate_score -- the MLP gate (aiproducthub.cn, section 事件详情; aisight.pl,
 * section "Jak to dziala").  For every row i in [0, n):
 *
 *     scores[i] = b2 + sum_j w2[j] * GELU( b1[j] + sum_k x[i,k] * w1[j,k] )
 *
 * with the exact GELU(t) = t * Phi(t) (Phi = standard normal CDF).  All n rows are
 * scored, question tokens included, since every kept token's score later biases
 * the attention.
 *   dtype     TG_F32 or TG_BF16: element type of x, w1, w2
 *   x         [n, d_model] row-major, row stride ldx elements (ldx >= d_model)
 *   w1        [d_hidden, d_model] row-major, contiguous (output-by-input layout)
 *   b1        [d_hidden] float32, or NULL for zero
 *   w2        [d_hidden] in dtype
 *   b2        (host) scalar
 *   scores    [n] float32 output
 * Arithmetic: bf16 operands with float32 accumulation (MFMA); GELU and the
 * 1-wide output dot in float32.  f32: float32 throughout.
 * Supported: n in [1, 2^31-1].  bf16: d_model % 64 == 0, d_hidden in {64, 128, 192, 256},
 * ldx % 8 == 0, x and w1 16-byte aligned.  f32: d_model % 4 == 0, ldx % 4 == 0,
 * d_hidden in [1, 256].  Otherwise TG_ERR_UNSUPPORTED.
 */
tg_status tg_gate_score(int32_t dtype, int64_t n, int32_t d_model, int32_t d_hidden,
                        const void* x, int64_t ldx, const void* w1, const float* b1,
                        const void* w2, float b2, float* scores, void* stream);

/*
 * tg_num_kept -- rows above the gate (host only).  The document is the span
 * [doc_begin, doc_end) of the prompt (the {state} placeholder, aisight.pl section
 * "Wdrozenie i zastrzezenia"); k is the document-token budget
 * (max_kept_prefill_tokens).  Returns (n - D) + min(k, D) with D = doc_end -
 * doc_begin, or -1 if the arguments are invalid (n < 0, k < 0, span outside [0, n]).
 */
int64_t tg_num_kept(int64_t n, int64_t doc_begin, int64_t doc_end, int64_t k);

/* Bytes of workspace the selection calls need for n scores (host only); 0 if n < 0.  One
 * workspace serves tg_select_topk, tg_select_gather, tg_select_topk_multi and
 * tg_select_random. */
size_t tg_select_workspace_bytes(int64_t n);

/*
 * tg_select_topk -- document-only top-K (aiproducthub.cn, section 事件详情: only the
 * document part of the prompt is prunable, the question never is).  Keeps every
 * position outside [doc_begin, doc_end) and the min(k, D) document positions ranked
 * first by (score descending, position ascending), and writes them to kept_idx in
 * ascending position order; m = tg_num_kept(n, doc_begin, doc_end, k) entries.
 * Ranking is exact: -0 equals +0, NaN ranks below every number (ties among NaNs
 * again by position).  K > D keeps the whole document; K = 0 keeps none of it.
 *   scores     [n] float32
 *   kept_idx   [m] int32 output
 *   workspace  >= tg_select_workspace_bytes(n) bytes, 256-byte aligned.  It must be
 *              zero-filled before its first use; every call leaves the parts that
 *              must start at zero (histograms, counters, flags) at zero again, so a
 *              workspace can be reused for any n it is large enough for.
 * The selection is one launch whose workgroups wait for each other; every wait is
 * bounded.  If a wait gives up (possible only when other work occupies the device so
 * that not all of the launch's workgroups are resident at once), or if the call finds
 * the workspace not zero-filled, the workspace's sticky failure word is set, the
 * outputs are invalid, and every later selection on that workspace exits without
 * writing until the caller zero-fills it again; tg_select_check reports the word.
 * Test hook: a non-zero uint32 at byte offset 12 of the workspace bounds each wait to
 * that many polls; 0xFFFFFFFF makes every wait give up at once (a zero-filled
 * workspace waits up to 2^22 polls).
 * m = 0 (the whole prompt is a document and k = 0) is a no-op.
 * Supported: n in [1, 2^31-1].
 */
tg_status tg_select_topk(int64_t n, const float* scores, int64_t doc_begin, int64_t doc_end,
                         int64_t k, int32_t* kept_idx, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * tg_select_gather -- tg_select_topk and tg_gather_kept in one launch: the kept
 * positions, the kept rows of x and their scores (aiproducthub.cn, section 事件详情:
 * the top-K selector keeps the best tokens and layers above the gate see only those;
 * aisight.pl, section "Jak to dziala").
 *     kept_idx[r] = r-th kept position (ascending),   x_kept[r, :] = x[kept_idx[r], :],
 *     s_kept[r] = scores[kept_idx[r]]                 (r < m = tg_num_kept(n, ..., k))
 *   dtype      TG_F32 or TG_BF16: element type of x and x_kept
 *   x          [n, d_model], row stride ldx >= d_model
 *   x_kept     [m, d_model] output, row stride ld_out >= d_model
 *   s_kept     [m] float32 output (required)
 * Selection, workspace, failure reporting and errors as tg_select_topk; the copy is
 * bit-exact.  m = 0 is a no-op.
 */
tg_status tg_select_gather(int32_t dtype, int64_t n, int32_t d_model, const float* scores,
                           int64_t doc_begin, int64_t doc_end, int64_t k, const void* x, int64_t ldx,
                           int32_t* kept_idx, void* x_kept, int64_t ld_out, float* s_kept,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * tg_select_gather_noalloc -- tg_select_gather without a workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, serving loops that
 * must not call hipMalloc, harnesses that forbid allocation.  The workspace is a static
 * device array of tg_select_workspace_bytes' fixed size (218 KiB, enough for every n: the
 * selection's layout does not depend on n), one per device, held by the library until the
 * process ends.  Each call clears it on `stream` with a small fill kernel before selecting,
 * so a call that gave up leaves nothing behind for the next.  Calls that overlap on one
 * device (two streams, or two host threads) share that array and race: serialise them.
 * Calls no hipMalloc, hipFree or other allocating routine.
 *   status  NULL, or one device int32 that the call sets to 0 on the stream and to 1 if a
 *           wait of the selection gave up (its outputs are then invalid); not touched when
 *           nothing is kept (m = 0)
 * Other arguments, outputs and errors as tg_select_gather.
 */
tg_status tg_select_gather_noalloc(int32_t dtype, int64_t n, int32_t d_model, const float* scores,
                                   int64_t doc_begin, int64_t doc_end, int64_t k, const void* x, int64_t ldx,
                                   int32_t* kept_idx, void* x_kept, int64_t ld_out, float* s_kept,
                                   int32_t* status, void* stream);

/*
 * tg_select_check -- whether every selection enqueued so far on `workspace` completed.
 * Synchronises `stream` (the host blocks until the stream's work is done), then reads
 * the workspace's sticky failure word: TG_OK if it is clear; TG_ERR_INCOMPLETE if a
 * selection gave up waiting or found the workspace not zero-filled (its outputs are
 * invalid; zero-fill the workspace before reusing it); TG_ERR_HIP on a runtime error.
 */
tg_status tg_select_check(const void* workspace, size_t workspace_bytes, void* stream);

/*
 * tg_select_topk_multi -- tg_select_topk for several budgets of the same scores in one
 * launch (one trained gate serves every budget: aiproducthub.cn, section 事件详情;
 * aisight.pl, section "Wyniki").  Budget b's kept list (m_b = tg_num_kept(n, doc_begin,
 * doc_end, ks[b]) ascending positions, exactly tg_select_topk's) is written at
 * kept_idx + sum_{c < b} m_c.
 *   ks         (host) [n_budgets] budgets, each >= 0; 1 <= n_budgets <= 8
 *   kept_idx   [sum_b m_b] int32 output
 * Other arguments, workspace and errors as tg_select_topk.
 */
tg_status tg_select_topk_multi(int64_t n, const float* scores, int64_t doc_begin, int64_t doc_end,
                               const int64_t* ks, int32_t n_budgets, int32_t* kept_idx, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * tg_select_random -- the pages' random-K selector (aiproducthub.cn, section 事件详情;
 * news.chathome.org, section "ベンチマーク"): every position outside the document plus a
 * uniformly random min(k, D)-subset of the document, ascending.  Position i draws the key
 * (uint32) of the high half of output i (counting from 0) of SplitMix64 seeded with
 * `seed`: x_i = seed + (i + 1) * 0x9E3779B97F4A7C15 (mod 2^64), then
 *     z = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9;  z = (z ^ (z >> 27)) * 0x94D049BB133111EB;
 *     z ^= z >> 31;  key = z >> 32
 * and the min(k, D) largest document keys are kept (equal keys: lower position first).
 * Deterministic for a given seed.  Arguments, workspace and errors as tg_select_topk.
 */
tg_status tg_select_random(int64_t n, int64_t doc_begin, int64_t doc_end, int64_t k, uint64_t seed,
                           int32_t* kept_idx, void* workspace, size_t workspace_bytes, void* stream);

/*
 * tg_gather_kept -- compaction of the kept rows: layers above the gate see only the
 * kept tokens and pruned tokens create no KV entries (aiproducthub.cn, section
 * 事件详情; aisight.pl, section "Jak to dziala").
 *     x_kept[r, :] = x[kept_idx[r], :],   s_kept[r] = scores[kept_idx[r]]   (r < m)
 *   x          [n, d_model] (row stride ldx), dtype elements
 *   kept_idx   [m] int32, entries in [0, n); a row whose index is outside [0, n) is
 *              skipped (its output row and score are left untouched)
 *   x_kept     [m, d_model] output, row stride ld_out >= d_model
 *   scores, s_kept  both NULL, or both set ([n] in, [m] out, float32)
 * A bit-exact copy.  m = 0 is a no-op.
 */
tg_status tg_gather_kept(int32_t dtype, int64_t n, int32_t d_model, const void* x, int64_t ldx,
                         const int32_t* kept_idx, int64_t m, void* x_kept, int64_t ld_out,
                         const float* scores, float* s_kept, void* stream);

/*
 * tg_gated_attention -- token-gated attention over the m kept tokens (aiproducthub.cn,
 * section 事件详情; aisight.pl, section "Jak to dziala": each kept token's score becomes
 * a bias on the attention logits, with a learnable per-head gain and a learnable
 * temperature).  Adopted form, for query head h and key/value head g = h / (Hq/Hkv):
 *
 *     logit[i,j] = q[i,h,:].k[j,g,:] / (sqrt(head_dim) * tau) + gain[h] * s_kept[j]
 *     out[i,h,:] = sum_{j : pos[j] <= pos[i]} softmax_j(logit[i,:]) * v[j,g,:]
 *
 *   q          [m, n_q_heads, head_dim], contiguous
 *   k, v       [m, n_kv_heads, head_dim], contiguous
 *   pos        [m] int32 original positions, strictly increasing (the output of
 *              tg_select_topk); NULL means 0..m-1.  Key tiles wholly after a query
 *              tile are skipped, which is exact only under this precondition.
 *   s_kept     [m] float32 and gain [n_q_heads] float32: both set, or both NULL
 *              (bias off)
 *   tau        (host) temperature, finite and > 0
 *   out        [m, n_q_heads, head_dim] in dtype (bf16 rounded to nearest even)
 * Arithmetic (bf16): Q is scaled by log2(e)/(sqrt(head_dim) tau) and rounded to bf16;
 * Q.K^T and P.V run on bf16 MFMA with float32 accumulation; the bias enters the same
 * accumulation with the score and gain each split into two bf16 parts (relative error
 * below 2^-16); online softmax in float32 (exp2), P rounded to bf16 for the P.V product.
 * q, k, v, s_kept and gain must be finite (NaN inputs give undefined output).
 * Supported: head_dim in {64, 128}; n_q_heads % n_kv_heads == 0; q, k, v, out
 * 16-byte aligned.  m = 0 is a no-op.
 * Launch (bf16): up to 768 workgroups of query tiles (a few thousand kept rows), each
 * workgroup walks its keys with two groups of waves and combines their softmax states
 * (tg_gated_attention_split's key groups); beyond, one group.
 */
tg_status tg_gated_attention(int32_t dtype, int64_t m, int32_t n_q_heads, int32_t n_kv_heads,
                             int32_t head_dim, const void* q, const void* k, const void* v,
                             const int32_t* pos, const float* s_kept, const float* gain, float tau,
                             void* out, void* stream);

/*
 * tg_gated_attention_lse -- tg_gated_attention that also writes each row's natural-log
 * log-sum-exp of its visible logits, lse [m, n_q_heads] float32 (what
 * tg_gated_attention_backward needs).  bf16 only (TG_ERR_UNSUPPORTED for float32);
 * otherwise as tg_gated_attention.
 */
tg_status tg_gated_attention_lse(int32_t dtype, int64_t m, int32_t n_q_heads, int32_t n_kv_heads,
                                 int32_t head_dim, const void* q, const void* k, const void* v,
                                 const int32_t* pos, const float* s_kept, const float* gain, float tau,
                                 void* out, float* lse, void* stream);

/*
 * tg_gated_attention_split -- tg_gated_attention (the same logits and mask: aiproducthub.cn,
 * section 事件详情; aisight.pl, section "Jak to dziala") with the library's launch plan for
 * few kept rows or few heads.  Without it, the query tile holding the last rows walks every
 * key before it in sequence, so at a few thousand kept rows the launch is as long as that
 * one walk while most of the GPU idles.  Two remedies, chosen by split_tiles:
 *   - key groups: each workgroup runs two groups of waves that walk alternate key tiles
 *     (64 keys each) of its query tile and combine their softmax states in LDS at the end
 *     (no workspace);
 *   - runs: each query tile's key tiles are cut into runs of split_tiles, walked by
 *     different workgroups; every run writes its partial softmax state to the workspace
 *     (its normalised output row Y_j = O_j / l_j, its running max m_j and row sum l_j, all
 *     float32) and a second kernel combines the runs of a row: w_j = 2^(m_j - M) l_j with
 *     M = max m_j, out = sum w_j Y_j / sum w_j, in run order (deterministic).  Query tiles
 *     with one run are written directly.
 *   split_tiles  0: chosen by the library: with at most 768 workgroups of query tiles and
 *                at least 4 head slots each, key groups; with fewer head slots, runs of
 *                max(8, ceil(total key-tile work / 256)) tiles (key groups if that is not
 *                shorter than the longest walk); beyond 768 workgroups (long contexts)
 *                neither, i.e. the tg_gated_attention kernel itself.
 *                < 0: no runs (key groups up to 768 workgroups, as tg_gated_attention does).
 *                > 0: runs of split_tiles key tiles, one key group (when that leaves one
 *                run per query tile: as < 0).
 *   lse          NULL, or [m, n_q_heads] float32 as in tg_gated_attention_lse.
 *   workspace    device, 256-byte aligned, at least
 *                tg_gated_attention_split_workspace_bytes(m, n_q_heads, n_kv_heads, head_dim,
 *                split_tiles) bytes (0 when that plan has no runs; the pointer may then be
 *                NULL).  Contents on entry are ignored; no zero-fill needed.
 * bf16 only; float32 runs the plain float32 kernel and ignores split_tiles and the workspace.
 * Other arguments, precision and errors as tg_gated_attention; TG_ERR_WORKSPACE if the
 * workspace is smaller than the plan needs.
 */
size_t tg_gated_attention_split_workspace_bytes(int64_t m, int32_t n_q_heads, int32_t n_kv_heads,
                                                int32_t head_dim, int32_t split_tiles);
tg_status tg_gated_attention_split(int32_t dtype, int64_t m, int32_t n_q_heads, int32_t n_kv_heads,
                                   int32_t head_dim, const void* q, const void* k, const void* v,
                                   const int32_t* pos, const float* s_kept, const float* gain, float tau,
                                   void* out, float* lse, int32_t split_tiles, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * tg_gated_attention_backward -- gradient of the token-gated attention: the path by which
 * the loss reaches the scorer through the score bias, and trains the per-head gain and
 * the temperature (aiproducthub.cn, section 事件详情; aisight.pl, section "Jak to dziala";
 * news.chathome.org, section "トークンゲート付きアテンションとは").  For dout = dL/dout,
 * with P the row softmax of the visible logits, dZ = P (dout v^T - rowsum(dout * out)):
 *     dq = dZ k / (sqrt(d) tau)        dk = dZ^T q / (sqrt(d) tau)     dv = P^T dout
 *     ds_kept[j] = sum_h gain[h] sum_i dZ_h[i,j]    dgain[h] = sum_j s_kept[j] sum_i dZ_h[i,j]
 *     dtau = -(1/tau) sum_{h,i,j} dZ_h[i,j] q_i.k_j / (sqrt(d) tau)
 * (dk, dv summed over the query heads of each key/value head.)
 *   q, k, v, pos, s_kept, gain, tau   the forward's inputs
 *   out, lse   the forward's output and tg_gated_attention_lse's log-sum-exp
 *   dout       [m, n_q_heads, head_dim] bf16
 *   dq, dk, dv outputs, shaped like q, k, v, bf16 (float32 accumulation)
 *   ds_kept [m], dgain [n_q_heads]: float32 outputs, set iff s_kept / gain are
 *   dtau       float32 output (one value) or NULL
 *   workspace  tg_gated_attention_backward_workspace_bytes(m, n_q_heads, n_kv_heads,
 *              head_dim) bytes, 256-byte aligned, no initial contents needed
 * Deterministic (fixed-order reductions, no float atomics).  Supported: bf16, head_dim in
 * {64, 128}, 16-byte aligned tensors; pos strictly increasing as for the forward.
 */
size_t tg_gated_attention_backward_workspace_bytes(int64_t m, int32_t n_q_heads, int32_t n_kv_heads,
                                                   int32_t head_dim);
tg_status tg_gated_attention_backward(int32_t dtype, int64_t m, int32_t n_q_heads, int32_t n_kv_heads,
                                      int32_t head_dim, const void* q, const void* k, const void* v,
                                      const int32_t* pos, const float* s_kept, const float* gain, float tau,
                                      const void* out, const float* lse, const void* dout, void* dq, void* dk,
                                      void* dv, float* ds_kept, float* dgain, float* dtau, void* workspace,
                                      size_t workspace_bytes, void* stream);

/*
 * tg_qkv_rope -- the step after the gather: project the kept rows to queries, keys and
 * values, rotate queries and keys by each kept token's ORIGINAL position, and write the
 * keys, values and positions into a KV cache that holds kept tokens only (layers above
 * the gate see only kept tokens and pruned tokens create no KV entries: aiproducthub.cn,
 * section 事件详情; aisight.pl, section "Jak to dziala").
 *     C = x_kept W_qkv^T (+ b_qkv)     W_qkv [(Hq + 2 Hkv) d, d_model]: rows of the Hq query
 *                                      heads, then the Hkv key heads, then the Hkv value heads
 *     rotary (rotate-half): for i < d/2, a = pos[j] * theta^(-2i/d),
 *         y_i = c_i cos a - c_{i+d/2} sin a,   y_{i+d/2} = c_{i+d/2} cos a + c_i sin a
 *     q_out[j, h, :]            = rotated query head h of row j
 *     k_cache[slot0 + j, h, :]  = rotated key head h;  v_cache[slot0 + j, h, :] = value head h
 *     pos_cache[slot0 + j]      = pos[j]   (if pos_cache is not NULL)
 *   x_kept   [m, ldx] bf16 (the gathered rows)     w_qkv, b_qkv (float32 or NULL) as above
 *   pos      [m] int32, the kept tokens' original positions (tg_select_topk's kept_idx)
 *   q_out    [m, Hq, d] bf16;  k_cache, v_cache [cache_capacity, Hkv, d] bf16; rows outside
 *            slot0 .. slot0 + m - 1 are not touched
 *   workspace  tg_qkv_rope_workspace_bytes(m, d) bytes, 256-byte aligned (the rotation table)
 * The angle is formed and reduced modulo 2 pi in float64, so positions up to 2^31 keep
 * full float32 accuracy in cos / sin.  Supported: bf16, d in {64, 128}, (Hq + 2 Hkv) d a
 * multiple of 128, d_model a multiple of 64, ldx a multiple of 8, 16-byte aligned
 * tensors; rope_theta > 1.  cache_slot0 + m <= cache_capacity, else TG_ERR_INVALID_ARG.
 */
size_t tg_qkv_rope_workspace_bytes(int64_t m, int32_t head_dim);
tg_status tg_qkv_rope(int32_t dtype, int64_t m, int32_t d_model, const void* x_kept, int64_t ldx,
                      const void* w_qkv, const float* b_qkv, int32_t n_q_heads, int32_t n_kv_heads,
                      int32_t head_dim, const int32_t* pos, float rope_theta, void* q_out, void* k_cache,
                      void* v_cache, int32_t* pos_cache, int64_t cache_slot0, int64_t cache_capacity,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * tg_check_positions -- the attention's precondition on pos (kept tokens keep their order
 * and the causal mask is on original positions: aiproducthub.cn, section 事件详情):
 *     *violations = #{i in [1, m) : pos[i] <= pos[i-1]} + #{i : pos[i] < 0}
 *   pos         [m] int32 (device)
 *   violations  one int32 (device), written (not accumulated); 0 means pos is strictly
 *               increasing and non-negative
 * One workgroup; asynchronous like every call.  TG_ERR_INVALID_ARG for m < 0 or a NULL
 * pointer (pos may be NULL when m == 0).
 */
tg_status tg_check_positions(const int32_t* pos, int64_t m, int32_t* violations, void* stream);

/* 1 if this library was built with TG_DEBUG: then tg_gated_attention, _lse, _split and
 * _backward run tg_check_positions on pos first, synchronise the stream, and return
 * TG_ERR_INVALID_ARG (nothing else enqueued) if pos is not strictly increasing. */
int32_t tg_debug_build(void);

#ifdef __cplusplus
}
#endif

#endif /* TOKENGATE_H */
