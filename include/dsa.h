/*
 * dsa.h -- C ABI of libdsa.so: one DeepSeek-Sparse-Attention (DSA) layer and
 * its sliding-window (SWA) sibling on an AMD Instinct MI355X (gfx950).
 *
 * Pages defining the operations (cited by title and section):
 *  [AXK2]    "Transformers 中的 AXK2 架构解析" (A.X-K2 in HF Transformers):
 *            "注意力前向的骨架：MLA + 显式稀疏掩码" (MLA forward with an explicit
 *            sparse mask), "三大改进" §1 Sparse Gated Attention (lightning
 *            indexer), §3 Attention output gate, and the AXK2Config section
 *            (index_topk, index_head_dim, index_n_heads).
 *  [SPARK]   Spark-X2.5-1.7B headwise attention output gate: "前向流程" steps
 *            1-3 and "为什么要加这一层门控" (sliding_window 512).
 *  [DSV2]    DeepSeek-V2 attention constructor parameters: items 4-6
 *            (qk_nope_head_dim, qk_rope_head_dim, v_head_dim).
 *  [PANGU]   openPangu-2.0 technical-report walkthrough: §3.2 (DSA-SWA-SWA,
 *            window 512), §3.3 (lightning indexer, fixed top-K), §3.4 (PAS
 *            attention sinks), §3.5 Table 1.
 *
 * Conventions shared by every entry point
 *  - Dtypes: DSA_F32 or DSA_BF16 applies to every floating input and to the
 *    attention output. Scores are always fp32, indices always int32.
 *  - Layouts are dense row-major with no padding. Caches are token-major:
 *    k_cache [B,T,H,Dqk], v_cache [B,T,H,Dv]; q [B,S,H,Dqk]. The last
 *    dimension of q and K is the nope slice followed by the rope slice
 *    ([DSV2] items 4-5); v_dim is separate ([DSV2] item 6).
 *  - Positions: query s of a call sits at absolute position p = past_len + s
 *    and may see keys t <= p (itself included). The caller has already
 *    appended this call's K/V rows and index keys to the caches
 *    ([AXK2] cache note), so T >= past_len + S.
 *  - Ownership: the caller allocates every buffer (inputs, outputs and the
 *    workspace) in device memory. The library never allocates or frees
 *    memory and keeps no pointer after a call returns.
 *  - Streams: every call only enqueues work on `stream` (0 = the default
 *    stream) and returns; outputs are valid once the stream reaches that
 *    point. Inputs must stay unchanged until then. Outputs must not alias
 *    inputs. Calls on different streams may run concurrently as long as they
 *    do not share a workspace.
 *  - Errors: every call validates its arguments on the host before touching
 *    the device and returns a status code (DSA_OK = 0). On error nothing is
 *    enqueued, and dsa_last_error() returns a message for the calling thread.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define DSA_OK 0
#define DSA_ERR_INVALID_ARG 1 /* null pointer, bad size, bad enum, T < past_len + S, ... */
#define DSA_ERR_UNSUPPORTED 2 /* valid but not implemented (head dims, topk > DSA_MAX_TOPK) */
#define DSA_ERR_WORKSPACE 3   /* workspace pointer null or smaller than the *_workspace_size */
#define DSA_ERR_HIP 4         /* a HIP launch failed; dsa_last_error() holds the message */
#define DSA_ERR_CHECK 5       /* debug builds only: a device-side check failed (see below) */

/* dtype */
#define DSA_F32 0
#define DSA_BF16 1

/* relu_mode of the indexer: where the ReLU sits relative to the head sum */
#define DSA_RELU_PER_HEAD 0 /* sum_h w_h * relu(u_h)  (default) */
#define DSA_RELU_NONE 1     /* sum_h w_h * u_h        (the printed formula) */
#define DSA_RELU_POST_SUM 2 /* relu(sum_h w_h * u_h) */

/* limits */
#define DSA_MAX_TOPK 2048
#define DSA_MAX_HEAD_DIM 256
#define DSA_MAX_SINKS 256
/* Size limits every call applies (DSA_ERR_UNSUPPORTED beyond them): query
 * rows B * S <= DSA_MAX_ROWS; keys T, and positions past_len + S, <=
 * DSA_MAX_KEYS; attention heads <= DSA_MAX_HEADS; index heads <=
 * DSA_MAX_INDEX_HEADS. The *_workspace_size queries return 0 for sizes their
 * calls reject. */
#define DSA_MAX_ROWS (0x7FFFFFFF / 64)
#define DSA_MAX_KEYS (1 << 30)
#define DSA_MAX_HEADS 65535
#define DSA_MAX_INDEX_HEADS 1024

/*
 * Lightning-indexer scores with causal mask ([AXK2] §1: per-head dot products
 * of the index query with the shared index key, weighted by the learned
 * per-head weights and summed; causality by an upper-triangle mask;
 * [PANGU] §3.3).
 *   score[b,s,t] = sum_h w[b,s,h] * relu(scale * q_idx[b,s,h,:] . k_idx[b,t,:])
 *   for t <= p = past_len + s, and -inf for p < t < T.
 * q_idx  [B,S,n_idx_heads,idx_dim]   dtype
 * k_idx  [B,T,idx_dim]               dtype (the indexer's own key cache)
 * w      [B,S,n_idx_heads]           dtype (per-head weights)
 * scores [B,S,T] fp32, written in full (every element, including the -inf
 *        triangle).
 * scale  > 0 and finite; the conventional value is idx_dim^-1/2.
 * relu_mode one of DSA_RELU_*.
 * Supported: idx_dim in {32, 64, 128}; 1 <= n_idx_heads <= DSA_MAX_INDEX_HEADS.
 */
int dsa_index_scores(const void* q_idx, const void* k_idx, const void* w, float* scores, int B,
                     int S, int T, int past_len, int n_idx_heads, int idx_dim, float scale,
                     int relu_mode, int dtype, hipStream_t stream);

/*
 * The indexer on FP8 operands ([AXK2] implementation notes: the reference
 * indexer rotates q and k with a Hadamard transform and scores FP8-quantised
 * copies; the rotation cancels in the dot products, so the scores
 * approximate dsa_index_scores). Two calls:
 *
 * dsa_index_quant_fp8 rotates each row of x [rows, dim] (bf16) by the
 * Sylvester-ordered Walsh-Hadamard matrix with +-1 entries (fast transform in
 * fp32, stride 1 first), picks the row scale 2^e with the smallest e such
 * that max|y| * 2^-e <= 448 (1 for an all-zero row), and stores
 *   codes [rows, dim]  OCP FP8 E4M3 (e4m3fn) of y * 2^-e, round to nearest even
 *   scales [rows]      fp32 2^e: a row's value is code * scale
 * Use it on q_idx (rows = B*S*n_idx_heads) every call and on the new rows of
 * the indexer key cache (rows = B*T, or just the appended ones) when they are
 * written. dim in {32, 64, 128}; dtype must be DSA_BF16 (DSA_F32 is
 * DSA_ERR_UNSUPPORTED).
 *
 * dsa_index_scores_fp8 computes, with the causal mask of dsa_index_scores,
 *   score[b,s,t] = sum_h w[b,s,h] * relu(scale / idx_dim * (qh . kt))
 *   qh = q_codes[b,s,h,:] * q_scales[b,s,h],  kt = k_codes[b,t,:] * k_scales[b,t]
 * (the 1 / idx_dim undoes the unnormalised rotation). q_codes
 * [B,S,n_idx_heads,idx_dim], q_scales [B,S,n_idx_heads], k_codes [B,T,idx_dim],
 * k_scales [B,T], w [B,S,n_idx_heads] (dtype), scores [B,S,T] fp32 written in
 * full. Supported: idx_dim 128, dtype DSA_BF16; every relu_mode.
 */
int dsa_index_quant_fp8(const void* x, uint8_t* codes, float* scales, long long rows, int dim,
                        int dtype, hipStream_t stream);
int dsa_index_scores_fp8(const uint8_t* q_codes, const float* q_scales, const uint8_t* k_codes,
                         const float* k_scales, const void* w, float* scores, int B, int S, int T,
                         int past_len, int n_idx_heads, int idx_dim, float scale, int relu_mode,
                         int dtype, hipStream_t stream);

/*
 * Per-query top-k of the score rows ([AXK2] §1: the indexer returns the top
 * index_topk positions as int32 [B,S,topk]; AXK2Config: index_topk, clamped
 * to the number of keys by the caller).
 * indices[b,s,j] lists the topk positions with the largest scores, ordered by
 * score descending and, among equal scores, position ascending (-0.0 equals
 * +0.0). A slot whose score is -inf (a causally invisible key) holds -1.
 * Every row is independent; results are bit-identical from run to run.
 * scores  [B,S,T] fp32, finite or -inf (NaN is outside the contract)
 * indices [B,S,topk] int32
 * 1 <= topk <= min(T, DSA_MAX_TOPK).
 * workspace: at least dsa_topk_workspace_size(...) bytes (may be 0 bytes, in
 * which case workspace may be NULL; the size query returns 0 for sizes the
 * call rejects).
 */
size_t dsa_topk_workspace_size(int B, int S, int T, int topk);
int dsa_topk(const float* scores, int32_t* indices, int B, int S, int T, int topk,
             void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The same selection as dsa_topk ([AXK2] §1) without the final ordering:
 * indices[b,s,0..n) hold the n = min(topk, finite scores in the row)
 * selected positions in an unspecified order that is identical from run to
 * run, and the remaining slots hold -1. The attention calls take index lists
 * as sets, so a layer may use either call; this one skips the sort. Same
 * arguments, limits, workspace (dsa_topk_workspace_size) and status codes as
 * dsa_topk.
 */
int dsa_topk_unsorted(const float* scores, int32_t* indices, int B, int S, int T, int topk,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Indexer and top-k in one call ([AXK2] "Sparse Gated Attention": the
 * indexer's scores exist only to choose each query's index_topk positions).
 * indices[b,s,:] are exactly what dsa_index_scores followed by dsa_topk
 * (sorted = 1) or dsa_topk_unsorted (sorted = 0) return on the same inputs.
 * The scores live in the workspace, and only the causally visible part of
 * each row (t <= past_len + s) is written and read: the -inf upper triangle
 * of the two-call path is neither stored nor scanned.
 * Arguments, limits and status codes: those of dsa_index_scores (without
 * `scores`) and of dsa_topk; `sorted` must be 0 or 1. workspace: at least
 * dsa_index_topk_workspace_size(B, S, T, topk) bytes (B*S*T fp32 scores,
 * then the top-k's own workspace); the size query returns 0 for sizes the
 * call rejects.
 */
size_t dsa_index_topk_workspace_size(int B, int S, int T, int topk);
int dsa_index_topk(const void* q_idx, const void* k_idx, const void* w, int32_t* indices, int B,
                   int S, int T, int past_len, int n_idx_heads, int idx_dim, float scale,
                   int relu_mode, int dtype, int topk, int sorted, void* workspace,
                   size_t workspace_bytes, hipStream_t stream);

/*
 * Sparse MLA attention over the selected expanded K/V rows, prefill
 * ([AXK2] "MLA + explicit sparse mask" steps 3-5: the cache holds expanded
 * K/V; the indexer's positions form an additive mask, combined with the
 * causal mask, so each query attends only to its selected, visible keys;
 * the result is multiplied by a sigmoid gate; [SPARK] steps 2-3: the gate is
 * one scalar per token and head, sigmoid taken in fp32).
 * For each (b, s, h), with Sel = { t in indices[b,s,:] : 0 <= t <= p }:
 *   out[b,s,h,:] = sigmoid(g) * sum_{t in Sel} softmax_t(sm_scale * q.K[t]) V[t]
 * where g = gate[b,s,h] (gate_dim 1) or gate[b,s,h,:] (gate_dim = v_dim), or
 * no gate (gate_dim 0, gate may be NULL). An empty Sel gives 0. Index lists
 * are sets: -1 and out-of-range entries are ignored; a position may appear at
 * most once per row (dsa_topk never repeats one).
 * q [B,S,H,Dqk], k_cache [B,T,H,Dqk], v_cache [B,T,H,Dv], indices
 * [B,S,topk] int32, gate as above, out [B,S,H,Dv]; Dqk = qk_nope_dim +
 * qk_rope_dim. sm_scale > 0 and finite (conventionally Dqk^-1/2).
 * Supported: Dqk and v_dim multiples of 16, at most DSA_MAX_HEAD_DIM;
 * topk <= DSA_MAX_TOPK.
 * workspace: at least dsa_sparse_attn_prefill_workspace_size(...) bytes, with
 * qk_dim = Dqk (a per-query selection bitmap for the MFMA path; per-split
 * partial softmax states when S is small or dtype is fp32).
 */
size_t dsa_sparse_attn_prefill_workspace_size(int B, int S, int T, int H, int qk_dim, int v_dim,
                                              int topk, int dtype);
int dsa_sparse_attn_prefill(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* indices, const void* gate, void* out, int B, int S,
                            int T, int past_len, int H, int qk_nope_dim, int qk_rope_dim,
                            int v_dim, int topk, float sm_scale, int gate_dim, int dtype,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The same attention for one new token per sequence (decode): S = 1 and
 * past_len = T - 1, so every cached key is causally visible.
 * q [B,1,H,Dqk], caches [B,T,H,*], indices [B,1,topk], gate [B,1,H(,Dv)],
 * out [B,1,H,Dv].
 * workspace: at least dsa_sparse_attn_decode_workspace_size(...) bytes
 * (per-split partial softmax states; bf16 calls with B * H >= 256 combine
 * their partial states on chip and leave the workspace untouched, but the
 * required size is the same).
 */
size_t dsa_sparse_attn_decode_workspace_size(int B, int H, int v_dim, int topk);
int dsa_sparse_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* indices, const void* gate, void* out, int B, int T,
                           int H, int qk_nope_dim, int qk_rope_dim, int v_dim, int topk,
                           float sm_scale, int gate_dim, int dtype, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/*
 * Sliding-window attention ([SPARK] sliding_window 512; [PANGU] §3.2: SWA
 * layers see a fixed local window of 512 tokens). Query at p attends to the
 * keys max(0, p-window+1) .. p, then the same gate as above.
 * The K/V buffers may hold only a suffix of the sequence: buffer row j is
 * absolute position kv_offset + j, and T_buf = past_len + S - kv_offset
 * rows are present. kv_offset must satisfy
 *   0 <= kv_offset <= max(0, past_len - window + 1)
 * so that every query's window lies inside the buffer.
 * q [B,S,H,Dqk], k_buf [B,T_buf,H,Dqk], v_buf [B,T_buf,H,Dv], gate, out as
 * above. Both prefill (S > 1) and decode (S = 1) shapes are accepted.
 * workspace: at least swa_attn_workspace_size(...) bytes, with qk_dim = Dqk
 * (0 for the MFMA path: bf16 with S >= 16).
 */
size_t swa_attn_workspace_size(int B, int S, int H, int qk_dim, int v_dim, int window,
                               int dtype);
int swa_attn(const void* q, const void* k_buf, const void* v_buf, const void* gate, void* out,
             int B, int S, int T_buf, int past_len, int kv_offset, int H, int qk_nope_dim,
             int qk_rope_dim, int v_dim, int window, float sm_scale, int gate_dim, int dtype,
             void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Parametric attention sinks ([PANGU] §3.4: every layer learns 128 key-value
 * pairs that absorb redundant attention; at inference they are a fixed set of
 * virtual KV entries, in DSA and SWA layers alike, at negligible cost).
 * The *_pas entry points are the three attention calls above with n_sink
 * extra rows that every query attends to besides its selected (or windowed)
 * keys: the softmax runs over the sinks and those keys together. Sinks carry
 * no position (no causal mask applies to them) and are shared by every
 * sequence of the batch:
 *   sink_k [n_sink,H,Dqk], sink_v [n_sink,H,Dv]   same dtype and head layout
 *                                                 as the caches
 *   0 <= n_sink <= DSA_MAX_SINKS; with n_sink = 0 the pointers may be NULL
 *   and each call equals its plain counterpart.
 * All other arguments, the workspace rule and the errors are those of the
 * plain entry point (with the *_pas_workspace_size functions). An empty
 * selection with n_sink > 0 attends to the sinks alone.
 */
size_t dsa_sparse_attn_prefill_pas_workspace_size(int B, int S, int T, int H, int qk_dim,
                                                  int v_dim, int topk, int n_sink, int dtype);
int dsa_sparse_attn_prefill_pas(const void* q, const void* k_cache, const void* v_cache,
                                const void* sink_k, const void* sink_v, int n_sink,
                                const int32_t* indices, const void* gate, void* out, int B, int S,
                                int T, int past_len, int H, int qk_nope_dim, int qk_rope_dim,
                                int v_dim, int topk, float sm_scale, int gate_dim, int dtype,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);
size_t dsa_sparse_attn_decode_pas_workspace_size(int B, int H, int v_dim, int topk, int n_sink);
int dsa_sparse_attn_decode_pas(const void* q, const void* k_cache, const void* v_cache,
                               const void* sink_k, const void* sink_v, int n_sink,
                               const int32_t* indices, const void* gate, void* out, int B, int T,
                               int H, int qk_nope_dim, int qk_rope_dim, int v_dim, int topk,
                               float sm_scale, int gate_dim, int dtype, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);
size_t swa_attn_pas_workspace_size(int B, int S, int H, int qk_dim, int v_dim, int window,
                                   int n_sink, int dtype);
int swa_attn_pas(const void* q, const void* k_buf, const void* v_buf, const void* sink_k,
                 const void* sink_v, int n_sink, const void* gate, void* out, int B, int S,
                 int T_buf, int past_len, int kv_offset, int H, int qk_nope_dim, int qk_rope_dim,
                 int v_dim, int window, float sm_scale, int gate_dim, int dtype, void* workspace,
                 size_t workspace_bytes, hipStream_t stream);

/*
 * Sliding-window attention with grouped KV heads ([SPARK] "为什么要加这一层门控":
 * 8 query heads share 2 KV heads, head_dim 256, sliding_window 512, one
 * sigmoid gate per head). swa_attn with caches that hold H_kv heads:
 *   k_buf [B,T_buf,H_kv,Dqk], v_buf [B,T_buf,H_kv,Dv]; q, gate, out as in
 *   swa_attn with H query heads.
 * Query head h reads cache head h / (H / H_kv): consecutive query heads form
 * the groups. 1 <= H_kv <= H and H_kv must divide H (else
 * DSA_ERR_INVALID_ARG); H_kv = H is swa_attn. All other arguments, the
 * workspace rule and the errors are those of swa_attn (workspace from
 * swa_attn_gqa_workspace_size, which takes the query head count).
 */
size_t swa_attn_gqa_workspace_size(int B, int S, int H, int qk_dim, int v_dim, int window,
                                   int dtype);
int swa_attn_gqa(const void* q, const void* k_buf, const void* v_buf, const void* gate, void* out,
                 int B, int S, int T_buf, int past_len, int kv_offset, int H, int H_kv,
                 int qk_nope_dim, int qk_rope_dim, int v_dim, int window, float sm_scale,
                 int gate_dim, int dtype, void* workspace, size_t workspace_bytes,
                 hipStream_t stream);

/*
 * The indexer's projections, in front of dsa_index_scores ([AXK2] §1 SGA: the
 * indexer's own light projections, wq_b on the query LoRA bottleneck, wk
 * followed by a LayerNorm (k_norm) on the key, per-head weights from
 * weights_proj, and its own key cache appended to by update_indexer; [AXK2]
 * "two RoPE layouts": the indexer's rotary embedding is non-interleaved,
 * half-split). For the S tokens of a call (positions past_len + s):
 *   q_idx[b,s,h,:] = RoPE_p((q_lora[b,s,:] . wq_b^T)[h * idx_dim ...])
 *   k_idx_cache[b, past_len + s, :] = RoPE_p(LayerNorm(hidden[b,s,:] . wk^T))
 *   w[b,s,:] = hidden[b,s,:] . weights_proj^T
 * Weights use the nn.Linear layout [out_features, in_features]:
 *   wq_b [n_idx_heads * idx_dim, q_lora_rank], wk [idx_dim, hidden_dim],
 *   weights_proj [n_idx_heads, hidden_dim], k_norm_weight / k_norm_bias
 *   [idx_dim] (LayerNorm with mean and biased variance over idx_dim, ln_eps).
 * RoPE acts on the last rope_dim dims of each index head and of the key
 * (rope_dim even, 0 = none): with half = rope_dim / 2 and j < half, the pair
 * (x_j, x_{j+half}) of that slice becomes (x_j c - x_{j+half} s,
 * x_{j+half} c + x_j s), c = rope_cos[p * half + j], s = rope_sin[p * half + j]
 * (fp32 tables [T, half]: the caller's frequency schedule).
 * q_lora [B,S,q_lora_rank], hidden [B,S,hidden_dim], q_idx [B,S,n_idx_heads,
 * idx_dim], k_idx_cache [B,T,idx_dim] (rows past_len .. past_len + S - 1 are
 * written), w [B,S,n_idx_heads]; all bf16 (dtype DSA_BF16; DSA_F32 is
 * DSA_ERR_UNSUPPORTED). The key projection is rounded to bf16 before its
 * LayerNorm, as the page's bf16 modules do; LayerNorm and RoPE compute in
 * fp32. q_idx is rounded once, after its RoPE, when rope_dim is 32 or 64 (the
 * GEMM applies it), else rounded and then rotated.
 * Supported: idx_dim 64 or 128; q_lora_rank and hidden_dim multiples of 32.
 * workspace: at least dsa_indexer_prologue_workspace_size(B, S, idx_dim)
 * bytes (the key projection before its LayerNorm).
 */
size_t dsa_indexer_prologue_workspace_size(int B, int S, int idx_dim);
int dsa_indexer_prologue(const void* q_lora, const void* hidden, const void* wq_b, const void* wk,
                         const void* k_norm_weight, const void* k_norm_bias,
                         const void* weights_proj, const float* rope_cos, const float* rope_sin,
                         void* q_idx, void* k_idx_cache, void* w, int B, int S, int T,
                         int past_len, int q_lora_rank, int hidden_dim, int n_idx_heads,
                         int idx_dim, int rope_dim, float ln_eps, int dtype, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/*
 * The main attention's projections, in front of the sparse attention calls
 * ([AXK2] "MLA + explicit sparse mask" steps 1-3: q_gate_proj produces the
 * query and the attention output gate together, kv_a_proj_with_mqa
 * compresses K/V to the kv_lora_rank latent plus one RoPE key shared by all
 * heads, expand_kv expands the latent into the full per-head K/V that the
 * caches hold; "Attention output gate": the fused projection reads
 * [q_resid, q_compressed] and splits its output into a qk_head_dim query and
 * a v_head_dim gate; "two RoPE layouts": the main attention's rotary layout
 * is interleaved). For the S tokens of a call (positions past_len + s), with
 * Dqk = qk_nope_dim + qk_rope_dim (N + R):
 *   [qry_h | gate_h]      = ([q_resid, q_compressed] . wq_gate^T)[h*(Dqk+Dv) ...]
 *   [latent | rope key]   = hidden . wkv_a^T
 *   [k_nope_h | v_h]      = (latent . wkv_b^T)[h*(N+Dv) ...]
 *   q[b,s,h,:]                    = [qry_h[:N] | RoPE_p(qry_h[N:])]
 *   gate[b,s,h,:]                 = gate_h        (use gate_dim = v_dim)
 *   k_cache[b,past_len+s,h,:]     = [k_nope_h | RoPE_p(rope key)]
 *   v_cache[b,past_len+s,h,:]     = v_h
 * RoPE_p rotates each interleaved pair (x_2j, x_2j+1) of a rope slice to
 * (x_2j c - x_2j+1 s, x_2j+1 c + x_2j s), c = rope_cos[p * R/2 + j],
 * s = rope_sin[p * R/2 + j] (fp32 tables [T, R/2], the caller's schedule).
 * Weights use the nn.Linear layout [out, in]: wq_gate [H*(Dqk+v_dim),
 * q_resid_dim + q_comp_dim], wkv_a [kv_lora_rank + R, hidden_dim], wkv_b
 * [H*(N+v_dim), kv_lora_rank]. q_resid [B,S,q_resid_dim], q_compressed
 * [B,S,q_comp_dim], hidden [B,S,hidden_dim]; q [B,S,H,Dqk], gate
 * [B,S,H,v_dim], k_cache [B,T,H,Dqk], v_cache [B,T,H,v_dim] (rows past_len ..
 * past_len + S - 1 are written, no other). All bf16 (DSA_F32 is
 * DSA_ERR_UNSUPPORTED); each projection is accumulated in fp32 and rounded
 * once to bf16, after its RoPE where it has one. No normalisation sits between
 * kv_a_proj_with_mqa and expand_kv (none is named on the page).
 * Supported: q_resid_dim, q_comp_dim, hidden_dim, kv_lora_rank multiples of
 * 32; N, R, v_dim multiples of 16 with N + R and v_dim at most
 * DSA_MAX_HEAD_DIM (R = 0: no RoPE, the tables may be NULL).
 * workspace: at least dsa_mla_prologue_workspace_size(B, S, kv_lora_rank)
 * bytes (the latent).
 */
size_t dsa_mla_prologue_workspace_size(int B, int S, int kv_lora_rank);
int dsa_mla_prologue(const void* q_resid, const void* q_compressed, const void* hidden,
                     const void* wq_gate, const void* wkv_a, const void* wkv_b,
                     const float* rope_cos, const float* rope_sin, void* q, void* gate,
                     void* k_cache, void* v_cache, int B, int S, int T, int past_len,
                     int q_resid_dim, int q_comp_dim, int hidden_dim, int kv_lora_rank, int H,
                     int qk_nope_dim, int qk_rope_dim, int v_dim, int dtype, void* workspace,
                     size_t workspace_bytes, hipStream_t stream);

/*
 * The work plan the MFMA prefill path (bf16, S >= 16) launches for a call
 * with these sizes, for inspection; host arithmetic only, no GPU call. A
 * query tile is 128 consecutive queries; tile qt sees the 64-key blocks of
 * its causal range (DSA, window <= 0) or of its window range. When the grid
 * would be small, long tiles are split into work items of at most
 * *max_blocks blocks each (*max_blocks = INT_MAX when nothing is split).
 * Outputs: *n_tiles, *n_items (workgroups per head and batch row) and, when
 * cap >= *n_tiles + 1 and item_start is not NULL, item_start[o] = the first
 * item of the o-th longest tile (tile n_tiles - 1 - o), item_start[n_tiles] =
 * n_items (items of a tile are its consecutive key ranges, first to last).
 * The prefill workspace is sized from the plan of past_len = T - S, which
 * has the most items any call with this T can have.
 * A selection-mask call (window <= 0) without sinks whose plan splits
 * nothing, with qk dim <= 192 and v dim <= 128, runs instead as 256-query
 * tiles (two 128-query halves per workgroup, same key ranges) when
 * B * H * ceil(S / 256) >= 1024; this function reports the 128-query plan,
 * whose tile ranges those workgroups cover in pairs.
 * Returns DSA_OK, or DSA_ERR_INVALID_ARG for null outputs or bad sizes.
 */
int dsa_prefill_work_plan(int B, int S, int T, int past_len, int H, int kv_offset, int window,
                          int* n_tiles, int* n_items, int* max_blocks, int* item_start, int cap);

/*
 * dsa_sparse_attn_decode without a workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Arguments, layouts, results and status
 * codes are those of dsa_sparse_attn_decode minus the workspace; the split
 * partial states live in a static device buffer of DSA_STATIC_SCRATCH_BYTES
 * that the library holds on every GPU it runs on until the process ends (its
 * address is looked up once per device; no call allocates or frees memory).
 * A call whose partial states need more than that buffer (see
 * dsa_sparse_attn_decode_workspace_size) returns DSA_ERR_UNSUPPORTED. Every
 * call on one GPU uses the same buffer: calls that may overlap on one GPU
 * (different streams, or host threads) race and must be ordered by the
 * caller. Each call writes all the scratch it reads, so nothing carries over
 * from the previous call.
 */
#define DSA_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
int dsa_sparse_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* indices, const void* gate, void* out, int B,
                                   int T, int H, int qk_nope_dim, int qk_rope_dim, int v_dim,
                                   int topk, float sm_scale, int gate_dim, int dtype,
                                   hipStream_t stream);

/* Debug builds. libdsa_debug.so is the same library compiled with
 * -DDSA_DEBUG: its kernels also check the invariants they rely on (indices
 * inside their buffers, the number of keys a selection must hold, work items
 * inside the launch plan). A failed check does not stop the kernel; it is
 * counted in device memory, and every call of a debug build then
 * synchronizes the device (so it must not be captured into a graph) and
 * returns DSA_ERR_CHECK, with dsa_last_error() naming the source file, line
 * and two values of the first failure. Outputs of a debug build are
 * bit-identical to the release build's. Returns 1 in a debug build, else 0.
 * Callers: tests and tools that want the checks; production code links the
 * release build. */
int dsa_debug_build(void);

/* Text of a status code (static storage). */
const char* dsa_status_string(int status);
/* Message of the last failed call on this thread ("" if none). */
const char* dsa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H_ */
