// kernels.h -- host launchers of the libdsa kernels. Arguments are validated
// by the C-ABI layer (abi.cpp) before any of these is called.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

// Lightning-indexer scores (index_scores.hip).
// fill_masked = false leaves the entries above each row's causal bound
// (t > past_len + s) unwritten, for callers that read only t <= past_len + s.
hipError_t launch_index_scores(const void* q_idx, const void* k_idx, const void* w, float* scores,
                               int B, int S, int T, int past_len, int HI, int DI, float scale,
                               int relu_mode, int dtype, hipStream_t stream,
                               bool fill_masked = true);

// FP8 indexer (index_fp8.hip): Hadamard rotation + E4M3 codes with one
// power-of-two scale per row (dim 32, 64 or 128, bf16 input); scores from
// the codes (idx_dim 128, bf16 weights).
hipError_t launch_quant_fp8(const void* x, uint8_t* codes, float* scales, int64_t rows, int dim,
                            hipStream_t stream);
hipError_t launch_index_scores_fp8(const uint8_t* q_codes, const float* q_scales,
                                   const uint8_t* k_codes, const float* k_scales, const void* w,
                                   float* scores, int B, int S, int T, int P, int HI, int DI,
                                   float scale, int relu_mode, hipStream_t stream);

// Indexer prologue (prologue.hip): bf16 GEMM with nn.Linear weights
// (C = A W^T, K % 32 == 0), then RoPE / LayerNorm + RoPE + cache append.
hipError_t launch_gemm_bf16(const void* A, const void* W, void* C, int M, int N, int K, int ldc,
                            hipStream_t stream);
hipError_t launch_indexer_prologue(const void* q_lora, const void* hidden, const void* wq_b,
                                   const void* wk, const void* k_norm_weight,
                                   const void* k_norm_bias, const void* weights_proj,
                                   const float* rope_cos, const float* rope_sin, void* q_idx,
                                   void* k_idx_cache, void* w, int B, int S, int T, int past_len,
                                   int q_lora_rank, int hidden_dim, int HI, int DI, int R,
                                   float eps, void* workspace, hipStream_t stream);

// The main attention's projections (prologue.hip): kv_a_proj_with_mqa (latent
// into the workspace [B*S, L] bf16, rotated rope key into every head's cache
// row), expand_kv (k_nope and v into the cache rows), q_gate_proj on
// [q_resid, q_comp] (query with its rope slice rotated, gate). Widths: Qr, Qc,
// Hd, L multiples of 32; N, R, Dv multiples of 16.
hipError_t launch_mla_prologue(const void* q_resid, const void* q_comp, const void* hidden,
                               const void* wq_gate, const void* wkv_a, const void* wkv_b,
                               const float* rope_cos, const float* rope_sin, void* q, void* gate,
                               void* k_cache, void* v_cache, int B, int S, int T, int past_len,
                               int Qr, int Qc, int Hd, int L, int H, int N, int R, int Dv,
                               void* workspace, hipStream_t stream);

// Per-row top-k (topk.hip).
size_t topk_workspace_bytes(int B, int S, int T, int topk);
// order 0: by score descending (ties: lower position first); 1: the same
// selection unsorted (a fixed, repeatable order), -1 slots last. causal_P >= 0:
// row r = b S + s holds only min(T, causal_P + s + 1) valid scores (the rest
// of its T are never read), which selects exactly what -inf there would.
hipError_t launch_topk(const float* scores, int32_t* indices, int B, int S, int T, int topk,
                       void* workspace, hipStream_t stream, int order = 0, int causal_P = -1);

// Selection bitmap + MFMA flash attention with a bitmap or window mask
// (attn_prefill.hip). Requires bf16 and a (Dqk, Dv) pair that
// prefill_mfma_supported accepts. The caches hold Hkv heads; query head h
// reads cache head h / (H / Hkv) (Hkv divides H; Hkv = H for expanded K/V).
size_t bitmap_bytes(int B, int S, int T);
size_t prefill_mfma_workspace_bytes(int B, int S, int T, int H, int Dv);
// sink_k [n_sink,Hkv,Dqk] / sink_v [n_sink,Hkv,Dv]: attention sinks every query
// attends to (n_sink may be 0, then the pointers are unused).
hipError_t launch_prefill_mfma(const void* q, const void* k, const void* v, const void* sink_k,
                               const void* sink_v, int n_sink, const int32_t* indices,
                               const void* gate, void* out, int B, int S, int T, int past_len,
                               int kv_offset, int H, int Hkv, int Dqk, int Dv, int topk,
                               int window, float sm_scale, int gate_dim, void* workspace,
                               hipStream_t stream);
bool prefill_mfma_supported(int dtype, int S, int Dqk, int Dv);
// The launch plan of launch_prefill_mfma (host only): query tiles, work items,
// blocks per item, and the first item of each tile (longest tile first) when
// cap allows; returns false if the table does not fit (tiles are not split).
void prefill_work_plan(int B, int S, int T, int P, int H, int kv_offset, int window, int* n_tiles,
                       int* n_items, int* max_blocks, int* item_start, int cap);

// Split-K row-gather attention + merge (attn_gather.hip); any dtype, any S.
// window > 0 selects the implicit window list, else `indices` is used; the
// n_sink sink rows are entries in front of that list. Cache heads as above.
size_t gather_workspace_bytes(int64_t rows, int H, int Dv, int64_t nentries);
hipError_t launch_gather(const void* q, const void* k, const void* v, const void* sink_k,
                         const void* sink_v, int n_sink, const int32_t* indices,
                         const void* gate, void* out, int B, int S, int T, int past_len,
                         int kv_offset, int H, int Hkv, int Dqk, int Dv, int topk, int window,
                         float sm_scale, int gate_dim, int dtype, void* workspace,
                         hipStream_t stream);

// Static device scratch (scratch.hip) for dsa_sparse_attn_decode_noalloc:
// kStaticScratchBytes per GPU, held from module load to process exit. Returns
// the current device's address of it (looked up once per device).
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
hipError_t static_scratch(void** ptr);

// Device-side checks of -DDSA_DEBUG builds (common.h: DSA_CHECK). Each kernel
// file keeps one record in device memory: the number of failed checks since it
// was last read, and the first failure's source line and two values.
struct DebugRecord {
  unsigned int count;
  int line;
  long long a, b;
};
#ifdef DSA_DEBUG
// Copy a file's record to *out and clear it (synchronous). Returns 1 if a
// check failed, 0 if none did, -1 if the copy failed.
int debug_take_attn_gather(DebugRecord* out);
int debug_take_attn_prefill(DebugRecord* out);
int debug_take_index_fp8(DebugRecord* out);
int debug_take_index_scores(DebugRecord* out);
int debug_take_prologue(DebugRecord* out);
int debug_take_topk(DebugRecord* out);
#endif

}  // namespace dsa
