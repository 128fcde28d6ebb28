"""The workloads, as shapes plus the distribution of every input tensor.

Every tensor is drawn from the seeded generator in this package: a normal
N(0, scale^2) stream keyed by (seed, tensor id). Seed = workload number - 1.

  tiny-fp32     B 1, S = T = 256 causal prefill; 4 heads (nope 32, rope 16,
                v 32); indexer 2 heads x 32; top-k 64; fp32; all N(0,1),
                index weights / sqrt(2), gate logits N(0,1).
  mla-s4k       B 1, S = T = 4096; 20 heads (64, 64, v 128); indexer 4 x 64;
                top-k 512; bf16; every tensor N(0,1) / sqrt(d) where d is its
                innermost size (q, K: 128; V: 128; q_idx, k_idx: 64), index
                weights / sqrt(4); gate logits unscaled N(0,1).
  dsa-s32k      B 1, S = T = 32768; 128 heads (128, 64, v 128); indexer 64 x
                128; top-k 2048; bf16; N(0,1), index weights / sqrt(64), gate
                logits N(0,1).
  decode-b8     B 8 x 131072 cached tokens, one new query each (S 1, past_len
                131071); heads and indexer as dsa-s32k; top-k 2048.
  hybrid-512k   B 1; 524288 cached tokens; DSA layer with 32 heads (128, 64,
                v 128), indexer 32 x 128, top-k 2048; two SWA layers, window
                512; a 4096-token chunk (past_len 524288) then one decode
                token (position 528384); index weights / sqrt(32).
  mla-s4k-pas, hybrid-512k-pas
                the same with 128 attention sinks per layer (sink K/V drawn
                like the cache's K/V, tensor ids 10 and 11).
  dsa-s32k-fp8  dsa-s32k with the FP8 indexer: q_idx and k_idx are rotated and
                quantised to E4M3 codes every step, then scored from the codes.
  prologue-s32k the indexer's projections (wq_b from a 1536-wide query
                bottleneck, wk + LayerNorm and weights_proj from a 7168-wide
                hidden state, RoPE on 64 dims) for 32768 tokens; inputs N(0,1),
                weights N(0,1) / sqrt(fan-in), LayerNorm weight N(0,1) and
                bias N(0,1) / 10, RoPE angles p * 10000^(-2j/64).
  mla-prologue-s32k
                the main attention's projections for the dsa-s32k tokens and
                heads: q_gate_proj on [q_resid 1536, q_compressed 1536] to 128
                heads of (query 192, gate 128), kv_a_proj_with_mqa from a
                7168-wide hidden state to a 512-wide latent and the 64-dim
                rope key, expand_kv to (k_nope 128, v 128) per head,
                interleaved RoPE with angles p * 10000^(-2j/64); inputs
                N(0,1), weights N(0,1) / sqrt(fan-in), tensor ids 40-45.
  spark-swa     one sliding-window layer with grouped KV heads (Spark-X2.5
                page: 8 query heads over 2 KV heads, head_dim 256, window 512,
                one gate logit per head): a 4096-token chunk after 131072
                cached tokens, then one decode token; the K/V buffers hold
                the window suffix only. N(0,1) inputs.

Element (b, t, h, d) of a cache is element ((b*T_alloc + t)*H + h)*D + d of
its stream, so a window buffer starting at absolute position kv_offset is the
stream from kv_offset*H*D on (B = 1).
"""
from __future__ import annotations

import math
import dataclasses
from dataclasses import dataclass

F32, BF16 = 0, 1


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: int
    B: int
    S: int
    past_len: int
    H: int
    nope: int
    rope: int
    v: int
    HI: int
    DI: int
    topk: int
    seed: int
    window: int = 512
    n_swa: int = 0            # SWA layers in the stack (hybrid: 2)
    decode_after: bool = False  # hybrid: one decode token after the chunk
    n_sink: int = 0            # attention sinks per layer (PAS), shared by the batch
    H_kv: int = 0              # KV heads of grouped-KV SWA layers (0: H)
    swa_only: bool = False     # one SWA layer and no DSA stages
    idx_fp8: bool = False      # indexer on FP8 codes (Hadamard rotation + E4M3)
    prologue_only: bool = False  # the indexer's projections alone
    q_lora: int = 0            # query LoRA rank (prologue input width)
    hidden: int = 0            # hidden size (prologue input width)
    rope_idx: int = 0          # rotary dims of each index head and key
    mla_prologue_only: bool = False  # the main attention's projections alone
    q_comp: int = 0            # q_compressed width (the second q_gate_proj input)
    kv_lora: int = 0           # kv_lora_rank (the latent of kv_a_proj_with_mqa)
    scale_q: float = 1.0
    scale_k: float = 1.0
    scale_v: float = 1.0
    scale_qidx: float = 1.0
    scale_kidx: float = 1.0
    scale_w: float = 1.0
    scale_gate: float = 1.0
    notes: str = ""

    @property
    def T(self) -> int:
        return self.past_len + self.S

    @property
    def Dqk(self) -> int:
        return self.nope + self.rope

    @property
    def dtype_name(self) -> str:
        return "f32" if self.dtype == F32 else "bf16"


WORKLOADS = {
    "tiny-fp32": Workload("tiny-fp32", F32, B=1, S=256, past_len=0, H=4, nope=32, rope=16, v=32,
                          HI=2, DI=32, topk=64, seed=0, scale_w=1 / math.sqrt(2)),
    "mla-s4k": Workload("mla-s4k", BF16, B=1, S=4096, past_len=0, H=20, nope=64, rope=64, v=128,
                        HI=4, DI=64, topk=512, seed=1, scale_q=1 / math.sqrt(128),
                        scale_k=1 / math.sqrt(128), scale_v=1 / math.sqrt(128),
                        scale_qidx=1 / 8.0, scale_kidx=1 / 8.0, scale_w=0.5),
    "dsa-s32k": Workload("dsa-s32k", BF16, B=1, S=32768, past_len=0, H=128, nope=128, rope=64,
                         v=128, HI=64, DI=128, topk=2048, seed=2, scale_w=1 / 8.0),
    "decode-b8": Workload("decode-b8", BF16, B=8, S=1, past_len=131071, H=128, nope=128, rope=64,
                          v=128, HI=64, DI=128, topk=2048, seed=3, scale_w=1 / 8.0),
    "hybrid-512k": Workload("hybrid-512k", BF16, B=1, S=4096, past_len=524288, H=32, nope=128,
                            rope=64, v=128, HI=32, DI=128, topk=2048, seed=4, n_swa=2,
                            decode_after=True, scale_w=1 / math.sqrt(32)),
}
# The same layers with 128 parametric attention sinks per layer (openPangu-2.0
# page §3.4: 128 learnable KV pairs in every DSA and SWA layer).
WORKLOADS["mla-s4k-pas"] = dataclasses.replace(WORKLOADS["mla-s4k"], name="mla-s4k-pas",
                                               n_sink=128)
WORKLOADS["hybrid-512k-pas"] = dataclasses.replace(WORKLOADS["hybrid-512k"],
                                                   name="hybrid-512k-pas", n_sink=128)

# The dsa-s32k layer with the FP8 indexer (A.X-K2 page implementation notes):
# q_idx and the chunk's k_idx rows are rotated and quantised every step.
WORKLOADS["dsa-s32k-fp8"] = dataclasses.replace(WORKLOADS["dsa-s32k"], name="dsa-s32k-fp8",
                                                idx_fp8=True)
# The indexer's projections for the dsa-s32k tokens: wq_b on a 1536-wide query
# bottleneck, wk + LayerNorm and weights_proj on a 7168-wide hidden state
# (DeepSeek-V3-sized synthetic shapes), half-split RoPE on 64 of the 128 dims.
WORKLOADS["prologue-s32k"] = Workload("prologue-s32k", BF16, B=1, S=32768, past_len=0, H=0, nope=0,
                                      rope=0, v=0, HI=64, DI=128, topk=0, seed=6,
                                      prologue_only=True, q_lora=1536, hidden=7168, rope_idx=64)
# The main attention's projections for the dsa-s32k tokens and heads:
# q_gate_proj on [q_resid (1536), q_compressed (1536)], kv_a_proj_with_mqa from
# a 7168-wide hidden state to a 512-wide latent plus the 64-dim rope key,
# expand_kv to 128 heads of (nope 128, v 128); interleaved RoPE on 64 dims.
WORKLOADS["mla-prologue-s32k"] = Workload("mla-prologue-s32k", BF16, B=1, S=32768, past_len=0, H=128,
                                          nope=128, rope=64, v=128, HI=0, DI=0, topk=0, seed=7,
                                          mla_prologue_only=True, q_lora=1536, q_comp=1536,
                                          hidden=7168, kv_lora=512)
WORKLOADS["spark-swa"] = Workload("spark-swa", BF16, B=1, S=4096, past_len=131072, H=8, nope=128,
                                  rope=128, v=256, HI=0, DI=0, topk=0, seed=5, n_swa=1,
                                  decode_after=True, H_kv=2, swa_only=True)

ORDER = ["tiny-fp32", "mla-s4k", "dsa-s32k", "decode-b8", "hybrid-512k", "mla-s4k-pas",
         "hybrid-512k-pas", "spark-swa", "dsa-s32k-fp8", "prologue-s32k", "mla-prologue-s32k"]
