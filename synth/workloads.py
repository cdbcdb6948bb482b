"""Parameter lists and run settings of the five synthetic workloads.

Shapes only: these are the model *shapes* the shard step is exercised on
(no weights, no data).  Registration order is the order listed; the bucket
planner visits them in reverse (gradients of later layers are ready first in
backward: "Parallelisms", section Data parallel).

  tiny_mlp      2-layer MLP, 525,568 params, 1 MiB buckets, N=2, R=2, 10 steps
  gpt2_small    GPT-2-small shape (12 x d768, ffn 3072, vocab 50257, tied
                head), 124,439,808 params, 25 MiB buckets, ZeRO-2 shard N=8, R=8
  llama3_8b     Llama-3-8B shape (32 x d4096, ffn 14336, GQA 32q/8kv x 128,
                vocab 128256, untied head), 8,030,261,248 params, 25 MiB
                buckets, ZeRO-3 shard N=8, R=8
  gpt_7b5       "7.5B"-labelled GPT shape (32 x d4096, ffn 16384, vocab 50000,
                tied head; the dims give 6,648,963,072 params), shard N=64,
                R=8, 4 microbatches, valid-token normalisation
  llama3_8b_dp  llama3_8b as a full DP replica (N=1), R=2, pack + step
"""

from dataclasses import dataclass, field
from math import prod


@dataclass(frozen=True)
class AdamW:
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01


@dataclass(frozen=True)
class Workload:
    name: str
    params: tuple  # ((name, shape), ...) in registration order
    bucket_cap_bytes: int
    world_n: int  # shard divisor N
    R: int  # gradient contributions reduced into the shard
    K: int = 1  # microbatches
    norm: str = "mean"  # "mean" (1/(R*K)) or "tokens" (1/sum of valid tokens)
    grad_sigma: float = 1e-3
    master_sigma: float = 0.02
    steps: int = 1
    shard_index: int = 0
    pack: bool = False  # rank 0's contribution comes from packing per-tensor grads
    adamw: AdamW = field(default_factory=AdamW)

    @property
    def numels(self):
        return [int(prod(s)) for _, s in self.params]

    @property
    def names(self):
        return [n for n, _ in self.params]

    @property
    def psi(self):
        return sum(self.numels)


def _mlp():
    return (("W1", (256, 1024)), ("b1", (1024,)), ("W2", (1024, 256)), ("b2", (256,)))


def _gpt2_small(d=768, ffn=3072, vocab=50257, ctx=1024, layers=12):
    p = [("wte", (vocab, d)), ("wpe", (ctx, d))]
    for i in range(layers):
        h = f"h{i}"
        p += [
            (f"{h}.ln_1.w", (d,)), (f"{h}.ln_1.b", (d,)),
            (f"{h}.attn.c_attn.w", (d, 3 * d)), (f"{h}.attn.c_attn.b", (3 * d,)),
            (f"{h}.attn.c_proj.w", (d, d)), (f"{h}.attn.c_proj.b", (d,)),
            (f"{h}.ln_2.w", (d,)), (f"{h}.ln_2.b", (d,)),
            (f"{h}.mlp.c_fc.w", (d, ffn)), (f"{h}.mlp.c_fc.b", (ffn,)),
            (f"{h}.mlp.c_proj.w", (ffn, d)), (f"{h}.mlp.c_proj.b", (d,)),
        ]
    p += [("ln_f.w", (d,)), ("ln_f.b", (d,))]
    return tuple(p)


def _llama3_8b(d=4096, ffn=14336, heads=32, kv_heads=8, head_dim=128,
               vocab=128256, layers=32):
    kv = kv_heads * head_dim
    p = [("embed", (vocab, d))]
    for i in range(layers):
        l = f"l{i}"
        p += [
            (f"{l}.attn_norm", (d,)), (f"{l}.q", (heads * head_dim, d)),
            (f"{l}.k", (kv, d)), (f"{l}.v", (kv, d)), (f"{l}.o", (d, heads * head_dim)),
            (f"{l}.mlp_norm", (d,)), (f"{l}.gate", (ffn, d)), (f"{l}.up", (ffn, d)),
            (f"{l}.down", (d, ffn)),
        ]
    p += [("final_norm", (d,)), ("lm_head", (vocab, d))]
    return tuple(p)


def _gpt_7b5(d=4096, ffn=16384, vocab=50000, layers=32):
    p = [("wte", (vocab, d))]
    for i in range(layers):
        l = f"l{i}"
        p += [
            (f"{l}.ln1.w", (d,)), (f"{l}.ln1.b", (d,)),
            (f"{l}.qkv.w", (3 * d, d)), (f"{l}.qkv.b", (3 * d,)),
            (f"{l}.proj.w", (d, d)), (f"{l}.proj.b", (d,)),
            (f"{l}.ln2.w", (d,)), (f"{l}.ln2.b", (d,)),
            (f"{l}.fc1.w", (ffn, d)), (f"{l}.fc1.b", (ffn,)),
            (f"{l}.fc2.w", (d, ffn)), (f"{l}.fc2.b", (d,)),
        ]
    p += [("ln_f.w", (d,)), ("ln_f.b", (d,))]
    return tuple(p)


MiB = 1 << 20

WORKLOADS = {
    "tiny_mlp": Workload("tiny_mlp", _mlp(), 1 * MiB, world_n=2, R=2,
                         grad_sigma=1e-2, steps=10),
    "gpt2_small": Workload("gpt2_small", _gpt2_small(), 25 * MiB, world_n=8, R=8),
    "llama3_8b": Workload("llama3_8b", _llama3_8b(), 25 * MiB, world_n=8, R=8),
    "gpt_7b5": Workload("gpt_7b5", _gpt_7b5(), 25 * MiB, world_n=64, R=8, K=4,
                        norm="tokens"),
    "llama3_8b_dp": Workload("llama3_8b_dp", _llama3_8b(), 25 * MiB, world_n=1,
                             R=2, pack=True),
}

# valid-token counts per rank and step are uniform integers on this range
TOKENS_LO, TOKENS_HI = 1000, 4000

SEED = 20260101
