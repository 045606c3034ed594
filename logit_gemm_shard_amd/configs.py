"""The workloads the library is checked and measured on.

Each entry names one tensor-parallel rank's unit of work at the shapes of a
model the pages discuss: the 8.3B-parameter GPT-style model trained with an
8-way split and a 51,200-entry padded vocabulary ("LIT-022: Megatron-LM ...",
dmarx anthology, "Key takeaways"), and a 70B dense decoder with hidden size
8,192 at sequence length 4,096 and micro-batch 1 ("Megatron-LM, in depth",
aicassindra, "Worked example: 70B parameters on 512 GPUs").

The attention projections are those of Llama-3-70B as that page gives them
("The Multi-Head Attention Block"): 64 query heads and 8 key/value heads, 8
and 1 per rank at t = 8, head size 8,192 / 64 = 128.

The gated (SwiGLU) MLP block is that of Llama-3-70B, hidden size 8,192, as the
mohashari.github.io page on tensor parallelism for fine-tuning 70B models with
Megatron-LM describes it ("The MLP Block"; sequence length 4,096 and batch
size 1 in its introduction), with the inner width 28,672 of the 70B GeLU
workload, split 8 ways.

Initialisation follows the same "Key takeaways": N(0, 0.02) (standard
deviation 0.02) for every weight, and the weight just before each residual
(here the row-parallel B) scaled by 1/sqrt(2N), N the number of attention plus
MLP blocks.
"""

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "mlp_fwd" | "mlp_bwd" | "xent" | "swiglu_fwd" | "swiglu_bwd" | "attn"
    b: int
    s: int
    h: int
    t: int
    dtype: str           # "f32" | "bf16"
    seed: int
    ffn: int = 0         # MLP inner width (all ranks)
    vocab: int = 0       # padded vocabulary (all ranks)
    n_blocks: int = 0    # N of the 1/sqrt(2N) residual scaling
    dz_seed: int = 0     # backward: seed of the incoming gradient
    dz_std: float = 0.0  # backward: its standard deviation
    n_heads: int = 0     # attention: query heads (all ranks)
    n_kv_heads: int = 0  # attention: key/value heads (all ranks)
    head_dim: int = 0
    note: str = field(default="", compare=False)

    @property
    def M(self):
        return self.b * self.s

    @property
    def f_i(self):
        return self.ffn // self.t

    @property
    def v_r(self):
        return self.vocab // self.t


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_mlp_t2_f32", "mlp_fwd", b=2, s=64, h=256, t=2, dtype="f32", seed=1,
                 ffn=1024, n_blocks=2,
                 note="tiny GeLU MLP block, both shards run and summed, fp32"),
        Workload("mlp_8p3b_fwd", "mlp_fwd", b=8, s=1024, h=3072, t=8, dtype="bf16", seed=2,
                 ffn=12288, n_blocks=144,
                 note="8.3B-shape MLP shard forward, one rank of t=8"),
        Workload("xent_8p3b", "xent", b=8, s=1024, h=3072, t=8, dtype="bf16", seed=3,
                 vocab=51200,
                 note="vocab-parallel fused cross-entropy, one rank of t=8"),
        Workload("mlp_70b_fwd", "mlp_fwd", b=1, s=4096, h=8192, t=8, dtype="bf16", seed=4,
                 ffn=28672, n_blocks=160,
                 note="70B-shape GeLU MLP shard forward, one rank of t=8"),
        Workload("mlp_70b_bwd", "mlp_bwd", b=1, s=4096, h=8192, t=8, dtype="bf16", seed=4,
                 ffn=28672, n_blocks=160, dz_seed=5, dz_std=0.01,
                 note="70B-shape MLP shard backward, one rank of t=8"),
        Workload("swiglu_70b_fwd", "swiglu_fwd", b=1, s=4096, h=8192, t=8, dtype="bf16", seed=6,
                 ffn=28672, n_blocks=160,
                 note="70B-shape SwiGLU MLP shard forward, one rank of t=8"),
        Workload("swiglu_70b_bwd", "swiglu_bwd", b=1, s=4096, h=8192, t=8, dtype="bf16", seed=6,
                 ffn=28672, n_blocks=160, dz_seed=7, dz_std=0.01,
                 note="70B-shape SwiGLU MLP shard backward, one rank of t=8"),
        Workload("attn_70b", "attn", b=1, s=4096, h=8192, t=8, dtype="bf16", seed=8, n_blocks=160,
                 n_heads=64, n_kv_heads=8, head_dim=128, dz_seed=9, dz_std=0.01,
                 note="70B-shape attention projections (QKV column-parallel, W_O row-parallel), "
                      "one rank of t=8, forward and backward"),
    ]
}
