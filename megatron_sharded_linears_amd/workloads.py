"""The five workloads the library is tested and measured on.

Model dimensions are the public configs of Llama-3.1-8B (hidden 4096, 32
layers, 8 KV heads and vocab 128256 are the values page "张量、流水线与数据并行"
uses in section "每 token 的通信量（估算）") and Qwen2.5-32B (named on page
"第 9 章 多进程与张量并行", section 2.1). Each workload is one rank's share of a
t-way split, computed on one GPU.
"""

from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    hidden: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    t: int
    tokens: int
    layers: int
    lm_positions: int      # sampled positions fed to the LM head
    has_vocab: bool        # whether the workload includes embedding + LM head

    def cfg(self):
        return {"hidden": self.hidden, "num_q_heads": self.num_q_heads,
                "num_kv_heads": self.num_kv_heads, "head_dim": self.head_dim,
                "intermediate": self.intermediate, "vocab": self.vocab}


WORKLOADS = [
    Workload(0, "tiny_t2_m16", 256, 8, 2, 32, 1024, 1000, 2, 16, 1, 16, True),
    # Llama-3.1-8B decode at t=8, 16 tokens; embedding and LM head use the
    # model's vocab (128256) over all 16 positions.
    Workload(1, "llama8b_t8_decode_m16", 4096, 32, 8, 128, 14336, 128256, 8, 16, 32, 16, True),
    Workload(2, "llama8b_t2_prefill_m2048", 4096, 32, 8, 128, 14336, 128256, 2, 2048, 32, 1, False),
    Workload(3, "llama8b_t16_kvrepl_decode_m64", 4096, 32, 8, 128, 14336, 128256, 16, 64, 32, 64, True),
    # Qwen2.5-32B prefill at t=8, one 4096-token chunk of one request: the LM
    # head runs on its last position only.
    Workload(4, "qwen32b_t8_prefill_m4096", 5120, 40, 8, 128, 27648, 152064, 8, 4096, 64, 1, True),
]

BY_NAME = {w.name: w for w in WORKLOADS}
