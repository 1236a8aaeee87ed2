"""Communication-volume arithmetic of a Megatron-split decoder, as page
"张量、流水线与数据并行" estimates it in section "每 token 的通信量（估算）":
reported by the benchmark as context for the all-reduce the reducer stands in
for. Host-side arithmetic only.

- every all-reduce moves the hidden vector: hidden x bytes per token;
- two all-reduces per layer (after o_proj and down_proj) plus one for the
  vocab-parallel embedding;
- a ring all-reduce sends 2 (t - 1) / t times the payload per rank;
- the logits all-gather delivers (t - 1) / t of the vocab's logits per sampled
  token to each rank.
"""

KIB = 1024
MIB = 1024 * 1024


def all_reduces_per_forward(layers):
    return 2 * layers + 1


def payload_per_token(hidden, bytes_per_elem=2):
    """Bytes of one all-reduce per token."""
    return hidden * bytes_per_elem


def payload_per_token_per_forward(hidden, layers, bytes_per_elem=2):
    return payload_per_token(hidden, bytes_per_elem) * all_reduces_per_forward(layers)


def ring_factor(t):
    return 2.0 * (t - 1) / t


def ring_sent_per_rank_per_token(hidden, layers, t, bytes_per_elem=2):
    return ring_factor(t) * payload_per_token_per_forward(hidden, layers, bytes_per_elem)


def logits_gather_received_per_token(vocab, t, bytes_per_elem=2):
    return (t - 1) / t * vocab * bytes_per_elem


def per_step(tokens, hidden, layers, bytes_per_elem=2):
    """(bytes of one all-reduce, bytes of all of a forward's all-reduces)."""
    one = tokens * payload_per_token(hidden, bytes_per_elem)
    return one, one * all_reduces_per_forward(layers)
