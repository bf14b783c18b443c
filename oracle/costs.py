"""Token-layer pass counts of a gated prefill (test infrastructure only).

Follows the worked example on the explainer page "Prune prefill tokens to
cut TTFT up to 11.3x with TokenGate -- Token-gated attention -- What does it
mean?" (section on how the savings compose): the layers up to and including
the gate layer see every token, every layer above sees only the kept ones,
and per-layer attention work scales with the square of the token count.
"""


def token_layer_passes(n_layers: int, n_tokens: int, gate_layer: int, kept: int):
    """(unpruned passes, gated passes) for a model of n_layers layers."""
    full = n_layers * n_tokens
    below = gate_layer + 1                         # layers 0..L see everything
    gated = below * n_tokens + (n_layers - below) * kept
    return full, gated


def attention_pair_ratio(n_tokens: int, kept: int) -> float:
    """Per-layer reduction of pairwise attention work above the gate."""
    return (n_tokens / kept) ** 2


def causal_attention_flops(seqlens, hq: int, dh: int) -> int:
    """Exact multiply-add flops of causal attention: per query head and causal
    (query, key) pair, dh MACs for q.k and dh for p.v, i.e. 4*dh flops, with
    T(T+1)/2 pairs per sequence of T kept tokens."""
    return sum(2 * dh * hq * t * (t + 1) for t in seqlens)
