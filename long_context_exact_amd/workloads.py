"""The five workloads of the ring-attention hot path and their algorithmic
work (FLOPs and bytes) used by the benchmark's roofline figures."""
from __future__ import annotations

from dataclasses import dataclass

TENSOR_Q, TENSOR_K, TENSOR_V = 0, 1, 2


@dataclass(frozen=True)
class Workload:
    """One of the five workloads of the ring-attention hot path."""
    cfg: int
    name: str
    kind: str          # "prefill" or "decode"
    B: int
    Hq: int
    Hkv: int
    d: int
    S: int             # prefill: sequence length; decode: KV length
    P: int             # ranks (prefill) or KV shards (decode)
    layout: str        # "contiguous" | "zigzag" | "zigzag<k>" | "striped" (prefill)
    causal: bool
    dtype: str         # "f32" | "bf16"
    Sq: int = 1        # decode queries per sequence

    def seed(self, tensor_id: int) -> tuple:
        return (self.cfg, tensor_id)

    @property
    def q_shape(self):
        return (self.B, self.S if self.kind == "prefill" else self.Sq, self.Hq, self.d)

    @property
    def kv_shape(self):
        return (self.B, self.S, self.Hkv, self.d)


WORKLOADS = {
    1: Workload(1, "mha_s1k_d64_p4_contig_noncausal_fp32", "prefill", 1, 2, 2, 64, 1024, 4,
                "contiguous", False, "f32"),
    2: Workload(2, "mha_h8_s8k_p8_contig_causal_bf16", "prefill", 1, 8, 8, 128, 8192, 8,
                "contiguous", True, "bf16"),
    3: Workload(3, "mha_h16_s32k_p8_zigzag_causal_bf16", "prefill", 1, 16, 16, 128, 32768, 8,
                "zigzag", True, "bf16"),
    4: Workload(4, "gqa_hq32_hkv8_s128k_p8_zigzag_causal_bf16", "prefill", 1, 32, 8, 128, 131072, 8,
                "zigzag", True, "bf16"),
    5: Workload(5, "decode_b8_hq64_hkv8_kv1m_p8_shards_bf16", "decode", 8, 64, 8, 128, 1 << 20, 8,
                "contiguous", False, "bf16", Sq=1),
}


def layout_kind(layout: str) -> tuple[str, int]:
    """"contiguous" -> (contiguous, 1); "zigzag" -> (zigzag, 2);
    "zigzag<k>" -> (zigzag, k); "striped" -> (striped, 0)."""
    if layout == "contiguous":
        return "contiguous", 1
    if layout == "zigzag":
        return "zigzag", 2
    if layout == "striped":
        return "striped", 0
    if layout.startswith("zigzag") and layout[6:].isdigit() and int(layout[6:]) >= 1:
        return "zigzag", int(layout[6:])
    raise ValueError(f"unknown layout {layout!r}")


def causal_pairs_rank(S: int, P: int, layout: str, rank: int) -> int:
    """Closed-form count of unmasked (query, key) pairs of one rank under the
    global causal mask (used for FLOP accounting).

    contiguous, n = S/P:   rank r scores r*n*n + n(n+1)/2 pairs;
    zig-zag, c = S/(2P):   every rank scores 2P*c*c + c pairs;
    zig-zag with k chunks of c = S/(kP) tokens: a chunk with global id g
                           scores c*c*g + c(c+1)/2 pairs, summed over the
                           rank's chunks (even picks g = (i/2)P + r, odd
                           picks g = kP-1-(i/2)P-r for local index i);
    striped, n = S/P:      query j of rank r sits at r + jP, so the rank
                           scores n(r+1) + P n(n-1)/2 pairs.
    """
    kind, k = layout_kind(layout)
    if kind == "contiguous":
        n = S // P
        return rank * n * n + n * (n + 1) // 2
    if kind == "striped":
        n = S // P
        return n * (rank + 1) + P * n * (n - 1) // 2
    if k == 2:
        c = S // (2 * P)
        return 2 * P * c * c + c
    c = S // (k * P)
    total = 0
    for i in range(k):
        g = (i // 2) * P + rank if i % 2 == 0 else k * P - 1 - (i // 2) * P - rank
        total += c * c * g + c * (c + 1) // 2
    return total


def prefill_flops(w: Workload, rank: int | None = None) -> int:
    """Algorithmic FLOPs: 4 * d * Hq * B per scored (query, key) pair (QK^T and
    PV, two FLOPs per multiply-add each), with causal pairs counted exactly."""
    ranks = range(w.P) if rank is None else [rank]
    pairs = 0
    for r in ranks:
        pairs += causal_pairs_rank(w.S, w.P, w.layout, r) if w.causal else (w.S // w.P) * w.S
    return 4 * w.d * w.Hq * w.B * pairs


def decode_bytes(w: Workload, n_parts: int, elem_bytes: int = 2, out_bytes: int = 4) -> dict:
    """Algorithmic HBM bytes of one decode step (KV-sharded attention of one
    query per sequence, then the merge of the per-part partials):

      K and V read once, Q read once, partials (O fp32 d-vector + lse fp32
      per row and part) written once and read once by the merge, merged O
      (input dtype) and lse (fp32) written once.
    """
    rows = w.B * w.Sq * w.Hq
    kv = 2 * w.B * w.S * w.Hkv * w.d * elem_bytes
    q = rows * w.d * elem_bytes
    partials = n_parts * rows * (w.d + 1) * 4
    out = rows * (w.d * out_bytes + 4)
    return {"kv": kv, "q": q, "partials": partials, "out": out,
            "attn_partial": kv + q + partials,
            "merge": partials + out,
            "total": kv + q + 2 * partials + out}


def decode_flops(w: Workload) -> int:
    """4 * d FLOPs per (query row, key) pair, every query head."""
    return 4 * w.d * w.B * w.Sq * w.Hq * w.S
