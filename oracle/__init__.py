"""fp64 CPU oracle for exact ring attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The HIP library never
imports, links or calls it, and it imports nothing from the HIP library.

Contents
  * ring plan (pure Python, from the exercise of lesson 8 "Context
    Parallelism (CP)", hpc.payai.win): ring visiting order, sequential and
    zig-zag chunk assignments, per-rank causal workload, and the exact count
    of unmasked (query, key) pairs;
  * the attention definition in fp64 (C library ``attn_oracle.c`` through
    ctypes, and a numpy twin for tiny inputs);
  * the online-softmax fold of lesson 8, section 3, written as the pages state
    it (O renormalised at every step) -- used only to pin the definition
    against the pages' own update rule;
  * the merge of (O, lse) partials over disjoint key shards.

Every function names the passage it follows.  Points the pages leave open
are taken as stated in ``attn_oracle.c``'s header.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

ELEM_F32, ELEM_BF16, ELEM_F64 = 0, 1, 2


# ----------------------------------------------------------------------------
# Ring plan (lesson 8: section 2 "ring flow", section 4 "causal / zig-zag",
# worked example, exercise and its answer)
# ----------------------------------------------------------------------------

def ring_order(P: int, rank: int) -> list[int]:
    """Source shard visited by ``rank`` at steps t = 0..P-1.

    Lesson 8, section 2: K/V move from rank r to r+1 each step while Q stays
    put, so after t steps rank r holds the block that started at r - t
    (mod P).  Step 0 is the rank's own block.
    """
    return [(rank - t) % P for t in range(P)]


def sequential_assignment(P: int, chunks_per_rank: int) -> dict[int, list[int]]:
    """Naive contiguous split: rank r owns chunks r*k .. r*k+k-1 (lesson 8,
    section 4A and the worked example)."""
    return {r: list(range(r * chunks_per_rank, (r + 1) * chunks_per_rank)) for r in range(P)}


def zigzag_assignment(P: int, chunks_per_rank: int = 2) -> dict[int, list[int]]:
    """Zig-zag split (lesson 8, section 4B and the exercise).

    With 2 chunks per rank, rank r owns chunks r and 2P-1-r, in that local
    order.  For more chunks per rank the even-numbered picks count forward
    from the front in rounds of P and the odd-numbered picks count back from
    the end.
    """
    total = P * chunks_per_rank
    out = {}
    for r in range(P):
        picks = []
        for k in range(chunks_per_rank):
            rnd = k // 2
            if k % 2 == 0:
                picks.append(rnd * P + r)
            else:
                picks.append(total - 1 - rnd * P - r)
        out[r] = picks
    return out


def causal_chunk_workload(assign: dict[int, list[int]]) -> dict[int, int]:
    """Chunk pairs a rank computes under the causal mask: query chunk q sees
    key chunks 0..q, i.e. q+1 of them (lesson 8, section 4B and worked
    example).  A diagonal pair counts once."""
    return {r: sum(q + 1 for q in qs) for r, qs in assign.items()}


def parse_layout(layout: str) -> tuple[str, int]:
    """Layout name -> (kind, chunks per rank).

    "contiguous"      P chunks, one per rank (lesson 8, section 4A);
    "zigzag"          2 chunks per rank, r and 2P-1-r (section 4B);
    "zigzag<k>"       k chunks per rank by the exercise's general rule
                      (``zigzag_assignment``), e.g. "zigzag4";
    "striped"         tokens dealt round-robin: rank r holds positions
                      r, r+P, r+2P, ... .  The pages only name striped
                      attention as a rebalancing variant; this one-token
                      stripe is the plain reading of the name.
    For "striped" the chunk count is None (one token per chunk).
    """
    if layout == "contiguous":
        return "contiguous", 1
    if layout == "zigzag":
        return "zigzag", 2
    if layout.startswith("zigzag") and layout[6:].isdigit() and int(layout[6:]) >= 1:
        return "zigzag", int(layout[6:])
    if layout == "striped":
        return "striped", None
    raise ValueError(layout)


def local_chunks(layout: str, P: int, rank: int) -> list[int]:
    """Global chunk ids a rank stores, in local order (chunked layouts).

    contiguous: P chunks of S/P tokens, rank r stores chunk r;
    zigzag<k>:  kP chunks of S/(kP) tokens, rank r stores
                ``zigzag_assignment(P, k)[r]`` ([r, 2P-1-r] for k = 2).
    """
    kind, k = parse_layout(layout)
    if kind == "contiguous":
        return [rank]
    if kind == "zigzag":
        return zigzag_assignment(P, k)[rank]
    raise ValueError(layout)


def chunk_len(layout: str, S: int, P: int) -> int:
    kind, k = parse_layout(layout)
    n_chunks = S if kind == "striped" else P * k
    if S % n_chunks or S % P:
        raise ValueError("sequence does not split evenly")
    return S // n_chunks


def natural_positions(S: int, P: int, layout: str) -> np.ndarray:
    """pos[k] = natural (global) position of row k of the rank-sharded order.

    Rank r's rows come after those of ranks 0..r-1; inside a rank the local
    chunks follow ``local_chunks`` (striped: the rank's positions in order).
    """
    c = chunk_len(layout, S, P)
    pos = []
    for r in range(P):
        if parse_layout(layout)[0] == "striped":
            pos.append(np.arange(r, S, P, dtype=np.int64))
            continue
        for ch in local_chunks(layout, P, r):
            pos.append(np.arange(ch * c, (ch + 1) * c, dtype=np.int64))
    return np.concatenate(pos)


def ulysses_scatter_heads(x: np.ndarray, P: int) -> np.ndarray:
    """The all-to-all of DeepSpeed Ulysses (lesson 8, section 5): [B, S, H, ...]
    in sequence order -> [P, B, S, H/P, ...], rank g holding head group g
    (heads g*H/P .. (g+1)*H/P - 1) of every token.  The heads must divide by
    the number of ranks."""
    B, S, H = x.shape[:3]
    if H % P:
        raise ValueError(f"{H} heads do not divide over {P} ranks")
    out = np.empty((P, B, S, H // P) + x.shape[3:], dtype=x.dtype)
    for g in range(P):
        out[g] = x[:, :, g * (H // P):(g + 1) * (H // P)]
    return out


def ulysses_gather_heads(y: np.ndarray) -> np.ndarray:
    """Inverse of ``ulysses_scatter_heads``: [P, B, S, H/P, ...] -> [B, S, H, ...]."""
    P = y.shape[0]
    return np.concatenate([y[g] for g in range(P)], axis=2)


def helix_round_robin(total: int, block: int, P: int) -> list[np.ndarray]:
    """Sequence positions each device of a KV-parallel group stores, in its
    local order, when the KV of new tokens is appended round-robin (Helix
    article, KV cache section: the first block of new tokens goes to device
    0, the next block to device 1, and so on).  The blocks are dealt in
    sequence order; the last one may be short."""
    shards: list[list[int]] = [[] for _ in range(P)]
    dev = 0
    for start in range(0, total, block):
        shards[dev].extend(range(start, min(start + block, total)))
        dev = (dev + 1) % P
    return [np.asarray(x, dtype=np.int64) for x in shards]


def unmasked_pairs(S: int, P: int, layout: str, rank: int, causal: bool = True) -> int:
    """Exact number of (query, key) pairs rank ``rank`` must score, counted by
    brute force over its query positions (global causal mask, section 4)."""
    n = S // P
    pos = natural_positions(S, P, layout)[rank * n:(rank + 1) * n]
    if not causal:
        return n * S
    return int(np.sum(pos + 1))


def chunk_pairs_touched(S: int, P: int, layout: str, rank: int, n_chunks: int) -> int:
    """Brute-force count of (query chunk, key chunk) pairs, with chunks of
    S/n_chunks tokens, that contain at least one unmasked (query, key) pair
    for the queries of ``rank``.  This is the quantity the lesson counts as
    'i+1 blocks' (naive) and '2P+1 blocks' (zig-zag)."""
    n = S // P
    cl = S // n_chunks
    pos = natural_positions(S, P, layout)[rank * n:(rank + 1) * n]
    count = 0
    for qc in sorted(set((pos // cl).tolist())):
        qmax = int(pos[(pos // cl) == qc].max())
        for kc in range(n_chunks):
            if kc * cl <= qmax:
                count += 1
    return count


# ----------------------------------------------------------------------------
# Attention definition, fp64 (C library)
# ----------------------------------------------------------------------------

def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(_LIB_PATH)
        i64, vp, dp = ctypes.c_int64, ctypes.c_void_p, ctypes.POINTER(ctypes.c_double)
        lib.oracle_attention_rows.argtypes = [vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, i64,
                                              i64, ctypes.c_int, i64, vp, vp, vp, vp]
        lib.oracle_attention_rows.restype = ctypes.c_int
        lib.oracle_merge.argtypes = [vp, vp, i64, i64, i64, vp, vp]
        lib.oracle_merge.restype = ctypes.c_int
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_num_threads.restype = None
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads the C oracle's parallel regions use from now on."""
    _load().oracle_set_num_threads(int(n))


def _elem(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return ELEM_F32
    if a.dtype == np.uint16:
        return ELEM_BF16
    if a.dtype == np.float64:
        return ELEM_F64
    raise TypeError(f"oracle input dtype {a.dtype}: use float32, float64 or uint16 bf16 bits")


def attention_rows(Q, K, V, causal: bool, rows_b, rows_i):
    """Exact attention of selected query rows, every query head, in fp64.

    Q [B, Sq, Hq, d], K/V [B, Skv, Hkv, d], natural order, all of one dtype
    (float32, float64, or uint16 holding bf16 bits).  Returns
    O [n, Hq, d] and lse [n, Hq] (float64) for rows (rows_b[n], rows_i[n]).
    """
    Q = np.ascontiguousarray(Q)
    K = np.ascontiguousarray(K)
    V = np.ascontiguousarray(V)
    if not (Q.dtype == K.dtype == V.dtype):
        raise TypeError("Q, K, V must share a dtype")
    B, Sq, Hq, d = Q.shape
    Bk, Skv, Hkv, dk = K.shape
    if (Bk, dk) != (B, d) or V.shape != K.shape:
        raise ValueError("shape mismatch")
    rb = np.ascontiguousarray(np.asarray(rows_b, dtype=np.int64))
    ri = np.ascontiguousarray(np.asarray(rows_i, dtype=np.int64))
    n = rb.shape[0]
    O = np.empty((n, Hq, d), np.float64)
    lse = np.empty((n, Hq), np.float64)
    rc = _load().oracle_attention_rows(Q.ctypes.data, K.ctypes.data, V.ctypes.data, _elem(Q),
                                       B, Sq, Skv, Hq, Hkv, d, int(bool(causal)), n,
                                       rb.ctypes.data, ri.ctypes.data, O.ctypes.data,
                                       lse.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_attention_rows rejected its arguments")
    return O, lse


def attention(Q, K, V, causal: bool):
    """All rows: O [B, Sq, Hq, d], lse [B, Hq, Sq] (fp64, natural order)."""
    B, Sq, Hq, d = Q.shape
    bb, ii = np.meshgrid(np.arange(B), np.arange(Sq), indexing="ij")
    O, lse = attention_rows(Q, K, V, causal, bb.ravel(), ii.ravel())
    return O.reshape(B, Sq, Hq, d), lse.reshape(B, Sq, Hq).transpose(0, 2, 1).copy()


def merge(O_parts, lse_parts):
    """Merge partials over disjoint key shards (fp64).

    O_parts [n_parts, rows, d], lse_parts [n_parts, rows] -> O [rows, d], lse [rows].
    """
    O_parts = np.ascontiguousarray(O_parts, dtype=np.float64)
    lse_parts = np.ascontiguousarray(lse_parts, dtype=np.float64)
    n_parts, rows, d = O_parts.shape
    O = np.empty((rows, d), np.float64)
    lse = np.empty((rows,), np.float64)
    rc = _load().oracle_merge(O_parts.ctypes.data, lse_parts.ctypes.data, n_parts, rows, d,
                              O.ctypes.data, lse.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_merge rejected its arguments")
    return O, lse


# ----------------------------------------------------------------------------
# numpy twin and the pages' own update rule (tiny inputs only)
# ----------------------------------------------------------------------------

def bf16_bits_to_f64(u16: np.ndarray) -> np.ndarray:
    return (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_f64(a: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def attention_np(Q, K, V, causal: bool):
    """The same definition as ``attention`` in numpy fp64, for tiny inputs.
    Returns O [B, Sq, Hq, d], lse [B, Hq, Sq]."""
    Q, K, V = to_f64(Q), to_f64(K), to_f64(V)
    B, Sq, Hq, d = Q.shape
    Skv, Hkv = K.shape[1], K.shape[2]
    G = Hq // Hkv
    O = np.zeros((B, Sq, Hq, d))
    lse = np.full((B, Hq, Sq), -np.inf)
    for b in range(B):
        for h in range(Hq):
            kh = h // G
            s = Q[b, :, h, :] @ K[b, :, kh, :].T / math.sqrt(d)
            if causal:
                s = np.where(np.arange(Skv)[None, :] <= np.arange(Sq)[:, None], s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            ok = np.isfinite(m[:, 0])
            e = np.where(ok[:, None], np.exp(s - np.where(ok[:, None], m, 0.0)), 0.0)
            l = e.sum(axis=1)
            O[b, ok, h, :] = (e[ok] @ V[b, :, kh, :]) / l[ok, None]
            lse[b, h, ok] = m[ok, 0] + np.log(l[ok])
    return O, lse


def fold_init(rows: int, d: int):
    """Initial online-softmax state (m, l, O) = (-inf, 0, 0) (lesson 8,
    section 3 leaves the start state implicit; this is its neutral element)."""
    return np.full(rows, -np.inf), np.zeros(rows), np.zeros((rows, d))


def fold_step(state, s_new, v_new):
    """One online-softmax update exactly as lesson 8, section 3 writes it:

      m~  = max(m, rowmax(S_new))
      l'  = l * exp(m - m~) + rowsum(exp(S_new - m~))
      O'  = O * exp(m - m~) * l / l'  +  exp(S_new - m~) / l' @ V_new
      m   := m~

    s_new [rows, n] holds already scaled scores (masked entries -inf);
    v_new [n, d].  A row whose state and new block are all masked is left as
    it was (its exponentials are taken as 0).
    """
    m, l, O = state
    m_new = np.maximum(m, s_new.max(axis=1) if s_new.shape[1] else m)
    ok = np.isfinite(m_new)
    safe = np.where(ok, m_new, 0.0)
    alpha = np.where(ok & np.isfinite(m), np.exp(m - safe), 0.0)
    p = np.where(ok[:, None], np.exp(s_new - safe[:, None]), 0.0)
    l_new = l * alpha + p.sum(axis=1)
    O_new = np.zeros_like(O)
    pos = l_new > 0
    O_new[pos] = (O[pos] * (alpha[pos] * l[pos] / l_new[pos])[:, None]
                  + (p[pos] / l_new[pos, None]) @ v_new)
    return np.where(ok, m_new, m), l_new, O_new


def fold_finish(state):
    m, l, O = state
    lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return O, lse
