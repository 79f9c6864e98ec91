"""Pins of the fp64 CPU oracle against what the pages and the mathematics fix.

None of these needs a GPU.  Each pin checks the oracle against something
other than itself: numbers printed on the pages (tests/golden), closed forms,
a library routine (torch's CPU scaled_dot_product_attention in float64), a
pure-Python brute force, and the pages' own online-softmax update rule.
The last group plants plausible mistakes in a copy of the oracle and checks
that some pin catches each of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from long_context_exact_amd import synthetic
from long_context_exact_amd.workloads import causal_pairs_rank

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "lesson08_exercise.json")


def _rand(shape, seed, dtype="f32"):
    return synthetic.normal_tensor(shape, (900, *seed), dtype)


# ---------------------------------------------------------------- ring plan

def test_golden_exercise_output():
    g = json.load(open(GOLDEN))
    P, k = g["P"], g["chunks_per_rank"]
    seq = oracle.sequential_assignment(P, k)
    zz = oracle.zigzag_assignment(P, k)
    assert {str(r): v for r, v in seq.items()} == g["sequential"]
    assert {str(r): v for r, v in zz.items()} == g["zigzag"]
    w_seq = oracle.causal_chunk_workload(seq)
    w_zz = oracle.causal_chunk_workload(zz)
    assert {str(r): v for r, v in w_seq.items()} == g["sequential_workload"]
    assert {str(r): v for r, v in w_zz.items()} == g["zigzag_workload"]
    assert max(w_seq.values()) / min(w_seq.values()) == g["sequential_max_over_min"]
    assert oracle.ring_order(P, 2) == g["rank2_rotation"]


@pytest.mark.parametrize("P", list(range(1, 17)))
def test_zigzag_workload_closed_form(P):
    # lesson 8, section 4B: every rank's causal workload is 2P+1 chunk pairs
    w = oracle.causal_chunk_workload(oracle.zigzag_assignment(P, 2))
    assert set(w.values()) == {2 * P + 1}
    # figure 8-1 / section 4A: naive split with one chunk per rank -> rank i does i+1
    w1 = oracle.causal_chunk_workload(oracle.sequential_assignment(P, 1))
    assert w1 == {i: i + 1 for i in range(P)}


@pytest.mark.parametrize("P", [1, 2, 3, 4, 8])
def test_ring_order_visits_every_shard_once(P):
    for r in range(P):
        order = oracle.ring_order(P, r)
        assert order[0] == r and sorted(order) == list(range(P))
        # K/V flow r-1 -> r: the block held at step t+1 is the one the
        # predecessor held at step t
        prev = oracle.ring_order(P, (r - 1) % P)
        assert all(order[t + 1] == prev[t] for t in range(P - 1))


@pytest.mark.parametrize("P,c", [(1, 3), (2, 2), (4, 3), (8, 2)])
def test_block_pair_counts_brute_force(P, c):
    # naive contiguous split, blocks of S/P: rank i touches i+1 blocks
    S = 2 * P * c
    for r in range(P):
        assert oracle.chunk_pairs_touched(S, P, "contiguous", r, P) == r + 1
    # zig-zag, 2P chunks: every rank touches 2P+1 chunk pairs
    for r in range(P):
        assert oracle.chunk_pairs_touched(S, P, "zigzag", r, 2 * P) == 2 * P + 1


@pytest.mark.parametrize("P,S", [(1, 8), (2, 8), (4, 16), (4, 40), (8, 64), (8, 8192)])
def test_exact_unmasked_pairs(P, S):
    # brute force over query positions vs the closed forms used for FLOPs:
    # contiguous r*n^2 + n(n+1)/2, zig-zag 2P c^2 + c
    for layout in ("contiguous", "zigzag"):
        for r in range(P):
            assert oracle.unmasked_pairs(S, P, layout, r) == causal_pairs_rank(S, P, layout, r)
    tot = sum(oracle.unmasked_pairs(S, P, "zigzag", r) for r in range(P))
    assert tot == S * (S + 1) // 2
    for layout in ("zigzag4", "striped"):
        if S % (4 * P):
            continue
        for r in range(P):
            assert oracle.unmasked_pairs(S, P, layout, r) == causal_pairs_rank(S, P, layout, r)


def test_natural_positions_small():
    pos = oracle.natural_positions(16, 4, "zigzag")
    expect = [0, 1, 14, 15, 2, 3, 12, 13, 4, 5, 10, 11, 6, 7, 8, 9]
    assert pos.tolist() == expect
    assert oracle.natural_positions(12, 3, "contiguous").tolist() == list(range(12))
    with pytest.raises(ValueError):
        oracle.natural_positions(10, 4, "zigzag")
    # four chunks per rank, P = 2, chunks of 2: rank 0 holds chunks 0, 7, 2, 5
    # and rank 1 holds 1, 6, 3, 4 (written out by hand from the rule)
    assert oracle.natural_positions(16, 2, "zigzag4").tolist() == [
        0, 1, 14, 15, 4, 5, 10, 11, 2, 3, 12, 13, 6, 7, 8, 9]
    # token round-robin: rank r holds r, r+P, r+2P, ...
    assert oracle.natural_positions(8, 2, "striped").tolist() == [0, 2, 4, 6, 1, 3, 5, 7]
    assert oracle.natural_positions(9, 3, "striped").tolist() == [0, 3, 6, 1, 4, 7, 2, 5, 8]
    with pytest.raises(ValueError):
        oracle.natural_positions(10, 4, "striped")
    with pytest.raises(ValueError):
        oracle.natural_positions(16, 4, "zigzag3")
    for bad in ("zigzag0", "zigzagx", "stripes", ""):
        with pytest.raises(ValueError):
            oracle.parse_layout(bad)


LAYOUTS = ["contiguous", "zigzag", "zigzag3", "zigzag4", "zigzag6", "striped"]


@pytest.mark.parametrize("P", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("layout", LAYOUTS)
def test_layouts_are_permutations(layout, P):
    # every layout deals every position to exactly one rank, S/P per rank
    S = 48 * P
    pos = oracle.natural_positions(S, P, layout)
    assert sorted(pos.tolist()) == list(range(S))
    n = S // P
    if layout == "striped":
        for r in range(P):
            assert (pos[r * n:(r + 1) * n] % P == r).all()


def test_zigzag_four_chunks_per_rank_explicit():
    # the exercise's general rule for more than two chunks per rank, P = 4,
    # k = 4, 16 chunks: even picks count forward from the front in rounds of
    # P, odd picks count back from the end (written out by hand)
    assert oracle.zigzag_assignment(4, 4) == {
        0: [0, 15, 4, 11], 1: [1, 14, 5, 10], 2: [2, 13, 6, 9], 3: [3, 12, 7, 8]}
    assert oracle.zigzag_assignment(3, 3) == {0: [0, 8, 3], 1: [1, 7, 4], 2: [2, 6, 5]}


@pytest.mark.parametrize("P", list(range(1, 13)))
def test_zigzag_even_k_balanced(P):
    # an even pick q and its odd partner total-1-q sum to total-1, so with an
    # even number of chunks per rank every rank does k/2 * (kP + 1) chunk pairs
    for k in (2, 4, 6, 8):
        w = oracle.causal_chunk_workload(oracle.zigzag_assignment(P, k))
        assert set(w.values()) == {k // 2 * (k * P + 1)}
    # an odd k leaves the last forward pick unpaired: unbalanced for P > 1
    w3 = oracle.causal_chunk_workload(oracle.zigzag_assignment(P, 3))
    assert (len(set(w3.values())) == 1) == (P == 1)


@pytest.mark.parametrize("P,S", [(1, 6), (2, 8), (3, 9), (4, 40), (8, 64), (8, 8192)])
def test_striped_unmasked_pairs_closed_form(P, S):
    # rank r's j-th query sits at r + jP and sees r + jP + 1 keys:
    # sum_j = n (r + 1) + P n (n - 1) / 2, n = S/P; all ranks sum to S(S+1)/2
    n = S // P
    tot = 0
    for r in range(P):
        got = oracle.unmasked_pairs(S, P, "striped", r)
        assert got == n * (r + 1) + P * n * (n - 1) // 2
        tot += got
    assert tot == S * (S + 1) // 2
    # ranks differ by exactly n pairs from one to the next
    assert oracle.unmasked_pairs(S, P, "striped", P - 1) - oracle.unmasked_pairs(
        S, P, "striped", 0) == n * (P - 1)


# ------------------------------------------------------ attention definition

def _sdpa_f64(Q, K, V, causal):
    """torch CPU float64 reference (math path); GQA by repeating K/V heads."""
    q = torch.from_numpy(oracle.to_f64(Q)).permute(0, 2, 1, 3)
    k = torch.from_numpy(oracle.to_f64(K)).permute(0, 2, 1, 3)
    v = torch.from_numpy(oracle.to_f64(V)).permute(0, 2, 1, 3)
    G = q.shape[1] // k.shape[1]
    k = k.repeat_interleave(G, dim=1).contiguous()
    v = v.repeat_interleave(G, dim=1).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal)
    s = (q @ k.transpose(-1, -2).contiguous()) / math.sqrt(q.shape[-1])
    if causal:
        m = torch.ones(s.shape[-2], s.shape[-1], dtype=torch.bool).tril()
        s = s.masked_fill(~m, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return o.permute(0, 2, 1, 3).numpy(), lse.numpy()


CASES = [  # B, S, Hq, Hkv, d, causal, dtype
    (1, 7, 2, 2, 4, False, "f32"),
    (2, 33, 4, 2, 16, True, "f32"),
    (1, 64, 8, 2, 64, True, "bf16"),
    (2, 50, 3, 1, 32, False, "bf16"),
    (1, 40, 6, 3, 128, True, "f64"),
]


@pytest.mark.parametrize("B,S,Hq,Hkv,d,causal,dt", CASES)
def test_attention_matches_torch_sdpa(B, S, Hq, Hkv, d, causal, dt):
    gen = "f32" if dt == "f64" else dt
    Q = _rand((B, S, Hq, d), (1, S, d), gen)
    K = _rand((B, S, Hkv, d), (2, S, d), gen)
    V = _rand((B, S, Hkv, d), (3, S, d), gen)
    if dt == "f64":
        Q, K, V = (x.astype(np.float64) for x in (Q, K, V))
    O, lse = oracle.attention(Q, K, V, causal)
    O_t, lse_t = _sdpa_f64(Q, K, V, causal)
    np.testing.assert_allclose(O, O_t, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_t, rtol=0, atol=1e-12)
    O_np, lse_np = oracle.attention_np(Q, K, V, causal)
    np.testing.assert_allclose(O, O_np, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_np, rtol=0, atol=1e-12)


def test_attention_pure_python_brute_force():
    B, S, Hq, Hkv, d = 2, 5, 4, 2, 3
    Q = _rand((B, S, Hq, d), (4,)).astype(np.float64)
    K = _rand((B, S, Hkv, d), (5,)).astype(np.float64)
    V = _rand((B, S, Hkv, d), (6,)).astype(np.float64)
    for causal in (False, True):
        O, lse = oracle.attention(Q, K, V, causal)
        for b in range(B):
            for i in range(S):
                for h in range(Hq):
                    kh = h // (Hq // Hkv)
                    js = range(i + 1) if causal else range(S)
                    sc = [sum(Q[b, i, h, e] * K[b, j, kh, e] for e in range(d)) / math.sqrt(d)
                          for j in js]
                    den = sum(math.exp(x) for x in sc)
                    for e in range(d):
                        num = sum(math.exp(x) * V[b, j, kh, e] for x, j in zip(sc, js))
                        assert abs(O[b, i, h, e] - num / den) < 1e-13
                    assert abs(lse[b, h, i] - math.log(den)) < 1e-13


def test_closed_forms():
    B, S, H, d = 1, 12, 2, 8
    V = _rand((B, S, H, d), (7,)).astype(np.float64)
    K = _rand((B, S, H, d), (8,)).astype(np.float64)
    # Q = 0: uniform weights over the visible keys
    Q0 = np.zeros((B, S, H, d))
    O, lse = oracle.attention(Q0, K, V, True)
    for i in range(S):
        np.testing.assert_allclose(O[0, i], V[0, :i + 1].mean(axis=0), atol=1e-14)
        np.testing.assert_allclose(lse[0, :, i], math.log(i + 1), atol=1e-14)
    O, lse = oracle.attention(Q0, K, V, False)
    np.testing.assert_allclose(O[0], np.broadcast_to(V[0].mean(axis=0), (S, H, d)), atol=1e-14)
    # causal row 0 sees only key 0: O = V_0, lse = s_00
    Q = _rand((B, S, H, d), (9,)).astype(np.float64)
    O, lse = oracle.attention(Q, K, V, True)
    np.testing.assert_allclose(O[0, 0], V[0, 0], atol=1e-14)
    s00 = (Q[0, 0] * K[0, 0]).sum(-1) / math.sqrt(d)
    np.testing.assert_allclose(lse[0, :, 0], s00, atol=1e-14)
    # identical keys: uniform weights, lse = s + ln(n)
    Kc = np.broadcast_to(K[:, :1], K.shape).copy()
    O, lse = oracle.attention(Q, Kc, V, False)
    np.testing.assert_allclose(O[0], np.broadcast_to(V[0].mean(axis=0), (S, H, d)), atol=1e-13)
    s = (Q[0] * Kc[0]).sum(-1) / math.sqrt(d)  # [S, H]
    np.testing.assert_allclose(lse[0], s.T + math.log(S), atol=1e-13)


def test_attention_rows_subset_and_errors():
    Q = _rand((2, 9, 4, 8), (10,))
    K = _rand((2, 9, 2, 8), (11,))
    V = _rand((2, 9, 2, 8), (12,))
    O, lse = oracle.attention(Q, K, V, True)
    rb, ri = [1, 0, 1], [8, 3, 0]
    Os, ls = oracle.attention_rows(Q, K, V, True, rb, ri)
    for n, (b, i) in enumerate(zip(rb, ri)):
        np.testing.assert_array_equal(Os[n], O[b, i])
        np.testing.assert_array_equal(ls[n], lse[b, :, i])
    with pytest.raises(ValueError):
        oracle.attention_rows(Q, K, V, True, [2], [0])
    with pytest.raises(ValueError):
        oracle.attention_rows(Q, K[:, :5], V[:, :5], True, [0], [0])


def test_decode_shape_and_shard_invariance():
    # one query per sequence over a long key set; splitting the keys into any
    # number of disjoint shards and merging gives the same result
    B, Skv, Hq, Hkv, d = 2, 300, 8, 2, 16
    Q = _rand((B, 1, Hq, d), (13,), "bf16")
    K = _rand((B, Skv, Hkv, d), (14,), "bf16")
    V = _rand((B, Skv, Hkv, d), (15,), "bf16")
    O, lse = oracle.attention(Q, K, V, False)
    O_t, lse_t = _sdpa_f64(Q, K, V, False)
    np.testing.assert_allclose(O, O_t, atol=1e-12)
    for n_parts in (1, 3, 8):
        cuts = np.linspace(0, Skv, n_parts + 1).astype(int)
        Op, lp = [], []
        for a, b in zip(cuts[:-1], cuts[1:]):
            o, l = oracle.attention(Q, K[:, a:b], V[:, a:b], False)
            Op.append(o.reshape(B * Hq, d))
            lp.append(l.transpose(0, 2, 1).reshape(B * Hq))
        Om, lm = oracle.merge(np.stack(Op), np.stack(lp))
        np.testing.assert_allclose(Om, O.reshape(B * Hq, d), atol=1e-13)
        np.testing.assert_allclose(lm, lse.transpose(0, 2, 1).reshape(B * Hq), atol=1e-13)


# -------------------------------------------- the pages' online update rule

def _fold_rows(Q, K, V, causal, qpos, blocks):
    """Fold key blocks (lists of natural key positions) in the given order
    with the lesson's update rule, for query positions qpos (B = 1, head 0)."""
    d = Q.shape[-1]
    q = oracle.to_f64(Q)[0, qpos, 0, :]
    state = oracle.fold_init(len(qpos), d)
    for blk in blocks:
        k = oracle.to_f64(K)[0, blk, 0, :]
        v = oracle.to_f64(V)[0, blk, 0, :]
        s = q @ k.T / math.sqrt(d)
        if causal:
            s = np.where(np.asarray(blk)[None, :] <= np.asarray(qpos)[:, None], s, -np.inf)
        state = oracle.fold_step(state, s, v)
    return oracle.fold_finish(state)


@pytest.mark.parametrize("P", [2, 3, 4])
@pytest.mark.parametrize("causal", [False, True])
def test_online_fold_equals_definition_in_every_order(P, causal):
    S, d = 4 * P, 8
    Q = _rand((1, S, 1, d), (16, P))
    K = _rand((1, S, 1, d), (17, P))
    V = _rand((1, S, 1, d), (18, P))
    O, lse = oracle.attention(Q, K, V, causal)
    n = S // P
    blocks = [list(range(s * n, (s + 1) * n)) for s in range(P)]
    qpos = list(range(S))
    for order in itertools.permutations(range(P)):
        Of, lf = _fold_rows(Q, K, V, causal, qpos, [blocks[s] for s in order])
        np.testing.assert_allclose(Of, O[0, :, 0, :], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lf, lse[0, 0, :], rtol=0, atol=1e-12)


@pytest.mark.parametrize("layout", ["contiguous", "zigzag", "zigzag3", "zigzag4", "striped"])
def test_ring_fold_per_rank_p8(layout):
    # each rank keeps its own query rows and folds the P shards in ring order
    P, S, d = 8, 96, 16
    Q = _rand((1, S, 1, d), (19,), "bf16")
    K = _rand((1, S, 1, d), (20,), "bf16")
    V = _rand((1, S, 1, d), (21,), "bf16")
    O, lse = oracle.attention(Q, K, V, True)
    pos = oracle.natural_positions(S, P, layout)
    n = S // P
    for r in range(P):
        qpos = pos[r * n:(r + 1) * n].tolist()
        blocks = [pos[s * n:(s + 1) * n].tolist() for s in oracle.ring_order(P, r)]
        Of, lf = _fold_rows(Q, K, V, True, qpos, blocks)
        np.testing.assert_allclose(Of, O[0, qpos, 0, :], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lf, lse[0, 0, qpos], rtol=0, atol=1e-12)


def test_fold_with_fully_masked_block_first():
    # a block that is entirely in the future of every query leaves the state
    # untouched, whichever position it takes in the order
    S, d = 8, 4
    Q = _rand((1, S, 1, d), (22,))
    K = _rand((1, S, 1, d), (23,))
    V = _rand((1, S, 1, d), (24,))
    O, lse = oracle.attention(Q, K, V, True)
    qpos = [0, 1, 2, 3]
    Of, lf = _fold_rows(Q, K, V, True, qpos, [[4, 5, 6, 7], [0, 1, 2, 3]])
    np.testing.assert_allclose(Of, O[0, :4, 0], atol=1e-12)
    np.testing.assert_allclose(lf, lse[0, 0, :4], atol=1e-12)


# --------------------------------------------------------------------- merge

def test_merge_permutation_and_partition():
    B, Skv, Hq, Hkv, d = 1, 40, 4, 4, 8
    Q = _rand((B, 1, Hq, d), (25,))
    K = _rand((B, Skv, Hkv, d), (26,))
    V = _rand((B, Skv, Hkv, d), (27,))
    O, lse = oracle.attention(Q, K, V, False)
    rng = np.random.default_rng(5)
    perm = rng.permutation(Skv)
    parts = np.array_split(perm, 5)  # disjoint, non-contiguous key sets
    Op, lp = [], []
    for keys in parts:
        o, l = oracle.attention(Q, K[:, keys], V[:, keys], False)
        Op.append(o.reshape(Hq, d))
        lp.append(l.reshape(Hq))
    Op, lp = np.stack(Op), np.stack(lp)
    ref_O, ref_l = O.reshape(Hq, d), lse.reshape(Hq)
    for order in itertools.permutations(range(5)):
        Om, lm = oracle.merge(Op[list(order)], lp[list(order)])
        np.testing.assert_allclose(Om, ref_O, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lm, ref_l, rtol=0, atol=1e-13)


def test_merge_empty_shards():
    d = 4
    Op = np.array([[[1.0, 2, 3, 4]], [[9.0, 9, 9, 9]], [[5.0, 6, 7, 8]]])
    lp = np.array([[0.5], [-np.inf], [0.5]])
    Om, lm = oracle.merge(Op, lp)
    np.testing.assert_allclose(Om[0], [3, 4, 5, 6])
    np.testing.assert_allclose(lm[0], 0.5 + math.log(2))
    Om, lm = oracle.merge(Op, np.full((3, 1), -np.inf))
    assert np.all(Om == 0) and lm[0] == -np.inf
    # a row that sees no key at all (all shards empty) is O = 0, lse = -inf
    Q = _rand((1, 1, 1, d), (28,))
    K = np.zeros((1, 0, 1, d), np.float32)
    O, lse = oracle.attention_rows(Q, K, K, False, [0], [0])
    assert np.all(O == 0) and lse[0, 0] == -np.inf


# ---------------------------------------------------------- input generator

def test_bf16_rne_matches_torch():
    x = np.concatenate([
        synthetic.normal_range((31,), 0, 100000),
        # exact ties: halfway between two bf16 values, even and odd lsb
        (np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x40498000], np.uint32)).view(np.float32),
    ])
    ours = synthetic.bf16_rne_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_generator_ranges_are_consistent():
    seed = (77, 1)
    n = synthetic.CHUNK * 2 + 1000
    full = synthetic.normal_range(seed, 0, n)
    a, b = synthetic.CHUNK - 10, synthetic.CHUNK * 2 + 5
    np.testing.assert_array_equal(synthetic.normal_range(seed, a, b), full[a:b])
    bits = synthetic.normal_range(seed, a, b, "bf16")
    np.testing.assert_array_equal(bits, synthetic.bf16_rne_bits(full[a:b]))
    assert abs(full.mean()) < 1e-3 and abs(full.std() - 1) < 1e-3


# --------------------------------------------- planted mistakes are caught

def _mutant_attention(kind):
    def f(Q, K, V, causal):
        Q, K, V = oracle.to_f64(Q), oracle.to_f64(K), oracle.to_f64(V)
        B, Sq, Hq, d = Q.shape
        Skv, Hkv = K.shape[1], K.shape[2]
        G = Hq // Hkv
        O = np.zeros((B, Sq, Hq, d))
        lse = np.zeros((B, Hq, Sq))
        for b in range(B):
            for h in range(Hq):
                kh = (h % Hkv) if kind == "gqa_mod" else h // G
                sc = 1.0 if kind == "no_scale" else 1 / math.sqrt(d)
                s = Q[b, :, h] @ K[b, :, kh].T * sc
                if causal:
                    keep = (np.arange(Skv)[None] < np.arange(Sq)[:, None]) if kind == "strict_mask" \
                        else (np.arange(Skv)[None] <= np.arange(Sq)[:, None])
                    if kind == "strict_mask":
                        keep[0, 0] = True
                    s = np.where(keep, s, -np.inf)
                m = s.max(1, keepdims=True)
                e = np.exp(s - m)
                l = e.sum(1)
                vv = V[b, :, kh]
                if kind == "transposed_pv":
                    vv = vv[::-1]
                O[b, :, h] = e @ vv / l[:, None]
                lse[b, h] = m[:, 0] + np.log(l) + (0.0 if kind != "lse_log2" else np.log(l) * 0.4427)
        return O, lse
    return f


@pytest.mark.parametrize("kind", ["no_scale", "gqa_mod", "strict_mask", "transposed_pv", "lse_log2"])
def test_planted_mistakes_fail_a_pin(kind):
    B, S, Hq, Hkv, d = 1, 16, 4, 2, 8
    Q = _rand((B, S, Hq, d), (40,))
    K = _rand((B, S, Hkv, d), (41,))
    V = _rand((B, S, Hkv, d), (42,))
    O_t, lse_t = _sdpa_f64(Q, K, V, True)
    O_m, lse_m = _mutant_attention(kind)(Q, K, V, True)
    caught = (np.abs(O_m - O_t).max() > 1e-6) or (np.abs(lse_m - lse_t).max() > 1e-6)
    assert caught, kind


def test_planted_plan_mistakes_fail_golden():
    g = json.load(open(GOLDEN))
    wrong_dir = [(2 + t) % 4 for t in range(4)]
    assert wrong_dir != g["rank2_rotation"]
    swapped = {r: [2 * 4 - 1 - r, r] for r in range(4)}  # local order swapped
    assert {str(r): v for r, v in swapped.items()} != g["zigzag"]
    off_by_one = {r: sum(q for q in qs) for r, qs in oracle.zigzag_assignment(4, 2).items()}
    assert {str(r): v for r, v in off_by_one.items()} != g["zigzag_workload"]


def test_planted_fold_mistake_fails():
    # dropping the rescale of the old O (a classic online-softmax slip) breaks
    # the equality with the definition
    S, d, P = 12, 4, 3
    Q = _rand((1, S, 1, d), (43,))
    K = _rand((1, S, 1, d), (44,))
    V = _rand((1, S, 1, d), (45,))
    O, _ = oracle.attention(Q, K, V, False)
    q, k, v = (oracle.to_f64(x)[0, :, 0] for x in (Q, K, V))
    m = np.full(S, -np.inf); l = np.zeros(S); o = np.zeros((S, d))
    for s0 in range(0, S, S // P):
        sc = q @ k[s0:s0 + S // P].T / math.sqrt(d)
        mn = np.maximum(m, sc.max(1))
        p = np.exp(sc - mn[:, None])
        ln = l * np.exp(m - mn) + p.sum(1)
        o = o * (l / ln)[:, None] + p / ln[:, None] @ v[s0:s0 + S // P]   # missing exp(m - m~)
        m, l = mn, ln
    assert np.abs(o - O[0, :, 0]).max() > 1e-6


def test_planted_layout_mistakes_fail_a_pin():
    # odd picks counted from the wrong end / with the rank's sign flipped
    def mutant(P, k, sign):
        total = P * k
        return {r: [(i // 2) * P + r if i % 2 == 0 else total - 1 - (i // 2) * P + sign * r
                    for i in range(k)] for r in range(P)}
    good = oracle.zigzag_assignment(4, 4)
    assert mutant(4, 4, -1) == good
    assert mutant(4, 4, +1) != good
    # a striped split read as contiguous blocks breaks the striped closed form
    S, P = 64, 4
    n = S // P
    contiguous_as_striped = [sum(range(r * n + 1, (r + 1) * n + 1)) for r in range(P)]
    assert contiguous_as_striped != [n * (r + 1) + P * n * (n - 1) // 2 for r in range(P)]


# ------------------------------------------------------ round-robin KV cache

def test_helix_round_robin_hand_written():
    # 10 tokens in blocks of 2 over 3 devices: blocks 0..4 go to devices
    # 0, 1, 2, 0, 1 (written out by hand)
    got = [x.tolist() for x in oracle.helix_round_robin(10, 2, 3)]
    assert got == [[0, 1, 6, 7], [2, 3, 8, 9], [4, 5]]
    # a short last block
    got = [x.tolist() for x in oracle.helix_round_robin(7, 3, 2)]
    assert got == [[0, 1, 2, 6], [3, 4, 5]]
    assert [x.tolist() for x in oracle.helix_round_robin(0, 4, 2)] == [[], []]


@pytest.mark.parametrize("total,block,P", [(1, 1, 1), (100, 16, 8), (1000, 7, 3), (4096, 64, 8),
                                           (33, 40, 4)])
def test_helix_round_robin_balance(total, block, P):
    sh = oracle.helix_round_robin(total, block, P)
    allpos = np.concatenate(sh)
    assert sorted(allpos.tolist()) == list(range(total))     # every token exactly once
    lens = [len(x) for x in sh]
    assert max(lens) - min(lens) <= block                    # memory grows evenly
    assert lens[0] == max(lens)                              # device 0 is served first
    for x in sh:
        assert np.all(np.diff(x) > 0)                        # local order is sequence order
    # appending one token at a time deals the same positions
    inc = [[] for _ in range(P)]
    for t in range(total):
        inc[(t // block) % P].append(t)
    assert [x.tolist() for x in sh] == inc


def test_decode_over_round_robin_shards_equals_full():
    # the merge of per-device partials over the round-robin shards is the
    # attention over all keys, whatever the dealing
    B, Skv, Hq, Hkv, d = 2, 57, 4, 2, 8
    Q = _rand((B, 1, Hq, d), (50,))
    K = _rand((B, Skv, Hkv, d), (51,))
    V = _rand((B, Skv, Hkv, d), (52,))
    O, lse = oracle.attention(Q, K, V, False)
    parts_O, parts_l = [], []
    for pos in oracle.helix_round_robin(Skv, 5, 4):
        Op, lp = oracle.attention(Q, K[:, pos], V[:, pos], False)
        parts_O.append(Op.reshape(B * Hq, d))
        parts_l.append(lp.reshape(B * Hq))
    Om, lm = oracle.merge(np.stack(parts_O), np.stack(parts_l))
    np.testing.assert_allclose(Om, O.reshape(B * Hq, d), atol=1e-12)
    np.testing.assert_allclose(lm, lse.reshape(B * Hq), atol=1e-12)


# ----------------------------------------------------------- Ulysses heads

def test_ulysses_scatter_hand_written():
    # B1, S2, H4 (d = 1) over 2 ranks: rank 0 gets heads 0, 1 of both tokens,
    # rank 1 heads 2, 3 (written out by hand)
    x = np.array([[[[0], [1], [2], [3]], [[10], [11], [12], [13]]]])
    y = oracle.ulysses_scatter_heads(x, 2)
    assert y[..., 0].tolist() == [[[[0, 1], [10, 11]]], [[[2, 3], [12, 13]]]]
    assert np.array_equal(oracle.ulysses_gather_heads(y), x)
    with pytest.raises(ValueError):
        oracle.ulysses_scatter_heads(x, 3)       # heads must divide by the ranks


def test_ulysses_memory_equals_ring():
    # section 5: per rank the attention phase holds s * h / N, the ring's (s / N) * h
    B, S, H, d, P = 1, 64, 8, 4, 4
    x = np.zeros((B, S, H, d))
    y = oracle.ulysses_scatter_heads(x, P)
    assert y[0].size == oracle.natural_positions(S, P, "contiguous")[: S // P].size * H * d


@pytest.mark.parametrize("Hq,Hkv,P", [(4, 4, 2), (8, 2, 2), (16, 4, 4)])
def test_ulysses_attention_equals_full(Hq, Hkv, P):
    # attention per head group over the whole sequence, gathered back, is full
    # causal attention (GQA groups stay together since P divides Hkv)
    B, S, d = 1, 24, 8
    Q = _rand((B, S, Hq, d), (60, Hq))
    K = _rand((B, S, Hkv, d), (61, Hkv))
    V = _rand((B, S, Hkv, d), (62, Hkv))
    O_t, lse_t = _sdpa_f64(Q, K, V, True)
    Qg, Kg, Vg = (oracle.ulysses_scatter_heads(x, P) for x in (Q, K, V))
    Og = np.stack([oracle.attention(Qg[g], Kg[g], Vg[g], True)[0] for g in range(P)])
    Lg = np.stack([oracle.attention(Qg[g], Kg[g], Vg[g], True)[1] for g in range(P)])
    np.testing.assert_allclose(oracle.ulysses_gather_heads(Og), O_t, atol=1e-12)
    np.testing.assert_allclose(np.concatenate(list(Lg), axis=1), lse_t, atol=1e-12)
