"""GPU parity at the five workload sizes of the hot path, in the launch
configuration the benchmark times.

Small workloads are checked on every output row; the 32k and 128k-token
workloads on seeded sampled rows (per rank: the first and last row of each
of its chunks plus 60 rows drawn with numpy.random.default_rng([cfg, 3,
rank])), every query head; the 1M-key decode on all 8 of its sequences, every
head (one query row per sequence and head)."""
import dataclasses

import numpy as np
import pytest
import torch

import long_context_exact_amd as ra
import oracle
from gpu_helpers import check, fmt, from_dev, log, sample_rows, shard, to_dev, unshard
from long_context_exact_amd import synthetic
from long_context_exact_amd.workloads import WORKLOADS

pytestmark = pytest.mark.gpu

ROWS_PER_RANK = 60  # drawn rows per rank of the sampled workloads (besides chunk ends)


def _inputs(w):
    Q = synthetic.normal_tensor(w.q_shape, w.seed(0), w.dtype)
    K = synthetic.normal_tensor(w.kv_shape, w.seed(1), w.dtype)
    V = synthetic.normal_tensor(w.kv_shape, w.seed(2), w.dtype)
    return Q, K, V


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


@pytest.mark.parametrize("cfg,layout", [(1, None), (2, None), (3, None), (4, None),
                                        (3, "zigzag4"), (3, "striped")])
def test_prefill_workload(cfg, layout):
    """layout: None for the workload's own split; otherwise the same inputs and
    shape under another split (the causal rebalancing variants)."""
    w = WORKLOADS[cfg]
    if layout is not None:
        w = dataclasses.replace(w, layout=layout, name=f"{w.name}-as-{layout}")
    log(f"workload {cfg} {w.name}: generating inputs")
    Qn, Kn, Vn = _inputs(w)
    S, P, lay = w.S, w.P, w.layout
    Qs, Ks, Vs = (to_dev(shard(x, S, P, lay)) for x in (Qn, Kn, Vn))
    # fp32 output: the accumulator unrounded (a bf16 output is the same values
    # rounded to nearest even, checked below)
    O = torch.empty(w.B, S, w.Hq, w.d, dtype=torch.float32, device="cuda")
    L = torch.empty(w.B, w.Hq, S, dtype=torch.float32, device="cuda")
    log(f"workload {cfg}: ra_fwd_all")
    ra.ra_fwd_all(Qs, Ks, Vs, O, L, P, w.causal, lay)
    torch.cuda.synchronize()

    # each rank alone (the benchmark times ra_fwd_rank) equals ra_fwd_all bit for bit
    n = S // P
    ranks = range(P) if cfg <= 3 else [0, P - 1]
    for r in ranks:
        log(f"workload {cfg}: ra_fwd_rank({r})")
        Qr = Qs[:, r * n:(r + 1) * n]
        Or = torch.empty(Qr.shape, dtype=torch.float32, device="cuda")
        Lr = torch.empty(w.B, w.Hq, n, dtype=torch.float32, device="cuda")
        ra.ra_fwd_rank(Qr, Ks, Vs, Or, Lr, P, r, w.causal, lay)
        torch.cuda.synchronize()
        assert torch.equal(Or, O[:, r * n:(r + 1) * n]), f"rank {r}"
        assert torch.equal(Lr, L[:, :, r * n:(r + 1) * n]), f"rank {r} LSE"
        del Or, Lr
    if w.dtype == "bf16":
        Ob = torch.empty(O.shape, dtype=torch.bfloat16, device="cuda")
        Lb = torch.empty_like(L)
        ra.ra_fwd_all(Qs, Ks, Vs, Ob, Lb, P, w.causal, lay)
        torch.cuda.synchronize()
        assert torch.equal(_bits(Ob), _bits(O.to(torch.bfloat16))) and torch.equal(Lb, L)
        del Ob, Lb

    O_h = unshard(from_dev(O), S, P, lay, axis=1)
    L_h = unshard(from_dev(L), S, P, lay, axis=2)
    del Qs, Ks, Vs, O, L
    torch.cuda.empty_cache()
    if cfg <= 2:
        log(f"workload {cfg}: oracle on all {S} rows")
        O_ref, L_ref = oracle.attention(Qn, Kn, Vn, w.causal)
        e = check(O_h, O_ref, L_h, L_ref, w.dtype, w.name)
    else:
        rows = sample_rows(S, P, lay, ROWS_PER_RANK, [cfg, 3])
        log(f"workload {cfg}: oracle on {len(rows)} sampled rows")
        O_ref, L_ref = oracle.attention_rows(Qn, Kn, Vn, w.causal, np.zeros_like(rows), rows)
        e = check(O_h[0, rows], O_ref, L_h[0][:, rows].T, L_ref, w.dtype, w.name)
    log(f"workload {cfg}: ok {fmt(e)}")


def _check_decode_sequences(w, qh, O_g, L_g, what):
    """Every sequence of the decode workload against the oracle: its query
    row of every head over all of its keys.  Each sequence's K/V are
    regenerated on the host from the same seeded ranges."""
    per_seq = w.S * w.Hkv * w.d
    for b in range(w.B):
        log(f"workload 5 {what}: oracle on sequence {b}")
        Kb = synthetic.normal_range(w.seed(1), b * per_seq, (b + 1) * per_seq, "bf16")
        Vb = synthetic.normal_range(w.seed(2), b * per_seq, (b + 1) * per_seq, "bf16")
        Kb = Kb.reshape(1, w.S, w.Hkv, w.d)
        Vb = Vb.reshape(1, w.S, w.Hkv, w.d)
        O_ref, L_ref = oracle.attention_rows(qh[b:b + 1], Kb, Vb, False, [0], [0])
        e = check(O_g[b][None], O_ref, L_g[b][None], L_ref, "bf16", f"{what} sequence {b}")
        log(f"workload 5 {what} sequence {b}: ok {fmt(e)}")
        del Kb, Vb


def test_decode_workload():
    w = WORKLOADS[5]
    parts = 64            # 8 shards x 8 parts, as the benchmark runs it
    log(f"workload 5 {w.name}: generating 2 x 16 GiB of K/V")
    Q = synthetic.to_device(w.q_shape, w.seed(0), "bf16")
    K = synthetic.to_device(w.kv_shape, w.seed(1), "bf16")
    V = synthetic.to_device(w.kv_shape, w.seed(2), "bf16")
    rows = w.B * w.Sq * w.Hq
    Op = torch.empty(parts, rows, w.d, dtype=torch.float32, device="cuda")
    lp = torch.empty(parts, rows, dtype=torch.float32, device="cuda")
    O = torch.empty(rows, w.d, dtype=torch.float32, device="cuda")
    Ob = torch.empty(rows, w.d, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(rows, dtype=torch.float32, device="cuda")
    log("workload 5: ra_attn_partial + ra_merge_partials")
    ra.ra_attn_partial(Q, K, V, Op, lp, parts)
    ra.ra_merge_partials(Op, lp, O, lse)
    ra.ra_merge_partials(Op, lp, Ob)
    # the two-level combine a sharded deployment would do: merge each shard's
    # 8 parts, then merge the 8 shard results
    shard_O = torch.empty(w.P, rows, w.d, dtype=torch.float32, device="cuda")
    shard_l = torch.empty(w.P, rows, dtype=torch.float32, device="cuda")
    per = parts // w.P
    for s in range(w.P):
        ra.ra_merge_partials(Op[s * per:(s + 1) * per].contiguous(),
                             lp[s * per:(s + 1) * per].contiguous(), shard_O[s], shard_l[s])
    O2 = torch.empty_like(O)
    lse2 = torch.empty_like(lse)
    ra.ra_merge_partials(shard_O, shard_l, O2, lse2)
    torch.cuda.synchronize()
    assert torch.equal(Ob.view(torch.int16), O.to(torch.bfloat16).view(torch.int16))
    O_g = from_dev(O).reshape(w.B, w.Hq, w.d)
    L_g = from_dev(lse).reshape(w.B, w.Hq)
    O2_g = from_dev(O2).reshape(w.B, w.Hq, w.d)
    assert np.abs(O2_g - O_g).max() <= 1e-5 * max(1.0, np.abs(O_g).max())
    assert np.abs(from_dev(lse2).reshape(w.B, w.Hq) - L_g).max() <= 1e-5
    qh = Q.cpu().view(torch.int16).numpy().view(np.uint16)
    del K, V, Op, lp, shard_O, shard_l
    torch.cuda.empty_cache()
    _check_decode_sequences(w, qh, O_g, L_g, "contiguous cache")


def test_decode_workload_round_robin_cache():
    """The 1M-key decode workload with its cache dealt round-robin in blocks
    of 64 tokens over the 8 shards (built by ra_kv_append_rr), 8 parts per
    shard, merged; checked against the oracle on all 8 sequences."""
    w = WORKLOADS[5]
    block, pps = 64, 8
    log(f"workload 5 {w.name}: round-robin cache, blocks of {block}")
    Q = synthetic.to_device(w.q_shape, w.seed(0), "bf16")
    shards = oracle.helix_round_robin(w.S, block, w.P)
    cap = max(len(x) for x in shards)
    Kc = torch.empty(w.P, w.B, cap, w.Hkv, w.d, dtype=torch.bfloat16, device="cuda")
    Vc = torch.empty_like(Kc)
    K = synthetic.to_device(w.kv_shape, w.seed(1), "bf16")
    V = synthetic.to_device(w.kv_shape, w.seed(2), "bf16")
    cut = 777_777  # two appends, the second starting inside a block
    ra.ra_kv_append_rr(Kc, Vc, K[:, :cut].contiguous(), V[:, :cut].contiguous(), 0, block)
    ra.ra_kv_append_rr(Kc, Vc, K[:, cut:].contiguous(), V[:, cut:].contiguous(), cut, block)
    torch.cuda.synchronize()
    del K, V
    torch.cuda.empty_cache()
    rows = w.B * w.Sq * w.Hq
    parts = w.P * pps
    Op = torch.empty(parts, rows, w.d, dtype=torch.float32, device="cuda")
    lp = torch.empty(parts, rows, dtype=torch.float32, device="cuda")
    O = torch.empty(rows, w.d, dtype=torch.float32, device="cuda")
    lse = torch.empty(rows, dtype=torch.float32, device="cuda")
    log("workload 5: ra_attn_partial_rr + ra_merge_partials")
    ra.ra_attn_partial_rr(Q, Kc, Vc, Op, lp, w.S, block, pps)
    ra.ra_merge_partials(Op, lp, O, lse)
    torch.cuda.synchronize()
    O_g = from_dev(O).reshape(w.B, w.Hq, w.d)
    L_g = from_dev(lse).reshape(w.B, w.Hq)
    qh = Q.cpu().view(torch.int16).numpy().view(np.uint16)
    del Kc, Vc, Op, lp
    torch.cuda.empty_cache()
    _check_decode_sequences(w, qh, O_g, L_g, "round-robin cache")
