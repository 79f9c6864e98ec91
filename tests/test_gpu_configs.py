"""GPU parity at the five workload sizes of the hot path, in the launch
configurations the benchmark times (for the prefill: the plain entry points
and the _ws ones with the automatic key-range count).

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
    # the benchmark's first stage: the layout kernel gathers the natural-order
    # tensors on the device into the sharded order, equal to the host's
    for name, x, xs in (("Q", Qn, Qs), ("K", Kn, Ks), ("V", Vn, Vs)):
        xn = to_dev(x)
        xg = torch.empty_like(xn)
        ra.ra_layout_gather(xn, xg, S, P, lay, inverse=False)
        torch.cuda.synchronize()
        raw = torch.int16 if xg.dtype == torch.bfloat16 else torch.int32
        assert torch.equal(xg.view(raw), xs.view(raw)), f"layout gather of {name}"
        del xn, xg
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

    # The benchmark times the _ws entry points with the automatic key-range
    # count: each rank's share (ra_fwd_rank_ws) and all ranks in one launch
    # (ra_fwd_all_ws).  Where the count is one they are the launches above, bit
    # for bit; otherwise their results go to the oracle as well.
    outs = [("ra_fwd_all", O, L)]
    code = ra.DTYPE_BF16 if w.dtype == "bf16" else ra.DTYPE_F32
    nb_r = ra.ra_fwd_workspace_bytes(w.B, w.Hq, w.Hkv, S, w.d, P, False, w.causal, lay, code, 0)
    nb_a = ra.ra_fwd_workspace_bytes(w.B, w.Hq, w.Hkv, S, w.d, P, True, w.causal, lay, code, 0)
    ws_r = torch.full((max(nb_r, 16) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    O_r = torch.empty_like(O)
    L_r = torch.empty_like(L)
    for r in ranks:
        log(f"workload {cfg}: ra_fwd_rank_ws({r}), automatic ranges")
        Qr = Qs[:, r * n:(r + 1) * n]
        Orw = torch.empty(Qr.shape, dtype=torch.float32, device="cuda")
        Lrw = torch.empty(w.B, w.Hq, n, dtype=torch.float32, device="cuda")
        ra.ra_fwd_rank_ws(Qr, Ks, Vs, Orw, Lrw, P, r, w.causal, lay, 0, ws_r if nb_r else None)
        torch.cuda.synchronize()
        O_r[:, r * n:(r + 1) * n] = Orw
        L_r[:, :, r * n:(r + 1) * n] = Lrw
        if nb_r == 0:
            assert torch.equal(Orw, O[:, r * n:(r + 1) * n]) and torch.equal(Lrw, L[:, :, r * n:(r + 1) * n])
        del Orw, Lrw
    del ws_r
    if nb_r and len(ranks) == P:
        outs.append(("ra_fwd_rank_ws", O_r, L_r))
    else:
        del O_r, L_r
    log(f"workload {cfg}: ra_fwd_all_ws, automatic ranges")
    ws_a = torch.full((max(nb_a, 16) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    O_a = torch.empty_like(O)
    L_a = torch.empty_like(L)
    ra.ra_fwd_all_ws(Qs, Ks, Vs, O_a, L_a, P, w.causal, lay, 0, ws_a if nb_a else None)
    torch.cuda.synchronize()
    del ws_a
    if nb_a == 0:
        assert torch.equal(O_a, O) and torch.equal(L_a, L)
        del O_a, L_a
    else:
        outs.append(("ra_fwd_all_ws", O_a, L_a))
    del Qs, Ks, Vs, O, L
    hosts = []
    for what, Od, Ld in outs:
        hosts.append((what, unshard(from_dev(Od), S, P, lay, axis=1), unshard(from_dev(Ld), S, P, lay, axis=2)))
    del outs, Od, Ld
    torch.cuda.empty_cache()
    if cfg <= 2:
        log(f"workload {cfg}: oracle on all {S} rows")
        O_ref, L_ref = oracle.attention(Qn, Kn, Vn, w.causal)
        for what, O_h, L_h in hosts:
            e = check(O_h, O_ref, L_h, L_ref, w.dtype, f"{w.name} {what}")
            log(f"workload {cfg} {what}: ok {fmt(e)}")
    else:
        rows = sample_rows(S, P, lay, ROWS_PER_RANK, [cfg, 3])
        log(f"workload {cfg}: oracle on {len(rows)} sampled rows")
        O_ref, L_ref = oracle.attention_rows(Qn, Kn, Vn, w.causal, np.zeros_like(rows), rows)
        for what, O_h, L_h in hosts:
            e = check(O_h[0, rows], O_ref, L_h[0][:, rows].T, L_ref, w.dtype, f"{w.name} {what}")
            log(f"workload {cfg} {what}: ok {fmt(e)}")


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


@pytest.mark.parametrize("cfg", [3, 4])
def test_ring_steps_workload(cfg):
    """The ring-step launches the benchmark times (``--ring-steps``): rank 0's
    P steps of the 32k and 128k-token workloads, each on a copy of the block
    that has arrived, with one key range (ra_ring_step) and with the automatic
    count (ra_ring_step_ws).  Both against the oracle on rank 0's sampled
    rows (the first and last row of each of its chunks plus 60 drawn with
    numpy.random.default_rng([cfg, 4, 0])), every query head."""
    w = WORKLOADS[cfg]
    log(f"workload {cfg} {w.name}: ring steps, generating inputs")
    Qn, Kn, Vn = _inputs(w)
    S, P, lay = w.S, w.P, w.layout
    Qs, Ks, Vs = (to_dev(shard(x, S, P, lay)) for x in (Qn, Kn, Vn))
    n, r = S // P, 0
    Qr = Qs[:, :n].contiguous()
    code = ra.DTYPE_BF16 if w.dtype == "bf16" else ra.DTYPE_F32
    nb = ra.ra_fwd_workspace_bytes(w.B, w.Hq, w.Hkv, S, w.d, P, False, w.causal, lay, code, 0)
    ws = torch.full((max(nb, 16) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    outs = []
    for splits in (None, 0):
        O = torch.empty(w.B, n, w.Hq, w.d, dtype=torch.float32, device="cuda")
        L = torch.empty(w.B, w.Hq, n, dtype=torch.float32, device="cuda")
        for t in range(P):
            s = (r - t) % P
            Kb = Ks[:, s * n:(s + 1) * n].contiguous()
            Vb = Vs[:, s * n:(s + 1) * n].contiguous()
            if splits is None:
                ra.ra_ring_step(Qr, Kb, Vb, O, L, S, P, r, t, w.causal, lay)
            else:
                ra.ra_ring_step_ws(Qr, Kb, Vb, O, L, S, P, r, t, w.causal, lay, splits, ws)
            del Kb, Vb
        torch.cuda.synchronize()
        outs.append(("ra_ring_step" if splits is None else "ra_ring_step_ws", from_dev(O), from_dev(L)))
        del O, L
    del Qs, Ks, Vs, Qr, ws
    torch.cuda.empty_cache()
    # rank 0's local rows: the two ends of each chunk and 60 drawn rows
    pos = oracle.natural_positions(S, P, lay)[:n]
    c = oracle.chunk_len(lay, S, P)
    local = [k for k0 in range(0, n, c) for k in (k0, k0 + c - 1)]
    local += list(np.random.default_rng([cfg, 4, 0]).choice(n, size=ROWS_PER_RANK, replace=False))
    local = np.unique(np.asarray(local, dtype=np.int64))
    log(f"workload {cfg}: oracle on {len(local)} rows of rank 0")
    O_ref, L_ref = oracle.attention_rows(Qn, Kn, Vn, w.causal, np.zeros_like(local), pos[local])
    for what, O_h, L_h in outs:
        e = check(O_h[0, local], O_ref, L_h[0][:, local].T, L_ref, w.dtype, f"{w.name} {what}")
        log(f"workload {cfg} {what}: ok {fmt(e)}")


@pytest.mark.parametrize("cfg", [3, 4])
def test_ulysses_workload(cfg):
    """The Ulysses launches the benchmark times (``--ulysses``) on the 32k and
    128k-token workloads: all-to-all of Q, K, V from natural order to P head
    groups (ra_head_a2a), attention of the groups as one batch over the whole
    sequence (ra_fwd_all_ws, one shard, automatic key ranges), all-to-all of
    O and LSE back; against the oracle on the sampled rows of
    test_prefill_workload, every query head."""
    w = WORKLOADS[cfg]
    log(f"workload {cfg} {w.name}: Ulysses, generating inputs")
    Qn, Kn, Vn = _inputs(w)
    B, S, P, d = w.B, w.S, w.P, w.d
    Gq, Gkv = w.Hq // P, w.Hkv // P
    Qd, Kd, Vd = to_dev(Qn), to_dev(Kn), to_dev(Vn)
    Qh = torch.empty(P * B, S, Gq, d, dtype=Qd.dtype, device="cuda")
    Kh = torch.empty(P * B, S, Gkv, d, dtype=Kd.dtype, device="cuda")
    Vh = torch.empty_like(Kh)
    es = Qd.element_size()
    ra.ra_head_a2a(Qd, Qh, B, S, P, Gq * d * es, False)
    ra.ra_head_a2a(Kd, Kh, B, S, P, Gkv * d * es, False)
    ra.ra_head_a2a(Vd, Vh, B, S, P, Gkv * d * es, False)
    del Qd, Kd, Vd
    Oh = torch.empty(P * B, S, Gq, d, dtype=torch.float32, device="cuda")
    Lh = torch.empty(P * B, Gq, S, dtype=torch.float32, device="cuda")
    code = ra.DTYPE_BF16 if w.dtype == "bf16" else ra.DTYPE_F32
    nb = ra.ra_fwd_workspace_bytes(P * B, Gq, Gkv, S, d, 1, True, w.causal, "contiguous", code, 0)
    ws = torch.full((max(nb, 16) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    log(f"workload {cfg}: ra_fwd_all_ws over {P} head groups, {nb} workspace bytes")
    ra.ra_fwd_all_ws(Qh, Kh, Vh, Oh, Lh, 1, w.causal, "contiguous", 0, ws if nb else None)
    del Qh, Kh, Vh, ws
    O = torch.empty(B, S, w.Hq, d, dtype=torch.float32, device="cuda")
    L = torch.empty(B, w.Hq, S, dtype=torch.float32, device="cuda")
    ra.ra_head_a2a(Oh, O, B, S, P, Gq * d * 4, True)
    ra.ra_head_a2a(Lh, L, B, 1, P, Gq * S * 4, True)
    torch.cuda.synchronize()
    del Oh, Lh
    rows = sample_rows(S, P, w.layout, ROWS_PER_RANK, [cfg, 3])
    idx = torch.as_tensor(rows, device="cuda")
    O_h = from_dev(O[0, idx])
    L_h = from_dev(L[0][:, idx]).T
    del O, L
    torch.cuda.empty_cache()
    log(f"workload {cfg}: oracle on {len(rows)} sampled rows")
    O_ref, L_ref = oracle.attention_rows(Qn, Kn, Vn, w.causal, np.zeros_like(rows), rows)
    e = check(O_h, O_ref, L_h, L_ref, w.dtype, f"{w.name} Ulysses")
    log(f"workload {cfg} Ulysses: ok {fmt(e)}")
