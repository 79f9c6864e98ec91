"""GPU parity of the three kernels against the fp64 oracle on small shapes
that span several tiles and ragged tails, in every layout / mask / dtype /
head-dim combination, plus the structural checks: ra_fwd_all equals the
concatenated ra_fwd_rank bit for bit, runs are deterministic, and writes stay
inside their outputs."""
import numpy as np
import pytest
import torch

import long_context_exact_amd as ra
import oracle
from gpu_helpers import (BF16_O_MAX, F32_O_MAX, check, fmt, from_dev, log, qkv, scale_bf16, shard,
                         to_dev, unshard)

pytestmark = pytest.mark.gpu

PREFILL = [  # B, S, Hq, Hkv, d, P, layout, causal, dtype
    (1, 1024, 2, 2, 64, 4, "contiguous", False, "f32"),
    (1, 1024, 2, 2, 64, 4, "contiguous", True, "f32"),
    (1, 520, 4, 2, 64, 4, "zigzag", True, "f32"),       # chunks of 65: ragged tiles
    (2, 384, 2, 1, 128, 3, "zigzag", True, "f32"),
    (1, 2048, 8, 8, 128, 8, "contiguous", True, "bf16"),
    (2, 640, 4, 2, 128, 4, "zigzag", True, "bf16"),     # chunks of 80
    (1, 96, 3, 1, 64, 3, "contiguous", True, "bf16"),   # shards of 32
    (2, 1200, 4, 4, 128, 5, "zigzag", False, "bf16"),   # chunks of 120
    (1, 300, 2, 2, 128, 1, "contiguous", True, "bf16"), # one rank
    (1, 300, 2, 2, 64, 1, "zigzag", True, "bf16"),      # one rank, two chunks
    (1, 512, 2, 2, 64, 16, "zigzag", True, "bf16"),     # chunks of 16
    (1, 4096, 8, 2, 128, 4, "zigzag", True, "bf16"),    # GQA, chunks of 512
    # k chunks per rank and the striped split
    (1, 768, 2, 2, 64, 4, "zigzag3", True, "f32"),      # chunks of 64
    (1, 520, 2, 1, 64, 2, "striped", True, "f32"),      # shards of 260
    (2, 1280, 4, 2, 128, 4, "zigzag4", True, "bf16"),   # chunks of 80
    (1, 2304, 4, 4, 128, 8, "zigzag3", True, "bf16"),   # chunks of 96, unbalanced k
    (1, 1040, 4, 2, 128, 4, "striped", True, "bf16"),   # shards of 260: ragged tiles
    (1, 1536, 2, 2, 64, 3, "striped", False, "bf16"),
    (1, 600, 2, 2, 128, 1, "zigzag6", True, "bf16"),    # one rank, six chunks of 100
    (1, 512, 2, 2, 64, 1, "striped", True, "bf16"),     # one rank: the identity
    (1, 4096, 8, 2, 128, 8, "striped", True, "bf16"),   # GQA
    (1, 4096, 8, 2, 128, 4, "zigzag8", True, "bf16"),   # chunks of 128
]


def _id(c):
    B, S, Hq, Hkv, d, P, lay, causal, dt = c
    return f"B{B}-S{S}-Hq{Hq}-Hkv{Hkv}-d{d}-P{P}-{lay}-{'causal' if causal else 'full'}-{dt}"


def _run_prefill(Qn, Kn, Vn, P, layout, causal, dtype, out="f32"):
    B, S, Hq, d = Qn.shape
    Qs, Ks, Vs = (to_dev(shard(x, S, P, layout)) for x in (Qn, Kn, Vn))
    tdt = torch.bfloat16 if out == "bf16" else torch.float32
    O = torch.empty(B, S, Hq, d, dtype=tdt, device="cuda")
    L = torch.empty(B, Hq, S, dtype=torch.float32, device="cuda")
    ra.ra_fwd_all(Qs, Ks, Vs, O, L, P, causal, layout)
    torch.cuda.synchronize()
    return (Qs, Ks, Vs), O, L


@pytest.mark.parametrize("case", PREFILL, ids=[_id(c) for c in PREFILL])
def test_prefill_parity(case):
    B, S, Hq, Hkv, d, P, layout, causal, dtype = case
    log(f"prefill {_id(case)}")
    Qn, Kn, Vn = qkv(B, S, S, Hq, Hkv, d, dtype, (1000, S, P))
    (Qs, Ks, Vs), O, L = _run_prefill(Qn, Kn, Vn, P, layout, causal, dtype)
    O_ref, lse_ref = oracle.attention(Qn, Kn, Vn, causal)
    O_nat = unshard(from_dev(O), S, P, layout, axis=1)
    L_nat = unshard(from_dev(L), S, P, layout, axis=2)
    e = check(O_nat, O_ref, L_nat, lse_ref, dtype, _id(case))
    log(f"  ok {fmt(e)}")

    # every rank alone gives the same rows bit for bit
    n = S // P
    for r in range(P):
        Qr = Qs[:, r * n:(r + 1) * n].contiguous()
        Or = torch.empty(Qr.shape, dtype=O.dtype, device="cuda")
        Lr = torch.empty(B, Hq, n, dtype=torch.float32, device="cuda")
        ra.ra_fwd_rank(Qr, Ks, Vs, Or, Lr, P, r, causal, layout)
        torch.cuda.synchronize()
        assert torch.equal(Or, O[:, r * n:(r + 1) * n]), f"rank {r} differs from ra_fwd_all"
        assert torch.equal(Lr, L[:, :, r * n:(r + 1) * n])

    # deterministic
    _, O2, L2 = _run_prefill(Qn, Kn, Vn, P, layout, causal, dtype)
    assert torch.equal(O, O2)
    assert torch.equal(L, L2)

    if dtype == "bf16":
        # a bf16 output is the same fp32 result rounded to nearest even
        _, Ob, Lb = _run_prefill(Qn, Kn, Vn, P, layout, causal, dtype, out="bf16")
        assert torch.equal(Ob.view(torch.int16), O.to(torch.bfloat16).view(torch.int16))
        assert torch.equal(Lb, L)
        check(unshard(from_dev(Ob), S, P, layout, axis=1), O_ref, L_nat, lse_ref, dtype,
              _id(case) + " bf16 out", o_rounded=True)


STRESS = ["peaky", "late_max", "zero_q"]


@pytest.mark.parametrize("kind", STRESS)
@pytest.mark.parametrize("layout", ["contiguous", "zigzag", "zigzag4", "striped"])
def test_prefill_stress_inputs(kind, layout):
    B, S, Hq, Hkv, d, P = 1, 1024, 4, 2, 128, 4
    log(f"stress {kind} {layout}")
    Qn, Kn, Vn = qkv(B, S, S, Hq, Hkv, d, "bf16", (1100, len(kind)))
    if kind == "peaky":      # large scores: big rescales between tiles
        Qn = scale_bf16(Qn, 8.0)
    elif kind == "late_max":  # a dominant key in the last shard of the ring order
        last = oracle.natural_positions(S, P, layout)[(S // P) * 1 + 3]
        Kn = Kn.copy()
        Kn[:, last] = scale_bf16(Kn[:, last], 6.0)
        Qn = scale_bf16(Qn, 3.0)
    else:
        Qn = np.zeros_like(Qn)
    _, O, L = _run_prefill(Qn, Kn, Vn, P, layout, True, "bf16")
    O_ref, lse_ref = oracle.attention(Qn, Kn, Vn, True)
    e = check(unshard(from_dev(O), S, P, layout), O_ref,
              unshard(from_dev(L), S, P, layout, axis=2), lse_ref, "bf16", kind)
    log(f"  ok {fmt(e)}")


def test_prefill_output_guard_bands():
    B, S, Hq, Hkv, d, P, layout = 1, 640, 4, 2, 128, 4, "zigzag"
    Qn, Kn, Vn = qkv(B, S, S, Hq, Hkv, d, "bf16", (1200,))
    Qs, Ks, Vs = (to_dev(shard(x, S, P, layout)) for x in (Qn, Kn, Vn))
    g = 4096
    n_o, n_l = B * S * Hq * d, B * Hq * S
    Obuf = torch.full((n_o + 2 * g,), 7.0, dtype=torch.float32, device="cuda")
    Lbuf = torch.full((n_l + 2 * g,), 7.0, dtype=torch.float32, device="cuda")
    O = Obuf[g:g + n_o].view(B, S, Hq, d)
    L = Lbuf[g:g + n_l].view(B, Hq, S)
    ra.ra_fwd_all(Qs, Ks, Vs, O, L, P, True, layout)
    torch.cuda.synchronize()
    for buf, n in ((Obuf, n_o), (Lbuf, n_l)):
        assert torch.all(buf[:g] == 7.0) and torch.all(buf[g + n:] == 7.0)


DECODE = [  # B, Sq, Hq, Hkv, d, Skv, n_parts, dtype
    (2, 1, 8, 2, 128, 1000, 3, "bf16"),
    (1, 2, 8, 1, 64, 777, 5, "bf16"),      # 16 query rows per kv head
    (1, 1, 32, 1, 128, 4099, 4, "bf16"),   # 32 rows: the full MFMA width
    (3, 1, 4, 4, 128, 70, 8, "f32"),
    (1, 1, 8, 2, 64, 5, 8, "bf16"),        # more parts than keys: empty parts
    (2, 1, 16, 2, 128, 2048, 1, "f32"),
]


@pytest.mark.parametrize("case", DECODE, ids=[str(c) for c in DECODE])
def test_decode_partials_and_merge(case):
    B, Sq, Hq, Hkv, d, Skv, n_parts, dtype = case
    log(f"decode {case}")
    Qn, Kn, Vn = qkv(B, Sq, Skv, Hq, Hkv, d, dtype, (1300, Skv))
    Q, K, V = to_dev(Qn), to_dev(Kn), to_dev(Vn)
    rows = B * Sq * Hq
    Op = torch.empty(n_parts, rows, d, dtype=torch.float32, device="cuda")
    lp = torch.empty(n_parts, rows, dtype=torch.float32, device="cuda")
    ra.ra_attn_partial(Q, K, V, Op, lp, n_parts)
    O = torch.empty(rows, d, dtype=torch.float32, device="cuda")
    lse = torch.empty(rows, dtype=torch.float32, device="cuda")
    ra.ra_merge_partials(Op, lp, O, lse)
    Ob = torch.empty(rows, d, dtype=torch.bfloat16, device="cuda")
    ra.ra_merge_partials(Op, lp, Ob)
    torch.cuda.synchronize()
    # a bf16 output is the fp32 result rounded to nearest even
    assert torch.equal(Ob.view(torch.int16), O.to(torch.bfloat16).view(torch.int16))

    # each part against the oracle on its own key range
    plen = -(-Skv // n_parts)
    Op_h, lp_h = from_dev(Op), from_dev(lp)
    for p in range(n_parts):
        a, b = min(Skv, p * plen), min(Skv, (p + 1) * plen)
        if a == b:
            assert np.all(Op_h[p] == 0) and np.all(lp_h[p] == -np.inf)
            continue
        o_ref, l_ref = oracle.attention(Qn, Kn[:, a:b], Vn[:, a:b], False)
        check(Op_h[p].reshape(B, Sq, Hq, d), o_ref, lp_h[p].reshape(B, Sq, Hq).transpose(0, 2, 1),
              l_ref, "f32" if dtype == "f32" else "bf16", f"part {p}")
    O_ref, lse_ref = oracle.attention(Qn, Kn, Vn, False)
    e = check(from_dev(O).reshape(B, Sq, Hq, d), O_ref,
              from_dev(lse).reshape(B, Sq, Hq).transpose(0, 2, 1), lse_ref, dtype, "merged")
    log(f"  ok {fmt(e)}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("n_parts,rows", [(7, 1000), (2, 999), (70, 1000)])  # few-parts and wave paths
def test_merge_kernel_vs_oracle(d, out, n_parts, rows):
    rng = np.random.default_rng([1400, d, n_parts])
    Op = rng.standard_normal((n_parts, rows, d)).astype(np.float32)
    lp = (rng.standard_normal((n_parts, rows)) * 5).astype(np.float32)
    lp[rng.random((n_parts, rows)) < 0.2] = -np.inf   # empty shards
    lp[:, :3] = -np.inf                                # rows with no key at all
    O = torch.empty(rows, d, dtype=torch.bfloat16 if out == "bf16" else torch.float32, device="cuda")
    lse = torch.empty(rows, dtype=torch.float32, device="cuda")
    ra.ra_merge_partials(to_dev(Op), to_dev(lp), O, lse)
    O_ref, l_ref = oracle.merge(Op.astype(np.float64), lp.astype(np.float64))
    O_g, l_g = from_dev(O), from_dev(lse)
    assert np.all(O_g[:3] == 0) and np.all(l_g[:3] == -np.inf)
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(l_g), fin)
    if out == "f32":
        assert np.abs(O_g - O_ref).max() <= 1e-6 * max(1.0, np.abs(O_ref).max())
    else:  # one bf16 rounding of the output
        assert np.all(np.abs(O_g - O_ref) <= np.abs(O_ref) * 2.0 ** -8 + 1e-6)
    assert np.abs(l_g[fin] - l_ref[fin]).max() <= 1e-6 * max(1.0, np.abs(l_ref[fin]).max())


@pytest.mark.parametrize("layout", ["contiguous", "zigzag", "zigzag4", "striped"])
def test_layout_gather_multi_range_chunks(layout):
    """Chunks of 40 rows x 2 KiB (80 KiB) span two 64 KiB copy ranges, the
    second one ragged; two outer slices."""
    outer, S, P, inner = 2, 160, 2, 2048
    rng = np.random.default_rng(1501)
    x = rng.integers(0, 256, size=(outer, S, inner), dtype=np.uint8)
    src = torch.from_numpy(x).cuda()
    dst = torch.empty_like(src)
    back = torch.empty_like(src)
    ra.ra_layout_gather(src, dst, S, P, layout, inverse=False)
    ra.ra_layout_gather(dst, back, S, P, layout, inverse=True)
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy(), x[:, oracle.natural_positions(S, P, layout)])
    assert np.array_equal(back.cpu().numpy(), x)


@pytest.mark.parametrize("inner", [16, 4, 6, 256, 80])
@pytest.mark.parametrize("layout", ["contiguous", "zigzag", "zigzag3", "zigzag4", "striped"])
def test_layout_gather_bit_exact(inner, layout):
    outer, S, P = 3, 96, 4
    rng = np.random.default_rng([1500, inner])
    x = rng.integers(0, 256, size=(outer, S, inner), dtype=np.uint8)
    src = torch.from_numpy(x).cuda()
    dst = torch.empty_like(src)
    back = torch.empty_like(src)
    ra.ra_layout_gather(src, dst, S, P, layout, inverse=False)
    ra.ra_layout_gather(dst, back, S, P, layout, inverse=True)
    torch.cuda.synchronize()
    expect = x[:, oracle.natural_positions(S, P, layout)]
    assert np.array_equal(dst.cpu().numpy(), expect)
    assert np.array_equal(back.cpu().numpy(), x)


@pytest.mark.parametrize("inner", [2048, 80, 65552])
def test_layout_gather_striped_rows(inner):
    """Striped row copy: rows of 2 KiB (32 rows a work-group), of 80 bytes
    (5 units, most lanes idle) and of 64 KiB + 16 bytes (4 rows a
    work-group, a ragged last work-group); S = 1000 over P = 8."""
    outer, P = 2, 8
    S = 1000 if inner <= 2048 else 40
    rng = np.random.default_rng([1502, inner])
    x = rng.integers(0, 256, size=(outer, S, inner), dtype=np.uint8)
    src = torch.from_numpy(x).cuda()
    dst = torch.empty_like(src)
    back = torch.empty_like(src)
    ra.ra_layout_gather(src, dst, S, P, "striped", inverse=False)
    ra.ra_layout_gather(dst, back, S, P, "striped", inverse=True)
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy(), x[:, oracle.natural_positions(S, P, "striped")])
    assert np.array_equal(back.cpu().numpy(), x)


SPLIT = [  # B, S, Hq, Hkv, d, P, layout, causal, dtype
    (1, 2048, 4, 4, 128, 4, "zigzag", True, "bf16"),     # chunks of 256: one query tile each
    (2, 640, 4, 2, 128, 4, "zigzag", True, "bf16"),      # chunks of 80
    (1, 1024, 2, 2, 64, 8, "contiguous", True, "bf16"),  # shards of 128
    (1, 1040, 4, 2, 128, 4, "striped", True, "bf16"),
    (1, 1200, 2, 1, 128, 5, "zigzag", False, "bf16"),
    (1, 520, 4, 2, 64, 4, "zigzag", True, "f32"),
    (1, 384, 2, 2, 128, 3, "zigzag4", True, "f32"),
]


@pytest.mark.parametrize("case", SPLIT, ids=[_id(c) for c in SPLIT])
def test_prefill_key_range_splits(case):
    """ra_fwd_rank_ws / ra_fwd_all_ws: every split count agrees with the
    oracle; one split is bit-identical to the unsplit entry points; the rows
    of a rank launch equal those of the all-ranks launch for the same count;
    a bf16 output is the fp32 result rounded; the workspace may hold garbage."""
    B, S, Hq, Hkv, d, P, layout, causal, dtype = case
    log(f"splits {_id(case)}")
    Qn, Kn, Vn = qkv(B, S, S, Hq, Hkv, d, dtype, (1200, S, P))
    (Qs, Ks, Vs), O1, L1 = _run_prefill(Qn, Kn, Vn, P, layout, causal, dtype)
    O_ref, lse_ref = oracle.attention(Qn, Kn, Vn, causal)
    n = S // P
    code = 1 if dtype == "bf16" else 0
    for splits in (1, 2, 3, 7, 0):
        nb = ra.ra_fwd_workspace_bytes(B, Hq, Hkv, S, d, P, True, causal, layout, code, splits)
        ws = torch.full((max(nb, 16) // 4,), float("nan"), dtype=torch.float32, device="cuda")
        O = torch.empty_like(O1)
        L = torch.empty_like(L1)
        ra.ra_fwd_all_ws(Qs, Ks, Vs, O, L, P, causal, layout, splits, ws)
        torch.cuda.synchronize()
        if splits == 1:
            assert torch.equal(O, O1) and torch.equal(L, L1)
        e = check(unshard(from_dev(O), S, P, layout, axis=1), O_ref,
                  unshard(from_dev(L), S, P, layout, axis=2), lse_ref, dtype,
                  f"{_id(case)} splits={splits}")
        log(f"  splits={splits} ok {fmt(e)}")
        if splits == 0:
            continue
        for r in (0, P - 1):
            nbr = ra.ra_fwd_workspace_bytes(B, Hq, Hkv, S, d, P, False, causal, layout, code, splits)
            wsr = torch.full((max(nbr, 16) // 4,), float("nan"), dtype=torch.float32, device="cuda")
            Qr = Qs[:, r * n:(r + 1) * n].contiguous()
            Or = torch.empty(Qr.shape, dtype=O.dtype, device="cuda")
            Lr = torch.empty(B, Hq, n, dtype=torch.float32, device="cuda")
            ra.ra_fwd_rank_ws(Qr, Ks, Vs, Or, Lr, P, r, causal, layout, splits, wsr)
            torch.cuda.synchronize()
            assert torch.equal(Or, O[:, r * n:(r + 1) * n]), f"rank {r} splits {splits}"
            assert torch.equal(Lr, L[:, :, r * n:(r + 1) * n])
        if dtype == "bf16" and splits == 3:
            Ob = torch.empty(O.shape, dtype=torch.bfloat16, device="cuda")
            Lb = torch.empty_like(L)
            ra.ra_fwd_all_ws(Qs, Ks, Vs, Ob, Lb, P, causal, layout, splits, ws)
            torch.cuda.synchronize()
            assert torch.equal(Ob.view(torch.int16), O.to(torch.bfloat16).view(torch.int16))
            assert torch.equal(Lb, L)


def test_prefill_auto_splits_fall_back_to_smaller_workspace():
    # a workspace that holds two ranges only: the automatic choice uses two
    B, S, Hq, Hkv, d, P = 1, 1024, 2, 2, 64, 8
    Qn, Kn, Vn = qkv(B, S, S, Hq, Hkv, d, "bf16", (1201,))
    (Qs, Ks, Vs), _, _ = _run_prefill(Qn, Kn, Vn, P, "contiguous", True, "bf16")
    O_ref, lse_ref = oracle.attention(Qn, Kn, Vn, True)
    two = ra.ra_fwd_workspace_bytes(B, Hq, Hkv, S, d, P, True, True, "contiguous", 1, 2)
    assert ra.ra_fwd_workspace_bytes(B, Hq, Hkv, S, d, P, True, True, "contiguous", 1, 0) > two
    ws = torch.empty(two, dtype=torch.uint8, device="cuda")
    outs = []
    for splits, w in ((0, ws), (2, ws), (0, None)):
        O = torch.empty(B, S, Hq, d, dtype=torch.float32, device="cuda")
        L = torch.empty(B, Hq, S, dtype=torch.float32, device="cuda")
        ra.ra_fwd_all_ws(Qs, Ks, Vs, O, L, P, True, "contiguous", splits, w)
        torch.cuda.synchronize()
        outs.append((O, L))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    check(from_dev(outs[2][0]), O_ref, from_dev(outs[2][1]), lse_ref, "bf16", "no workspace")
    check(from_dev(outs[0][0]), O_ref, from_dev(outs[0][1]), lse_ref, "bf16", "two ranges")


RING = [  # B, S, Hq, Hkv, d, P, layout, causal, dtype
    (2, 640, 4, 2, 128, 4, "zigzag", True, "bf16"),
    (1, 1024, 2, 2, 64, 8, "contiguous", True, "bf16"),
    (1, 1040, 4, 2, 128, 4, "striped", True, "bf16"),
    (1, 1200, 2, 1, 128, 5, "zigzag", False, "bf16"),
    (1, 520, 4, 2, 64, 4, "zigzag", True, "f32"),
    (1, 768, 2, 2, 128, 3, "zigzag4", True, "f32"),
]


def _ring_rank(Qs, Ks, Vs, S, P, r, causal, layout, order=None, splits=None):
    """Run rank r's P steps, each on a copy of the arriving block only
    (through ra_ring_step_ws with ``splits`` key ranges when given)."""
    B, _, Hq, d = Qs.shape
    Hkv = Ks.shape[2]
    n = S // P
    Qr = Qs[:, r * n:(r + 1) * n].contiguous()
    O = torch.empty(B, n, Hq, d, dtype=torch.float32, device="cuda")
    L = torch.empty(B, Hq, n, dtype=torch.float32, device="cuda")
    ws = None
    if splits is not None:
        dt = ra.DTYPE_BF16 if Qs.dtype == torch.bfloat16 else ra.DTYPE_F32
        nb = ra.ra_fwd_workspace_bytes(B, Hq, Hkv, S, d, P, False, causal, layout, dt, splits)
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda") if nb > 0 else None
    for t in (order or range(P)):
        s = (r - t) % P
        Kb = Ks[:, s * n:(s + 1) * n].contiguous()
        Vb = Vs[:, s * n:(s + 1) * n].contiguous()
        if splits is None:
            ra.ra_ring_step(Qr, Kb, Vb, O, L, S, P, r, t, causal, layout)
        else:
            ra.ra_ring_step_ws(Qr, Kb, Vb, O, L, S, P, r, t, causal, layout, splits, ws)
    torch.cuda.synchronize()
    return O, L


@pytest.mark.parametrize("case", RING, ids=[_id(c) for c in RING])
def test_ring_step_fold(case):
    """P calls of ra_ring_step, each seeing only the block that has arrived,
    reach the oracle's result (and ra_fwd_rank's within rounding); the steps
    after t = 0 may come in any order."""
    B, S, Hq, Hkv, d, P, layout, causal, dtype = case
    log(f"ring steps {_id(case)}")
    Qn, Kn, Vn = qkv(B, S, S, Hq, Hkv, d, dtype, (1300, S, P))
    (Qs, Ks, Vs), O_all, L_all = _run_prefill(Qn, Kn, Vn, P, layout, causal, dtype)
    O_ref, lse_ref = oracle.attention(Qn, Kn, Vn, causal)
    n = S // P
    O_g = torch.empty_like(O_all)
    L_g = torch.empty_like(L_all)
    for r in range(P):
        O, L = _ring_rank(Qs, Ks, Vs, S, P, r, causal, layout)
        O_g[:, r * n:(r + 1) * n] = O
        L_g[:, :, r * n:(r + 1) * n] = L
    e = check(unshard(from_dev(O_g), S, P, layout, axis=1), O_ref,
              unshard(from_dev(L_g), S, P, layout, axis=2), lse_ref, dtype, _id(case))
    log(f"  ok {fmt(e)}")
    # the two GPU paths round differently (each step normalises its own bf16
    # P); both meet the oracle bar above, and agree within it
    tol = BF16_O_MAX if dtype == "bf16" else F32_O_MAX
    assert (O_g - O_all).abs().max().item() <= tol
    fin = torch.isfinite(L_all)
    assert torch.equal(torch.isfinite(L_g), fin)
    assert (L_g[fin] - L_all[fin]).abs().max().item() <= tol
    # t = 0 first, the rest reversed
    r = P - 1
    O2, L2 = _ring_rank(Qs, Ks, Vs, S, P, r, causal, layout, order=[0] + list(range(P - 1, 0, -1)))
    assert (O2 - O_g[:, r * n:(r + 1) * n]).abs().max().item() <= tol
    assert (L2 - L_g[:, :, r * n:(r + 1) * n]).abs().max().item() <= tol


@pytest.mark.parametrize("case", [RING[0], RING[1], RING[2], RING[5]], ids=lambda c: _id(c))
def test_ring_step_key_range_splits(case):
    """ra_ring_step_ws: one range is ra_ring_step bit for bit; more ranges
    (and the automatic choice) fold the ranges and the running state in one
    merge and reach the oracle's result, in any order of the steps after
    t = 0."""
    B, S, Hq, Hkv, d, P, layout, causal, dtype = case
    log(f"ring steps with splits {_id(case)}")
    Qn, Kn, Vn = qkv(B, S, S, Hq, Hkv, d, dtype, (1350, S, P))
    (Qs, Ks, Vs), _, _ = _run_prefill(Qn, Kn, Vn, P, layout, causal, dtype)
    O_ref, lse_ref = oracle.attention(Qn, Kn, Vn, causal)
    n = S // P
    tol = BF16_O_MAX if dtype == "bf16" else F32_O_MAX
    for r in range(P):
        O1, L1 = _ring_rank(Qs, Ks, Vs, S, P, r, causal, layout)
        Ow, Lw = _ring_rank(Qs, Ks, Vs, S, P, r, causal, layout, splits=1)
        assert torch.equal(O1, Ow) and torch.equal(L1, Lw), f"rank {r}: one range differs"
    for splits in (3, 0):
        O_g = torch.empty(B, S, Hq, d, dtype=torch.float32, device="cuda")
        L_g = torch.empty(B, Hq, S, dtype=torch.float32, device="cuda")
        for r in range(P):
            O, L = _ring_rank(Qs, Ks, Vs, S, P, r, causal, layout, splits=splits)
            O_g[:, r * n:(r + 1) * n] = O
            L_g[:, :, r * n:(r + 1) * n] = L
            O1, L1 = _ring_rank(Qs, Ks, Vs, S, P, r, causal, layout)
            assert (O - O1).abs().max().item() <= tol
            fin = torch.isfinite(L1)
            assert torch.equal(torch.isfinite(L), fin)
            assert (L[fin] - L1[fin]).abs().max().item() <= tol
        e = check(unshard(from_dev(O_g), S, P, layout, axis=1), O_ref,
                  unshard(from_dev(L_g), S, P, layout, axis=2), lse_ref, dtype, f"{_id(case)} splits={splits}")
        log(f"  splits={splits} ok {fmt(e)}")
    # t = 0 first, the rest reversed
    r = P - 1
    O2, L2 = _ring_rank(Qs, Ks, Vs, S, P, r, causal, layout, order=[0] + list(range(P - 1, 0, -1)), splits=3)
    assert (O2 - O_g[:, r * n:(r + 1) * n]).abs().max().item() <= tol
    assert (L2 - L_g[:, :, r * n:(r + 1) * n]).abs().max().item() <= tol


def test_ring_step_automatic_and_many_ranges():
    """The automatic range count of a ring step on a block of 2048 keys is
    two (at most one range per 1024 keys of the block): its result differs
    from one range and equals an explicit kv_splits = 2 bit for bit, and
    every rank reaches the oracle.  Twelve explicit ranges take the merge's
    path for more than eight parts, which folds the running state as its
    first part; most of those ranges are empty on this small block."""
    B, S, Hq, Hkv, d, P, layout, causal, dtype = 1, 16384, 2, 2, 128, 8, "zigzag", True, "bf16"
    log("ring steps, automatic ranges on 2048-key blocks")
    Qn, Kn, Vn = qkv(B, S, S, Hq, Hkv, d, dtype, (1360, S, P))
    Qs, Ks, Vs = (to_dev(shard(x, S, P, layout)) for x in (Qn, Kn, Vn))
    O_ref, lse_ref = oracle.attention(Qn, Kn, Vn, causal)
    n = S // P
    O_g = torch.empty(B, S, Hq, d, dtype=torch.float32, device="cuda")
    L_g = torch.empty(B, Hq, S, dtype=torch.float32, device="cuda")
    for r in range(P):
        O0, L0 = _ring_rank(Qs, Ks, Vs, S, P, r, causal, layout, splits=0)
        O2, L2 = _ring_rank(Qs, Ks, Vs, S, P, r, causal, layout, splits=2)
        O1, L1 = _ring_rank(Qs, Ks, Vs, S, P, r, causal, layout)
        assert torch.equal(O0, O2) and torch.equal(L0, L2), f"rank {r}: automatic != 2 ranges"
        assert not torch.equal(O0, O1), f"rank {r}: automatic choice ran one range"
        O_g[:, r * n:(r + 1) * n] = O0
        L_g[:, :, r * n:(r + 1) * n] = L0
    e = check(unshard(from_dev(O_g), S, P, layout, axis=1), O_ref,
              unshard(from_dev(L_g), S, P, layout, axis=2), lse_ref, dtype, "automatic ranges")
    log(f"  automatic (2 ranges) ok {fmt(e)}")

    B, S, Hq, Hkv, d, P, layout, causal, dtype = RING[0]
    log(f"ring steps with 12 ranges {_id(RING[0])}")
    Qn, Kn, Vn = qkv(B, S, S, Hq, Hkv, d, dtype, (1370, S, P))
    Qs, Ks, Vs = (to_dev(shard(x, S, P, layout)) for x in (Qn, Kn, Vn))
    O_ref, lse_ref = oracle.attention(Qn, Kn, Vn, causal)
    n = S // P
    O_g = torch.empty(B, S, Hq, d, dtype=torch.float32, device="cuda")
    L_g = torch.empty(B, Hq, S, dtype=torch.float32, device="cuda")
    for r in range(P):
        order = [0] + list(range(P - 1, 0, -1)) if r % 2 else None
        O, L = _ring_rank(Qs, Ks, Vs, S, P, r, causal, layout, order=order, splits=12)
        O_g[:, r * n:(r + 1) * n] = O
        L_g[:, :, r * n:(r + 1) * n] = L
    e = check(unshard(from_dev(O_g), S, P, layout, axis=1), O_ref,
              unshard(from_dev(L_g), S, P, layout, axis=2), lse_ref, dtype, "12 ranges")
    log(f"  12 ranges ok {fmt(e)}")


def test_ring_step_without_visible_keys_keeps_the_state():
    """A step whose block holds no key visible to some query rows leaves those
    rows of the running state exactly as they were (the fold with an empty
    block is the identity), with one key range and with several; the rows
    that do see keys reach the oracle.  Zig-zag, P = 4: rank 0 holds chunks 0
    and 7, and after step 0 no later block has a key for chunk 0."""
    B, S, Hq, Hkv, d, P, layout, causal = 1, 4096, 4, 2, 128, 4, "zigzag", True
    log("ring steps with fully masked tiles")
    Qn, Kn, Vn = qkv(B, S, S, Hq, Hkv, d, "bf16", (1380, S, P))
    Qs, Ks, Vs = (to_dev(shard(x, S, P, layout)) for x in (Qn, Kn, Vn))
    O_ref, lse_ref = oracle.attention(Qn, Kn, Vn, causal)
    n, c, r = S // P, S // (2 * P), 0
    Qr = Qs[:, :n].contiguous()
    for splits in (None, 3):
        O = torch.empty(B, n, Hq, d, dtype=torch.float32, device="cuda")
        L = torch.empty(B, Hq, n, dtype=torch.float32, device="cuda")
        ws = None
        if splits is not None:
            nb = ra.ra_fwd_workspace_bytes(B, Hq, Hkv, S, d, P, False, causal, layout, ra.DTYPE_BF16, splits)
            ws = torch.full((nb // 4,), float("nan"), dtype=torch.float32, device="cuda")
        early = None
        for t in range(P):
            s = (r - t) % P
            Kb, Vb = Ks[:, s * n:(s + 1) * n].contiguous(), Vs[:, s * n:(s + 1) * n].contiguous()
            if splits is None:
                ra.ra_ring_step(Qr, Kb, Vb, O, L, S, P, r, t, causal, layout)
            else:
                ra.ra_ring_step_ws(Qr, Kb, Vb, O, L, S, P, r, t, causal, layout, splits, ws)
            torch.cuda.synchronize()
            if t == 0:
                early = (O[:, :c].clone(), L[:, :, :c].clone())
            else:
                assert torch.equal(O[:, :c], early[0]) and torch.equal(L[:, :, :c], early[1]), \
                    f"splits {splits}: step {t} changed the rows of chunk 0"
        # rank 0's rows: chunk 0 (positions 0..c-1) and chunk 7 (the last c)
        pos = np.concatenate([np.arange(c), np.arange(S - c, S)])
        e = check(from_dev(O), O_ref[:, pos], from_dev(L), lse_ref[:, :, pos], "bf16", f"splits {splits}")
        log(f"  splits={splits} ok {fmt(e)}")


def test_ring_step_double_buffered_streams():
    """The schedule a multi-GPU ring would run: while step t computes on one
    receive buffer, the next block is copied into the other on a second
    stream (standing in for the peer-to-peer receive), ordered by events.
    The result equals the single-stream loop bit for bit."""
    B, S, Hq, Hkv, d, P, layout = 1, 2048, 8, 2, 128, 4, "zigzag"
    Qn, Kn, Vn = qkv(B, S, S, Hq, Hkv, d, "bf16", (1301,))
    (Qs, Ks, Vs), _, _ = _run_prefill(Qn, Kn, Vn, P, layout, True, "bf16")
    n = S // P
    r = 1
    ref_O, ref_L = _ring_rank(Qs, Ks, Vs, S, P, r, True, layout)
    comp = torch.cuda.current_stream()
    copy = torch.cuda.Stream()
    Qr = Qs[:, r * n:(r + 1) * n].contiguous()
    bufK = [torch.empty(B, n, Hkv, d, dtype=Ks.dtype, device="cuda") for _ in range(2)]
    bufV = [torch.empty_like(bufK[0]) for _ in range(2)]
    arrived = [torch.cuda.Event() for _ in range(2)]
    free = [torch.cuda.Event() for _ in range(2)]
    O = torch.empty(B, n, Hq, d, dtype=torch.float32, device="cuda")
    L = torch.empty(B, Hq, n, dtype=torch.float32, device="cuda")

    def receive(t):
        s = (r - t) % P
        with torch.cuda.stream(copy):
            if t >= 2:
                copy.wait_event(free[t % 2])
            bufK[t % 2].copy_(Ks[:, s * n:(s + 1) * n])
            bufV[t % 2].copy_(Vs[:, s * n:(s + 1) * n])
            arrived[t % 2].record(copy)

    receive(0)
    for t in range(P):
        if t + 1 < P:
            receive(t + 1)
        comp.wait_event(arrived[t % 2])
        ra.ra_ring_step(Qr, bufK[t % 2], bufV[t % 2], O, L, S, P, r, t, True, layout)
        free[t % 2].record(comp)
    torch.cuda.synchronize()
    assert torch.equal(O, ref_O) and torch.equal(L, ref_L)


RR = [  # B, Sq, Hq, Hkv, d, P, block, total, dtype, parts_per_shard
    (2, 1, 16, 8, 128, 4, 16, 1000, "bf16", 2),
    (1, 2, 8, 1, 64, 3, 7, 200, "bf16", 3),
    (2, 1, 4, 2, 128, 8, 5, 37, "f32", 1),
    (1, 1, 8, 8, 128, 8, 5, 20, "bf16", 2),      # shards 4..7 stay empty
]


@pytest.mark.parametrize("case", RR, ids=[str(c) for c in RR])
def test_round_robin_cache_append_and_decode(case):
    """Tokens appended in uneven pieces land where the dealing of blocks
    puts them (bit-exact, other rows untouched); decoding over the P shard
    caches and merging the partials gives attention over all keys."""
    B, Sq, Hq, Hkv, d, P, block, total, dtype, pps = case
    log(f"round-robin cache {case}")
    Qn, Kn, Vn = qkv(B, Sq, total, Hq, Hkv, d, dtype, (1400, total, P))
    shards = oracle.helix_round_robin(total, block, P)
    cap = max(len(x) for x in shards) + 3
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    Kc = torch.empty(P, B, cap, Hkv, d, dtype=tdt, device="cuda")
    Vc = torch.empty_like(Kc)
    Kc.view(torch.uint8).fill_(0xAB)
    Vc.view(torch.uint8).fill_(0xCD)
    Kd, Vd = to_dev(Kn), to_dev(Vn)
    rng = np.random.default_rng(1401)
    pos = 0
    while pos < total:
        step = int(min(total - pos, rng.choice([1, 2, 5, 37, 130])))
        ra.ra_kv_append_rr(Kc, Vc, Kd[:, pos:pos + step].contiguous(), Vd[:, pos:pos + step].contiguous(),
                           pos, block)
        pos += step
    torch.cuda.synchronize()
    Kh = Kc.cpu().view(torch.uint8).numpy()
    Vh = Vc.cpu().view(torch.uint8).numpy()
    Kb = Kd.cpu().view(torch.uint8).numpy()
    Vb = Vd.cpu().view(torch.uint8).numpy()
    for p_, idx in enumerate(shards):
        L_ = len(idx)
        assert np.array_equal(Kh[p_, :, :L_], Kb[:, idx]), f"K shard {p_}"
        assert np.array_equal(Vh[p_, :, :L_], Vb[:, idx]), f"V shard {p_}"
        assert np.all(Kh[p_, :, L_:] == 0xAB) and np.all(Vh[p_, :, L_:] == 0xCD), f"shard {p_} tail"
    rows = B * Sq * Hq
    Op = torch.empty(P * pps, rows, d, dtype=torch.float32, device="cuda")
    lp = torch.empty(P * pps, rows, dtype=torch.float32, device="cuda")
    O = torch.empty(rows, d, dtype=torch.float32, device="cuda")
    lse = torch.empty(rows, dtype=torch.float32, device="cuda")
    ra.ra_attn_partial_rr(to_dev(Qn), Kc, Vc, Op, lp, total, block, pps)
    ra.ra_merge_partials(Op, lp, O, lse)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(Qn, Kn, Vn, False)
    O_g = from_dev(O).reshape(B, Sq, Hq, d)
    L_g = from_dev(lse).reshape(B, Sq, Hq).transpose(0, 2, 1)
    e = check(O_g, O_ref, L_g, L_ref, dtype, str(case))
    log(f"  ok {fmt(e)}")
    # partials of empty shards carry no weight
    for p_, idx in enumerate(shards):
        if len(idx) == 0:
            assert torch.all(torch.isneginf(lp[p_ * pps:(p_ + 1) * pps]))


@pytest.mark.parametrize("inverse", [False, True])
@pytest.mark.parametrize("B,S,P,run", [(2, 37, 4, 256), (1, 100, 8, 1024), (3, 5, 2, 16), (1, 9, 3, 2064),
                                       (2, 3, 4, 8240), (1, 1, 8, 65536)])  # runs over several 4 KiB segments
def test_head_a2a_bit_exact(B, S, P, run, inverse):
    rng = np.random.default_rng([1600, B, S, P, run])
    if not inverse:
        x = rng.integers(0, 256, size=(B, S, P, run), dtype=np.uint8)
        expect = np.ascontiguousarray(x.transpose(2, 0, 1, 3))
    else:
        x = rng.integers(0, 256, size=(P, B, S, run), dtype=np.uint8)
        expect = np.ascontiguousarray(x.transpose(1, 2, 0, 3))
    src = torch.from_numpy(x).cuda()
    dst = torch.empty(expect.shape, dtype=torch.uint8, device="cuda")
    ra.ra_head_a2a(src, dst, B, S, P, run, inverse)
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy(), expect)


ULYSSES = [  # B, S, Hq, Hkv, d, P, causal, dtype
    (1, 1024, 8, 2, 128, 2, True, "bf16"),
    (2, 640, 8, 8, 64, 4, True, "bf16"),
    (1, 520, 4, 4, 64, 4, False, "f32"),
]


@pytest.mark.parametrize("case", ULYSSES, ids=[str(c) for c in ULYSSES])
def test_ulysses_pipeline(case):
    """All-to-all of Q, K, V to head groups, full-sequence attention of every
    group in one launch (the P groups as a batch, one shard), all-to-all of O
    and LSE back: equals the oracle's attention."""
    B, S, Hq, Hkv, d, P, causal, dtype = case
    log(f"ulysses {case}")
    Qn, Kn, Vn = qkv(B, S, S, Hq, Hkv, d, dtype, (1601, S, P))
    es = 2 if dtype == "bf16" else 4
    Qd, Kd, Vd = to_dev(Qn), to_dev(Kn), to_dev(Vn)
    Qh = torch.empty(P * B, S, Hq // P, d, dtype=Qd.dtype, device="cuda")
    Kh = torch.empty(P * B, S, Hkv // P, d, dtype=Kd.dtype, device="cuda")
    Vh = torch.empty_like(Kh)
    ra.ra_head_a2a(Qd, Qh, B, S, P, Hq // P * d * es, False)
    ra.ra_head_a2a(Kd, Kh, B, S, P, Hkv // P * d * es, False)
    ra.ra_head_a2a(Vd, Vh, B, S, P, Hkv // P * d * es, False)
    Oh = torch.empty(P * B, S, Hq // P, d, dtype=torch.float32, device="cuda")
    Lh = torch.empty(P * B, Hq // P, S, dtype=torch.float32, device="cuda")
    ra.ra_fwd_all(Qh, Kh, Vh, Oh, Lh, 1, causal, "contiguous")
    O = torch.empty(B, S, Hq, d, dtype=torch.float32, device="cuda")
    L = torch.empty(B, Hq, S, dtype=torch.float32, device="cuda")
    ra.ra_head_a2a(Oh, O, B, S, P, Hq // P * d * 4, True)
    ra.ra_head_a2a(Lh, L, B, 1, P, Hq // P * S * 4, True)
    torch.cuda.synchronize()
    O_ref, lse_ref = oracle.attention(Qn, Kn, Vn, causal)
    e = check(from_dev(O), O_ref, from_dev(L), lse_ref, dtype, str(case))
    log(f"  ok {fmt(e)}")


def test_ring_step_state_checkpoint_resume():
    """The running (O, LSE) state is the whole carried state of the ring:
    saved to the host after step 3 and restored into fresh tensors, the
    remaining steps finish bit-identical to an uninterrupted run."""
    B, S, Hq, Hkv, d, P, layout = 1, 2048, 8, 2, 128, 8, "zigzag"
    Qn, Kn, Vn = qkv(B, S, S, Hq, Hkv, d, "bf16", (1302,))
    (Qs, Ks, Vs), _, _ = _run_prefill(Qn, Kn, Vn, P, layout, True, "bf16")
    n = S // P
    r = 5
    ref_O, ref_L = _ring_rank(Qs, Ks, Vs, S, P, r, True, layout)
    Qr = Qs[:, r * n:(r + 1) * n].contiguous()
    O = torch.empty(B, n, Hq, d, dtype=torch.float32, device="cuda")
    L = torch.empty(B, Hq, n, dtype=torch.float32, device="cuda")

    def step(t, O_, L_):
        s = (r - t) % P
        ra.ra_ring_step(Qr, Ks[:, s * n:(s + 1) * n].contiguous(), Vs[:, s * n:(s + 1) * n].contiguous(),
                        O_, L_, S, P, r, t, True, layout)

    for t in range(4):
        step(t, O, L)
    torch.cuda.synchronize()
    saved = (O.cpu().numpy().copy(), L.cpu().numpy().copy())
    del O, L
    O2 = torch.from_numpy(saved[0]).cuda()
    L2 = torch.from_numpy(saved[1]).cuda()
    for t in range(4, P):
        step(t, O2, L2)
    torch.cuda.synchronize()
    assert torch.equal(O2, ref_O) and torch.equal(L2, ref_L)


def _random_cases(n, seed):
    """Seeded random prefill shapes: every split, mask, dtype and head dim,
    GQA ratios 1-8, 1-8 ranks, ragged chunks; small enough for the oracle."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        P = int(rng.integers(1, 9))
        layout = str(rng.choice(["contiguous", "zigzag", "zigzag3", "zigzag4", "striped"]))
        k = {"contiguous": 1, "zigzag": 2, "zigzag3": 3, "zigzag4": 4, "striped": 1}[layout]
        c = int(rng.integers(1, 200))            # tokens per chunk (ragged against the tiles)
        S = c * k * P
        if S > 3000:
            continue
        Hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 2, 4, 8]))
        d = int(rng.choice([64, 128]))
        B = int(rng.integers(1, 3))
        dtype = str(rng.choice(["bf16", "bf16", "f32"]))
        causal = bool(rng.integers(0, 2))
        cases.append((B, S, Hkv * G, Hkv, d, P, layout, causal, dtype))
    return cases


RANDOM = _random_cases(24, 1700)


@pytest.mark.parametrize("case", RANDOM, ids=[_id(c) for c in RANDOM])
def test_prefill_random_shapes(case):
    """Fused launch, a key-range split launch and the ring-step path of one
    rank, each against the oracle."""
    B, S, Hq, Hkv, d, P, layout, causal, dtype = case
    log(f"random {_id(case)}")
    Qn, Kn, Vn = qkv(B, S, S, Hq, Hkv, d, dtype, (1701, S, P, Hq, d))
    (Qs, Ks, Vs), O, L = _run_prefill(Qn, Kn, Vn, P, layout, causal, dtype)
    O_ref, lse_ref = oracle.attention(Qn, Kn, Vn, causal)
    check(unshard(from_dev(O), S, P, layout, axis=1), O_ref, unshard(from_dev(L), S, P, layout, axis=2),
          lse_ref, dtype, _id(case))
    code = 1 if dtype == "bf16" else 0
    nb = ra.ra_fwd_workspace_bytes(B, Hq, Hkv, S, d, P, True, causal, layout, code, 3)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
    O3, L3 = torch.empty_like(O), torch.empty_like(L)
    ra.ra_fwd_all_ws(Qs, Ks, Vs, O3, L3, P, causal, layout, 3, ws)
    torch.cuda.synchronize()
    check(unshard(from_dev(O3), S, P, layout, axis=1), O_ref, unshard(from_dev(L3), S, P, layout, axis=2),
          lse_ref, dtype, _id(case) + " 3 ranges")
    r = P - 1
    n = S // P
    Or, Lr = _ring_rank(Qs, Ks, Vs, S, P, r, causal, layout)
    rows = oracle.natural_positions(S, P, layout)[r * n:(r + 1) * n]
    check(from_dev(Or), O_ref[:, rows], from_dev(Lr), lse_ref[:, :, rows], dtype, _id(case) + " ring steps")


def test_merge_unaligned_pointers():
    # partials that start 4 bytes into an allocation take the general path
    n_parts, rows, d = 3, 50, 64
    rng = np.random.default_rng(1402)
    Op = rng.standard_normal((n_parts, rows, d)).astype(np.float32)
    lp = rng.standard_normal((n_parts, rows)).astype(np.float32)
    big = torch.zeros(n_parts * rows * d + 1, dtype=torch.float32, device="cuda")
    big[1:] = to_dev(Op.reshape(-1))
    Ou = big[1:].view(n_parts, rows, d)
    O = torch.empty(rows, d, dtype=torch.float32, device="cuda")
    ra.ra_merge_partials(Ou, to_dev(lp), O)
    torch.cuda.synchronize()
    O_ref, _ = oracle.merge(Op.astype(np.float64), lp.astype(np.float64))
    assert np.abs(from_dev(O) - O_ref).max() <= 1e-6 * max(1.0, np.abs(O_ref).max())


def test_ring_step_state_to_bf16_as_documented():
    # the header's recipe: one part of weight 1 rounds O_acc to bf16 exactly
    B, S, Hq, Hkv, d, P, layout = 1, 512, 4, 2, 64, 4, "zigzag"
    Qn, Kn, Vn = qkv(B, S, S, Hq, Hkv, d, "bf16", (1303,))
    (Qs, Ks, Vs), _, _ = _run_prefill(Qn, Kn, Vn, P, layout, True, "bf16")
    O, L = _ring_rank(Qs, Ks, Vs, S, P, 2, True, layout)
    rows = O.numel() // d
    Ob = torch.empty(O.shape, dtype=torch.bfloat16, device="cuda")
    Z = torch.zeros(1, rows, dtype=torch.float32, device="cuda")
    ra.ra_merge_partials(O.view(1, rows, d), Z, Ob)
    torch.cuda.synchronize()
    assert torch.equal(Ob.view(torch.int16), O.to(torch.bfloat16).view(torch.int16))


def _random_decode_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        Hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 2, 4, 8, 16]))
        Sq = int(rng.integers(1, 5))
        if Sq * G > 32:
            continue
        B = int(rng.integers(1, 4))
        d = int(rng.choice([64, 128]))
        Skv = int(rng.integers(1, 3000))
        dtype = str(rng.choice(["bf16", "bf16", "f32"]))
        P = int(rng.integers(1, 9))
        block = int(rng.integers(1, 100))
        pps = int(rng.integers(1, 10))
        cases.append((B, Sq, Hkv * G, Hkv, d, Skv, dtype, P, block, pps))
    return cases


RANDOM_DECODE = _random_decode_cases(16, 1800)


@pytest.mark.parametrize("case", RANDOM_DECODE, ids=[str(c) for c in RANDOM_DECODE])
def test_decode_random_shapes(case):
    """Contiguous-cache decode with P*pps parts and the same keys dealt
    round-robin over P shard caches, both merged, against the oracle."""
    B, Sq, Hq, Hkv, d, Skv, dtype, P, block, pps = case
    log(f"random decode {case}")
    Qn, Kn, Vn = qkv(B, Sq, Skv, Hq, Hkv, d, dtype, (1801, Skv, Hq, d, Sq))
    O_ref, L_ref = oracle.attention(Qn, Kn, Vn, False)
    rows = B * Sq * Hq
    n_parts = P * pps
    Qd, Kd, Vd = to_dev(Qn), to_dev(Kn), to_dev(Vn)
    Op = torch.empty(n_parts, rows, d, dtype=torch.float32, device="cuda")
    lp = torch.empty(n_parts, rows, dtype=torch.float32, device="cuda")
    O = torch.empty(rows, d, dtype=torch.float32, device="cuda")
    lse = torch.empty(rows, dtype=torch.float32, device="cuda")
    ra.ra_attn_partial(Qd, Kd, Vd, Op, lp, n_parts)
    ra.ra_merge_partials(Op, lp, O, lse)
    torch.cuda.synchronize()
    check(from_dev(O).reshape(B, Sq, Hq, d), O_ref, from_dev(lse).reshape(B, Sq, Hq).transpose(0, 2, 1),
          L_ref, dtype, str(case) + " contiguous")
    cap = max(len(x) for x in oracle.helix_round_robin(Skv, block, P))
    Kc = torch.empty(P, B, cap, Hkv, d, dtype=Kd.dtype, device="cuda")
    Vc = torch.empty_like(Kc)
    ra.ra_kv_append_rr(Kc, Vc, Kd, Vd, 0, block)
    ra.ra_attn_partial_rr(Qd, Kc, Vc, Op, lp, Skv, block, pps)
    ra.ra_merge_partials(Op, lp, O, lse)
    torch.cuda.synchronize()
    check(from_dev(O).reshape(B, Sq, Hq, d), O_ref, from_dev(lse).reshape(B, Sq, Hq).transpose(0, 2, 1),
          L_ref, dtype, str(case) + " round-robin")


def test_graph_capture_and_replay():
    """The entry points allocate nothing and record no memsets, so a stream
    capture of one rank's P ring steps and of a split prefill launch replays
    to the eager results bit for bit; replays are interleaved with eager work
    and synchronisations, and every replay is checked."""
    B, S, Hq, Hkv, d, P, layout = 1, 2048, 8, 2, 128, 4, "zigzag"
    Qn, Kn, Vn = qkv(B, S, S, Hq, Hkv, d, "bf16", (1304,))
    (Qs, Ks, Vs), _, _ = _run_prefill(Qn, Kn, Vn, P, layout, True, "bf16")
    n = S // P
    r = 3
    Qr = Qs[:, r * n:(r + 1) * n].contiguous()
    blocks = [(Ks[:, s * n:(s + 1) * n].contiguous(), Vs[:, s * n:(s + 1) * n].contiguous())
              for s in range(P)]
    O = torch.empty(B, n, Hq, d, dtype=torch.float32, device="cuda")
    L = torch.empty(B, Hq, n, dtype=torch.float32, device="cuda")
    nb = ra.ra_fwd_workspace_bytes(B, Hq, Hkv, S, d, P, False, True, layout, 1, 3)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    O2 = torch.empty_like(O)
    L2 = torch.empty_like(L)

    def work():
        for t in range(P):
            Kb, Vb = blocks[(r - t) % P]
            ra.ra_ring_step(Qr, Kb, Vb, O, L, S, P, r, t, True, layout)
        ra.ra_fwd_rank_ws(Qr, Ks, Vs, O2, L2, P, r, True, layout, 3, ws)

    work()
    torch.cuda.synchronize()
    ref = (O.clone(), L.clone(), O2.clone(), L2.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        work()  # warm the side stream once before capture
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=side):
        work()
    torch.cuda.synchronize()
    for rep in range(3):
        for x in (O, L, O2, L2):
            x.fill_(float("nan"))           # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (O, L, O2, L2)
        assert all(torch.equal(a, b) for a, b in zip(got, ref)), f"replay {rep}"
