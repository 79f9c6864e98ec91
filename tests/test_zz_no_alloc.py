"""ra_fwd_rank_noalloc (the entry point for callers that cannot allocate:
its key-range partials live in the library's own device scratch) against
ra_fwd_rank_ws with a caller workspace, on two calls in a row, the second
with a smaller input; and the oracle on both."""
import numpy as np
import pytest
import torch

import long_context_exact_amd as ra
import oracle
from gpu_helpers import check, fmt, from_dev, log, qkv, shard, to_dev, unshard

pytestmark = pytest.mark.gpu

CASES = [  # B, S, Hq, Hkv, d, P, layout, causal, dtype, rank, kv_splits
    (1, 8192, 8, 2, 128, 4, "zigzag", True, "bf16", 1, 4),
    (2, 1200, 4, 4, 64, 3, "contiguous", True, "bf16", 2, 3),   # smaller: 2 x 400 rows, d = 64
]


def _rank_inputs(case):
    B, S, Hq, Hkv, d, P, layout, causal, dtype, rank, splits = case
    Qn, Kn, Vn = qkv(B, S, S, Hq, Hkv, d, dtype, (1400, S, P))
    Qs, Ks, Vs = (to_dev(shard(x, S, P, layout)) for x in (Qn, Kn, Vn))
    n = S // P
    Qr = Qs[:, rank * n:(rank + 1) * n].contiguous()
    O = torch.empty(B, n, Hq, d, dtype=torch.float32, device="cuda")
    L = torch.empty(B, Hq, n, dtype=torch.float32, device="cuda")
    return (Qn, Kn, Vn), (Qr, Ks, Vs, O, L)


@pytest.mark.parametrize("mode", ["explicit", "automatic"])
def test_noalloc_matches_workspace_entry_point(mode):
    results = []
    for case in CASES:
        B, S, Hq, Hkv, d, P, layout, causal, dtype, rank, splits = case
        k = splits if mode == "explicit" else 0
        log(f"noalloc {mode} {case}")
        (Qn, Kn, Vn), (Qr, Ks, Vs, O, L) = _rank_inputs(case)
        ra.ra_fwd_rank_noalloc(Qr, Ks, Vs, O, L, P, rank, causal, layout, kv_splits=k)
        torch.cuda.synchronize()
        # the same call through the caller-workspace entry point, with a
        # workspace of the scratch's size (the automatic choice sees the same bound)
        ws = torch.empty(ra.SCRATCH_BYTES, dtype=torch.uint8, device="cuda")
        O2 = torch.empty_like(O)
        L2 = torch.empty_like(L)
        ra.ra_fwd_rank_ws(Qr, Ks, Vs, O2, L2, P, rank, causal, layout, kv_splits=k, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(O, O2) and torch.equal(L, L2), f"{case}: differs from ra_fwd_rank_ws"
        del ws
        # and the oracle on the rank's rows
        n = S // P
        pos = oracle.natural_positions(S, P, layout)[rank * n:(rank + 1) * n]
        bb, ii = np.meshgrid(np.arange(B), pos, indexing="ij")
        O_ref, L_ref = oracle.attention_rows(Qn, Kn, Vn, causal, bb.ravel(), ii.ravel())
        e = check(from_dev(O).reshape(B * n, Hq, d), O_ref,
                  from_dev(L).transpose(0, 2, 1).reshape(B * n, Hq), L_ref, dtype, str(case))
        log(f"  ok {fmt(e)}")
        results.append(e)
    assert len(results) == 2
