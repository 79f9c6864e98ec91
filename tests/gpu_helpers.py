"""Shared helpers of the GPU parity tests: seeded inputs, host-side sharding
with the oracle's own index arithmetic, and the tolerance checks."""
from __future__ import annotations

import math
import time

import numpy as np
import torch

import oracle
from long_context_exact_amd import synthetic

# bf16 inputs: O max-abs <= 1e-2, O rel-L2 <= 5e-3, LSE abs <= 1e-3
BF16_O_MAX, BF16_O_REL, BF16_LSE = 1e-2, 5e-3, 1e-3
# fp32 inputs: O and LSE max-abs <= 1e-5
F32_O_MAX, F32_LSE = 1e-5, 1e-5


def log(msg: str) -> None:
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)


def to_dev(a: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.cuda()


def from_dev(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> float64 numpy (bf16 widened exactly)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return oracle.bf16_bits_to_f64(t.view(torch.int16).numpy().view(np.uint16))
    return t.double().numpy()


def qkv(B, Sq, Skv, Hq, Hkv, d, dtype, seed):
    Q = synthetic.normal_tensor((B, Sq, Hq, d), (*seed, 0), dtype)
    K = synthetic.normal_tensor((B, Skv, Hkv, d), (*seed, 1), dtype)
    V = synthetic.normal_tensor((B, Skv, Hkv, d), (*seed, 2), dtype)
    return Q, K, V


def scale_bf16(x: np.ndarray, s: float) -> np.ndarray:
    return synthetic.bf16_rne_bits(synthetic.bf16_bits_to_f32(x) * np.float32(s))


def shard(x: np.ndarray, S: int, P: int, layout: str) -> np.ndarray:
    """Natural -> sharded order along axis 1 (the oracle's index map)."""
    return np.ascontiguousarray(x[:, oracle.natural_positions(S, P, layout)])


def unshard(x: np.ndarray, S: int, P: int, layout: str, axis: int = 1) -> np.ndarray:
    pos = oracle.natural_positions(S, P, layout)
    out = np.empty_like(x)
    idx = [slice(None)] * x.ndim
    idx[axis] = pos
    out[tuple(idx)] = x
    return out


def check(O, O_ref, lse, lse_ref, dtype: str, what: str = "", o_rounded: bool = False) -> dict:
    """Compare GPU results (float64 arrays) with the oracle's, element by
    element, with the tolerances for the input dtype.  Returns the errors.

    o_rounded: O was stored in bf16.  Rounding to bf16 alone moves a value by
    up to 2**-8 of its magnitude (0.0156 at |O| = 4), more than the 1e-2
    bound, so that bound is widened by 2**-8 |O_ref| per element."""
    assert O.shape == O_ref.shape and lse.shape == lse_ref.shape
    assert np.all(np.isfinite(O)), f"{what}: non-finite O"
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse), fin), f"{what}: LSE finiteness differs"
    err = np.abs(O - O_ref)
    e = {
        "o_max": float(err.max()) if err.size else 0.0,
        "o_rel_l2": float(np.linalg.norm(err) / max(np.linalg.norm(O_ref), 1e-300)),
        "lse_max": float(np.abs(lse[fin] - lse_ref[fin]).max()) if fin.any() else 0.0,
    }
    if dtype == "bf16":
        if o_rounded:
            e["o_excess"] = float((err - (BF16_O_MAX + 2.0 ** -8 * np.abs(O_ref))).max()) if err.size else -1.0
            ok = e["o_excess"] <= 0 and e["o_rel_l2"] <= BF16_O_REL and e["lse_max"] <= BF16_LSE
        else:
            ok = e["o_max"] <= BF16_O_MAX and e["o_rel_l2"] <= BF16_O_REL and e["lse_max"] <= BF16_LSE
    else:
        ok = e["o_max"] <= F32_O_MAX and e["lse_max"] <= F32_LSE
    assert ok, f"{what}: parity failed {e}"
    return e


def sample_rows(S: int, P: int, layout: str, per_rank: int, seed) -> np.ndarray:
    """Natural positions to check: per rank the first and last row of each of
    its chunks plus ``per_rank`` rows drawn with the seeded generator
    ``numpy.random.default_rng([*seed, rank])``."""
    pos = oracle.natural_positions(S, P, layout)
    n = S // P
    # a striped rank's rows are one strided chunk
    c = n if layout == "striped" else oracle.chunk_len(layout, S, P)
    rows = []
    for r in range(P):
        rng = np.random.default_rng([*seed, r])
        mine = pos[r * n:(r + 1) * n]
        for k in range(0, n, c):
            rows += [mine[k], mine[k + c - 1]]
        rows += list(rng.choice(mine, size=min(per_rank, n), replace=False))
    return np.unique(np.asarray(rows, dtype=np.int64))


def prefill_flops(B, Hq, d, S, P, layout, causal) -> int:
    pairs = sum(oracle.unmasked_pairs(S, P, layout, r, causal) for r in range(P))
    return 4 * B * Hq * d * pairs


def fmt(e: dict) -> str:
    return " ".join(f"{k}={v:.3g}" for k, v in e.items())


def ceil_div(a, b):
    return -(-a // b)


def isclose_rel(a, b, tol):
    return math.isclose(a, b, rel_tol=tol)
