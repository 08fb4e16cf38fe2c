"""Shared helpers for the GPU parity tests: moving the seeded inputs to the
device, and the parity bar.

Parity bar (scores): the -inf mask is bit-exact (0xff800000), no NaN, no -0.0,
and every finite cell agrees with the oracle within
|gpu - ref| <= 2e-3 * max(1, |ref|).
Parity bar (top-k on given logits): bit-exact (integer work on identical
inputs).  Top-k on GPU-computed scores: the same number of picks, ascending,
distinct, -1 padded, every pick a visible block, and no pick whose oracle
score is more than 2e-3*max(1,|kth|) below the oracle's k-th best score.
"""
from __future__ import annotations

import numpy as np
import torch

NEG_INF_BITS = 0xFF800000
RTOL = 2e-3


def dev():
    return torch.device("cuda:0")


def bf16_to_device(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(dev()).view(torch.bfloat16)


def i32_to_device(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev())


def f32_bits(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)


def assert_scores_match(gpu, ref, what=""):
    g = gpu.detach().cpu().numpy() if isinstance(gpu, torch.Tensor) else np.asarray(gpu)
    r = np.asarray(ref)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    gb, rb = f32_bits(g), f32_bits(r)
    assert not np.isnan(g).any(), f"{what}: NaN in GPU output"
    mask_g, mask_r = gb == NEG_INF_BITS, rb == NEG_INF_BITS
    if not np.array_equal(mask_g, mask_r):
        bad = np.argwhere(mask_g != mask_r)
        raise AssertionError(f"{what}: -inf pattern differs at {len(bad)} cells, first {bad[:5].tolist()}")
    fin = ~mask_r
    assert not np.any(gb[fin] == 0x80000000), f"{what}: -0.0 in GPU output"
    err = np.abs(g[fin].astype(np.float64) - r[fin].astype(np.float64))
    lim = RTOL * np.maximum(1.0, np.abs(r[fin].astype(np.float64)))
    if err.size and not np.all(err <= lim):
        i = int(np.argmax(err - lim))
        raise AssertionError(f"{what}: max excess {float((err - lim)[i]):.3g}; gpu {g[fin][i]} ref {r[fin][i]}")


def assert_topk_valid(picks, ref_scores, k):
    """Top-k picks made on GPU scores, checked with the oracle's scores."""
    picks = picks.detach().cpu().numpy() if isinstance(picks, torch.Tensor) else np.asarray(picks)
    ref = np.asarray(ref_scores)
    for t in range(picks.shape[0]):
        row = ref[t]
        fin = np.nonzero(row > -np.inf)[0]
        want = min(k, len(fin))
        got = picks[t]
        sel = got[:want]
        assert np.all(got[want:] == -1), f"row {t}: padding"
        assert np.all(sel >= 0) and np.all(np.diff(sel) > 0), f"row {t}: not ascending/distinct"
        assert np.all(row[sel] > -np.inf), f"row {t}: picked a masked block"
        if want == 0:
            continue
        kth = np.sort(row[fin].astype(np.float64))[::-1][want - 1]
        floor = kth - RTOL * max(1.0, abs(kth))
        assert np.all(row[sel] >= floor), f"row {t}: pick below the k-th score by more than the tolerance"
