"""The seeded input generators: reproducible, shaped like the pages' workloads."""
import numpy as np
import torch

from workloads import (C3_CONTEXTS, WORKLOADS, bf16_bits, bits_to_f32, decode_inputs,
                       lognormal_contexts, pages_for)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100_000).astype(np.float32),
                        np.array([1.0, -2.5, 3.0039062, 1.00390625, 1.01171875], np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_bits(x), want)
    assert np.array_equal(bits_to_f32(bf16_bits(x)),
                          torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_c3_contexts_min_mean_max():
    ctx = C3_CONTEXTS
    assert len(ctx) == 16
    assert min(ctx) == 3508 and max(ctx) == 102400
    assert sum(ctx) == 16 * 51200
    assert ctx == sorted(ctx)
    assert lognormal_contexts(16, 3508, 51200, 102400, seed=1) == ctx


def test_decode_inputs_reproducible_and_paged():
    a = decode_inputs([1000, 37, 5000], 4, 16, 100, 3, 1300, seed=9)
    b = decode_inputs([1000, 37, 5000], 4, 16, 100, 3, 1300, seed=9)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.k_pool, b.k_pool)
    assert np.array_equal(a.page_table, b.page_table)
    used = []
    for r, ctx in enumerate([1000, 37, 5000]):
        n = pages_for(ctx, 16)
        assert np.all(a.page_table[r, :n] >= 0) and np.all(a.page_table[r, n:] == -1)
        used.extend(a.page_table[r, :n].tolist())
    assert len(set(used)) == len(used)            # no page shared
    assert a.k_pool.shape[0] == len(used) + 3     # plus the spare pages
    assert list(a.query_start_loc) == [0, 4, 8, 12]


def test_workload_shapes():
    c1 = WORKLOADS["tiny_decode"].make()
    assert c1.q.shape == (1, 1, 4, 128) and c1.k_pool.shape == (4, 16, 1, 128)
    assert c1.page_table.shape == (1, 4) and sorted(c1.page_table[0]) == [0, 1, 2, 3]
    c2 = WORKLOADS["decode_100k"].make()
    assert c2.k_pool.shape == (391 + 32, 64, 1, 128)
    assert (c2.page_table[0] >= 0).sum() == 391 and (c2.page_table[0] == -1).sum() == 9
    assert c2.out_cols == 25_000
