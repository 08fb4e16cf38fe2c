"""GPU parity: qsa_topk_blocks and qsa_build_metadata against the CPU oracle,
and one pass of the whole path (metadata -> scores -> top-k) on a mixed
decode + prefill batch."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from tests.parity import assert_scores_match, assert_topk_valid, bf16_to_device, i32_to_device
from workloads import WORKLOADS, decode_inputs, normal_bf16, prefill_inputs

pytestmark = pytest.mark.gpu


def _qsa():
    import block_indexer_scoring_amd as qsa
    qsa.load_library()
    return qsa


def _topk_gpu(x: np.ndarray, k: int):
    qsa = _qsa()
    xd = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    out = torch.full((x.shape[0], k), 12345, dtype=torch.int32, device="cuda")
    qsa.qsa_topk_blocks(xd, k, out=out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("cols,k", [(1, 1), (50, 7), (1000, 64), (4096, 512), (5000, 512),
                                    (26024, 512), (25600, 2048), (32768, 512), (40000, 512),
                                    (65535, 512), (65536, 512), (3000, 4000), (9000, 1)])
def test_topk_bit_exact_on_given_logits(cols, k):
    rng = np.random.default_rng(cols + k)
    x = (np.abs(rng.standard_normal((9, cols))) * 3).astype(np.float32)
    x[1, cols // 3:] = -np.inf                     # short row (causal tail)
    x[2] = -np.inf                                 # nothing visible
    x[3] = np.round(x[3] * 2) / 2                  # many exact ties
    x[4] = 1.0                                     # all tied
    x[5, ::2] = 0.0
    x[5, 1::2] = -0.0                              # -0 ties +0
    x[6] = rng.standard_normal(cols).astype(np.float32)  # negative values too
    x[7, ::5] = np.nan                             # NaN is never picked
    x[8] = np.arange(cols, dtype=np.float32)       # strictly increasing
    got = _topk_gpu(x, k)
    want = O.topk(x, k)
    assert np.array_equal(got, want), np.argwhere(got != want)[:5]


def _pattern_rows(rng, rows, cols):
    """Rows cycling through the edge patterns of the test above."""
    x = (np.abs(rng.standard_normal((rows, cols))) * 3).astype(np.float32)
    for r in range(rows):
        kind = r % 10
        if kind == 1:
            x[r, (r * 7919) % cols:] = -np.inf
        elif kind == 2:
            x[r] = -np.inf
        elif kind == 3:
            x[r] = np.round(x[r] * 2) / 2
        elif kind == 4:
            x[r] = 1.0
        elif kind == 5:
            x[r, ::2] = 0.0
            x[r, 1::2] = -0.0
        elif kind == 6:
            x[r] = rng.standard_normal(cols).astype(np.float32)
        elif kind == 7:
            x[r, ::5] = np.nan
        elif kind == 8:
            x[r] = np.arange(cols, dtype=np.float32)
        elif kind == 9:
            x[r] = np.round(x[r] * 64) / 64   # ties inside one 16-bit key prefix
    return x


@pytest.mark.parametrize("cols,k", [(5000, 512), (26024, 512), (32768, 512), (27048, 2048),
                                    (27047, 512), (5003, 100), (30001, 512), (4097, 4096)])
def test_topk_patterns_many_rows(cols, k):
    """Enough rows for the many-row launch shapes, with the edge patterns;
    column counts that are not a multiple of 4 take the element-load path
    (a ragged last 4-column chunk)."""
    rng = np.random.default_rng(cols ^ k)
    x = _pattern_rows(rng, 300, cols)
    got = _topk_gpu(x, k)
    want = O.topk(x, k)
    assert np.array_equal(got, want), np.argwhere(got != want)[:5]


@pytest.mark.parametrize("rows,cols,k", [(300, 27048, 512), (64, 25600, 512), (300, 27048, 2048), (300, 5000, 512)])
def test_topk_scores_spread_over_one_binade(rows, cols, k):
    """Scores spread evenly over one binade, or over a narrow part of one:
    the k-th largest sits in an 11-bit key bin holding most of the row, so
    the floor is taken to 16 bits; in the narrowest rows even that bin holds
    more keys than the list (the select then reads the row itself)."""
    rng = np.random.default_rng(rows * 7 + cols + k)
    x = np.empty((rows, cols), dtype=np.float32)
    for r in range(rows):
        kind = r % 4
        if kind == 0:
            x[r] = rng.uniform(2.0, 4.0, cols)          # one binade
        elif kind == 1:
            x[r] = rng.uniform(0.0, 3.0, cols)          # about two binades
        elif kind == 2:
            x[r] = rng.uniform(2.0, 2.001, cols)        # a sliver of one 16-bit key prefix
        else:
            x[r] = 2.0 + np.round(rng.uniform(0.0, 1.0, cols) * 256) / 256  # ties at 16-bit prefixes
    x[rows // 2, cols // 2:] = -np.inf                  # a short row among them
    got = _topk_gpu(x, k)
    want = O.topk(x, k)
    assert np.array_equal(got, want), np.argwhere(got != want)[:5]


@pytest.mark.parametrize("rows,cols,k", [(300, 27048, 512), (64, 25600, 512), (300, 26024, 512), (300, 5000, 100)])
def test_topk_outliers_over_many_binades(rows, cols, k):
    """Rows whose listed keys reach 16 or more binades above the floor (a
    few huge outliers over unit-range scores, or log-uniform scores over
    60 decades): the list is then counted by its top 11 bits and the select
    takes two radix passes, where rows within 2,048 top-half values of the
    floor take one."""
    rng = np.random.default_rng(rows * 13 + cols + k)
    x = rng.uniform(1.0, 2.0, (rows, cols)).astype(np.float32)
    for r in range(rows):
        kind = r % 4
        if kind == 0:    # fewer outliers than k: the k-th key is a unit-range one
            n = int(rng.integers(1, k))
            x[r, rng.choice(cols, n, replace=False)] = 10.0 ** rng.uniform(10, 30, n)
        elif kind == 1:  # more outliers than k, spread over 20 decades
            n = min(cols, 2 * k + int(rng.integers(0, k)))
            x[r, rng.choice(cols, n, replace=False)] = 10.0 ** rng.uniform(10, 30, n)
        elif kind == 2:  # log-uniform over 60 decades
            x[r] = (10.0 ** rng.uniform(-30, 30, cols)).astype(np.float32)
        else:            # outliers tied at one value, with -inf and NaN cells
            n = int(rng.integers(k // 2, 2 * k))
            x[r, rng.choice(cols, n, replace=False)] = 1e25
            x[r, ::7] = -np.inf
            x[r, 3::11] = np.nan
    got = _topk_gpu(x, k)
    want = O.topk(x, k)
    assert np.array_equal(got, want), np.argwhere(got != want)[:5]


def test_topk_many_rows_and_strided_logits():
    rng = np.random.default_rng(5)
    big = rng.standard_normal((300, 700)).astype(np.float32)
    qsa = _qsa()
    xd = torch.from_numpy(big).cuda()[:, 3:603]   # row stride 700
    out = qsa.qsa_topk_blocks(xd, 100)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), O.topk(big[:, 3:603], 100))


def test_metadata_matches_oracle():
    qsa = _qsa()
    rng = np.random.default_rng(6)
    for case in range(6):
        R = int(rng.integers(1, 40))
        qlens = rng.integers(0, 300, R)
        qlens[rng.random(R) < 0.5] = 4
        seq = qlens + rng.integers(0, 5000, R)
        qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
        T = int(qsl[-1]) + int(rng.integers(0, 9))          # padding tokens at the end
        offs = np.concatenate([[0], np.cumsum(seq // 4)[:-1]]).astype(np.int32)
        res = qsa.qsa_build_metadata(i32_to_device(qsl), i32_to_device(seq), T,
                                     key_offsets=i32_to_device(offs))
        torch.cuda.synchronize()
        req, pos, vis = O.token_metadata(qsl, seq.astype(np.int32), T)
        ks, ke = O.prefill_intervals(req, vis, offs)
        assert np.array_equal(res["token_to_req"].cpu().numpy(), req)
        assert np.array_equal(res["positions"].cpu().numpy(), pos)
        assert np.array_equal(res["visible"].cpu().numpy(), vis)
        assert np.array_equal(res["comp_lens"].cpu().numpy(), O.comp_lens(seq.astype(np.int32)))
        assert np.array_equal(res["row_k_start"].cpu().numpy(), ks)
        assert np.array_equal(res["row_k_end"].cpu().numpy(), ke)


@pytest.mark.parametrize("dql", [1, 3, 4, 16])
def test_decode_visible_blocks_matches_oracle(dql):
    """Uniform decode batches: compressed lengths and per-row visible blocks
    equal the oracle's token metadata for query_start_loc = 0, dql, 2 dql ..,
    including contexts shorter than dql, empty contexts, the golden visible
    table's contexts and the spec-decode batch's."""
    qsa = _qsa()
    rng = np.random.default_rng(dql)
    ctx = [0, 1, 2, 3, 4, 5, 7, 8, 10, 11, 256, 3508, 100_000, 102_400]
    ctx += rng.integers(0, 200_000, 200).tolist()
    ctx += [int(x) for x in WORKLOADS["specdecode_16x51k"].make().seq_lens]
    seq = np.array(ctx, np.int32)
    comp, vis = qsa.qsa_decode_visible_blocks(i32_to_device(seq), dql)
    torch.cuda.synchronize()
    qsl = (np.arange(len(seq) + 1) * dql).astype(np.int32)
    _, _, want = O.token_metadata(qsl, seq, len(seq) * dql)
    assert np.array_equal(vis.cpu().numpy(), want)
    assert np.array_equal(comp.cpu().numpy(), O.comp_lens(seq))


def test_whole_path_mixed_batch():
    """One step: split a mixed batch, build metadata on the GPU, score the
    decode rows through the page table and the prefill rows over packed keys,
    then take the top-k blocks of every row."""
    qsa = _qsa()
    dec = decode_inputs([3000, 1333, 804], 4, 64, table_cols=20, spare_pages=2, out_cols=800, seed=31)
    pre = prefill_inputs(2, 300, 1700, seed=32)
    R_dec, R_pre = dec.num_reqs, 2
    qlens = [4] * R_dec + [300, 300]
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    seq = np.concatenate([dec.seq_lens, pre.seq_lens]).astype(np.int32)
    order, nd, ndt, npf, npt, dql = qsa.qsa_split_batch(qsl.tolist(), 4)
    assert (nd, ndt, npf, npt, dql) == (3, 12, 2, 600, 4)
    assert (order, nd, ndt, npf, npt, dql) == O.split_batch(qsl, 4)
    offs = np.zeros(R_dec + R_pre, np.int32)
    offs[R_dec:] = pre.key_offsets
    meta = qsa.qsa_build_metadata(i32_to_device(qsl), i32_to_device(seq), int(qsl[-1]),
                                  key_offsets=i32_to_device(offs))
    vis_dec = meta["visible"][:ndt]
    dscores = qsa.qsa_mqa_decode(bf16_to_device(dec.q), bf16_to_device(dec.k_pool),
                                 i32_to_device(dec.page_table), meta["comp_lens"][:R_dec],
                                 vis_dec, out_cols=800)
    pscores = qsa.qsa_mqa_prefill(bf16_to_device(pre.q), bf16_to_device(pre.k),
                                  meta["row_k_start"][ndt:], meta["row_k_end"][ndt:],
                                  out_cols=pre.out_cols)
    dtop = qsa.qsa_topk_blocks(dscores, 64)
    ptop = qsa.qsa_topk_blocks(pscores, 64)
    torch.cuda.synchronize()

    req, _, vis = O.token_metadata(qsl, seq, int(qsl[-1]))
    ks, ke = O.prefill_intervals(req, vis, offs)
    dref = O.decode(dec.q, dec.k_pool, dec.page_table, O.comp_lens(dec.seq_lens), vis[:ndt], 800)
    pref = O.prefill(pre.q, pre.k, ks[ndt:], ke[ndt:], pre.out_cols)
    assert_scores_match(dscores, dref, "decode part")
    assert_scores_match(pscores, pref, "prefill part")
    assert_topk_valid(dtop, dref, 64)
    assert_topk_valid(ptop, pref, 64)
    # Top-k on identical logits is integer work: bit-exact.
    assert np.array_equal(dtop.cpu().numpy(), O.topk(dscores.cpu().numpy(), 64))
    assert np.array_equal(ptop.cpu().numpy(), O.topk(pscores.cpu().numpy(), 64))


def test_topk_on_prefill_4x4k_100k_all_rows():
    """Top-512 of all 16,384 rows of the 4x4K-over-100K prefill: bit-exact
    against the oracle's top-k of the same GPU scores on every row (integer
    work on identical inputs), and valid against the oracle's own scores on
    512 sampled rows."""
    qsa = _qsa()
    inp = WORKLOADS["prefill_4x4k_100k"].make()
    req, _, vis = O.token_metadata(inp.query_start_loc, inp.seq_lens, inp.q.shape[0])
    ks, ke = O.prefill_intervals(req, vis, inp.key_offsets)
    scores = qsa.qsa_mqa_prefill(bf16_to_device(inp.q), bf16_to_device(inp.k), i32_to_device(ks),
                                 i32_to_device(ke), out_cols=inp.out_cols)
    top = qsa.qsa_topk_blocks(scores, 512)
    torch.cuda.synchronize()
    top_host = top.cpu().numpy()
    T = inp.q.shape[0]
    for b in range(0, T, 4096):
        chunk = scores[b:b + 4096].cpu().numpy()
        assert np.array_equal(top_host[b:b + 4096], O.topk(chunk, 512)), f"rows {b}.."
    del chunk
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, 4095, 4096, 8191, 8192, 12287, 12288, 16383],
                                     rng.choice(T, 520, replace=False)]))
    assert len(rows) >= 512
    ref = O.prefill(inp.q, inp.k, ks, ke, inp.out_cols, rows=rows)
    assert_topk_valid(top_host[rows], ref, 512)
