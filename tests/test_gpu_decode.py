"""GPU parity: qsa_mqa_decode (paged decode scores) against the CPU oracle."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from tests.parity import assert_scores_match, bf16_to_device, f32_bits, i32_to_device
from workloads import WORKLOADS, DecodeInputs, decode_inputs, normal_bf16

pytestmark = pytest.mark.gpu


def _qsa():
    import block_indexer_scoring_amd as qsa
    qsa.load_library()
    return qsa


def _run_gpu(inp: DecodeInputs, visible, scale=None, q=None, out=None, poison=True):
    qsa = _qsa()
    qd = bf16_to_device(inp.q) if q is None else q
    kd = bf16_to_device(inp.k_pool)
    pt = i32_to_device(inp.page_table)
    comp = i32_to_device(O.comp_lens(inp.seq_lens))
    vis = None if visible is None else i32_to_device(visible)
    if out is None:
        out = torch.empty((inp.num_reqs * inp.dql, inp.out_cols), dtype=torch.float32, device="cuda")
    if poison:
        out.view(torch.int32).fill_(0x7FC00001)  # NaN: any cell left unwritten fails parity
    kw = {} if scale is None else {"scale": scale}
    qsa.qsa_mqa_decode(qd, kd, pt, comp, vis, out=out, **kw)
    torch.cuda.synchronize()
    return out


def _oracle(inp: DecodeInputs, visible, scale=None, q=None):
    return O.decode(inp.q if q is None else q, inp.k_pool, inp.page_table,
                    O.comp_lens(inp.seq_lens), visible, inp.out_cols, scale=scale)


def _visible(inp):
    _, _, vis = O.token_metadata(inp.query_start_loc, inp.seq_lens, inp.num_reqs * inp.dql)
    return vis


@pytest.mark.parametrize("name", ["tiny_decode", "decode_100k", "specdecode_16x51k"])
def test_decode_workloads_full(name):
    inp = WORKLOADS[name].make()
    vis = _visible(inp)
    gpu = _run_gpu(inp, vis)
    assert_scores_match(gpu, _oracle(inp, vis), name)


@pytest.mark.parametrize("dql", [1, 2, 3, 4, 5, 8, 13, 16])
def test_decode_dql(dql):
    ctx = [4 * 97 + (dql % 4), 1000, 3, 257]
    inp = decode_inputs(ctx, dql, 16, table_cols=20, spare_pages=5, out_cols=300, seed=dql)
    vis = _visible(inp)
    assert_scores_match(_run_gpu(inp, vis), _oracle(inp, vis), f"dql={dql}")


@pytest.mark.parametrize("page_size", [1, 3, 8, 16, 32, 49, 64, 128, 196])
def test_decode_page_sizes(page_size):
    ctx = [5000, 4 * 64 * 3, 4 * 64 * 3 + 3, 17, 2]
    table_cols = -(-(5000 // 4 + 1) // page_size) + 2
    inp = decode_inputs(ctx, 4, page_size, table_cols, spare_pages=7, out_cols=1300, seed=page_size)
    vis = _visible(inp)
    assert_scores_match(_run_gpu(inp, vis), _oracle(inp, vis), f"ps={page_size}")


def test_decode_page_holes_and_bad_ids():
    inp = decode_inputs([3000, 2900, 2500], 4, 16, table_cols=60, spare_pages=3, out_cols=800, seed=7)
    inp.page_table[0, 3] = -1
    inp.page_table[1, 0] = inp.k_pool.shape[0]        # one past the pool
    inp.page_table[2, 10] = 1 << 30
    inp.page_table[2, 11] = -7
    vis = _visible(inp)
    assert_scores_match(_run_gpu(inp, vis), _oracle(inp, vis), "holes")
    # Page table narrower than the visible range.
    narrow = DecodeInputs(inp.q, inp.k_pool, np.ascontiguousarray(inp.page_table[:, :20]),
                          inp.seq_lens, inp.query_start_loc, inp.page_size, inp.out_cols)
    assert_scores_match(_run_gpu(narrow, vis), _oracle(narrow, vis), "narrow table")


def test_decode_visible_none_and_odd_values():
    inp = decode_inputs([777, 64, 1], 2, 16, table_cols=20, spare_pages=2, out_cols=200, seed=8)
    assert_scores_match(_run_gpu(inp, None), _oracle(inp, None), "visible=None")
    odd = np.array([10_000, -3, 5, 0, 1, 7], np.int32)
    assert_scores_match(_run_gpu(inp, odd), _oracle(inp, odd), "odd visible")


def test_decode_scale():
    inp = decode_inputs([900, 333], 4, 16, table_cols=20, spare_pages=1, out_cols=230, seed=9)
    vis = _visible(inp)
    for scale in (1.0, 0.125, 3.7):
        assert_scores_match(_run_gpu(inp, vis, scale=scale), _oracle(inp, vis, scale=scale), f"scale {scale}")


def test_decode_strided_and_broadcast_q():
    inp = decode_inputs([1200, 640, 90], 4, 16, table_cols=24, spare_pages=2, out_cols=310, seed=10)
    vis = _visible(inp)
    # A padded view (rows of 136 features, 5 heads): still 16-byte aligned.
    wide = np.zeros((3, 4, 5, 136), np.uint16)
    wide[:, :, :4, :128] = inp.q
    qd = bf16_to_device(wide)[:, :, :4, :128]
    assert_scores_match(_run_gpu(inp, vis, q=qd), _oracle(inp, vis), "padded q view")
    # A view whose base is off the 16-byte grid (element loads).
    flat = np.zeros(3 * 4 * 4 * 128 + 3, np.uint16)
    flat[3:] = inp.q.reshape(-1)
    qd = bf16_to_device(flat)[3:].view(3, 4, 4, 128)
    assert_scores_match(_run_gpu(inp, vis, q=qd), _oracle(inp, vis), "misaligned q view")
    # Broadcast over requests and rows (stride 0).
    one = np.ascontiguousarray(inp.q[:1, :1])
    qd = bf16_to_device(one).expand(3, 4, 4, 128)
    q_bcast = np.broadcast_to(one, (3, 4, 4, 128))
    assert_scores_match(_run_gpu(inp, vis, q=qd), _oracle(inp, vis, q=q_bcast), "broadcast q")


def test_decode_out_views():
    inp = decode_inputs([1500, 200], 3, 16, table_cols=30, spare_pages=2, out_cols=390, seed=11)
    vis = _visible(inp)
    ref = _oracle(inp, vis)
    big = torch.full((6, 401), 1.25, dtype=torch.float32, device="cuda")
    out = big[:, 5:395]                      # row stride 401, base off the 16-byte grid
    _run_gpu(inp, vis, out=out, poison=False)
    assert_scores_match(out, ref, "strided out")
    host = big.cpu().numpy()
    assert np.all(host[:, :5] == 1.25) and np.all(host[:, 395:] == 1.25), "wrote outside out"


def test_decode_deterministic_and_page_permutation():
    inp = decode_inputs([4000, 2000, 100], 4, 64, table_cols=20, spare_pages=4, out_cols=1000, seed=12)
    vis = _visible(inp)
    a = f32_bits(_run_gpu(inp, vis))
    b = f32_bits(_run_gpu(inp, vis))
    assert np.array_equal(a, b)
    rng = np.random.default_rng(3)
    perm = rng.permutation(inp.k_pool.shape[0])
    pool2 = np.empty_like(inp.k_pool)
    pool2[perm] = inp.k_pool
    table2 = np.where(inp.page_table >= 0, perm[np.maximum(inp.page_table, 0)], -1).astype(np.int32)
    inp2 = DecodeInputs(inp.q, pool2, table2, inp.seq_lens, inp.query_start_loc, 64, inp.out_cols)
    assert np.array_equal(f32_bits(_run_gpu(inp2, vis)), a)


def test_decode_onehot_bit_exact():
    a = np.array([1.0, -1.0, 2.0, 0.5], np.float32)
    q = np.zeros((1, 1, 4, 128), np.float32)
    q[0, 0, :, 0] = a
    from workloads import bf16_bits
    pool = np.zeros((2, 16, 1, 128), np.float32)
    pool[1, :8, 0, 0] = np.arange(8) - 2
    inp = DecodeInputs(bf16_bits(q), bf16_bits(pool), np.array([[1]], np.int32),
                       np.array([32], np.int32), np.array([0, 1], np.int32), 16, 8)
    gpu = _run_gpu(inp, np.array([8], np.int32))
    want = [0x3E3504F3, 0x3DB504F3, 0x0, 0x3E9E6455, 0x3F1E6455, 0x3F6D967F, 0x3F9E6455, 0x3FC5FD6A]
    assert list(f32_bits(gpu)[0]) == want


def test_decode_empty_calls():
    qsa = _qsa()
    inp = decode_inputs([100], 1, 16, table_cols=4, spare_pages=0, out_cols=25, seed=13)
    q, kd = bf16_to_device(inp.q), bf16_to_device(inp.k_pool)
    pt, comp = i32_to_device(inp.page_table), i32_to_device(O.comp_lens(inp.seq_lens))
    out = torch.empty((1, 0), dtype=torch.float32, device="cuda")
    qsa.qsa_mqa_decode(q, kd, pt, comp, None, out=out)
    # No pages at all: every cell is -inf.
    empty_table = torch.empty((1, 0), dtype=torch.int32, device="cuda")
    out = qsa.qsa_mqa_decode(q, kd, empty_table, comp, None, out_cols=25)
    torch.cuda.synchronize()
    assert np.all(f32_bits(out) == 0xFF800000)


def test_launch_events_time_the_kernel():
    """qsa_set_launch_events: the attached events bracket the decode kernel
    and the scores are unchanged; clearing them leaves the events alone."""
    import bench
    qsa = _qsa()
    inp = WORKLOADS["tiny_decode"].make()
    _, _, vis = O.token_metadata(inp.query_start_loc, inp.seq_lens, inp.num_reqs * inp.dql)
    ev = bench.HipEvents(2)
    try:
        qsa.qsa_set_launch_events(ev.ev[0], ev.ev[1])
        try:
            out = _run_gpu(inp, vis)
        finally:
            qsa.qsa_set_launch_events(None, None)
        first = ev.elapsed_us(0, 1)
        assert 0.0 < first < 1e6
        assert_scores_match(out.cpu().numpy(), _oracle(inp, vis))
        _run_gpu(inp, vis)
        assert ev.elapsed_us(0, 1) == first
    finally:
        ev.close()
