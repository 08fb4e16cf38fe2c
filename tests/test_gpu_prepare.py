"""GPU parity: qsa_prepare_q (Gemma RMSNorm + NeoX/MRoPE rotary of the query
heads, bf16 or e4m3 store) against the oracle, bit for bit.

Both sides take the sum of squares as the fp32 rounding of the exact sum,
rrms as the fp32 rounding of 1/sqrt, round once per operation in the
table's type with no fused multiply-add, and encode bf16 and e4m3 with ties
to even; so every output bit is fixed and the comparison is exact (NaN
included: both write the canonical 0x7FC0 / 0x7F).
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from tests.parity import bf16_to_device
from workloads import bf16_bits, prepare_inputs

pytestmark = pytest.mark.gpu


def _qsa():
    import block_indexer_scoring_amd as qsa
    qsa.load_library()
    return qsa


def _table_to_device(a):
    return bf16_to_device(a) if a.dtype == np.uint16 else torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _gpu(inp, sec=None, out_format="bf16", out_scale=1.0, q_pad=0, head_pad=0, positions=None):
    qsa = _qsa()
    T, HD = inp.q.shape
    H = HD // 128
    qbuf = torch.zeros((T, HD + q_pad), dtype=torch.bfloat16, device="cuda")
    if T:
        qbuf[:, :HD] = bf16_to_device(inp.q)
    pos = inp.positions if positions is None else positions
    posd = torch.from_numpy(np.ascontiguousarray(pos, dtype=np.int64)).cuda()
    dt = torch.bfloat16 if out_format == "bf16" else torch.float8_e4m3fn
    obuf = torch.zeros((T, H, 128 + head_pad), dtype=torch.uint8 if dt != torch.bfloat16 else dt, device="cuda")
    out = obuf.view(dt)[:, :, :128] if head_pad else obuf.view(dt)
    qsa.qsa_prepare_q(qbuf[:, :HD], posd, _table_to_device(inp.cos_sin), _table_to_device(inp.weight), inp.eps,
                      mrope_section=sec, out=out, out_scale=out_scale)
    torch.cuda.synchronize()
    host = out.contiguous().cpu()
    return host.view(torch.int16).numpy().view(np.uint16) if out_format == "bf16" else host.view(torch.uint8).numpy()


def _oracle(inp, sec=None, out_format="bf16", out_scale=1.0, positions=None):
    pos = inp.positions if positions is None else positions
    return O.prepare_q(inp.q, pos, inp.cos_sin, inp.weight, inp.eps, mrope_section=sec, out_format=out_format,
                       out_scale=out_scale)


def _assert_same(got, want, what):
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        t, h, d = bad[0]
        raise AssertionError(f"{what}: {len(bad)} elements differ, first (token {t}, head {h}, feature {d}): "
                             f"gpu {got[t, h, d]:#x} oracle {want[t, h, d]:#x}")


@pytest.mark.parametrize("table", ["bf16", "fp32"])
@pytest.mark.parametrize("weight", ["bf16", "fp32"])
@pytest.mark.parametrize("out_format", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("rope", ["plain", "mrope_3axes", "mrope_1axis"])
def test_prepare_matches_oracle(table, weight, out_format, rope):
    # 301 tokens x 3 heads = 903 rows: many 16-row blocks and a ragged last one.
    inp = prepare_inputs(301, 3, seed=81, first_pos=5000, table_rows=6000, table=table, weight=weight,
                         mrope=rope == "mrope_3axes")
    sec = None if rope == "plain" else ((16, 8, 8) if rope == "mrope_3axes" else (12, 10, 10))
    scale = 0.0625 if out_format == "fp8_e4m3" else 1.0
    _assert_same(_gpu(inp, sec, out_format, scale), _oracle(inp, sec, out_format, scale),
                 f"{table}/{weight}/{out_format}/{rope}")


@pytest.mark.parametrize("out_format", ["bf16", "fp8_e4m3"])
def test_prepare_full_size(out_format):
    # One 8K-token prefill chunk after a 100K-token prefix, 4 indexer heads,
    # a 131,072-row bf16 table: the whole output against the oracle.
    inp = prepare_inputs(8192, 4, seed=82, first_pos=100_000, table_rows=131_072)
    scale = 0.03125 if out_format == "fp8_e4m3" else 1.0
    _assert_same(_gpu(inp, None, out_format, scale), _oracle(inp, None, out_format, scale), f"8K x 4 {out_format}")


def test_prepare_mrope_full_size():
    inp = prepare_inputs(8192, 4, seed=83, first_pos=100_000, table_rows=131_072, mrope=True)
    _assert_same(_gpu(inp, (16, 8, 8)), _oracle(inp, (16, 8, 8)), "8K x 4 MRoPE")


@pytest.mark.parametrize("T,H", [(1, 1), (7, 16), (33, 5), (1000, 1)])
def test_prepare_shapes_and_strides(T, H):
    # Padded q token stride and padded output head stride read and write the
    # same values as the packed layout.
    inp = prepare_inputs(T, H, seed=84 + T, first_pos=17, table_rows=2000)
    want = _oracle(inp)
    _assert_same(_gpu(inp), want, f"T={T} H={H}")
    _assert_same(_gpu(inp, q_pad=64, head_pad=128), want, f"T={T} H={H} padded")
    _assert_same(_gpu(inp, out_format="fp8_e4m3", out_scale=0.5, head_pad=8),
                 _oracle(inp, out_format="fp8_e4m3", out_scale=0.5), f"T={T} H={H} fp8 padded")


def test_prepare_edge_values():
    # Zero rows, a row of huge values (x^2 overflows fp32), subnormal-scale
    # rows, a large eps, a weight of -1 (gain 0) on some features, and
    # positions off the table (negative, == rows, far beyond) on single axes.
    T, H = 40, 4
    inp = prepare_inputs(T, H, seed=85, first_pos=0, table_rows=64, mrope=True)
    q = inp.q.reshape(T, H, 128)
    q[0] = 0
    q[1, 0] = bf16_bits(np.full(128, 3e38, np.float32))
    q[2, 1] = bf16_bits(np.full(128, 1e-39, np.float32))
    q[3] = bf16_bits(np.linspace(-1e-20, 1e-20, H * 128, dtype=np.float32).reshape(H, 128))
    w = inp.weight.copy()
    w[[3, 40, 100]] = bf16_bits(np.full(3, -1.0, np.float32))
    pos = inp.positions.copy()
    pos[0, 5], pos[1, 6], pos[2, 7], pos[0, 8] = -1, 64, 1 << 40, 63
    for eps in (1e-6, 4.0):
        case = type(inp)(inp.q, pos, inp.cos_sin, w, eps)
        got, want = _gpu(case, (16, 8, 8)), _oracle(case, (16, 8, 8))
        _assert_same(got, want, f"edges eps={eps}")
        nan = got == 0x7FC0
        assert nan[5:8, :, :64].any() and not nan[5:8, :, 64:].any()   # off-table pairs are NaN
        assert not nan[np.r_[0:5, 8:T]].any()
        assert np.all(got[0] == 0)                                      # zero row -> +0
    plain = type(inp)(inp.q, pos[0], inp.cos_sin, w, 1e-6)
    _assert_same(_gpu(plain), _oracle(plain), "edges plain rotary")
    _assert_same(_gpu(plain, out_format="fp8_e4m3", out_scale=1e-3), _oracle(plain, out_format="fp8_e4m3",
                                                                            out_scale=1e-3), "edges fp8 saturating")


def test_prepare_zero_tokens_and_table_rows():
    qsa = _qsa()
    out = torch.full((0, 4, 128), 1.0, dtype=torch.bfloat16, device="cuda")
    qsa.qsa_prepare_q(torch.empty((0, 512), dtype=torch.bfloat16, device="cuda"),
                      torch.empty(0, dtype=torch.int64, device="cuda"),
                      torch.zeros((8, 64), dtype=torch.bfloat16, device="cuda"),
                      torch.zeros(128, dtype=torch.bfloat16, device="cuda"), 1e-6, out=out)
    torch.cuda.synchronize()
    # A one-row table: every position but 0 is off the table.
    inp = prepare_inputs(5, 2, seed=86, first_pos=0, table_rows=1)
    _assert_same(_gpu(inp), _oracle(inp), "one-row table")
    # An empty table (NULL pointer): every rotated feature is NaN, the rest
    # is the norm.
    inp = prepare_inputs(5, 2, seed=87, first_pos=0, table_rows=0)
    out = torch.empty((5, 2, 128), dtype=torch.bfloat16, device="cuda")
    qsa.qsa_prepare_q(bf16_to_device(inp.q), torch.from_numpy(inp.positions).cuda(),
                      torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"), bf16_to_device(inp.weight),
                      inp.eps, out=out)
    torch.cuda.synchronize()
    got = out.cpu().view(torch.int16).numpy().view(np.uint16)
    _assert_same(got, _oracle(inp), "empty table")
    assert np.all(got[:, :, :64] == 0x7FC0) and not np.any(got[:, :, 64:] == 0x7FC0)


@pytest.mark.parametrize("table", ["bf16", "fp32"])
def test_prepare_non_finite_fp32_weights(table):
    # fp32 weights holding a NaN with a full payload, infinities and a huge
    # finite value: the non-finite results must come out exactly as the
    # oracle's (one NaN pattern, signed infinities), in every format.
    inp = prepare_inputs(24, 4, seed=88, first_pos=3, table_rows=40, table=table, weight="fp32")
    w = inp.weight.copy()
    w[[2, 40, 70]] = np.array([0x7FFFFFFF, 0xFF800000, 0x7F800000], np.uint32).view(np.float32)
    w[100] = np.float32(3e38)
    q = inp.q.copy()
    q[5, :128] = 0                                   # 0 * inf gain -> NaN
    case = type(inp)(q, inp.positions, inp.cos_sin, w, 1e-6)
    got, want = _gpu(case), _oracle(case)
    _assert_same(got, want, f"non-finite weights, {table} table")
    assert (got == 0x7FC0).any() and ((got & 0x7FFF) == 0x7F80).any()
    _assert_same(_gpu(case, out_format="fp8_e4m3", out_scale=0.5),
                 _oracle(case, out_format="fp8_e4m3", out_scale=0.5), f"non-finite weights e4m3, {table} table")
