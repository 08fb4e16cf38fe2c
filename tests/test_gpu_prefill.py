"""GPU parity: qsa_mqa_prefill (packed prefill scores) against the CPU oracle."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from tests.parity import assert_scores_match, bf16_to_device, f32_bits, i32_to_device
from workloads import WORKLOADS, bf16_bits, normal_bf16

pytestmark = pytest.mark.gpu


def _qsa():
    import block_indexer_scoring_amd as qsa
    qsa.load_library()
    return qsa


def _gpu(q_bits, k_bits, ks, ke, out_cols, scale=None, out=None, poison=True):
    qsa = _qsa()
    qd = bf16_to_device(q_bits) if isinstance(q_bits, np.ndarray) else q_bits
    kd = bf16_to_device(k_bits) if isinstance(k_bits, np.ndarray) else k_bits
    if out is None:
        out = torch.empty((qd.shape[0], out_cols), dtype=torch.float32, device="cuda")
    if poison:
        out.view(torch.int32).fill_(0x7FC00001)
    kw = {} if scale is None else {"scale": scale}
    qsa.qsa_mqa_prefill(qd, kd, i32_to_device(ks), i32_to_device(ke), out=out, **kw)
    torch.cuda.synchronize()
    return out


def _intervals(inp):
    T = inp.q.shape[0]
    req, _, vis = O.token_metadata(inp.query_start_loc, inp.seq_lens, T)
    return O.prefill_intervals(req, vis, inp.key_offsets)


def _sample_rows(T, seed, extra=96):
    rng = np.random.default_rng(seed)
    rows = set(range(min(T, 70))) | set(range(max(0, T - 70), T))
    rows |= set(rng.integers(0, T, extra).tolist())
    return np.array(sorted(rows), np.int64)


def _mask_pattern_all_rows(out_host, ks, ke, num_keys):
    """Every cell: -inf exactly where key ks+c is outside [0, min(ke, NK)),
    finite and >= +0 elsewhere."""
    T, C = out_host.shape
    cols = np.arange(C)[None, :]
    key = ks.astype(np.int64)[:, None] + cols
    valid = (key >= 0) & (key < num_keys) & (key < ke.astype(np.int64)[:, None])
    bits = out_host.view(np.uint32)
    assert np.array_equal(bits == 0xFF800000, ~valid), "mask pattern"
    # Finite and >= +0: also fails on the NaN poison of an unwritten cell.
    assert np.all(bits[valid] < 0x7F800000), "negative, -0, infinite or NaN score (or a cell left unwritten)"


@pytest.mark.parametrize("name", ["prefill_1x8k_8k", "prefill_4x4k_100k", "prefill_1x8k_100k"])
def test_prefill_workloads_sampled(name):
    inp = WORKLOADS[name].make()
    ks, ke = _intervals(inp)
    gpu = _gpu(inp.q, inp.k, ks, ke, inp.out_cols)
    host = gpu.cpu().numpy()
    del gpu
    _mask_pattern_all_rows(host, ks, ke, inp.k.shape[0])
    rows = _sample_rows(inp.q.shape[0], seed=len(name), extra=64 if "100k" in name else 160)
    ref = O.prefill(inp.q, inp.k, ks, ke, inp.out_cols, rows=rows)
    assert_scores_match(host[rows], ref, name)


def test_prefill_1x8k_8k_full():
    """1x8K queries over an 8K prefix: every cell against the oracle."""
    inp = WORKLOADS["prefill_1x8k_8k"].make()
    ks, ke = _intervals(inp)
    host = _gpu(inp.q, inp.k, ks, ke, inp.out_cols).cpu().numpy()
    T = inp.q.shape[0]
    for b in range(0, T, 2048):
        rows = np.arange(b, min(T, b + 2048))
        ref = O.prefill(inp.q, inp.k, ks, ke, inp.out_cols, rows=rows)
        assert_scores_match(host[rows], ref, f"prefill_1x8k_8k rows {b}..")


@pytest.mark.parametrize("T,NK,cols", [(1, 5, 5), (5, 70, 64), (63, 200, 65), (64, 64, 64),
                                         (65, 300, 1), (130, 1000, 999), (257, 129, 300)])
def test_prefill_small_full(T, NK, cols):
    rng = np.random.default_rng(T * 1000 + cols)
    q = normal_bf16(rng, (T, 4, 128))
    k = normal_bf16(rng, (NK, 128))
    ks = np.zeros(T, np.int32)
    ke = np.minimum(rng.integers(0, NK + 3, T), NK + 2).astype(np.int32)
    ke[0] = NK  # at least one full row
    gpu = _gpu(q, k, ks, ke, cols)
    assert_scores_match(gpu, O.prefill(q, k, ks, ke, cols), f"T={T} NK={NK} cols={cols}")


def test_prefill_mixed_starts_in_one_workgroup():
    # Packed requests whose boundaries fall inside workgroups, plus
    # negative starts, reversed and empty intervals and ends past the keys.
    rng = np.random.default_rng(21)
    T, NK, cols = 200, 900, 420
    q = normal_bf16(rng, (T, 4, 128))
    k = normal_bf16(rng, (NK, 128))
    bounds = [0, 30, 31, 100, 129, 200]
    offsets = [0, 300, 310, 500, 860]
    ks = np.zeros(T, np.int32)
    ke = np.zeros(T, np.int32)
    for r in range(5):
        for t in range(bounds[r], bounds[r + 1]):
            ks[t] = offsets[r]
            ke[t] = offsets[r] + int(rng.integers(0, 450))
    ks[5], ke[5] = -40, 100
    ks[6], ke[6] = 50, 20
    ks[7], ke[7] = 10, 10
    ks[8], ke[8] = 700, 5000
    gpu = _gpu(q, k, ks, ke, cols)
    assert_scores_match(gpu, O.prefill(q, k, ks, ke, cols), "mixed starts")


def test_prefill_strided_inputs_and_out():
    rng = np.random.default_rng(22)
    T, NK, cols = 150, 333, 333
    q = normal_bf16(rng, (T, 4, 128))
    k = normal_bf16(rng, (NK, 128))
    ks = np.zeros(T, np.int32)
    ke = rng.integers(1, NK + 1, T).astype(np.int32)
    ref = O.prefill(q, k, ks, ke, cols)
    # q rows padded to 5 heads x 136 features; k rows padded to 144 features.
    qw = np.zeros((T, 5, 136), np.uint16)
    qw[:, :4, :128] = q
    kw = np.zeros((NK, 144), np.uint16)
    kw[:, :128] = k
    qd = bf16_to_device(qw)[:, :4, :128]
    kd = bf16_to_device(kw)[:, :128]
    assert_scores_match(_gpu(qd, kd, ks, ke, cols), ref, "strided q/k")
    big = torch.full((T, 350), 9.0, dtype=torch.float32, device="cuda")
    out = big[:, 1:334]                              # stride 350, base off the 16-byte grid
    _gpu(q, k, ks, ke, cols, out=out, poison=False)
    assert_scores_match(out, ref, "strided out")
    host = big.cpu().numpy()
    assert np.all(host[:, 0] == 9.0) and np.all(host[:, 334:] == 9.0)


@pytest.mark.parametrize("pad", [0, 4, 8, 16])
def test_prefill_any_row_pitch_and_base(pad):
    """Line-aligned stores: rows are spaced so that a wave's rows share their
    offset within a 128-byte line, and lanes are rotated by that offset.
    Every row pitch residue (mod 32 floats) and several base offsets, over
    4 column chunks, 2 passes per workgroup, a ragged last tile and rows cut
    short (tiles that are -inf only); the cells around the view must stay
    untouched."""
    rng = np.random.default_rng(23)
    T, NK, cols = 300, 2600, 2000
    q = normal_bf16(rng, (T, 4, 128))
    k = normal_bf16(rng, (NK, 128))
    ks = np.where(np.arange(T) < 150, 0, 40).astype(np.int32)  # two starts in the second row block
    ke = (ks + rng.integers(0, cols + 50, T)).astype(np.int32)
    ke[:10] = ks[:10] + cols                                     # full rows
    ref = O.prefill(q, k, ks, ke, cols)
    stride = cols + pad
    for base in (0, 4, 12, 28):                                  # floats: 0, 16, 48, 112 bytes into a line
        buf = torch.full((T * stride + 64,), 5.0, dtype=torch.float32, device="cuda")
        out = buf[base:base + T * stride].view(T, stride)[:, :cols]
        _gpu(q, k, ks, ke, cols, out=out, poison=False)
        assert_scores_match(out, ref, f"stride {stride} base +{base}")
        host = buf.cpu().numpy()
        inside = np.zeros(host.shape, bool)
        idx = base + np.arange(T)[:, None] * stride + np.arange(cols)[None, :]
        inside[idx.ravel()] = True
        assert np.all(host[~inside] == 5.0), f"stride {stride} base +{base}: write outside the view"



def test_prefill_onehot_bit_exact_and_scale():
    a = np.array([1.0, -1.0, 2.0, 0.5], np.float32)
    q = np.zeros((3, 4, 128), np.float32)
    q[:, :, 0] = a
    keys = np.zeros((8, 128), np.float32)
    keys[:, 0] = np.arange(8) - 2
    ks = np.zeros(3, np.int32)
    ke = np.full(3, 8, np.int32)
    gpu = _gpu(bf16_bits(q), bf16_bits(keys), ks, ke, 8)
    want = [0x3E3504F3, 0x3DB504F3, 0x0, 0x3E9E6455, 0x3F1E6455, 0x3F6D967F, 0x3F9E6455, 0x3FC5FD6A]
    for t in range(3):
        assert list(f32_bits(gpu)[t]) == want
    rng = np.random.default_rng(23)
    qn, kn = normal_bf16(rng, (70, 4, 128)), normal_bf16(rng, (90, 128))
    ks, ke = np.zeros(70, np.int32), np.full(70, 90, np.int32)
    for scale in (1.0, 0.01):
        assert_scores_match(_gpu(qn, kn, ks, ke, 90, scale=scale),
                            O.prefill(qn, kn, ks, ke, 90, scale=scale), f"scale {scale}")


def test_prefill_equals_decode_on_gathered_keys():
    # The same request scored through the paged decode path and through
    # prefill over its gathered keys gives the same masks and scores.
    from workloads import decode_inputs
    qsa = _qsa()
    inp = decode_inputs([2222], 4, 16, table_cols=40, spare_pages=3, out_cols=560, seed=24)
    _, _, vis = O.token_metadata(inp.query_start_loc, inp.seq_lens, 4)
    comp = int(O.comp_lens(inp.seq_lens)[0])
    keys = np.stack([inp.k_pool[inp.page_table[0, c // 16], c % 16, 0] for c in range(comp)])
    dec = qsa.qsa_mqa_decode(bf16_to_device(inp.q), bf16_to_device(inp.k_pool),
                             i32_to_device(inp.page_table), i32_to_device([comp]),
                             i32_to_device(vis), out_cols=560)
    pre = _gpu(np.ascontiguousarray(inp.q[0]), keys, np.zeros(4, np.int32), vis.astype(np.int32), 560)
    torch.cuda.synchronize()
    assert np.array_equal(f32_bits(dec) == 0xFF800000, f32_bits(pre) == 0xFF800000)
    assert_scores_match(pre, dec.cpu().numpy(), "prefill vs decode")


def test_prefill_deterministic():
    inp = WORKLOADS["prefill_1x8k_8k"].make()
    ks, ke = _intervals(inp)
    a = f32_bits(_gpu(inp.q, inp.k, ks, ke, inp.out_cols))
    b = f32_bits(_gpu(inp.q, inp.k, ks, ke, inp.out_cols))
    assert np.array_equal(a, b)
