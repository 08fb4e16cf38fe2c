"""GPU parity: qsa_mqa_prefill_topk (fused prefill scores + per-row top-k).

The fused call must return exactly what qsa_topk_blocks returns on the
output of qsa_mqa_prefill with the same arguments (bit for bit: same scores,
same tie rule).  That composition is itself checked against the oracle in
test_gpu_prefill.py and test_gpu_topk_meta.py; here the fused picks are also
checked against the oracle's scores (the top-k tolerance rule) and, for
exact ties, against the oracle's selection rule run on the GPU scores.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from tests.parity import assert_topk_valid, bf16_to_device, i32_to_device
from workloads import WORKLOADS, normal_bf16

pytestmark = pytest.mark.gpu


def _qsa():
    import block_indexer_scoring_amd as qsa
    qsa.load_library()
    return qsa


def _both(q, k, ks, ke, out_cols, topk, workspace=None):
    """(fused picks, composed picks, scores) for the same arguments."""
    qsa = _qsa()
    qd = bf16_to_device(q) if isinstance(q, np.ndarray) else q
    kd = bf16_to_device(k) if isinstance(k, np.ndarray) else k
    ksd, ked = i32_to_device(ks), i32_to_device(ke)
    fused = torch.full((qd.shape[0], topk), -7, dtype=torch.int32, device="cuda")
    qsa.qsa_mqa_prefill_topk(qd, kd, ksd, ked, out_cols, topk, out=fused, workspace=workspace)
    scores = qsa.qsa_mqa_prefill(qd, kd, ksd, ked, out_cols)
    composed = qsa.qsa_topk_blocks(scores, topk)
    torch.cuda.synchronize()
    return fused, composed, scores


def _assert_same(fused, composed, what):
    if not torch.equal(fused, composed):
        diff = (fused != composed).any(dim=1).nonzero().flatten()
        t = int(diff[0])
        raise AssertionError(f"{what}: {diff.numel()} rows differ, first row {t}: "
                             f"fused {fused[t, :8].tolist()} composed {composed[t, :8].tolist()}")


def _intervals(inp):
    T = inp.q.shape[0]
    req, _, vis = O.token_metadata(inp.query_start_loc, inp.seq_lens, T)
    return O.prefill_intervals(req, vis, inp.key_offsets)


@pytest.mark.parametrize("name,topk", [("prefill_1x8k_8k", 512), ("prefill_1x8k_100k", 512),
                                       ("prefill_4x4k_100k", 512), ("prefill_1x8k_100k", 2048)])
def test_fused_equals_composition_full_size(name, topk):
    inp = WORKLOADS[name].make()
    ks, ke = _intervals(inp)
    fused, composed, _ = _both(inp.q, inp.k, ks, ke, inp.out_cols, topk)
    _assert_same(fused, composed, f"{name} top-{topk}")
    # Sampled rows checked with the oracle's own scores.
    rows = np.array([0, 1, 2, 127, 128, 4095, inp.q.shape[0] - 1])
    ref = O.prefill(inp.q, inp.k, ks, ke, inp.out_cols, rows=rows)
    assert_topk_valid(fused[torch.from_numpy(rows).cuda()], ref, topk)


@pytest.mark.parametrize("T,NK,cols,topk", [(200, 900, 420, 16), (130, 5000, 4999, 100), (64, 3000, 2050, 2048),
                                            (300, 1200, 1200, 1)])
def test_fused_small_against_oracle(T, NK, cols, topk):
    rng = np.random.default_rng(T + NK + topk)
    q = normal_bf16(rng, (T, 4, 128))
    k = normal_bf16(rng, (NK, 128))
    ks = rng.integers(-50, 60, T).astype(np.int32)
    ke = (ks + rng.integers(0, cols + 80, T)).astype(np.int32)
    fused, composed, _ = _both(q, k, ks, ke, cols, topk)
    _assert_same(fused, composed, f"T={T} NK={NK} cols={cols} k={topk}")
    assert_topk_valid(fused, O.prefill(q, k, ks, ke, cols), topk)


def test_fused_mixed_starts_short_and_empty_rows():
    # Requests whose boundaries fall inside a workgroup (one pass per start),
    # rows with fewer visible keys than k, empty and reversed intervals.
    rng = np.random.default_rng(31)
    T, NK, cols, topk = 300, 2000, 1500, 256
    q = normal_bf16(rng, (T, 4, 128))
    k = normal_bf16(rng, (NK, 128))
    bounds = [0, 40, 41, 150, 260, 300]
    offsets = [0, 300, 310, 800, 1400]
    ks = np.zeros(T, np.int32)
    ke = np.zeros(T, np.int32)
    for r in range(5):
        for t in range(bounds[r], bounds[r + 1]):
            ks[t] = offsets[r]
            ke[t] = offsets[r] + int(rng.integers(0, 1200))
    ks[5], ke[5] = -40, 100      # negative start
    ks[6], ke[6] = 50, 20        # reversed: all -inf
    ks[7], ke[7] = 10, 10        # empty
    ks[8], ke[8] = 700, 700 + 30  # fewer than k visible
    fused, composed, _ = _both(q, k, ks, ke, cols, topk)
    _assert_same(fused, composed, "mixed starts")
    ref = O.prefill(q, k, ks, ke, cols)
    assert_topk_valid(fused, ref, topk)
    host = fused.cpu().numpy()
    assert np.all(host[6] == -1) and np.all(host[7] == -1)
    assert np.array_equal(host[8, :30], np.arange(30)) and np.all(host[8, 30:] == -1)


def test_fused_exact_ties():
    # Duplicated keys give bit-identical scores in different columns, and an
    # all-zero query row makes every visible score +0: the picks must follow
    # the tie rule exactly (lower column first).
    rng = np.random.default_rng(41)
    T, cols, topk = 160, 1100, 300
    base = normal_bf16(rng, (50, 128))
    k = base[rng.integers(0, 50, cols)]            # every key repeats about 22 times
    q = normal_bf16(rng, (T, 4, 128))
    q[3] = 0                                       # all scores +0
    q[4, :2] = 0                                   # two heads zero
    ks = np.zeros(T, np.int32)
    ke = rng.integers(topk // 2, cols + 1, T).astype(np.int32)
    fused, composed, scores = _both(q, k, ks, ke, cols, topk)
    _assert_same(fused, composed, "ties")
    # The selection rule itself, run by the oracle on the GPU scores.
    want = O.topk(scores.cpu().numpy(), topk)
    assert np.array_equal(fused.cpu().numpy(), want)
    assert np.array_equal(fused[3, :min(topk, int(ke[3]))].cpu().numpy(), np.arange(min(topk, int(ke[3]))))


def test_fused_workspace_reuse_and_zero_columns():
    qsa = _qsa()
    rng = np.random.default_rng(51)
    T, NK, cols, topk = 140, 800, 700, 64
    q = normal_bf16(rng, (T, 4, 128))
    k = normal_bf16(rng, (NK, 128))
    ks = np.zeros(T, np.int32)
    ke = rng.integers(0, NK + 1, T).astype(np.int32)
    need = qsa.qsa_prefill_topk_workspace_bytes(T, cols, topk)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")  # garbage contents
    first, composed, _ = _both(q, k, ks, ke, cols, topk, workspace=ws)
    _assert_same(first, composed, "first call")
    second, _, _ = _both(q, k, ks, ke, cols, topk, workspace=ws)   # the same workspace again
    _assert_same(second, composed, "second call")
    # Zero columns: every row is -1 padding.
    out = torch.zeros((T, topk), dtype=torch.int32, device="cuda")
    qsa.qsa_mqa_prefill_topk(bf16_to_device(q), bf16_to_device(k), i32_to_device(ks), i32_to_device(ke), 0,
                             topk, out=out)
    torch.cuda.synchronize()
    assert torch.all(out == -1)


def test_fused_rows_left_to_the_fallback():
    # k = 2048 over rows of 5,000-12,000 visible keys: fewer than k of the
    # 8-key chunks bound the floor, so more than the in-register list holds
    # is listed, and those rows are rescored whole by the fallback (more rows
    # than it has workgroups, so each takes several).
    rng = np.random.default_rng(61)
    T, NK, cols, topk = 200, 12000, 12000, 2048
    q = normal_bf16(rng, (T, 4, 128))
    k = normal_bf16(rng, (NK, 128))
    ks = np.zeros(T, np.int32)
    ke = rng.integers(5000, NK + 1, T).astype(np.int32)
    ke[::7] = rng.integers(0, 2000, len(ke[::7]))  # and some rows the list holds
    fused, composed, _ = _both(q, k, ks, ke, cols, topk)
    _assert_same(fused, composed, "fallback rows")
    rows = np.array([0, 1, 7, 100, T - 1])
    assert_topk_valid(fused[torch.from_numpy(rows).cuda()], O.prefill(q, k, ks, ke, cols, rows=rows), topk)


def test_fused_wide_rows():
    # Rows wider than 32,768 columns take the group-maximum path.
    rng = np.random.default_rng(71)
    T, NK, cols, topk = 96, 41000, 40000, 512
    q = normal_bf16(rng, (T, 4, 128))
    k = normal_bf16(rng, (NK, 128))
    ks = rng.integers(-100, 900, T).astype(np.int32)
    ke = (ks + rng.integers(0, cols + 200, T)).astype(np.int32)
    fused, composed, _ = _both(q, k, ks, ke, cols, topk)
    _assert_same(fused, composed, "wide rows")
    rows = np.array([0, 5, T - 1])
    assert_topk_valid(fused[torch.from_numpy(rows).cuda()], O.prefill(q, k, ks, ke, cols, rows=rows), topk)


def test_fused_non_finite_inputs():
    # NaN and +-inf in queries and keys give NaN and +inf scores: a NaN cell
    # is never picked and +inf cells rank first, in the fused path (16-bit
    # key prefixes, rescored ties) as in the composition.
    rng = np.random.default_rng(81)
    T, NK, cols, topk = 160, 1500, 1400, 200
    q = normal_bf16(rng, (T, 4, 128))
    k = normal_bf16(rng, (NK, 128))
    nan, pinf, ninf = np.uint16(0x7FC0), np.uint16(0x7F80), np.uint16(0xFF80)
    q[3, 0, 5] = nan           # row 3: a NaN head, so every visible score is NaN or the other heads' sum
    q[7, :, :] = 0
    q[7, 1, 9] = pinf          # row 7: +inf x key feature -> +inf, NaN (x 0) or -inf dots
    k[11, 17] = nan            # key 11: NaN in every row's dot with it
    k[40, 2] = pinf
    k[41, 2] = ninf
    k[300:340] = k[299]        # a run of identical keys: ties across the picked boundary
    ks = np.zeros(T, np.int32)
    ke = rng.integers(topk // 2, cols + 1, T).astype(np.int32)
    ke[3] = ke[7] = cols
    fused, composed, scores = _both(q, k, ks, ke, cols, topk)
    _assert_same(fused, composed, "non-finite inputs")
    want = O.topk(scores.cpu().numpy(), topk)
    assert np.array_equal(fused.cpu().numpy(), want)
    assert 11 not in fused[5].cpu().numpy().tolist()   # the NaN key's cell is never picked


@pytest.mark.parametrize("cols", [28_700, 32_768, 32_769])
def test_fused_widest_key_select_rows(cols):
    # The key select's widest shape (64 key prefixes per thread, up to 32,768
    # columns) and the first width past it (the group-maximum path).
    rng = np.random.default_rng(cols)
    T, topk = 48, 512
    NK = cols + 300
    q = normal_bf16(rng, (T, 4, 128))
    k = normal_bf16(rng, (NK, 128))
    ks = rng.integers(-50, 250, T).astype(np.int32)
    ke = (ks + rng.integers(cols // 2, cols + 100, T)).astype(np.int32)
    fused, composed, _ = _both(q, k, ks, ke, cols, topk)
    _assert_same(fused, composed, f"{cols} columns")
    rows = np.array([0, T - 1])
    assert_topk_valid(fused[torch.from_numpy(rows).cuda()], O.prefill(q, k, ks, ke, cols, rows=rows), topk)


def _f16(bits_bf16):
    """bf16 bit patterns -> the same values as an fp16 device tensor (values
    drawn N(0,1) are well inside fp16's range; rounding to fp16 is fine: both
    sides of the comparison get the same fp16 inputs)."""
    f = torch.from_numpy(bits_bf16.astype(np.uint32) << 16).view(torch.float32)
    return f.to(torch.float16).cuda()


@pytest.mark.parametrize("name", ["prefill_1x8k_100k", None])
def test_fused_fp16_equals_typed_composition(name):
    qsa = _qsa()
    if name:
        inp = WORKLOADS[name].make()
        q, k, cols, topk = inp.q, inp.k, inp.out_cols, 512
        ks, ke = _intervals(inp)
    else:
        rng = np.random.default_rng(91)
        T, NK, cols, topk = 260, 3000, 2900, 300
        q = normal_bf16(rng, (T, 4, 128))
        base = normal_bf16(rng, (60, 128))
        k = base[rng.integers(0, 60, NK)]      # repeated keys: exact ties
        q[2] = 0                               # a row of +0 scores (the fallback)
        ks = rng.integers(-40, 80, T).astype(np.int32)
        ke = (ks + rng.integers(0, cols + 60, T)).astype(np.int32)
    qd, kd = _f16(q), _f16(k)
    ksd, ked = i32_to_device(ks), i32_to_device(ke)
    fused = qsa.qsa_mqa_prefill_topk(qd, kd, ksd, ked, cols, topk)
    scores = qsa.qsa_mqa_prefill_typed(qd, kd, ksd, ked, cols)
    composed = qsa.qsa_topk_blocks(scores, topk)
    torch.cuda.synchronize()
    _assert_same(fused, composed, f"fp16 {name or 'small with ties'}")
    if not name:
        assert np.array_equal(fused.cpu().numpy(), O.topk(scores.cpu().numpy(), topk))
