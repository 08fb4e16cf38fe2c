"""GPU: qsa_mqa_decode_static_plan (the decode whose task table lives in the
library's own device array) against qsa_mqa_decode_planned with a table the
caller allocated, on two calls in a row (the second with a smaller batch),
and its capacity limit."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from tests.parity import bf16_to_device, f32_bits, i32_to_device
from workloads import WORKLOADS, decode_inputs

pytestmark = pytest.mark.gpu


def _qsa():
    import block_indexer_scoring_amd as qsa
    qsa.load_library()
    return qsa


def _dev(inp):
    comp = O.comp_lens(inp.seq_lens)
    _, _, vis = O.token_metadata(inp.query_start_loc, inp.seq_lens, inp.num_reqs * inp.dql)
    return (bf16_to_device(inp.q), bf16_to_device(inp.k_pool), i32_to_device(inp.page_table),
            i32_to_device(comp), i32_to_device(vis))


def _planned(qsa, inp, dev):
    q, k, pt, comp, vis = dev
    plan = qsa.qsa_build_decode_plan(comp, pt, k.shape[0], inp.page_size, inp.out_cols)
    return qsa.qsa_mqa_decode_planned(plan, q, k, pt, vis, out_cols=inp.out_cols)


def test_static_plan_decode_two_calls_match_the_planned_decode():
    qsa = _qsa()
    big = WORKLOADS["specdecode_16x51k"].make()              # 16 x 400 = 6,400 table entries
    small = decode_inputs([5000, 17, 0, 900], 3, 64, table_cols=30, spare_pages=2, out_cols=700, seed=41)
    for inp in (big, small):
        dev = _dev(inp)
        q, k, pt, comp, vis = dev
        out = torch.full((inp.num_reqs * inp.dql, inp.out_cols), float("nan"), device="cuda")
        qsa.qsa_mqa_decode_static_plan(q, k, pt, comp, vis, out=out)
        ref = _planned(qsa, inp, dev)
        torch.cuda.synchronize()
        assert np.array_equal(f32_bits(out), f32_bits(ref)), inp.num_reqs


def test_static_plan_decode_page_size_16():
    """A page size that is not a multiple of 64 (per-key page lookups)."""
    qsa = _qsa()
    inp = decode_inputs([3000, 640, 2], 4, 16, table_cols=60, spare_pages=3, out_cols=800, seed=42)
    dev = _dev(inp)
    q, k, pt, comp, vis = dev
    out = qsa.qsa_mqa_decode_static_plan(q, k, pt, comp, vis, out_cols=inp.out_cols)
    ref = _planned(qsa, inp, dev)
    torch.cuda.synchronize()
    assert np.array_equal(f32_bits(out), f32_bits(ref))


def test_static_plan_decode_refuses_more_than_its_table_holds():
    qsa = _qsa()
    R = 1025                                   # 1,025 x 256 spans > 262,144 entries
    q = torch.zeros((R, 1, 4, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 64, 1, 128), dtype=torch.bfloat16, device="cuda")
    pt = torch.zeros((R, 1), dtype=torch.int32, device="cuda")
    comp = torch.zeros(R, dtype=torch.int32, device="cuda")
    out = torch.empty((R, 256 * 64), dtype=torch.float32, device="cuda")
    with pytest.raises(qsa.QSAError, match="262144"):
        qsa.qsa_mqa_decode_static_plan(q, k, pt, comp, None, out=out)
