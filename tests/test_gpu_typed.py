"""GPU parity: the typed entry points (qsa_mqa_decode_typed with bf16/fp16
queries and bf16/fp16/fp8-e4m3 keys; qsa_mqa_prefill_typed with fp16 queries
and keys) against the oracle's typed functions, plus bit-exact cross-checks
between formats on inputs every format holds exactly."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from tests.parity import assert_scores_match, bf16_to_device, f32_bits, i32_to_device
from workloads import (FP8_K_SCALE, WORKLOADS, bf16_bits, bits_to_f32, decode_inputs, fp8_e4m3_cache,
                       fp16_bits, normal_bf16)

pytestmark = pytest.mark.gpu


def _qsa():
    import block_indexer_scoring_amd as qsa
    qsa.load_library()
    return qsa


def _dev(bits, dtype):
    """Bit patterns (uint16 / uint8) -> device tensor of the given dtype."""
    a = np.ascontiguousarray(bits)
    if a.dtype == np.uint8:
        return torch.from_numpy(a).to("cuda").view(dtype)
    return torch.from_numpy(a.view(np.int16)).to("cuda").view(dtype)


_TORCH = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp8_e4m3": torch.float8_e4m3fn}


def _decode_typed(inp, q_bits, qf, k_bits, kf, k_scale, vis, comp, out_cols=None):
    qsa = _qsa()
    out_cols = inp.out_cols if out_cols is None else out_cols
    out = torch.full((inp.q.shape[0] * inp.q.shape[1], out_cols), float("nan"), device="cuda")
    qsa.qsa_mqa_decode_typed(_dev(q_bits, _TORCH[qf]), _dev(k_bits, _TORCH[kf]), i32_to_device(inp.page_table),
                             i32_to_device(comp), i32_to_device(vis), k_scale=k_scale, out=out)
    torch.cuda.synchronize()
    return out


def _meta(inp):
    T = inp.q.shape[0] * inp.q.shape[1]
    return O.token_metadata(inp.query_start_loc, inp.seq_lens, T)[2], O.comp_lens(inp.seq_lens)


def test_decode_fp8_keys_full_spec_decode_batch():
    # The 16-request spec-decode batch (DQL 4, contexts 3,508 .. 102,400,
    # page size 64) with its key cache written as e4m3 codes: every row.
    inp = WORKLOADS["specdecode_16x51k"].make()
    vis, comp = _meta(inp)
    k8 = fp8_e4m3_cache(inp.k_pool)
    gpu = _decode_typed(inp, inp.q, "bf16", k8, "fp8_e4m3", FP8_K_SCALE, vis, comp)
    ref = O.decode_typed(inp.q, "bf16", k8, "fp8_e4m3", inp.page_table, comp, vis, inp.out_cols,
                         k_scale=FP8_K_SCALE)
    assert_scores_match(gpu, ref, "fp8 keys, spec-decode batch")


@pytest.mark.parametrize("qf,kf,page_size", [("fp16", "fp16", 64), ("fp16", "fp16", 16), ("fp16", "fp8_e4m3", 64),
                                             ("fp16", "fp8_e4m3", 48), ("bf16", "fp8_e4m3", 16),
                                             ("bf16", "fp8_e4m3", 128), ("bf16", "bf16", 48)])
def test_decode_typed_small_with_missing_pages(qf, kf, page_size):
    rng = np.random.default_rng(page_size + len(qf + kf))
    inp = decode_inputs([3000, 517, 12, 4400], 3, page_size, 80, 4, 1200, seed=page_size)
    vis, comp = _meta(inp)
    pt = inp.page_table.copy()
    pt[1, 1] = -1                      # a missing page inside the visible range
    pt[3, 2] = inp.k_pool.shape[0] + 9  # an out-of-range page id
    inp.page_table[:] = pt
    qv = bits_to_f32(inp.q)
    q_bits = fp16_bits(qv) if qf == "fp16" else inp.q
    if kf == "fp8_e4m3":
        k_bits, k_scale = fp8_e4m3_cache(inp.k_pool, 0.0173), 0.0173
    elif kf == "fp16":
        k_bits, k_scale = fp16_bits(bits_to_f32(inp.k_pool)), 1.0
    else:
        k_bits, k_scale = inp.k_pool, 1.0
    gpu = _decode_typed(inp, q_bits, qf, k_bits, kf, k_scale, vis, comp)
    ref = O.decode_typed(q_bits, qf, k_bits, kf, inp.page_table, comp, vis, inp.out_cols, k_scale=k_scale)
    assert_scores_match(gpu, ref, f"{qf}/{kf} ps={page_size}")


def test_decode_typed_bf16_equals_untyped():
    qsa = _qsa()
    inp = decode_inputs([900, 2100], 4, 64, 40, 2, 600, seed=5)
    vis, comp = _meta(inp)
    typed = _decode_typed(inp, inp.q, "bf16", inp.k_pool, "bf16", 1.0, vis, comp)
    plain = qsa.qsa_mqa_decode(bf16_to_device(inp.q), bf16_to_device(inp.k_pool), i32_to_device(inp.page_table),
                               i32_to_device(comp), i32_to_device(vis), out_cols=inp.out_cols)
    torch.cuda.synchronize()
    assert np.array_equal(f32_bits(typed), f32_bits(plain))


@pytest.mark.parametrize("page_size", [64, 16])
def test_decode_formats_bit_exact_on_exact_values(page_size):
    """Integer queries and keys (|q| <= 8, e4m3 codes of integers |k| <= 15
    with k_scale 0.5): every partial sum is exact in fp32, so the fp8 and fp16
    paths must reproduce the bf16 kernel bit for bit; this also checks that
    the fp8 path reorders query features exactly as it reorders key codes."""
    rng = np.random.default_rng(page_size)
    inp = decode_inputs([700, 2600, 64], 4, page_size, 60, 2, 700, seed=7)
    vis, comp = _meta(inp)
    qv = rng.integers(-8, 9, inp.q.shape).astype(np.float32)
    kv = rng.integers(-15, 16, inp.k_pool.shape).astype(np.float32)
    k8 = torch.from_numpy(kv).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    base = _decode_typed(inp, bf16_bits(qv), "bf16", bf16_bits(kv * 0.5), "bf16", 1.0, vis, comp)
    for q_bits, qf, k_bits, kf in ((bf16_bits(qv), "bf16", k8, "fp8_e4m3"), (fp16_bits(qv), "fp16", k8, "fp8_e4m3"),
                                   (fp16_bits(qv), "fp16", fp16_bits(kv * 0.5), "fp16")):
        got = _decode_typed(inp, q_bits, qf, k_bits, kf, 0.5, vis, comp)
        assert np.array_equal(f32_bits(got), f32_bits(base)), (qf, kf)


def _prefill_typed(q_bits, k_bits, ks, ke, cols, dtype=torch.float16, out=None):
    qsa = _qsa()
    qd, kd = _dev(q_bits, dtype), _dev(k_bits, dtype)
    if out is None:
        out = torch.full((qd.shape[0], cols), float("nan"), device="cuda")
    qsa.qsa_mqa_prefill_typed(qd, kd, i32_to_device(ks), i32_to_device(ke), out=out)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("T,NK,cols", [(1, 5, 5), (63, 200, 65), (130, 1000, 999), (300, 2600, 2000)])
def test_prefill_fp16_small_full(T, NK, cols):
    rng = np.random.default_rng(T + cols)
    q = fp16_bits(bits_to_f32(normal_bf16(rng, (T, 4, 128))) * 1.37)
    k = fp16_bits(rng.standard_normal((NK, 128)).astype(np.float32))
    ks = rng.integers(-20, 30, T).astype(np.int32)
    ke = (ks + rng.integers(0, cols + 40, T)).astype(np.int32)
    gpu = _prefill_typed(q, k, ks, ke, cols)
    assert_scores_match(gpu, O.prefill_typed(q, "fp16", k, "fp16", ks, ke, cols), f"fp16 T={T}")


def test_prefill_fp16_1x8k_over_100k_sampled():
    # 1x8K queries over a 100K prefix, inputs rounded to fp16.
    inp = WORKLOADS["prefill_1x8k_100k"].make()
    T = inp.q.shape[0]
    req, _, vis = O.token_metadata(inp.query_start_loc, inp.seq_lens, T)
    ks, ke = O.prefill_intervals(req, vis, inp.key_offsets)
    q, k = fp16_bits(bits_to_f32(inp.q)), fp16_bits(bits_to_f32(inp.k))
    gpu = _prefill_typed(q, k, ks, ke, inp.out_cols)
    rows = np.array([0, 1, 2, 63, 64, 127, 128, 1000, 4095, 4096, 8000, T - 1])
    ref = O.prefill_typed(q, "fp16", k, "fp16", ks, ke, inp.out_cols, rows=rows)
    assert_scores_match(gpu[torch.from_numpy(rows).cuda()], ref, "fp16 NS sampled")
    # Every row: -inf exactly outside the interval, finite and >= +0 inside
    # (the output started as NaN, so an unwritten cell fails).
    bits = gpu.cpu().numpy().view(np.uint32)
    key = ks.astype(np.int64)[:, None] + np.arange(inp.out_cols)[None, :]
    valid = (key >= 0) & (key < inp.k.shape[0]) & (key < ke.astype(np.int64)[:, None])
    assert np.array_equal(bits == 0xFF800000, ~valid)
    assert np.all(bits[valid] < 0x7F800000)


@pytest.mark.parametrize("pad,base", [(4, 12), (8, 0), (16, 28)])
def test_prefill_fp16_row_pitch_and_base(pad, base):
    rng = np.random.default_rng(pad)
    T, NK, cols = 300, 2600, 2000
    q = fp16_bits(rng.standard_normal((T, 4, 128)).astype(np.float32))
    k = fp16_bits(rng.standard_normal((NK, 128)).astype(np.float32))
    ks = np.where(np.arange(T) < 150, 0, 40).astype(np.int32)
    ke = (ks + rng.integers(0, cols + 50, T)).astype(np.int32)
    stride = cols + pad
    buf = torch.full((T * stride + 64,), 5.0, dtype=torch.float32, device="cuda")
    out = buf[base:base + T * stride].view(T, stride)[:, :cols]
    _prefill_typed(q, k, ks, ke, cols, out=out)
    assert_scores_match(out, O.prefill_typed(q, "fp16", k, "fp16", ks, ke, cols), f"stride {stride}")
    host = buf.cpu().numpy()
    inside = np.zeros(host.shape, bool)
    inside[(base + np.arange(T)[:, None] * stride + np.arange(cols)[None, :]).ravel()] = True
    assert np.all(host[~inside] == 5.0)


def test_prefill_fp16_bit_exact_on_exact_values():
    rng = np.random.default_rng(3)
    T, NK, cols = 200, 900, 700
    qv = rng.integers(-8, 9, (T, 4, 128)).astype(np.float32)
    kv = rng.integers(-15, 16, (NK, 128)).astype(np.float32) * 0.5
    ks = np.zeros(T, np.int32)
    ke = rng.integers(0, NK + 1, T).astype(np.int32)
    f16 = _prefill_typed(fp16_bits(qv), fp16_bits(kv), ks, ke, cols)
    b16 = _prefill_typed(bf16_bits(qv), bf16_bits(kv), ks, ke, cols, dtype=torch.bfloat16)
    assert np.array_equal(f32_bits(f16), f32_bits(b16))


@pytest.mark.parametrize("dql,qf,kf", [(5, "bf16", "fp8_e4m3"), (8, "fp16", "fp8_e4m3"), (13, "fp16", "fp16"),
                                       (16, "bf16", "fp8_e4m3"), (16, "fp16", "fp16"), (9, "fp16", "fp8_e4m3")])
def test_decode_typed_query_lengths(dql, qf, kf):
    # 2, 3 and 4 query tiles per wave (DQL 5..16) in every format.
    inp = decode_inputs([2600, 700, 64 + dql, 5000], dql, 64, 90, 2, 1300, seed=100 + dql)
    vis, comp = _meta(inp)
    q_bits = fp16_bits(bits_to_f32(inp.q)) if qf == "fp16" else inp.q
    if kf == "fp8_e4m3":
        k_bits, k_scale = fp8_e4m3_cache(inp.k_pool, 0.011), 0.011
    else:
        k_bits, k_scale = fp16_bits(bits_to_f32(inp.k_pool)), 1.0
    gpu = _decode_typed(inp, q_bits, qf, k_bits, kf, k_scale, vis, comp)
    ref = O.decode_typed(q_bits, qf, k_bits, kf, inp.page_table, comp, vis, inp.out_cols, k_scale=k_scale)
    assert_scores_match(gpu, ref, f"DQL {dql} {qf}/{kf}")
