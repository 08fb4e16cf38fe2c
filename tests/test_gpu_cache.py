"""GPU parity: qsa_build_cache_metadata (compressed-cache slots, writer work
items) and qsa_gather_keys (paged keys into contiguous rows) against the
oracle; bit-exact (integer and copy work)."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from tests.oracle_pins import _CM_BT, _CM_QSL, _CM_SEQ, _read_golden
from tests.parity import bf16_to_device, f32_bits, i32_to_device
from workloads import FP8_K_SCALE, WORKLOADS, bf16_bits, decode_inputs, fp8_e4m3_cache

pytestmark = pytest.mark.gpu


def _qsa():
    import block_indexer_scoring_amd as qsa
    qsa.load_library()
    return qsa


def _meta(qsl, seq, T, bt, sbs, cr=4, common=None, max_work=0):
    qsa = _qsa()
    cm = None if common is None else torch.from_numpy(np.ascontiguousarray(common, np.int64)).cuda()
    slots = torch.full((T,), 12345, dtype=torch.int64, device="cuda")
    work = torch.full((max(max_work, 1), 2), 777, dtype=torch.int32, device="cuda")
    s, w = qsa.qsa_build_cache_metadata(i32_to_device(qsl), i32_to_device(seq), T, i32_to_device(bt), sbs, cr,
                                        common_slot_mapping=cm, max_num_work=max_work, slot_mapping=slots,
                                        k_work=work if max_work else None)
    torch.cuda.synchronize()
    return s.cpu().numpy(), (None if w is None else w.cpu().numpy())


def test_cache_metadata_golden_batch():
    rows = {r[0]: r[1:] for r in _read_golden("cache_metadata.txt")}
    common = np.zeros(19, np.int64)
    common[15] = -1
    slots, work = _meta(_CM_QSL, _CM_SEQ, 19, _CM_BT, 2, 4, common, max_work=12)
    assert slots.tolist() == [int(x) for x in rows["slots"]]
    assert work.tolist() == [[int(v) for v in it.split(",")] for it in rows["work"]]
    _, work5 = _meta(_CM_QSL, _CM_SEQ, 19, _CM_BT, 2, 4, common, max_work=5)
    assert np.array_equal(work5, work[:5])


@pytest.mark.parametrize("seed,cr,sbs,n", [(1, 4, 64, 40), (2, 4, 3, 300), (3, 2, 7, 9), (4, 1, 16, 2000),
                                           (5, 4, 16, 8192)])
def test_cache_metadata_random_batches(seed, cr, sbs, n):
    rng = np.random.default_rng(seed)
    qlens = rng.integers(0, 12, n)
    qlens[rng.integers(0, n)] = 900                        # one long prefill chunk
    seqs = (qlens + rng.integers(0, 5000, n)).astype(np.int32)
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    T = int(qsl[-1]) + 37                                   # padding tokens
    cols = int(seqs.max()) // cr // sbs + 2
    bt = rng.integers(-1, 1 << 20, (n, cols)).astype(np.int32)
    common = rng.integers(-1, 1 << 30, T).astype(np.int64)
    W = int(rng.integers(1, 3 * T))
    slots, work = _meta(qsl, seqs, T, bt, sbs, cr, common, max_work=W)
    assert np.array_equal(slots, O.cache_slots(qsl, seqs, T, bt, sbs, cr, common))
    assert np.array_equal(work, O.k_work(qsl, seqs, W, cr))
    slots2, _ = _meta(qsl, seqs, T, bt, sbs, cr)           # no main-cache slots
    assert np.array_equal(slots2, O.cache_slots(qsl, seqs, T, bt, sbs, cr))


def test_cache_metadata_mixed_step_batch():
    # The mixed step's batch: 16 decode requests (DQL 4) and one 8,192-token
    # prefill chunk over a 100,000-token prefix; page size 64.
    dec = WORKLOADS["specdecode_16x51k"].make()
    R, DQL = dec.q.shape[0], dec.q.shape[1]
    qlens = [DQL] * R + [8192]
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    seqs = np.concatenate([dec.seq_lens, [108192]]).astype(np.int32)
    cols = max(dec.page_table.shape[1], 108192 // 4 // 64 + 1)
    bt = np.full((R + 1, cols), -1, np.int32)
    bt[:R, :dec.page_table.shape[1]] = dec.page_table
    bt[R] = np.random.default_rng(9).permutation(cols) + 5000
    T = int(qsl[-1])
    slots, work = _meta(qsl, seqs, T, bt, 64, 4, max_work=4096)
    assert np.array_equal(slots, O.cache_slots(qsl, seqs, T, bt, 64, 4))
    assert np.array_equal(work, O.k_work(qsl, seqs, 4096, 4))
    assert (slots >= 0).sum() == R + 8192 // 4  # one closing token per decode request, 2,048 in the chunk


def _gather(pool, table, counts, offsets, max_keys, out):
    qsa = _qsa()
    qsa.qsa_gather_keys(pool, i32_to_device(table), i32_to_device(counts), i32_to_device(offsets), max_keys, out=out)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("fmt,page_size", [("bf16", 64), ("bf16", 5), ("fp16", 16), ("fp8_e4m3", 64), ("fp8_e4m3", 7)])
def test_gather_keys_against_oracle(fmt, page_size):
    rng = np.random.default_rng(page_size)
    inp = decode_inputs([3000, 517, 12, 8400, 0], 1, page_size, 500, 4, 2200, seed=page_size)
    table = inp.page_table.copy()
    table[1, 2] = -1
    table[3, 5] = inp.k_pool.shape[0] + 3
    counts = O.comp_lens(inp.seq_lens).astype(np.int32)
    counts[0] += 9                                          # runs past the request's pages into -1 entries
    # Disjoint destinations; the end of request 3 falls past the last row.
    offsets = np.array([5, 800, 950, 1000, 40], np.int32)
    rows = 3000
    if fmt == "fp8_e4m3":
        pool_bits = fp8_e4m3_cache(inp.k_pool)
        pool = torch.from_numpy(pool_bits).cuda().view(torch.float8_e4m3fn)
        out = torch.full((rows, 128), 0x5A, dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn)
        host = np.full((rows, 128), 0x5A, np.uint8)
    else:
        pool_bits = inp.k_pool
        dt = torch.bfloat16 if fmt == "bf16" else torch.float16
        pool = torch.from_numpy(pool_bits.view(np.int16)).cuda().view(dt)
        out = torch.full((rows, 128), 0x3A5A, dtype=torch.int16, device="cuda").view(dt)
        host = np.full((rows, 128), 0x3A5A, np.uint16)
    max_keys = int(counts.max())
    _gather(pool, table, counts, offsets, max_keys, out)
    # The oracle's gather, restricted to destinations inside the output.
    want = np.concatenate([host, np.zeros((4000, 128), host.dtype)])
    O.gather_keys(pool_bits, table, counts, offsets, want)
    want = want[:rows]
    got = out.view(torch.uint8 if fmt == "fp8_e4m3" else torch.int16).cpu().numpy().view(host.dtype)
    assert np.array_equal(got, want)
    # A smaller max_keys clamps every request's count.
    out2 = out.clone().view(torch.uint8 if fmt == "fp8_e4m3" else torch.int16).fill_(0x11).view(out.dtype)
    _gather(pool, table, counts, offsets, 100, out2)
    want2 = np.concatenate([np.full((rows, 128), 0x11 if fmt == "fp8_e4m3" else 0x0011, host.dtype),
                            np.zeros((4000, 128), host.dtype)])
    O.gather_keys(pool_bits, table, np.minimum(counts, 100), offsets, want2)
    got2 = out2.view(torch.uint8 if fmt == "fp8_e4m3" else torch.int16).cpu().numpy().view(host.dtype)
    assert np.array_equal(got2, want2[:rows])


def test_gather_then_prefill_equals_decode():
    # The spec-decode batch scored by decode over its paged cache, and by
    # prefill over the same keys gathered into one packed K: bit-exact.
    qsa = _qsa()
    inp = WORKLOADS["specdecode_16x51k"].make()
    R, DQL = inp.q.shape[0], inp.q.shape[1]
    _, _, vis = O.token_metadata(inp.query_start_loc, inp.seq_lens, R * DQL)
    comp = O.comp_lens(inp.seq_lens).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(comp[:-1])]).astype(np.int32)
    pool, table = bf16_to_device(inp.k_pool), i32_to_device(inp.page_table)
    k = torch.zeros((int(comp.sum()), 128), dtype=torch.bfloat16, device="cuda")
    qsa.qsa_gather_keys(pool, table, i32_to_device(comp), i32_to_device(offsets), int(comp.max()), out=k)
    dec = qsa.qsa_mqa_decode(bf16_to_device(inp.q), pool, table, i32_to_device(comp), i32_to_device(vis),
                             out_cols=inp.out_cols)
    req = np.repeat(np.arange(R), DQL)
    ks = offsets[req]
    pre = qsa.qsa_mqa_prefill(bf16_to_device(inp.q).reshape(R * DQL, 4, 128), k, i32_to_device(ks),
                              i32_to_device(ks + vis), out_cols=inp.out_cols)
    torch.cuda.synchronize()
    assert np.array_equal(f32_bits(pre), f32_bits(dec))


@pytest.mark.parametrize("widen,page_size", [("bf16", 64), ("fp16", 64), ("bf16", 7)])
def test_gather_widening_e4m3_against_oracle(widen, page_size):
    inp = decode_inputs([3000, 517, 12, 8400], 1, page_size, 500, 4, 2200, seed=page_size + 1)
    table = inp.page_table.copy()
    table[1, 1] = -1
    counts = O.comp_lens(inp.seq_lens).astype(np.int32)
    offsets = np.array([0, 800, 950, 1000], np.int32)
    rows = 3200
    codes = fp8_e4m3_cache(inp.k_pool)
    pool = torch.from_numpy(codes).cuda().view(torch.float8_e4m3fn)
    dt = torch.bfloat16 if widen == "bf16" else torch.float16
    out = torch.full((rows, 128), 0x2A2A, dtype=torch.int16, device="cuda").view(dt)
    _gather(pool, table, counts, offsets, int(counts.max()), out)
    want = np.full((rows, 128), 0x2A2A, np.uint16)
    O.gather_keys(codes, table, counts, offsets, want, widen=widen)
    assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), want)


def test_prefill_over_widened_e4m3_cache():
    # The spec-decode batch over its e4m3 cache: keys gathered and widened to
    # bf16, then the bf16 prefill with scale * k_scale, against the oracle's
    # typed prefill over the codes (and the e4m3 decode, within tolerance).
    from tests.parity import assert_scores_match
    qsa = _qsa()
    inp = WORKLOADS["specdecode_16x51k"].make()
    R, DQL = inp.q.shape[0], inp.q.shape[1]
    _, _, vis = O.token_metadata(inp.query_start_loc, inp.seq_lens, R * DQL)
    comp = O.comp_lens(inp.seq_lens).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(comp[:-1])]).astype(np.int32)
    codes = fp8_e4m3_cache(inp.k_pool)
    pool = torch.from_numpy(codes).cuda().view(torch.float8_e4m3fn)
    table = i32_to_device(inp.page_table)
    k = torch.zeros((int(comp.sum()), 128), dtype=torch.bfloat16, device="cuda")
    qsa.qsa_gather_keys(pool, table, i32_to_device(comp), i32_to_device(offsets), int(comp.max()), out=k)
    req = np.repeat(np.arange(R), DQL)
    ks = offsets[req]
    mult = float(np.float32(qsa.DEFAULT_SCALE) * np.float32(FP8_K_SCALE))
    q = bf16_to_device(inp.q).reshape(R * DQL, 4, 128)
    pre = qsa.qsa_mqa_prefill(q, k, i32_to_device(ks), i32_to_device(ks + vis), out_cols=inp.out_cols, scale=mult)
    dec = qsa.qsa_mqa_decode_typed(bf16_to_device(inp.q), pool, table, i32_to_device(comp), i32_to_device(vis),
                                   out_cols=inp.out_cols, k_scale=FP8_K_SCALE)
    torch.cuda.synchronize()
    k8 = np.zeros((int(comp.sum()), 128), np.uint8)
    O.gather_keys(codes, inp.page_table, comp, offsets, k8)
    rows = np.arange(0, R * DQL, 3)
    ref = O.prefill_typed(np.ascontiguousarray(inp.q.reshape(R * DQL, 4, 128)), "bf16", k8, "fp8_e4m3", ks, ks + vis,
                          inp.out_cols, k_scale=FP8_K_SCALE, rows=rows)
    assert_scores_match(pre[torch.from_numpy(rows).cuda()], ref, "prefill over the widened e4m3 cache")
    assert_scores_match(pre, dec.cpu().numpy(), "prefill vs e4m3 decode")


# ----------------------------------------------------------------------------
# Raw-key ring slots and key-cache writes


def test_ring_slots_golden_batch():
    qsa = _qsa()
    head = {r[0]: [int(x) for x in r[1:]] for r in _read_golden("ring_slots.txt")}
    bt = np.stack([head["block_col0"], head["block_col1"]], axis=1).astype(np.int32)
    got = qsa.qsa_build_ring_slots(i32_to_device(head["query_start_loc"]), i32_to_device(head["seq_lens"]),
                                   head["num_tokens"][0], i32_to_device(bt), head["ring_size"][0])
    torch.cuda.synchronize()
    assert got.cpu().numpy().tolist() == head["slots"]


@pytest.mark.parametrize("seed,n,ring", [(1, 7, 8), (2, 300, 4), (3, 8192, 12)])
def test_ring_slots_random_batches(seed, n, ring):
    qsa = _qsa()
    rng = np.random.default_rng(seed)
    qlens = rng.integers(0, 10, n)
    qlens[rng.integers(0, n)] = 700                         # one long prefill chunk
    seqs = np.maximum(qlens + rng.integers(-4, 5000, n), 0).astype(np.int32)
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    T = int(qsl[-1]) + 21                                   # padding tokens
    bt = rng.integers(0, 1 << 20, (n, 3)).astype(np.int32)
    bt[rng.random(n) < 0.1, 0] = 0                          # null blocks
    got = qsa.qsa_build_ring_slots(i32_to_device(qsl), i32_to_device(seqs), T, i32_to_device(bt), ring)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), O.ring_slots(qsl, seqs, T, bt, ring))


def _bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)


@pytest.mark.parametrize("fmt,width,with_pos", [("bf16", 128, False), ("bf16", 140, True), ("bf16", 136, False),
                                                ("fp8_e4m3", 128, False), ("fp8_e4m3", 132, False)])
def test_write_keys_matches_oracle(fmt, width, with_pos):
    qsa = _qsa()
    rng = np.random.default_rng(width + len(fmt))
    T, rows = 1500, 2048
    keys = bf16_bits_noise(rng, T)
    keys[5, :4] = bf16_bits(np.array([0.0, -0.0, 3e38, -1e-30], np.float32))
    slots = rng.permutation(rows + 200)[:T].astype(np.int64) - 100   # some negative, some past the cache
    pos = rng.integers(-(1 << 62), 1 << 62, (3, T)).astype(np.int64) if with_pos else None
    scale = 0.0173 if fmt == "fp8_e4m3" else 1.0
    if fmt == "bf16":
        cache0 = rng.integers(0, 1 << 16, (rows, width)).astype(np.uint16)
        dev = torch.from_numpy(cache0.view(np.int16)).to("cuda").view(torch.bfloat16)
    else:
        cache0 = rng.integers(0, 256, (rows, width)).astype(np.uint8)
        dev = torch.from_numpy(cache0).to("cuda").view(torch.float8_e4m3fn)
    key_dev = _bf16_dev(np.pad(keys, ((0, 0), (0, 8))))[:, :128]      # a padded row stride
    pos_dev = None if pos is None else torch.from_numpy(pos).to("cuda")
    qsa.qsa_write_keys(key_dev, torch.from_numpy(slots).to("cuda"), dev, scale=scale, positions=pos_dev)
    torch.cuda.synchronize()
    got = dev.view(torch.int16 if fmt == "bf16" else torch.uint8).cpu().numpy()
    want = O.write_keys(keys, slots, cache0, fmt=fmt, scale=scale, positions=pos)
    assert np.array_equal(got.view(want.dtype), want)


def bf16_bits_noise(rng, T):
    from workloads import normal_bf16
    return normal_bf16(rng, (T, 128))


@pytest.mark.parametrize("fmt", ["bf16", "fp8_e4m3"])
def test_compressed_keys_round_trip_through_decode(fmt):
    """A step's compressed keys written at the cache slots of
    qsa_build_cache_metadata into a paged cache that holds earlier keys,
    then decode over that cache: equal to the oracle's write and decode."""
    qsa = _qsa()
    rng = np.random.default_rng(51)
    R, ps, cr = 6, 16, 4
    qlens = np.array([4, 4, 4, 4, 37, 1], np.int64)            # decodes of DQL 4, a prefill chunk, one token
    seqs = np.array([403, 64, 1000, 7, 900, 129], np.int32)
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    T = int(qsl[-1])
    cols = int(seqs.max()) // cr // ps + 1
    pages = R * cols + 3
    bt = rng.permutation(pages)[:R * cols].reshape(R, cols).astype(np.int32)
    slots_dev, _ = qsa.qsa_build_cache_metadata(i32_to_device(qsl), i32_to_device(seqs), T, i32_to_device(bt), ps, cr,
                                                slot_mapping=torch.empty(T, dtype=torch.int64, device="cuda"))
    slots = O.cache_slots(qsl, seqs, T, bt, ps, cr)
    torch.cuda.synchronize()
    assert np.array_equal(slots_dev.cpu().numpy(), slots)
    new_keys = bf16_bits_noise(rng, T)
    old = bf16_bits_noise(rng, pages * ps).reshape(pages, ps, 1, 128)   # earlier steps' keys
    scale = FP8_K_SCALE
    if fmt == "bf16":
        cache0, dev = old, bf16_to_device(old)
    else:
        cache0 = fp8_e4m3_cache(old)
        dev = torch.from_numpy(cache0).to("cuda").view(torch.float8_e4m3fn)
    qsa.qsa_write_keys(_bf16_dev(new_keys), slots_dev, dev, scale=scale)
    want_cache = O.write_keys(new_keys, slots, cache0, fmt=fmt, scale=scale)
    # Decode rows of the first four requests (DQL 4) over the updated cache.
    dec_q = bf16_bits_noise(rng, 4 * 4 * 4).reshape(4, 4, 4, 128)
    comp = O.comp_lens(seqs[:4])
    dqsl = (np.arange(5) * 4).astype(np.int32)
    _, _, vis = O.token_metadata(dqsl, seqs[:4], 16)
    out = torch.full((16, 260), float("nan"), device="cuda")
    qsa.qsa_mqa_decode_typed(bf16_to_device(dec_q), dev, i32_to_device(bt[:4]), i32_to_device(comp),
                             i32_to_device(vis), k_scale=scale if fmt == "fp8_e4m3" else 1.0, out=out)
    torch.cuda.synchronize()
    got_cache = dev.view(torch.int16 if fmt == "bf16" else torch.uint8).cpu().numpy()
    assert np.array_equal(got_cache.view(want_cache.dtype), want_cache)
    ref = O.decode_typed(dec_q, "bf16", want_cache, fmt, bt[:4], comp, vis, 260,
                         k_scale=scale if fmt == "fp8_e4m3" else 1.0)
    from tests.parity import assert_scores_match
    assert_scores_match(out, ref, f"round trip {fmt}")
