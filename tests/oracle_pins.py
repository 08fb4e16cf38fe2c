"""Pins for the CPU oracle: checks against what the pages and the mathematics
fix, never against the oracle itself.

Each pin is a plain function that raises AssertionError on a mismatch.
``test_oracle_pins.py`` runs them against the oracle; ``test_oracle_mutants.py``
runs them against deliberately broken copies of the oracle and expects at
least one pin to fail for every plausible mistake.

Kinds of pin used here:
  * hand-worked values (tests/golden/*.txt, each with its citation);
  * closed forms (all-ones inputs);
  * brute force on tiny inputs in pure Python and in numpy float64 with an
    independent gather (a special case that reduces to a library matmul);
  * invariants the definition implies (page permutation, head permutation,
    negation symmetry, decode == prefill on gathered keys, DQL independence,
    scale linearity, mask pattern, non-negativity).
"""
from __future__ import annotations

import math
import os

import numpy as np

from oracle import oracle as O
from workloads import bf16_bits, bits_to_f32, decode_inputs, normal_bf16

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
NEG_INF_BITS = 0xFF800000
SCALE = float(np.float32(1.0 / math.sqrt(128.0)))


def _f32_bits(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _onehot_inputs(page_size=3):
    """q[h][0] = (1,-1,2,0.5)[h]; key n has feature 0 = n-2, others 0."""
    a = np.array([1.0, -1.0, 2.0, 0.5], np.float32)
    q = np.zeros((1, 1, 4, 128), np.float32)
    q[0, 0, :, 0] = a
    keys = np.zeros((8, 128), np.float32)
    keys[:, 0] = np.arange(8) - 2
    return bf16_bits(q), bf16_bits(keys)


def _paged(keys_bits, page_size, order=None, spare=0, seed=0):
    """Place keys [n,128] into a shuffled page pool; returns (pool, table).
    Unused rows and spare pages hold random noise."""
    rng = np.random.default_rng(seed)
    n = keys_bits.shape[0]
    pages = -(-n // page_size)
    total = pages + spare
    pool = normal_bf16(rng, (total, page_size, 1, 128))
    phys = rng.permutation(total) if order is None else np.asarray(order)
    for i in range(n):
        pool[phys[i // page_size], i % page_size, 0] = keys_bits[i]
    table = np.full((1, pages + 2), -1, np.int32)
    table[0, :pages] = phys[:pages]
    return pool, table


# ----------------------------------------------------------------------------
# hand-worked values and closed forms


def pin_onehot_decode():
    golden = _read_golden("onehot_scores.txt")
    expect = np.array([int(r[3], 16) for r in golden], np.uint32)
    q, keys = _onehot_inputs()
    for ps in (1, 3, 8):
        pool, table = _paged(keys, ps, seed=ps)
        out = O.decode(q, pool, table, np.array([8], np.int32), np.array([8], np.int32), 8,
                       scale=SCALE)
        assert np.array_equal(_f32_bits(out[0]), expect), (ps, _f32_bits(out[0]), expect)


def pin_onehot_prefill():
    golden = _read_golden("onehot_scores.txt")
    expect = np.array([int(r[3], 16) for r in golden], np.uint32)
    q, keys = _onehot_inputs()
    out = O.prefill(q[:, 0], keys, np.array([0], np.int32), np.array([8], np.int32), 8,
                    scale=SCALE)
    assert np.array_equal(_f32_bits(out[0]), expect)
    # The same keys behind an offset interval: column c is key start + c.
    padded = np.concatenate([bf16_bits(np.full((5, 128), 7.0, np.float32)), keys])
    out = O.prefill(q[:, 0], padded, np.array([5], np.int32), np.array([13], np.int32), 10,
                    scale=SCALE)
    assert np.array_equal(_f32_bits(out[0, :8]), expect)
    assert np.all(_f32_bits(out[0, 8:]) == NEG_INF_BITS)


def pin_all_ones_closed_form():
    # Every head dot is 128, so the score is 4*128*scale; with head 2 negated
    # its dot is -128 and ReLU drops it: 3*128*scale.
    q = bf16_bits(np.ones((1, 4, 128), np.float32))
    k = bf16_bits(np.ones((3, 128), np.float32))
    out = O.prefill(q, k, np.array([0], np.int32), np.array([3], np.int32), 3, scale=SCALE)
    assert np.all(_f32_bits(out) == 0x423504F3), _f32_bits(out)
    qn = np.ones((1, 4, 128), np.float32)
    qn[0, 2] = -1.0
    out = O.prefill(bf16_bits(qn), k, np.array([0], np.int32), np.array([3], np.int32), 3,
                    scale=SCALE)
    assert np.all(out == np.float32(384 * np.float64(SCALE)))


def pin_visible_golden():
    rows = _read_golden("visible_blocks.txt")
    # Each golden request alone, then all of them packed in one batch (so the
    # per-request query offset matters).
    ctxs, dqls, expects = [], [], []
    for ctx, dql, vis in rows:
        ctx, dql = int(ctx), int(dql)
        vis = [int(v) for v in vis.split(",")]
        qsl = np.array([0, dql], np.int32)
        _, pos, got = O.token_metadata(qsl, np.array([ctx], np.int32), dql)
        assert list(got) == vis, (ctx, dql, list(got), vis)
        assert list(pos) == list(range(ctx - dql, ctx))
        ctxs.append(ctx), dqls.append(dql), expects.extend(vis)
    qsl = np.concatenate([[0], np.cumsum(dqls)]).astype(np.int32)
    req, _, got = O.token_metadata(qsl, np.array(ctxs, np.int32), int(qsl[-1]) + 3)
    assert list(got[:-3]) == expects
    assert list(got[-3:]) == [0, 0, 0]  # padding tokens past the last request
    assert list(req[:-3]) == [r for r, d in enumerate(dqls) for _ in range(d)]
    assert list(O.comp_lens(np.array(ctxs, np.int32))) == [c // 4 for c in ctxs]


def pin_prefill_intervals_golden():
    """The packed batch of tests/golden/prefill_intervals.txt, worked by hand:
    request, position, visible count and key interval of every token,
    including an empty request, non-zero key offsets and padding tokens."""
    rows = _read_golden("prefill_intervals.txt")
    head = {r[0]: [int(x) for x in r[1:]] for r in rows if not r[0].lstrip("-").isdigit()}
    body = [[int(x) for x in r] for r in rows if r[0].lstrip("-").isdigit()]
    qsl = np.array(head["query_start_loc"], np.int32)
    seq = np.array(head["seq_lens"], np.int32)
    off = np.array(head["key_offsets"], np.int32)
    T = head["num_tokens"][0]
    req, pos, vis = O.token_metadata(qsl, seq, T)
    ks, ke = O.prefill_intervals(req, vis, off)
    want = np.array(body, np.int64)
    assert list(want[:, 0]) == list(range(T))
    assert list(req) == list(want[:, 1]), list(req)
    assert list(pos) == list(want[:, 2]), list(pos)
    assert list(vis) == list(want[:, 3]), list(vis)
    assert list(ks) == list(want[:, 4]), list(ks)
    assert list(ke) == list(want[:, 5]), list(ke)


def pin_ring_slots_golden():
    """tests/golden/ring_slots.txt: ring rows of a decode, a speculative
    decode, a prefill chunk longer than the ring, a request starting before
    position 0, a request on the null block, an empty request and padding."""
    head = {r[0]: [int(x) for x in r[1:]] for r in _read_golden("ring_slots.txt")}
    bt = np.stack([head["block_col0"], head["block_col1"]], axis=1).astype(np.int32)
    got = O.ring_slots(np.array(head["query_start_loc"], np.int32), np.array(head["seq_lens"], np.int32),
                       head["num_tokens"][0], bt, head["ring_size"][0])
    assert list(got) == head["slots"], list(got)


def pin_ring_slots_counting():
    """Random batches, characterised by counting: in every request with a
    non-null block, exactly its last min(ring, query_len) tokens with a
    position >= 0 get a slot, inside the request's own ring, at row pos %
    ring, all distinct; every other token gets -1."""
    rng = np.random.default_rng(11)
    for _ in range(40):
        R = int(rng.integers(1, 7))
        ring = int(rng.choice([4, 8, 12]))
        qlens = rng.integers(0, 20, R)
        seq = np.maximum(qlens + rng.integers(-3, 50, R), 0).astype(np.int32)
        qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
        T = int(qsl[-1]) + int(rng.integers(0, 4))
        bt = rng.integers(0, 9, (R, 2)).astype(np.int32)
        got = O.ring_slots(qsl, seq, T, bt, ring)
        want = np.full(T, -1, np.int64)
        for r in range(R):
            block = int(bt[r, 0])
            for i in range(int(qlens[r])):
                t = int(qsl[r]) + i
                pos = int(seq[r]) - int(qlens[r]) + i
                if block > 0 and pos >= 0 and i >= int(qlens[r]) - ring:
                    want[t] = block * ring + pos % ring
        assert np.array_equal(got, want)
        for r in range(R):
            mine = got[qsl[r]:qsl[r + 1]]
            mine = mine[mine >= 0]
            assert len(set(mine.tolist())) == len(mine)
            assert np.all(mine // ring == bt[r, 0])


def pin_write_keys_labels():
    """Labelled key rows: after the write, cache row s holds the key of the
    token whose slot is s, rows no token names keep their sentinel, slots
    outside the cache are skipped, and positions follow a ring row's key as
    exact int64."""
    rng = np.random.default_rng(12)
    T, rows = 30, 48
    keys = np.zeros((T, 128), np.uint16)
    keys[:, 0] = np.arange(T) + 1
    keys[:, 127] = 0x4000 + np.arange(T)
    slots = rng.permutation(rows)[:T].astype(np.int64)
    slots[3], slots[7], slots[11] = -1, rows, 1 << 40          # skipped
    cache = np.full((6, 8, 1, 140), 0xBEEF, np.uint16)
    pos = rng.integers(-(1 << 62), 1 << 62, (3, T)).astype(np.int64)
    out = O.write_keys(keys, slots, cache, positions=pos).reshape(rows, 140)
    written = set()
    for t in range(T):
        s = int(slots[t])
        if 0 <= s < rows:
            written.add(s)
            assert np.array_equal(out[s, :128], keys[t])
            assert np.array_equal(out[s, 128:140].copy().view(np.int64), pos[:, t])
    for s in range(rows):
        if s not in written:
            assert np.all(out[s] == 0xBEEF)
    plain = O.write_keys(keys, slots, np.full((rows, 128), 7, np.uint16))
    for t in range(T):
        if 0 <= int(slots[t]) < rows:
            assert np.array_equal(plain[int(slots[t])], keys[t])


def pin_write_keys_e4m3_matches_library():
    """The e4m3 cache write [_to_dst_dtype]: each bf16 key value divided by
    the scale in fp32, converted by torch's float8_e4m3fn (RNE) wherever the
    quotient is below 448 in magnitude; larger quotients saturate to 448."""
    import torch
    rng = np.random.default_rng(13)
    T = 64
    keys = bf16_bits(rng.standard_normal((T, 128)).astype(np.float32) * 3.0)
    keys[0, :4] = bf16_bits(np.array([0.0, -0.0, 1e-30, -7.5], np.float32))
    keys[1, :3] = bf16_bits(np.array([100.0, -100.0, 3e38], np.float32))
    scale = 0.0173
    slots = np.arange(T, dtype=np.int64)
    out = O.write_keys(keys, slots, np.zeros((T, 128), np.uint8), fmt="fp8_e4m3", scale=scale)
    with np.errstate(over="ignore"):                      # 3e38 / scale: +inf, which saturates
        q = (bits_to_f32(keys) / np.float32(scale)).astype(np.float32)
    small = np.abs(q) < 448.0
    lib = torch.from_numpy(np.where(small, q, 0.0).astype(np.float32)).to(torch.float8_e4m3fn)
    assert np.array_equal(out[small], lib.view(torch.uint8).numpy()[small])
    big = ~small
    assert big.any()
    assert np.all(out[big] & 0x7F == 0x7E)
    assert np.array_equal(out[big] >> 7, (q[big] < 0).astype(np.uint8))


def pin_visible_counts_complete_blocks():
    # Independent characterisation: the number of 4-token blocks whose last
    # token is at or before pos, among the blocks complete within seq_len.
    rng = np.random.default_rng(7)
    for _ in range(30):
        nreq = int(rng.integers(1, 5))
        qlens = rng.integers(1, 9, nreq)
        seq = qlens + rng.integers(0, 40, nreq)
        qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
        _, pos, vis = O.token_metadata(qsl, seq.astype(np.int32), int(qsl[-1]))
        t = 0
        for r in range(nreq):
            for i in range(qlens[r]):
                p = seq[r] - qlens[r] + i
                assert pos[t] == p
                count = sum(1 for n in range(seq[r]) if 4 * n + 3 <= p and 4 * n + 3 < seq[r])
                assert vis[t] == count, (seq[r], p, vis[t], count)
                t += 1


# ----------------------------------------------------------------------------
# brute force


def _numpy_decode_reference(inp, visible, out_cols, scale):
    """Dense float64 evaluation with an independent gather: for each request,
    walk its page table in Python, stack its keys, and use a numpy matmul for
    the dots."""
    q = bits_to_f32(inp.q).astype(np.float64)
    pool = bits_to_f32(inp.k_pool).astype(np.float64)
    R, dql = inp.q.shape[:2]
    ps = inp.page_size
    out = np.full((R * dql, out_cols), -np.inf, np.float32)
    comp = [int(s) // 4 for s in inp.seq_lens]
    for r in range(R):
        keys, ok = [], []
        for c in range(out_cols):
            slot = c // ps
            page = inp.page_table[r, slot] if slot < inp.page_table.shape[1] else -1
            good = 0 <= page < pool.shape[0]
            keys.append(pool[page, c % ps, 0] if good else np.zeros(128))
            ok.append(good)
        K = np.stack(keys)
        for j in range(dql):
            row = r * dql + j
            dots = q[r, j] @ K.T                                # [4, cols]
            s = np.maximum(dots, 0.0).sum(axis=0) * np.float64(scale)
            seen = min(max(int(visible[row]), 0), comp[r])
            for c in range(min(seen, out_cols)):
                if ok[c]:
                    out[row, c] = np.float32(s[c])
    return out


def _assert_close_exact_mask(got, ref, ulps=1):
    gb, rb = _f32_bits(got), _f32_bits(ref)
    ninf_g, ninf_r = gb == NEG_INF_BITS, rb == NEG_INF_BITS
    assert np.array_equal(ninf_g, ninf_r), "-inf pattern differs"
    fin = ~ninf_r
    diff = np.abs(gb[fin].astype(np.int64) - rb[fin].astype(np.int64))
    assert diff.size == 0 or diff.max() <= ulps, f"max ulp diff {diff.max()}"


def pin_bruteforce_numpy_decode():
    rng = np.random.default_rng(11)
    for case in range(8):
        R = int(rng.integers(1, 4))
        dql = int(rng.integers(1, 5))
        ps = [1, 3, 16, 5][case % 4]
        ctx = [int(x) for x in rng.integers(1, 800, R)]
        cols = max(c // 4 for c in ctx) + int(rng.integers(0, 5))
        table_cols = max(-(-(-(-c // 4)) // ps) for c in ctx) + 1
        inp = decode_inputs(ctx, dql, ps, table_cols, spare_pages=2, out_cols=cols,
                            seed=100 + case)
        # Knock out one page-table entry and plant an out-of-range id.
        if inp.page_table[0, 0] >= 0 and table_cols > 2:
            inp.page_table[0, 1] = -1
            inp.page_table[R - 1, 0] = inp.k_pool.shape[0] + 3
        _, _, vis = O.token_metadata(inp.query_start_loc, inp.seq_lens, R * dql)
        got = O.decode(inp.q, inp.k_pool, inp.page_table, O.comp_lens(inp.seq_lens), vis, cols,
                       scale=SCALE)
        ref = _numpy_decode_reference(inp, vis, cols, SCALE)
        _assert_close_exact_mask(got, ref)


def pin_bruteforce_python_loops():
    # Pure-Python loops on a tiny prefill case, same summation order as the
    # definition (features, then heads): bit-exact.
    rng = np.random.default_rng(12)
    q = normal_bf16(rng, (3, 4, 128))
    k = normal_bf16(rng, (7, 128))
    ks = np.array([0, 2, 5], np.int32)
    ke = np.array([4, 9, 3], np.int32)
    cols = 6
    got = O.prefill(q, k, ks, ke, cols, scale=SCALE)
    qf, kf = bits_to_f32(q), bits_to_f32(k)
    for t in range(3):
        for c in range(cols):
            n = int(ks[t]) + c
            if n < int(ke[t]) and 0 <= n < 7:
                total = 0.0
                for h in range(4):
                    dot = 0.0
                    for d in range(128):
                        dot += float(qf[t, h, d]) * float(kf[n, d])
                    total += dot if dot > 0.0 else 0.0
                want = np.float32(total * SCALE)
                assert _f32_bits(got[t, c]) == _f32_bits(want), (t, c, got[t, c], want)
            else:
                assert _f32_bits(got[t, c]) == NEG_INF_BITS, (t, c)


def pin_bruteforce_numpy_prefill():
    rng = np.random.default_rng(13)
    T, NK, cols = 9, 40, 30
    q = normal_bf16(rng, (T, 4, 128))
    k = normal_bf16(rng, (NK, 128))
    ks = rng.integers(-3, 25, T).astype(np.int32)
    ke = (ks + rng.integers(-2, 35, T)).astype(np.int32)
    got = O.prefill(q, k, ks, ke, cols, scale=SCALE)
    qf = bits_to_f32(q).astype(np.float64)
    kf = bits_to_f32(k).astype(np.float64)
    ref = np.full((T, cols), -np.inf, np.float32)
    for t in range(T):
        s = np.maximum(qf[t] @ kf.T, 0).sum(axis=0) * SCALE      # [NK]
        for c in range(cols):
            n = ks[t] + c
            if 0 <= n < NK and n < ke[t]:
                ref[t, c] = np.float32(s[n])
    _assert_close_exact_mask(got, ref)


# ----------------------------------------------------------------------------
# invariants


def _small_decode(seed=21, dql=3, ps=7, ctx=(301, 77, 5)):
    ctx = list(ctx)
    inp = decode_inputs(ctx, dql, ps, table_cols=12, spare_pages=4,
                        out_cols=max(ctx) // 4 + 3, seed=seed)
    _, _, vis = O.token_metadata(inp.query_start_loc, inp.seq_lens, len(ctx) * dql)
    return inp, vis


def _run_decode(inp, vis, scale=SCALE, q=None):
    return O.decode(inp.q if q is None else q, inp.k_pool, inp.page_table,
                    O.comp_lens(inp.seq_lens), vis, inp.out_cols, scale=scale)


def pin_mask_pattern_and_sign():
    inp, vis = _small_decode()
    out = _run_decode(inp, vis)
    bits = _f32_bits(out)
    comp = [int(s) // 4 for s in inp.seq_lens]
    for row in range(out.shape[0]):
        r = row // inp.dql
        seen = min(int(vis[row]), comp[r])
        assert np.all(bits[row, seen:] == NEG_INF_BITS)
        assert np.all(np.isfinite(out[row, :seen]))
        assert np.all(bits[row, :seen] < 0x80000000)   # >= +0.0, never -0.0
    # Some cells must be exactly +0 (all four heads negative) and most positive.
    fin = out[np.isfinite(out)]
    assert (fin > 0).mean() > 0.5


def pin_page_permutation_invariance():
    inp, vis = _small_decode()
    base = _run_decode(inp, vis)
    rng = np.random.default_rng(5)
    perm = rng.permutation(inp.k_pool.shape[0])          # new_pool[perm[p]] = pool[p]
    pool2 = np.empty_like(inp.k_pool)
    pool2[perm] = inp.k_pool
    table2 = np.where(inp.page_table >= 0, perm[np.maximum(inp.page_table, 0)], -1)
    inp2 = type(inp)(inp.q, pool2, table2.astype(np.int32), inp.seq_lens,
                     inp.query_start_loc, inp.page_size, inp.out_cols)
    assert np.array_equal(_f32_bits(_run_decode(inp2, vis)), _f32_bits(base))


def pin_head_permutation():
    inp, vis = _small_decode()
    base = _run_decode(inp, vis)
    perm = _run_decode(inp, vis, q=np.ascontiguousarray(inp.q[:, :, [2, 0, 3, 1]]))
    _assert_close_exact_mask(perm, base, ulps=1)


def pin_negation_symmetry():
    inp, vis = _small_decode()
    base = _run_decode(inp, vis)
    neg = type(inp)(inp.q ^ np.uint16(0x8000), inp.k_pool ^ np.uint16(0x8000), inp.page_table,
                    inp.seq_lens, inp.query_start_loc, inp.page_size, inp.out_cols)
    assert np.array_equal(_f32_bits(_run_decode(neg, vis)), _f32_bits(base))


def pin_strided_q():
    inp, vis = _small_decode()
    base = _run_decode(inp, vis)
    R, dql = inp.q.shape[:2]
    wide = np.zeros((R, dql + 1, 5, 136), np.uint16)
    wide[:, :dql, :4, :128] = inp.q
    view = wide[:, :dql, :4, :128]
    assert not view.flags.c_contiguous
    assert np.array_equal(_f32_bits(_run_decode(inp, vis, q=view)), _f32_bits(base))


def pin_dql_independence():
    inp, vis = _small_decode(dql=4, ctx=(123, 64))
    base = _run_decode(inp, vis)
    comp = O.comp_lens(inp.seq_lens)
    for r in range(2):
        for j in range(4):
            row = r * 4 + j
            one = O.decode(np.ascontiguousarray(inp.q[r:r + 1, j:j + 1]), inp.k_pool,
                           inp.page_table[r:r + 1], comp[r:r + 1], vis[row:row + 1],
                           inp.out_cols, scale=SCALE)
            assert np.array_equal(_f32_bits(one[0]), _f32_bits(base[row]))


def pin_decode_equals_prefill():
    inp, vis = _small_decode()
    base = _run_decode(inp, vis)
    ps = inp.page_size
    for r in range(inp.num_reqs):
        n = int(inp.seq_lens[r]) // 4
        keys = np.stack([inp.k_pool[inp.page_table[r, c // ps], c % ps, 0] for c in range(n)]) \
            if n else np.zeros((0, 128), np.uint16)
        keys = np.concatenate([keys, np.zeros((1, 128), np.uint16)])  # never read
        for j in range(inp.dql):
            row = r * inp.dql + j
            got = O.prefill(np.ascontiguousarray(inp.q[r, j:j + 1]), keys,
                            np.array([0], np.int32), np.array([vis[row]], np.int32),
                            inp.out_cols, scale=SCALE)
            assert np.array_equal(_f32_bits(got[0]), _f32_bits(base[row])), (r, j)


def pin_scale_linearity():
    inp, vis = _small_decode()
    base = _run_decode(inp, vis)
    dbl = _run_decode(inp, vis, scale=2 * SCALE)
    fin = np.isfinite(base)
    assert np.array_equal(dbl[fin], 2 * base[fin])
    assert np.array_equal(np.isfinite(dbl), fin)


def pin_invalid_pages_mask():
    inp, vis = _small_decode(ctx=(301, 300, 299))
    base = _run_decode(inp, vis)
    table = inp.page_table.copy()
    table[0, 2] = -1
    table[1, 0] = inp.k_pool.shape[0]          # one past the pool
    table[2, 5] = 1 << 30
    inp2 = type(inp)(inp.q, inp.k_pool, table, inp.seq_lens, inp.query_start_loc,
                     inp.page_size, inp.out_cols)
    got = _run_decode(inp2, vis)
    ps, dql = inp.page_size, inp.dql
    expect = base.copy()
    expect[0 * dql:1 * dql, 2 * ps:3 * ps] = -np.inf
    expect[1 * dql:2 * dql, 0:ps] = -np.inf
    expect[2 * dql:3 * dql, 5 * ps:6 * ps] = -np.inf
    assert np.array_equal(_f32_bits(got), _f32_bits(expect))
    # A page table narrower than the visible range masks the columns past it.
    narrow = np.ascontiguousarray(inp.page_table[:, :3])
    inp3 = type(inp)(inp.q, inp.k_pool, narrow, inp.seq_lens, inp.query_start_loc,
                     inp.page_size, inp.out_cols)
    got = _run_decode(inp3, vis)
    expect = base.copy()
    expect[:, 3 * ps:] = -np.inf
    assert np.array_equal(_f32_bits(got), _f32_bits(expect))


def pin_decode_visible_override():
    # No visible array: each row sees comp_len; a visible value above comp_len
    # is clamped; a negative one masks the whole row.
    inp, vis = _small_decode(dql=2, ctx=(90, 41))
    comp = O.comp_lens(inp.seq_lens)
    full = O.decode(inp.q, inp.k_pool, inp.page_table, comp, None, inp.out_cols, scale=SCALE)
    want = _run_decode(inp, np.repeat(comp, 2))
    assert np.array_equal(_f32_bits(full), _f32_bits(want))
    odd = np.array([10_000, -5, 3, 0], np.int32)
    got = _run_decode(inp, odd)
    assert np.array_equal(_f32_bits(got[0]), _f32_bits(full[0]))
    assert np.all(_f32_bits(got[1]) == NEG_INF_BITS)
    assert np.array_equal(_f32_bits(got[2, :3]), _f32_bits(full[2, :3]))
    assert np.all(_f32_bits(got[2, 3:]) == NEG_INF_BITS)
    assert np.all(_f32_bits(got[3]) == NEG_INF_BITS)


def pin_prefill_degenerate_intervals():
    rng = np.random.default_rng(31)
    q = normal_bf16(rng, (4, 4, 128))
    k = normal_bf16(rng, (10, 128))
    ks = np.array([3, 5, -2, 8], np.int32)
    ke = np.array([3, 2, 4, 50], np.int32)
    got = O.prefill(q, k, ks, ke, 6, scale=SCALE)
    bits = _f32_bits(got)
    assert np.all(bits[0] == NEG_INF_BITS)             # empty interval
    assert np.all(bits[1] == NEG_INF_BITS)             # end before start
    assert np.all(bits[2, :2] == NEG_INF_BITS)         # keys -2, -1 do not exist
    assert np.all(np.isfinite(got[2, 2:6]))            # keys 0..3
    assert np.all(np.isfinite(got[3, :2]))             # keys 8, 9
    assert np.all(bits[3, 2:] == NEG_INF_BITS)         # past the last key


# ----------------------------------------------------------------------------
# top-k


def _topk_by_sort(x, k):
    out = np.full((x.shape[0], k), -1, np.int32)
    for t in range(x.shape[0]):
        cols = np.nonzero(x[t] > -np.inf)[0]
        vals = x[t, cols].astype(np.float64) + 0.0      # -0.0 and +0.0 compare equal
        order = np.lexsort((cols, -vals))                # score desc, column asc
        pick = np.sort(cols[order[:k]])
        out[t, :len(pick)] = pick
    return out


def pin_topk_against_sort():
    rng = np.random.default_rng(41)
    for cols, k in ((50, 7), (300, 64), (1000, 512), (20, 30), (1, 1)):
        x = rng.standard_normal((6, cols)).astype(np.float32)
        x[1, cols // 2:] = -np.inf                     # short row
        x[2] = -np.inf                                 # nothing to pick
        x[3] = np.round(x[3] * 2) / 2                  # many exact ties
        x[4, ::3] = 0.0
        x[4, 1::3] = -0.0                              # -0 ties +0
        x[5] = np.abs(x[5])
        got = O.topk(x, k)
        assert np.array_equal(got, _topk_by_sort(x, k)), (cols, k)


def pin_topk_ties_lowest_index():
    x = np.full((1, 40), 1.5, np.float32)
    x[0, 7] = 2.0
    got = O.topk(x, 5)
    assert list(got[0]) == [0, 1, 2, 3, 7]
    x = np.array([[3.0, -np.inf, 3.0, 1.0, 3.0]], np.float32)
    assert list(O.topk(x, 6)[0]) == [0, 2, 3, 4, -1, -1]
    assert list(O.topk(x, 2)[0]) == [0, 2]


def pin_split_batch():
    # Decodes first, uniform length: two DQL-4 decodes then prefills.
    assert O.split_batch([0, 4, 8, 9, 9, 17], 4) == (None, 2, 8, 3, 9, 4)
    # Plain decode batch (threshold 1, one token each).
    assert O.split_batch([0, 1, 2, 3], 1) == (None, 3, 3, 0, 0, 1)
    # All prefills.
    assert O.split_batch([0, 10, 30], 4) == (None, 0, 0, 2, 30, 0)
    # Non-uniform decode lengths: the run ends at the first other length.
    assert O.split_batch([0, 2, 4, 7, 9], 4) == (None, 2, 4, 2, 5, 2)
    # Reordering moves qualifying requests first, stably.
    order, nd, ndt, npf, npt, dql = O.split_batch([0, 9, 11, 12, 14, 14], 2, reorder=True)
    assert order == [1, 3, 0, 2, 4] and (nd, ndt, npf, npt, dql) == (2, 4, 3, 10, 2)
    # Empty batch.
    assert O.split_batch([0], 4) == (None, 0, 0, 0, 0, 0)


# ---------------------------------------------------------------------------
# Typed inputs (fp16 queries/keys, fp8 e4m3 keys with a cache scale).


def _row_unit(n, value_bits, dtype):
    """n rows [n, 4, 128]: head 0, feature 0 holds value_bits[i]; all else 0."""
    q = np.zeros((n, 4, 128), dtype)
    q[:, 0, 0] = value_bits
    return q


def _relu_pair(v):
    """Scores of a unit query against keys +v and -v at scale 1: relu(v), relu(-v)."""
    v = np.asarray(v, np.float64)
    return np.maximum(v, 0.0).astype(np.float32), np.maximum(-v, 0.0).astype(np.float32)


def pin_fp16_decoding_all_codes():
    """Every binary16 code, as a query element and as a key element, against
    numpy's float16 conversion (a library routine).  NaN codes are skipped."""
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = codes.view(np.float16).astype(np.float64)
    keep = ~np.isnan(vals)
    want_pos, want_neg = _relu_pair(vals[keep])
    one, minus_one = 0x3C00, 0xBC00  # binary16 +1, -1
    # As a query element: rows hold the codes, keys are +1 and -1.
    q = _row_unit(len(codes), codes, np.uint16)[keep]
    k = np.zeros((2, 128), np.uint16)
    k[0, 0], k[1, 0] = one, minus_one
    n = len(q)
    got = O.prefill_typed(q, "fp16", k, "fp16", np.zeros(n, np.int32), np.full(n, 2, np.int32), 2,
                          scale=1.0)
    assert np.array_equal(_f32_bits(got[:, 0]), _f32_bits(want_pos))
    assert np.array_equal(_f32_bits(got[:, 1]), _f32_bits(want_neg))
    # As a key element: one query row +1 against every code.
    qk = _row_unit(2, [one, minus_one], np.uint16)
    keys = np.zeros((int(keep.sum()), 128), np.uint16)
    keys[:, 0] = codes[keep]
    m = len(keys)
    got = O.prefill_typed(qk, "fp16", keys, "fp16", np.zeros(2, np.int32), np.full(2, m, np.int32), m,
                          scale=1.0)
    assert np.array_equal(_f32_bits(got[0]), _f32_bits(want_pos))
    assert np.array_equal(_f32_bits(got[1]), _f32_bits(want_neg))


def pin_e4m3_decoding_all_codes():
    """Every OCP e4m3 code as a key element, against torch's float8_e4m3fn
    conversion (a library routine), at k_scale 1 and at k_scale 0.375 (the
    products are exact in fp32).  NaN codes are skipped."""
    import torch
    codes = np.arange(256, dtype=np.uint16).astype(np.uint8)
    vals = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    keep = ~np.isnan(vals)
    keys = np.zeros((int(keep.sum()), 128), np.uint8)
    keys[:, 0] = codes[keep]
    m = len(keys)
    q = _row_unit(2, [0x3F80, 0xBF80], np.uint16)  # bf16 +1, -1
    for k_scale in (1.0, 0.375):
        want_pos, want_neg = _relu_pair(vals[keep] * k_scale)
        got = O.prefill_typed(q, "bf16", keys, "fp8_e4m3", np.zeros(2, np.int32), np.full(2, m, np.int32),
                              m, k_scale=k_scale, scale=1.0)
        assert np.array_equal(_f32_bits(got[0]), _f32_bits(want_pos)), k_scale
        assert np.array_equal(_f32_bits(got[1]), _f32_bits(want_neg)), k_scale
    # Range facts of the format: largest finite 448, smallest subnormal 2^-9.
    fin = vals[keep]
    assert fin.max() == 448.0 and np.min(np.abs(fin[fin != 0])) == 2.0 ** -9


def _exact_case(seed=31):
    """Values every format holds exactly: queries are integers in [-8, 8],
    fp8 key codes are integers in [-15, 15] with k_scale 0.5, so every key
    value is a multiple of 0.5 below 8 in magnitude."""
    import torch
    rng = np.random.default_rng(seed)
    inp = decode_inputs([37, 201, 90], 3, 5, 20, 2, 60, seed=seed)
    qv = rng.integers(-8, 9, inp.q.shape).astype(np.float32)
    kv = rng.integers(-15, 16, inp.k_pool.shape).astype(np.float32)
    k8 = torch.from_numpy(kv).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return inp, qv, kv, k8


def pin_typed_equal_bf16_on_exact_values():
    """On inputs every format represents exactly, the typed decode and
    prefill equal the bf16 oracle bit for bit: fp16 q and keys, and fp8 keys
    whose codes times k_scale equal the bf16 keys."""
    inp, qv, kv, k8 = _exact_case()
    vis = O.token_metadata(inp.query_start_loc, inp.seq_lens, inp.q.shape[0] * inp.q.shape[1])[2]
    comp = O.comp_lens(inp.seq_lens)
    q16, qh = bf16_bits(qv), qv.astype(np.float16).view(np.uint16)
    kb, kh = bf16_bits(kv * 0.5), (kv * 0.5).astype(np.float16).view(np.uint16)
    base = O.decode(q16, kb, inp.page_table, comp, vis, inp.out_cols, scale=SCALE)
    for qb, qf, kbits, kf in ((q16, "bf16", kb, "bf16"), (qh, "fp16", kh, "fp16"),
                              (q16, "bf16", k8, "fp8_e4m3"), (qh, "fp16", k8, "fp8_e4m3")):
        got = O.decode_typed(qb, qf, kbits, kf, inp.page_table, comp, vis, inp.out_cols,
                             k_scale=0.5, scale=SCALE)
        assert np.array_equal(_f32_bits(got), _f32_bits(base)), (qf, kf)
    # Prefill over the flattened pool, keys read through a padded row stride.
    T = 7
    qp = qv.reshape(-1, 4, 128)[:T]
    flat = kv.reshape(-1, 128)
    nk = flat.shape[0]
    ks = np.array([0, 3, -2, 5, 0, 10, 1], np.int32)
    ke = np.array([nk, 40, 9, 5, 77, nk + 5, 2], np.int32)
    cols = nk + 3
    base = O.prefill(bf16_bits(qp), bf16_bits(flat * 0.5), ks, ke, cols, scale=SCALE)
    padded = np.zeros((nk, 144), np.uint8)
    padded[:, :128] = k8.reshape(-1, 128)
    kh_pad = np.zeros((nk, 136), np.uint16)
    kh_pad[:, :128] = (flat * 0.5).astype(np.float16).view(np.uint16)
    for qb, qf, kbits, kf in ((qp.astype(np.float16).view(np.uint16), "fp16", kh_pad[:, :128], "fp16"),
                              (bf16_bits(qp), "bf16", padded[:, :128], "fp8_e4m3")):
        got = O.prefill_typed(qb, qf, kbits, kf, ks, ke, cols, k_scale=0.5, scale=SCALE)
        assert np.array_equal(_f32_bits(got), _f32_bits(base)), (qf, kf)


# ---------------------------------------------------------------------------
# Compressed-cache metadata and the paged key gather.

_CM_QSL = np.array([0, 6, 8, 11, 15, 16, 17, 18, 18], np.int32)
_CM_SEQ = np.array([12, 8, 12, 24, 4, 4, 2, 9], np.int32)
_CM_BT = np.array([[5, 2], [7, -1], [4, -1], [1, 0], [3, 6], [0, 10], [11, 12], [13, 14]], np.int32)


def pin_cache_metadata_golden():
    rows = {r[0]: r[1:] for r in _read_golden("cache_metadata.txt")}
    common = np.zeros(19, np.int64)
    common[15] = -1
    got = O.cache_slots(_CM_QSL, _CM_SEQ, 19, _CM_BT, 2, 4, common)
    assert got.tolist() == [int(x) for x in rows["slots"]], got.tolist()
    want = [[int(v) for v in item.split(",")] for item in rows["work"]]
    assert O.k_work(_CM_QSL, _CM_SEQ, 12).tolist() == want
    assert O.k_work(_CM_QSL, _CM_SEQ, 5).tolist() == want[:5]  # truncated list
    # Without main-cache slots token 15 keeps its slot 3*2+0.
    assert O.cache_slots(_CM_QSL, _CM_SEQ, 19, _CM_BT, 2, 4)[15] == 6


def pin_cache_metadata_counting():
    """Random batches against an independent characterisation: the tokens
    with a slot are exactly the group-closing tokens (positions 3, 7, 11, ...)
    whose block exists, each such slot names the block that holds its
    compressed row, no two tokens share a slot, and each request owns as many
    work items as it has group-closing tokens (at least one when it has query
    tokens)."""
    rng = np.random.default_rng(41)
    for cr, sbs in ((4, 16), (4, 3), (2, 5), (1, 7)):
        n = 9
        qlens = rng.integers(0, 40, n)
        seqs = (qlens + rng.integers(0, 200, n)).astype(np.int32)
        qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
        T = int(qsl[-1]) + 2
        cols = int(seqs.max()) // cr // sbs + 1
        perm = rng.permutation(n * cols).astype(np.int32).reshape(n, cols)
        perm[rng.random(perm.shape) < 0.15] = -1
        slots = O.cache_slots(qsl, seqs, T, perm, sbs, cr)
        seen = set()
        for r in range(n):
            for i in range(int(qlens[r])):
                t = int(qsl[r]) + i
                pos = int(seqs[r]) - int(qlens[r]) + i
                closes = pos >= 0 and pos % cr == cr - 1
                blk = perm[r, (pos // cr) // sbs] if closes else -1
                if closes and blk >= 0:
                    assert slots[t] >= 0 and slots[t] // sbs == blk and slots[t] % sbs == (pos // cr) % sbs
                    assert int(slots[t]) not in seen
                    seen.add(int(slots[t]))
                else:
                    assert slots[t] == -1, (cr, sbs, r, i)
        assert np.all(slots[int(qsl[-1]):] == -1)
        work = O.k_work(qsl, seqs, 4000, cr)
        live = work[work[:, 0] >= 0]
        for r in range(n):
            closing = sum(1 for p in range(int(seqs[r]) - int(qlens[r]), int(seqs[r])) if p % cr == cr - 1)
            mine = live[live[:, 0] == r]
            want = max(closing, 1) if qlens[r] > 0 else 0
            assert len(mine) == want and mine[:, 1].tolist() == list(range(want)), (cr, r)
        assert live[:, 0].tolist() == sorted(live[:, 0].tolist())
        assert np.all(work[len(live):] == -1)


def _labelled_pool(num_pages, page_size, seed):
    """A pool whose every row is distinct noise except feature 0, which holds
    a label set per test."""
    rng = np.random.default_rng(seed)
    return normal_bf16(rng, (num_pages, page_size, 1, 128))


def pin_gather_keys_labels():
    """Keys labelled with their request and logical index land at rows
    key_offsets[r] + c in order; missing pages give zero rows; rows no
    request covers are untouched."""
    rng = np.random.default_rng(5)
    ps, R = 5, 4
    counts = np.array([13, 0, 7, 22], np.int32)
    pages = [(int(c) + ps - 1) // ps for c in counts]
    P = sum(pages) + 3
    order = rng.permutation(P)
    pool = np.zeros((P, ps, 1, 128), np.uint16)
    table = np.full((R, 6), -1, np.int32)
    k = 0
    for r in range(R):
        for j in range(pages[r]):
            table[r, j] = order[k]
            for i in range(ps):
                pool[order[k], i, 0, 0] = 1000 * (r + 1) + j * ps + i   # label (as bits)
            k += 1
    table[3, 2] = -1                                                   # a missing page
    offsets = np.array([4, 40, 17, 60], np.int32)
    out = np.full((90, 128), 7, np.uint16)
    O.gather_keys(pool, table, counts, offsets, out)
    for r in range(R):
        for c in range(int(counts[r])):
            row = out[offsets[r] + c]
            if r == 3 and c // ps == 2:
                assert np.all(row == 0)
            else:
                assert row[0] == 1000 * (r + 1) + c and np.all(row[1:] == 0)
    covered = {int(offsets[r]) + c for r in range(R) for c in range(int(counts[r]))}
    for row in range(90):
        if row not in covered:
            assert np.all(out[row] == 7)


def pin_gather_then_prefill_equals_decode():
    """Prefill over the gathered keys, each row seeing [offset_r, offset_r +
    visible), reproduces decode over the paged cache bit for bit."""
    inp, vis = _small_decode()
    comp = O.comp_lens(inp.seq_lens)
    offsets = np.concatenate([[0], np.cumsum(comp[:-1])]).astype(np.int32) + 3
    k = np.zeros((int(comp.sum()) + 5, 128), np.uint16)
    O.gather_keys(inp.k_pool, inp.page_table, comp, offsets, k)
    base = _run_decode(inp, vis)
    rows = inp.q.shape[0] * inp.q.shape[1]
    q = np.ascontiguousarray(inp.q.reshape(rows, 4, 128))
    req = np.repeat(np.arange(inp.q.shape[0]), inp.q.shape[1])
    ks = offsets[req]
    got = O.prefill(q, k, ks, ks + vis, inp.out_cols, scale=SCALE)
    assert np.array_equal(_f32_bits(got), _f32_bits(base))


def pin_widened_gather_then_prefill_equals_typed_prefill():
    """e4m3 keys gathered with widening to bf16, then the bf16 prefill with
    scale * k_scale, equal the typed prefill over the codes bit for bit (the
    widening is exact and k_scale is a positive factor of every dot)."""
    import torch
    inp, vis = _small_decode()
    k8 = torch.from_numpy(bits_to_f32(inp.k_pool) * 16).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    comp = O.comp_lens(inp.seq_lens)
    offsets = np.concatenate([[0], np.cumsum(comp[:-1])]).astype(np.int32)
    kw = np.zeros((int(comp.sum()) + 1, 128), np.uint16)
    O.gather_keys(k8, inp.page_table, comp, offsets, kw, widen="bf16")
    k8g = np.zeros((int(comp.sum()) + 1, 128), np.uint8)
    O.gather_keys(k8, inp.page_table, comp, offsets, k8g)
    rows = inp.q.shape[0] * inp.q.shape[1]
    q = np.ascontiguousarray(inp.q.reshape(rows, 4, 128))
    req = np.repeat(np.arange(inp.q.shape[0]), inp.q.shape[1])
    ks = offsets[req]
    k_scale = 0.0625  # a power of two: scale * k_scale is exact in fp32
    a = O.prefill(q, kw, ks, ks + vis, inp.out_cols, scale=float(np.float32(SCALE * k_scale)))
    b = O.prefill_typed(q, "bf16", k8g, "fp8_e4m3", ks, ks + vis, inp.out_cols, k_scale=k_scale, scale=SCALE)
    assert np.array_equal(_f32_bits(a), _f32_bits(b))


# ---- Query preparation [QSA-PREP _norm_rope, _store_rotated, _to_dst_dtype] ----

def _torch_round(x32, dtype_name):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(getattr(torch, dtype_name))
    return t.view(torch.uint8 if dtype_name == "float8_e4m3fn" else torch.int16).numpy()


def pin_bf16_rounding_matches_library():
    # torch's float -> bfloat16 conversion (nearest, ties to even) is the
    # library routine; exact ties with odd and even kept parts included.
    rng = np.random.default_rng(71)
    x = (rng.standard_normal(20000) * 3.0).astype(np.float32)
    kept = np.arange(0x3F00, 0x4100, dtype=np.uint32)
    ties = ((kept << 16) | 0x8000).view(np.float32)
    near = np.concatenate([((kept << 16) | 0x7FFF), ((kept << 16) | 0x8001)]).view(np.float32)
    tiny = np.array([1e-40, -3e-39, 0.0, -0.0, 3.0e38, -3.3e38], np.float32)
    for v in (x, ties, near, tiny):
        assert np.array_equal(O.round_bf16(v), _torch_round(v, "bfloat16").view(np.uint16))


def pin_e4m3_rounding_matches_library_and_saturates():
    # Below 448 torch's float8_e4m3fn conversion (nearest, ties to even) is
    # the library routine: random values, every midpoint between two
    # neighbouring codes, and values just beside the midpoints.
    rng = np.random.default_rng(72)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-9, 5, 20000))).astype(np.float32)
    x = x[np.abs(x) < 440]
    import torch
    vals = torch.arange(0, 127, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    beside = np.concatenate([np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    for v in (x, mids, -mids, beside):
        v = v[np.abs(v) < 448]
        assert np.array_equal(O.round_e4m3(v), _torch_round(v, "float8_e4m3fn"))
    # The largest finite magnitude is 448: everything beyond saturates.
    big = np.array([448.0, 449.0, 463.9, 464.0, 480.0, 1e6, np.inf], np.float32)
    assert np.all(O.round_e4m3(big) == 0x7E) and np.all(O.round_e4m3(-big) == 0xFE)
    assert O.round_e4m3(np.array([np.nan], np.float32))[0] == 0x7F


def _identity_table(rows, fmt):
    cs = np.zeros((rows, 64), np.float32)
    cs[:, :32] = 1.0
    return cs if fmt == "fp32" else bf16_bits(cs)


def _rope_table(rows, seed=None):
    # cos/sin of position * 10000^(-j/32), rounded to fp32 (a real table).
    j = np.arange(32)
    ang = np.arange(rows)[:, None] * (10000.0 ** (-j / 32.0))[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def _library_norm(q_bits, weight, eps):
    import torch
    x = torch.from_numpy(bits_to_f32(q_bits).astype(np.float64)).reshape(q_bits.shape[0], -1, 128)
    w = torch.from_numpy(np.asarray(weight, np.float64) + 1.0)
    return torch.nn.functional.rms_norm(x, (128,), weight=w, eps=eps).numpy()


def _prep_inputs(seed, T=7, H=3):
    rng = np.random.default_rng(seed)
    q = normal_bf16(rng, (T, H * 128))
    q[1] = bf16_bits(bits_to_f32(q[1]) * np.float32(1e-3))   # small row: eps matters
    w_f = (rng.standard_normal(128) * 0.3).astype(np.float32)
    return q, bf16_bits(w_f), bits_to_f32(bf16_bits(w_f)), rng


def pin_prepare_norm_matches_library():
    # With cos 1 and sin 0 the output is the Gemma RMSNorm itself:
    # torch.nn.functional.rms_norm in float64 with weight (w + 1), to bf16
    # precision; eps large enough that its placement shows.
    q, w_bits, w_f, _ = _prep_inputs(73)
    for eps in (0.25, 1e-6):
        pos = np.zeros(q.shape[0], np.int64)
        got = bits_to_f32(O.prepare_q(q, pos, _identity_table(2, "fp32"), w_bits, eps)).astype(np.float64)
        ref = _library_norm(q, w_f, eps)
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30), eps


def pin_prepare_rotation_is_complex_product():
    # NeoX pairs (j, j + 32) turn by the table's angle: y_j + i*y_{j+32}
    # times c + i*s (numpy complex128), the last 64 features unchanged.
    q, w_bits, w_f, rng = _prep_inputs(74)
    table = _rope_table(50)
    pos = rng.integers(0, 50, q.shape[0]).astype(np.int64)
    got = bits_to_f32(O.prepare_q(q, pos, table, w_bits, 1e-6)).astype(np.float64)
    y = _library_norm(q, w_f, 1e-6)
    c = table[pos, :32].astype(np.float64)[:, None, :]
    s = table[pos, 32:].astype(np.float64)[:, None, :]
    z = (y[..., :32] + 1j * y[..., 32:64]) * (c + 1j * s)
    want = np.concatenate([z.real, z.imag, y[..., 64:]], axis=-1)
    mag = np.concatenate([np.abs(y[..., :32]) + np.abs(y[..., 32:64])] * 2 + [np.abs(y[..., 64:])], axis=-1)
    assert np.all(np.abs(got - want) <= 2.0 ** -7 * mag + 1e-30)


def pin_prepare_closed_forms():
    # Every feature 2.0, weight w: mean(x^2) = 4, so the output is
    # (w + 1) / sqrt(4 + eps) wherever cos is 1 and sin 0.
    q = np.full((2, 256), 0x4000, np.uint16)               # bf16 2.0
    pos = np.array([0, 1], np.int64)
    for eps, w, want in ((0.0, 0.0, 1.0), (12.0, 0.0, 0.5), (12.0, 0.5, 0.75), (60.0, -0.5, 0.125)):
        out = bits_to_f32(O.prepare_q(q, pos, _identity_table(2, "bf16"), bf16_bits(np.full(128, w, np.float32)),
                                      eps))
        assert np.all(out == np.float32(want)), (eps, w)


def _worked_example(table_format):
    # Hand-worked rounding example.  Features 5 = 1 + 2^-7, 37 = -2^-4,
    # 9 = 1 + 2^-7 and 70 = 1.1875, all others 0; eps = 1 - sum(x^2)/128
    # (exact in fp32) so rrms = 1; weight 0 except w_9 = w_70 = -2^-10, so
    # y_9 = (1 + 2^-7)(1 - 2^-10) and y_70 = 1.1875 (1 - 2^-10).
    # Table row 0: pair 5 has cos 1 - 2^-8, sin 2^-4; pair 9 cos 1.5, sin 0;
    # every other pair cos 1, sin 0.
    x = np.zeros(128, np.float32)
    x[5], x[37], x[9], x[70] = 1 + 2.0 ** -7, -(2.0 ** -4), 1 + 2.0 ** -7, 1.1875
    s = float(np.sum(x.astype(np.float64) ** 2))
    eps = float(np.float32(1.0) - np.float32(s / 128))
    w = np.zeros(128, np.float32)
    w[9] = w[70] = -(2.0 ** -10)
    cs = np.zeros((1, 64), np.float32)
    cs[0, :32] = 1.0
    cs[0, 5], cs[0, 32 + 5] = 1 - 2.0 ** -8, 2.0 ** -4
    cs[0, 9] = 1.5
    table = bf16_bits(cs) if table_format == "bf16" else cs
    return bf16_bits(x)[None, :], bf16_bits(w), table, eps


def pin_prepare_worked_rounding_example():
    # bf16 table, one rounding per operation:
    #   out_5  = bf16(1 + 2^-8 - 2^-15) - bf16(-2^-8) = 1 + 2^-8 -> tie -> 1
    #   out_37 = (-2^-4 + 2^-12) + (2^-4 + 2^-11) = 3 * 2^-12
    #   y_9 rounds to 1 + 2^-7; times 1.5 is the tie 1.5 + 2^-7 + 2^-8,
    #   which goes to the even 1.5 + 2^-6.
    # fp32 table (rounded to bf16 only at the end):
    #   out_5 = bf16(1 + 2^-7 - 2^-15) = 1 + 2^-7
    #   out_9 = bf16(1.5 (1 + 2^-7)(1 - 2^-10)), just below the tie: 1.5 + 2^-7.
    pos = np.zeros(1, np.int64)
    for fmt, o5, o9 in (("bf16", 1.0, 1.5 + 2.0 ** -6), ("fp32", 1 + 2.0 ** -7, 1.5 + 2.0 ** -7)):
        q, w, table, eps = _worked_example(fmt)
        out = bits_to_f32(O.prepare_q(q, pos, table, w, eps))[0, 0]
        want = np.zeros(128, np.float32)
        want[5], want[37], want[9], want[70] = o5, 3 * 2.0 ** -12, o9, 1.1875
        assert np.array_equal(out, want), (fmt, np.nonzero(out != want))
    # The e4m3 store divides the bf16 value by the scale.  bf16 table, scale
    # 2: 1/2 -> 0x30; (1.5 + 2^-6)/2 = 0.7578125 -> 0.75 = 0x34; 1.1875/2 is
    # the tie between 0.5625 (odd code 0x31) and 0.625 (even, 0x32);
    # 3*2^-13 -> 0 (below half of 2^-9).
    q, w, table, eps = _worked_example("bf16")
    codes = O.prepare_q(q, pos, table, w, eps, out_format="fp8_e4m3", out_scale=2.0)[0, 0]
    want = np.zeros(128, np.uint8)
    want[5], want[9], want[70] = 0x30, 0x34, 0x32
    assert np.array_equal(codes, want)
    # fp32 table, scale 1: y_70 = 1.1875 - 1.1875 * 2^-10 lies below the
    # e4m3 midpoint 1.1875, but its bf16 rounding is 1.1875, the tie between
    # 1.125 (0x39) and 1.25 (even, 0x3A): the store gives 0x3A.  Feature 5
    # -> 1.0 (0x38), feature 9 -> 1.5 (0x3C).
    q, w, table, eps = _worked_example("fp32")
    codes = O.prepare_q(q, pos, table, w, eps, out_format="fp8_e4m3", out_scale=1.0)[0, 0]
    want = np.zeros(128, np.uint8)
    want[5], want[9], want[70] = 0x38, 0x3C, 0x3A
    assert np.array_equal(codes, want)


def pin_prepare_mrope_axes():
    # Table row p: cos 2^-p, sin 0, so output feature j (and j + 32) of an
    # all-ones row is 2^-(position of pair j's axis).  Positions t=1, h=2,
    # w=3 name the axis.  Interleaved MRoPE: each axis gets as many pairs as
    # its section entry, pairs 0, 3, 6, ... are temporal, the first triples
    # run (t, h, w), and pairs past the interleaved part are temporal.
    cs = np.zeros((4, 64), np.float32)
    cs[:, :32] = (2.0 ** -np.arange(4))[:, None]
    q = np.full((1, 128), 0x3F80, np.uint16)                # bf16 1.0
    pos = np.array([[1], [2], [3]], np.int64)
    for sec in ((16, 8, 8), (12, 10, 10), (24, 8, 0), (32, 0, 0), (20, 6, 6)):
        out = bits_to_f32(O.prepare_q(q, pos, bf16_bits(cs), np.zeros(128, np.uint16), 0.0,
                                      mrope_section=sec))[0, 0]
        axis = np.round(-np.log2(out[:32])).astype(int) - 1
        assert np.array_equal(out[:32], out[32:64])
        assert [int((axis == a).sum()) for a in range(3)] == list(sec), sec
        assert np.all(axis[0::3] == 0)
        m = 3 * min(sec[1], sec[2])
        assert np.array_equal(axis[:m], np.arange(m) % 3)
        assert np.all(axis[3 * max(sec[1], sec[2]):] == 0)
    # One position per token with a section: every axis reads the same row,
    # which is plain rotary.
    q, w_bits, _, rng = _prep_inputs(75)
    p1 = rng.integers(0, 50, q.shape[0]).astype(np.int64)
    table = bf16_bits(_rope_table(50))
    plain = O.prepare_q(q, p1, table, w_bits, 1e-6)
    assert np.array_equal(O.prepare_q(q, p1, table, w_bits, 1e-6, mrope_section=(16, 8, 8)), plain)
    assert np.array_equal(O.prepare_q(q, np.stack([p1] * 3), table, w_bits, 1e-6, mrope_section=(12, 10, 10)),
                          plain)


def pin_prepare_layout_invariants():
    # Heads and tokens are independent: permuting heads (and tokens with
    # their positions) permutes the output; a padded token stride reads the
    # same values.  A position outside the table turns exactly the rotated
    # features of the pairs that use it into NaN.
    q, w_bits, _, rng = _prep_inputs(76, T=9, H=4)
    table = bf16_bits(_rope_table(40))
    pos = rng.integers(0, 40, q.shape[0]).astype(np.int64)
    base = O.prepare_q(q, pos, table, w_bits, 1e-6)
    hp, tp = np.array([2, 0, 3, 1]), rng.permutation(q.shape[0])
    qh = q.reshape(9, 4, 128)[:, hp].reshape(9, 512)
    assert np.array_equal(O.prepare_q(qh, pos, table, w_bits, 1e-6), base[:, hp])
    assert np.array_equal(O.prepare_q(q[tp], pos[tp], table, w_bits, 1e-6), base[tp])
    padded = np.zeros((9, 512 + 64), np.uint16)
    padded[:, :512] = q
    assert np.array_equal(O.prepare_q(padded[:, :512], pos, table, w_bits, 1e-6), base)
    pos3 = np.stack([pos, pos, pos])
    pos3[1, 4] = 40                                          # height position off the table
    out = bits_to_f32(O.prepare_q(q, pos3, table, w_bits, 1e-6, mrope_section=(16, 8, 8)))
    h_pairs = np.array([j for j in range(32) if j % 3 == 1 and j < 24])
    bad = np.zeros(128, bool)
    bad[h_pairs] = bad[h_pairs + 32] = True
    assert np.all(np.isnan(out[4][:, bad])) and not np.any(np.isnan(out[4][:, ~bad]))
    assert not np.any(np.isnan(np.delete(out, 4, axis=0)))
    # The e4m3 store takes the bf16 result divided by the scale.
    codes = O.prepare_q(q, pos, table, w_bits, 1e-6, out_format="fp8_e4m3", out_scale=0.05)
    assert np.array_equal(codes, O.round_e4m3(bits_to_f32(base) / np.float32(0.05)))


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
