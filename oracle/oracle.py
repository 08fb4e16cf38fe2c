"""Python side of the plain CPU oracle for the QSA MQA indexer.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this module.  The product library
never loads it and shares no code with it.

``qsa_oracle.c`` holds the score, metadata and top-k arithmetic (plain loops,
double accumulation).  This module compiles it with gcc, marshals numpy arrays
into it, and splits rows over threads (ctypes releases the GIL for the call,
and rows are independent).  The batch split is host bookkeeping and is written
here in plain Python.

Sources (page title, section):
  "vLLM/vllm/models/qwen4_exp/common/qsa_cache.py", QSAMetadataBuilder.__init__
  and .build: decode threshold 1 with speculative tokens counted as decode,
  decodes ordered first, one uniform decode query length over the non-empty
  decode requests.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qsa_oracle.c")
LIB = os.path.join(HERE, "libqsa_oracle.so")

HEADS = 4
DIM = 128

_lib = None


def build(src: str = SRC, out: str = LIB) -> str:
    """Compile the oracle with gcc.  No fast-math and no FP contraction, so the
    double arithmetic is exactly what the source says."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _declare(lib: ctypes.CDLL) -> ctypes.CDLL:
    P = ctypes.c_void_p
    i32, i64, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    lib.oracle_token_metadata.argtypes = [P, P, i32, i32, i32, P, P, P]
    lib.oracle_token_metadata.restype = None
    lib.oracle_comp_lens.argtypes = [P, i32, i32, P]
    lib.oracle_comp_lens.restype = None
    lib.oracle_prefill_intervals.argtypes = [P, P, P, i32, P, P]
    lib.oracle_prefill_intervals.restype = None
    lib.oracle_decode.argtypes = [P, i64, i64, i64, P, i64, i32, P, i64, i32, P, P,
                                  i32, i32, f32, P, i64, i32, i32, i32]
    lib.oracle_decode.restype = None
    lib.oracle_prefill.argtypes = [P, i64, i64, P, i64, i64, P, P, i32, f32, P, i64,
                                   i32, i32, i32]
    lib.oracle_prefill.restype = None
    lib.oracle_topk.argtypes = [P, i64, i32, i32, P, i64, i32, i32]
    lib.oracle_topk.restype = ctypes.c_int
    lib.oracle_cache_slots.argtypes = [P, P, i32, i32, i32, P, i64, i32, i32, P, P]
    lib.oracle_cache_slots.restype = None
    lib.oracle_k_work.argtypes = [P, P, i32, i32, P, i32]
    lib.oracle_k_work.restype = None
    f64 = ctypes.c_double
    lib.oracle_decode_typed.argtypes = [P, ctypes.c_int, i64, i64, i64, P, ctypes.c_int, f64, i64,
                                        i32, P, i64, i32, P, P, i32, i32, f32, P, i64, i32, i32, i32]
    lib.oracle_decode_typed.restype = None
    lib.oracle_prefill_typed.argtypes = [P, ctypes.c_int, i64, i64, P, ctypes.c_int, f64, i64, i64,
                                         P, P, i32, f32, P, i64, i32, i32, i32]
    lib.oracle_prefill_typed.restype = None
    lib.oracle_round_bf16.argtypes = [P, i64, P]
    lib.oracle_round_bf16.restype = None
    lib.oracle_round_e4m3.argtypes = [P, i64, P]
    lib.oracle_round_e4m3.restype = None
    lib.oracle_prepare_q.argtypes = [P, i64, i32, P, i64, i64, P, ctypes.c_int, i64, P, ctypes.c_int, f32,
                                     P, P, ctypes.c_int, f32, i64, i64, i32, i32]
    lib.oracle_prepare_q.restype = None
    lib.oracle_ring_slots.argtypes = [P, P, i32, i32, P, i64, i32, i32, P]
    lib.oracle_ring_slots.restype = None
    lib.oracle_write_keys.argtypes = [P, i64, i32, P, P, ctypes.c_int, i64, i64, f32, P, i64, i64]
    lib.oracle_write_keys.restype = None
    return lib


def load(path: str | None = None) -> ctypes.CDLL:
    """Load the compiled oracle, building it first if it is missing or older
    than its source."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        _lib = _declare(ctypes.CDLL(LIB))
    return _lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data


def _threads(threads: int | None) -> int:
    if threads is None:
        threads = (int(os.environ.get("QSA_ORACLE_THREADS", "0"))
                   or int(os.environ.get("OMP_NUM_THREADS", "0"))
                   or len(os.sched_getaffinity(0)))
    return max(1, int(threads))


def _run_rows(fn, num_rows: int, threads: int | None) -> int:
    """Call fn(row_begin, row_end) over [0, num_rows) on a thread pool.
    Returns the number of threads used."""
    n = min(_threads(threads), max(num_rows, 1))
    if n <= 1 or num_rows <= 1:
        fn(0, num_rows)
        return 1
    bounds = np.linspace(0, num_rows, n + 1).astype(np.int64)
    with ThreadPoolExecutor(max_workers=n) as pool:
        list(pool.map(lambda i: fn(int(bounds[i]), int(bounds[i + 1])), range(n)))
    return n


# ----------------------------------------------------------------------------
# a1: batch split and per-token metadata


def split_batch(query_start_loc, decode_threshold: int, reorder: bool = False):
    """Decode/prefill split of one batch.

    A request qualifies as a decode when its query length is between 1 and
    ``decode_threshold`` and equals the decode query length (DQL): the length
    of the first request (in batch order) whose length is in that range.
    Empty requests are not decodes.

    ``reorder=False``: the batch is taken as ordered decodes-first, and the
    decodes are its longest qualifying prefix.  ``reorder=True``: returns the
    stable order that puts every qualifying request first.

    Returns (order or None, num_decodes, num_decode_tokens, num_prefills,
    num_prefill_tokens, dql)."""
    qsl = [int(x) for x in query_start_loc]
    num_reqs = len(qsl) - 1
    lens = [qsl[r + 1] - qsl[r] for r in range(num_reqs)]
    dql = 0
    for n in lens:
        if 1 <= n <= decode_threshold:
            dql = n
            break
    qualifies = [dql > 0 and n == dql for n in lens]
    if reorder:
        order = [r for r in range(num_reqs) if qualifies[r]] + \
                [r for r in range(num_reqs) if not qualifies[r]]
        num_decodes = sum(qualifies)
        lens_in_order = [lens[r] for r in order]
    else:
        order = None
        num_decodes = 0
        while num_decodes < num_reqs and qualifies[num_decodes]:
            num_decodes += 1
        lens_in_order = lens
    num_decode_tokens = sum(lens_in_order[:num_decodes])
    num_prefill_tokens = sum(lens_in_order[num_decodes:])
    if num_decodes == 0:
        dql = 0
    return (order, num_decodes, num_decode_tokens, num_reqs - num_decodes,
            num_prefill_tokens, dql)


def token_metadata(query_start_loc, seq_lens, num_tokens: int, compress_ratio: int = 4):
    """Per-token (request, logical position, visible blocks)."""
    lib = load()
    qsl = np.ascontiguousarray(query_start_loc, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    req = np.empty(num_tokens, np.int32)
    pos = np.empty(num_tokens, np.int64)
    vis = np.empty(num_tokens, np.int32)
    lib.oracle_token_metadata(_ptr(qsl), _ptr(sl), len(sl), num_tokens, compress_ratio,
                              _ptr(req), _ptr(pos), _ptr(vis))
    return req, pos, vis


def comp_lens(seq_lens, compress_ratio: int = 4):
    lib = load()
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    out = np.empty(len(sl), np.int32)
    lib.oracle_comp_lens(_ptr(sl), len(sl), compress_ratio, _ptr(out))
    return out


def prefill_intervals(token_to_req, visible, key_offsets):
    lib = load()
    req = np.ascontiguousarray(token_to_req, dtype=np.int32)
    vis = np.ascontiguousarray(visible, dtype=np.int32)
    off = np.ascontiguousarray(key_offsets, dtype=np.int32)
    ks = np.empty(len(req), np.int32)
    ke = np.empty(len(req), np.int32)
    lib.oracle_prefill_intervals(_ptr(req), _ptr(vis), _ptr(off), len(req), _ptr(ks), _ptr(ke))
    return ks, ke


# ----------------------------------------------------------------------------
# a2/a4: decode, a3/a4: prefill, a5: top-k


def default_scale() -> float:
    """1/sqrt(head_dim) for head_dim 128, as an fp32 multiplier."""
    return float(np.float32(1.0 / np.sqrt(np.float64(DIM))))


def _row_list(rows, total):
    """None -> every row as one contiguous range; else the given row indices."""
    if rows is None:
        return None
    rows = np.asarray(rows, dtype=np.int64).reshape(-1)
    assert np.all((rows >= 0) & (rows < total))
    return rows


def decode(q_bits, k_pool_bits, page_table, comp_lens_arr, visible, out_cols: int,
           scale: float | None = None, rows=None, threads: int | None = None):
    """Decode scores.

    q_bits: uint16 [R, DQL, 4, 128] (any strides, unit feature stride);
    k_pool_bits: uint16 [P, page_size, 1, 128]; page_table int32 [R, W];
    comp_lens_arr int32 [R]; visible int32 [R*DQL] or None.
    rows: None for every row, else a sequence of row indices r*DQL+j.
    Returns fp32 [len(rows) or R*DQL, out_cols]."""
    lib = load()
    q = np.asarray(q_bits)
    assert q.dtype == np.uint16 and q.ndim == 4 and q.shape[2:] == (HEADS, DIM)
    assert q.strides[3] == 2
    kp = np.ascontiguousarray(k_pool_bits, dtype=np.uint16)
    assert kp.ndim == 4 and kp.shape[2:] == (1, DIM)
    pt = np.ascontiguousarray(page_table, dtype=np.int32)
    assert pt.ndim == 2
    cl = np.ascontiguousarray(comp_lens_arr, dtype=np.int32)
    vis = None if visible is None else np.ascontiguousarray(visible, dtype=np.int32)
    num_reqs, dql = q.shape[0], q.shape[1]
    sr, sj, sh = (s // 2 for s in q.strides[:3])
    scale = default_scale() if scale is None else float(scale)
    total = num_reqs * dql
    sel = _row_list(rows, total)
    out = np.empty((total if sel is None else len(sel), out_cols), np.float32)

    def call(row_begin, row_end, dst_row):
        lib.oracle_decode(_ptr(q), sr, sj, sh, _ptr(kp), kp.shape[0], kp.shape[1],
                          _ptr(pt), pt.shape[1], pt.shape[1], _ptr(cl), _ptr(vis),
                          num_reqs, dql, scale, out.ctypes.data + dst_row * out_cols * 4,
                          out_cols, out_cols, row_begin, row_end)

    if sel is None:
        _run_rows(lambda b, e: call(b, e, b), total, threads)
    else:
        _run_rows(lambda b, e: [call(int(sel[i]), int(sel[i]) + 1, i) for i in range(b, e)],
                  len(sel), threads)
    return out


def prefill(q_bits, k_bits, row_k_start, row_k_end, out_cols: int, scale: float | None = None,
            rows=None, threads: int | None = None):
    """Prefill scores.

    q_bits: uint16 [T, 4, 128] (unit feature stride); k_bits: uint16 [NK, 128]
    (unit feature stride); row_k_start/row_k_end int32 [T].
    rows: None for all rows, else a sequence of row indices.
    Returns fp32 [len(rows) or T, out_cols]."""
    lib = load()
    q = np.asarray(q_bits)
    assert q.dtype == np.uint16 and q.ndim == 3 and q.shape[1:] == (HEADS, DIM)
    assert q.strides[2] == 2
    k = np.asarray(k_bits)
    assert k.dtype == np.uint16 and k.ndim == 2 and k.shape[1] == DIM and k.strides[1] == 2
    ks = np.ascontiguousarray(row_k_start, dtype=np.int32)
    ke = np.ascontiguousarray(row_k_end, dtype=np.int32)
    num_rows = q.shape[0]
    scale = default_scale() if scale is None else float(scale)
    sq, sh = q.strides[0] // 2, q.strides[1] // 2
    sk = k.strides[0] // 2
    sel = _row_list(rows, num_rows)
    out = np.empty((num_rows if sel is None else len(sel), out_cols), np.float32)

    def call(row_begin, row_end, dst_row):
        lib.oracle_prefill(_ptr(q), sq, sh, _ptr(k), sk, k.shape[0], _ptr(ks), _ptr(ke),
                           num_rows, scale, out.ctypes.data + dst_row * out_cols * 4,
                           out_cols, out_cols, row_begin, row_end)

    if sel is None:
        _run_rows(lambda b, e: call(b, e, b), num_rows, threads)
    else:
        _run_rows(lambda b, e: [call(int(sel[i]), int(sel[i]) + 1, i) for i in range(b, e)],
                  len(sel), threads)
    return out


# Element formats of the typed functions: name -> (code, numpy container dtype).
FORMATS = {"bf16": (0, np.uint16), "fp16": (1, np.uint16), "fp8_e4m3": (2, np.uint8)}


def _typed(bits, fmt):
    code, container = FORMATS[fmt]
    a = np.asarray(bits)
    assert a.dtype == container, f"{fmt} elements are {np.dtype(container).name} bit patterns"
    return code, a


def decode_typed(q_bits, q_format: str, k_pool_bits, k_format: str, page_table, comp_lens_arr,
                 visible, out_cols: int, k_scale: float = 1.0, scale: float | None = None,
                 rows=None, threads: int | None = None):
    """decode() for typed elements: q in "bf16" or "fp16", the key pool in
    "bf16", "fp16" or "fp8_e4m3" (bit patterns: uint16, or uint8 for fp8).
    An fp8 key element stands for its value times k_scale."""
    lib = load()
    qf, q = _typed(q_bits, q_format)
    assert q.ndim == 4 and q.shape[2:] == (HEADS, DIM) and q.strides[3] == q.itemsize
    kf, kp = _typed(k_pool_bits, k_format)
    kp = np.ascontiguousarray(kp)
    assert kp.ndim == 4 and kp.shape[2:] == (1, DIM)
    pt = np.ascontiguousarray(page_table, dtype=np.int32)
    cl = np.ascontiguousarray(comp_lens_arr, dtype=np.int32)
    vis = None if visible is None else np.ascontiguousarray(visible, dtype=np.int32)
    num_reqs, dql = q.shape[0], q.shape[1]
    sr, sj, sh = (st // q.itemsize for st in q.strides[:3])
    scale = default_scale() if scale is None else float(scale)
    total = num_reqs * dql
    sel = _row_list(rows, total)
    out = np.empty((total if sel is None else len(sel), out_cols), np.float32)

    def call(row_begin, row_end, dst_row):
        lib.oracle_decode_typed(_ptr(q), qf, sr, sj, sh, _ptr(kp), kf, float(k_scale), kp.shape[0],
                                kp.shape[1], _ptr(pt), pt.shape[1], pt.shape[1], _ptr(cl), _ptr(vis),
                                num_reqs, dql, scale, out.ctypes.data + dst_row * out_cols * 4,
                                out_cols, out_cols, row_begin, row_end)

    if sel is None:
        _run_rows(lambda b, e: call(b, e, b), total, threads)
    else:
        _run_rows(lambda b, e: [call(int(sel[i]), int(sel[i]) + 1, i) for i in range(b, e)],
                  len(sel), threads)
    return out


def prefill_typed(q_bits, q_format: str, k_bits, k_format: str, row_k_start, row_k_end,
                  out_cols: int, k_scale: float = 1.0, scale: float | None = None, rows=None,
                  threads: int | None = None):
    """prefill() for typed elements (formats as in decode_typed)."""
    lib = load()
    qf, q = _typed(q_bits, q_format)
    assert q.ndim == 3 and q.shape[1:] == (HEADS, DIM) and q.strides[2] == q.itemsize
    kf, k = _typed(k_bits, k_format)
    assert k.ndim == 2 and k.shape[1] == DIM and k.strides[1] == k.itemsize
    ks = np.ascontiguousarray(row_k_start, dtype=np.int32)
    ke = np.ascontiguousarray(row_k_end, dtype=np.int32)
    num_rows = q.shape[0]
    scale = default_scale() if scale is None else float(scale)
    sq, sh = q.strides[0] // q.itemsize, q.strides[1] // q.itemsize
    sk = k.strides[0] // k.itemsize
    sel = _row_list(rows, num_rows)
    out = np.empty((num_rows if sel is None else len(sel), out_cols), np.float32)

    def call(row_begin, row_end, dst_row):
        lib.oracle_prefill_typed(_ptr(q), qf, sq, sh, _ptr(k), kf, float(k_scale), sk, k.shape[0],
                                 _ptr(ks), _ptr(ke), num_rows, scale,
                                 out.ctypes.data + dst_row * out_cols * 4, out_cols, out_cols,
                                 row_begin, row_end)

    if sel is None:
        _run_rows(lambda b, e: call(b, e, b), num_rows, threads)
    else:
        _run_rows(lambda b, e: [call(int(sel[i]), int(sel[i]) + 1, i) for i in range(b, e)],
                  len(sel), threads)
    return out


def cache_slots(query_start_loc, seq_lens, num_tokens: int, block_table, storage_block_size: int,
                compress_ratio: int = 4, common_slot_mapping=None):
    """int64 [num_tokens]: the compressed-cache slot each token writes, or -1
    (see oracle_cache_slots)."""
    lib = load()
    qsl = np.ascontiguousarray(query_start_loc, dtype=np.int32)
    seq = np.ascontiguousarray(seq_lens, dtype=np.int32)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    assert bt.ndim == 2
    common = None if common_slot_mapping is None else np.ascontiguousarray(common_slot_mapping, dtype=np.int64)
    out = np.empty(num_tokens, np.int64)
    lib.oracle_cache_slots(_ptr(qsl), _ptr(seq), len(seq), num_tokens, compress_ratio, _ptr(bt), bt.shape[1],
                           bt.shape[1], storage_block_size, _ptr(common), _ptr(out))
    return out


def k_work(query_start_loc, seq_lens, max_num_work: int, compress_ratio: int = 4):
    """int32 [max_num_work, 2]: (request, index) work items, (-1, -1) past the last."""
    lib = load()
    qsl = np.ascontiguousarray(query_start_loc, dtype=np.int32)
    seq = np.ascontiguousarray(seq_lens, dtype=np.int32)
    out = np.empty((max_num_work, 2), np.int32)
    lib.oracle_k_work(_ptr(qsl), _ptr(seq), len(seq), compress_ratio, _ptr(out), max_num_work)
    return out


def ring_slots(query_start_loc, seq_lens, num_tokens: int, block_table, ring_size: int):
    """int64 [num_tokens]: the raw-key ring row each token writes, or -1
    (see oracle_ring_slots)."""
    lib = load()
    qsl = np.ascontiguousarray(query_start_loc, dtype=np.int32)
    seq = np.ascontiguousarray(seq_lens, dtype=np.int32)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    assert bt.ndim == 2 and ring_size >= 1
    out = np.empty(num_tokens, np.int64)
    lib.oracle_ring_slots(_ptr(qsl), _ptr(seq), len(seq), num_tokens, _ptr(bt), bt.shape[1], bt.shape[1],
                          int(ring_size), _ptr(out))
    return out


def write_keys(keys, slots, cache, fmt: str = "bf16", scale: float = 1.0, positions=None):
    """Key rows written to cache rows (see oracle_write_keys), on a copy of
    `cache`, which is returned.  keys: uint16 bf16 bits [T, 128]; slots:
    int64 [T]; cache: [..., W] rows of uint16 (fmt "bf16", W >= 128, or
    W >= 140 with positions) or uint8 e4m3 codes (fmt "fp8_e4m3", W >= 128);
    positions: int64 [3, T] or None."""
    lib = load()
    k = np.ascontiguousarray(keys, dtype=np.uint16)
    assert k.ndim == 2 and k.shape[1] == DIM
    sl = np.ascontiguousarray(slots, dtype=np.int64)
    assert sl.shape == (k.shape[0],)
    out = np.array(cache, copy=True)
    width = out.shape[-1]
    if fmt == "fp8_e4m3":
        assert out.dtype == np.uint8 and width >= DIM and positions is None
        code = FORMATS["fp8_e4m3"][0]
    else:
        assert fmt == "bf16" and out.dtype == np.uint16 and width >= DIM
        code = FORMATS["bf16"][0]
    pos = None
    if positions is not None:
        pos = np.ascontiguousarray(positions, dtype=np.int64)
        assert pos.shape == (3, k.shape[0]) and width >= DIM + 12
    lib.oracle_write_keys(_ptr(k), DIM, k.shape[0], _ptr(sl), out.ctypes.data, code, width, out.size // width,
                          float(np.float32(scale)), _ptr(pos), k.shape[0] if pos is not None else 0, 1)
    return out


def e4m3_to_16bit(codes, fmt: str):
    """OCP e4m3 codes (uint8) -> the same values as bf16 or fp16 bit patterns
    (uint16); exact (every e4m3 value is representable in both).  The
    decoding is torch's float8_e4m3fn, a library routine."""
    import torch
    vals = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    dt = torch.bfloat16 if fmt == "bf16" else torch.float16
    return vals.to(dt).view(torch.int16).numpy().view(np.uint16)


def gather_keys(k_pool, page_table, key_counts, key_offsets, out, widen: str | None = None):
    """Paged compressed keys gathered into contiguous rows, in place in `out`
    ([rows, 128] of the pool's element type): row key_offsets[r] + c holds
    request r's compressed key c for c < key_counts[r], i.e. row c % page_size
    of page page_table[r][c // page_size]; a missing page (negative id, id
    >= the pool's pages, or past the table's columns) gives a zero row.
    Rows no request covers are left as they are.  widen ("bf16" or "fp16"):
    the pool holds e4m3 codes and `out` receives their values in that 16-bit
    format."""
    pool = np.asarray(k_pool)
    if widen is not None:
        pool = e4m3_to_16bit(pool, widen)
    assert pool.ndim == 4 and pool.shape[2] == 1
    num_pages, page_size = pool.shape[0], pool.shape[1]
    pt = np.asarray(page_table)
    for r in range(len(key_counts)):
        for c in range(int(key_counts[r])):
            slot = c // page_size
            page = int(pt[r, slot]) if slot < pt.shape[1] else -1
            row = int(key_offsets[r]) + c
            out[row] = pool[page, c % page_size, 0] if 0 <= page < num_pages else 0
    return out


def topk(logits, k: int, threads: int | None = None):
    """Per-row top-k columns of fp32 logits [T, C]: int32 [T, k], ascending,
    -1 padded."""
    lib = load()
    x = np.ascontiguousarray(logits, dtype=np.float32)
    assert x.ndim == 2 and k >= 1
    out = np.empty((x.shape[0], k), np.int32)

    def fn(b, e):
        rc = lib.oracle_topk(x.ctypes.data, x.shape[1], x.shape[1], k,
                             out.ctypes.data + b * k * 4, k, b, e)
        if rc != 0:
            raise MemoryError("oracle_topk: allocation failed")
    _run_rows(fn, x.shape[0], threads)
    return out


def round_bf16(x):
    """fp32 values -> bf16 bit patterns (uint16), nearest with ties to even."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(a.shape, np.uint16)
    load().oracle_round_bf16(_ptr(a), a.size, _ptr(out))
    return out


def round_e4m3(x):
    """fp32 values -> OCP e4m3 codes (uint8): nearest finite value, ties to
    the even code (so beyond 448 the result is +-448); NaN -> 0x7F."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(a.shape, np.uint8)
    load().oracle_round_e4m3(_ptr(a), a.size, _ptr(out))
    return out


def _rot_table(a):
    """(code, array) of a cos/sin table or norm weight: bf16 bit patterns
    (uint16) or float32 values."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return FORMATS["bf16"][0], a
    assert a.dtype == np.float32, "bf16 bit patterns (uint16) or float32"
    return 3, a


def prepare_q(q_bits, positions, cos_sin, weight, eps: float, mrope_section=None,
              out_format: str = "bf16", out_scale: float = 1.0, threads: int | None = None):
    """Query preparation (see oracle_prepare_q): q_bits [T, H*128] bf16 bit
    patterns (uint16; the token stride may exceed H*128), positions int64 [T]
    or [3, T], cos_sin [rows, 64] (bf16 bits or float32), weight [128] (bf16
    bits or float32).  Returns [T, H, 128]: uint16 bf16 patterns, or uint8
    e4m3 codes of value / out_scale when out_format is "fp8_e4m3"."""
    lib = load()
    q = np.asarray(q_bits)
    assert q.dtype == np.uint16 and q.ndim == 2 and q.strides[1] == 2 and q.shape[1] % DIM == 0
    T, H = q.shape[0], q.shape[1] // DIM
    pos = np.ascontiguousarray(positions, dtype=np.int64)
    if pos.ndim == 1:
        assert pos.shape == (T,)
        sa, st = 0, 1
    else:
        assert pos.shape == (3, T)
        sa, st = T, 1
    rf, cs = _rot_table(cos_sin)
    assert cs.ndim == 2 and cs.shape[1] == 64
    wf, w = _rot_table(weight)
    assert w.shape == (DIM,)
    sec = None if mrope_section is None else np.ascontiguousarray(mrope_section, dtype=np.int32)
    assert sec is None or (sec.shape == (3,) and int(sec.sum()) == 32)
    of = FORMATS[out_format][0]
    assert out_format in ("bf16", "fp8_e4m3")
    out = np.empty((T, H, DIM), FORMATS[out_format][1])
    sq = q.strides[0] // 2

    def fn(b, e):
        lib.oracle_prepare_q(_ptr(q), sq, H, _ptr(pos), sa, st, _ptr(cs), rf, cs.shape[0], _ptr(w), wf,
                             float(eps), _ptr(sec), _ptr(out), of, float(out_scale), H * DIM, DIM, b, e)
    _run_rows(fn, T, threads)
    return out
