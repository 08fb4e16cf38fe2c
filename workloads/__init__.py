"""Seeded synthetic inputs for the QSA indexer workloads.

Both the HIP path and the oracle consume these inputs, so this module holds
none of the scoring arithmetic: no dot products, no masks, no visibility
formula, no top-k.  It draws random numbers, rounds them to bf16 bit patterns,
picks context lengths, allocates pages and shuffles page tables.

Shapes follow the pages' workloads: the decode microbenchmarks of vLLM PR 54513
("[Qwen3.8-Flash-Next] Separate prefill and decode paths for QSA indexer",
section "Microbenchmarks": single request at 100K context, 16 requests with
log-normal contexts of min/mean/max 3,508 / 51,200 / 102,400 tokens at DQL 4)
and its prefill table (1x8K and 4x4K query layouts over 8K and 100K
prefixes); the compressed-key page layout [pages, page_size, 1, 128] from the
MATE "QSA (Qwen Sparse Attention)" page, section "MQA score".
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

HEADS = 4
DIM = 128
TOKENS_PER_ROW = 4  # each compressed-cache row stores one 4-token group


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even.  Inputs
    here are finite normals, so NaN handling is not needed."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def fp16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> IEEE binary16 bit patterns (uint16), round to nearest even
    (numpy's conversion)."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


# Cache scale of the synthetic fp8 key caches: 448 * scale = 5.6, so N(0,1)
# keys essentially never saturate.
FP8_K_SCALE = float(np.float32(0.0125))


def fp8_e4m3_cache(k_bf16_bits: np.ndarray, k_scale: float = FP8_K_SCALE) -> np.ndarray:
    """bf16 key bit patterns -> OCP e4m3 codes (uint8) by the fp8 cache write
    rule of qsa_prepare ("_to_dst_dtype": round to bf16, divide by the cache
    scale in fp32, convert to fp8); the conversion is torch's float8_e4m3fn
    (round to nearest even).  Magnitudes above 448 saturate to 448."""
    import torch
    x = bits_to_f32(k_bf16_bits) / np.float32(k_scale)
    x = np.clip(x, -448.0, 448.0).astype(np.float32)
    return torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    """i.i.d. N(0,1) drawn in float32, stored as bf16 bit patterns."""
    return bf16_bits(rng.standard_normal(size=shape, dtype=np.float32))


def lognormal_contexts(n: int, lo: int, mean: int, hi: int, seed: int = 1) -> list[int]:
    """Skewed context lengths with exact min, mean and max.

    Sorted exp(N(0,1)) draws; the extremes are set to lo and hi; the inner
    draws are scaled (bisection on the factor, clipped to [lo, hi]) so that the
    total is n*mean; values are rounded and the rounding residue goes to the
    element at index n//2."""
    rng = np.random.default_rng(seed)
    x = np.sort(np.exp(rng.standard_normal(n)))
    inner = x[1:-1]
    target = n * mean - lo - hi
    a, b = 0.0, 1e9
    for _ in range(200):
        s = 0.5 * (a + b)
        if np.clip(s * inner, lo, hi).sum() < target:
            a = s
        else:
            b = s
    v = np.round(np.clip(s * inner, lo, hi)).astype(np.int64)
    ctx = np.concatenate([[lo], v, [hi]])
    ctx[n // 2] += target - v.sum()
    return [int(c) for c in ctx]


# ----------------------------------------------------------------------------
# Decode inputs: paged compressed keys


@dataclass
class DecodeInputs:
    q: np.ndarray            # uint16 [R, DQL, 4, 128]
    k_pool: np.ndarray       # uint16 [P, page_size, 1, 128]
    page_table: np.ndarray   # int32 [R, W]; -1 = unused
    seq_lens: np.ndarray     # int32 [R] tokens in context (query tokens included)
    query_start_loc: np.ndarray  # int32 [R+1]: DQL query tokens per request
    page_size: int
    out_cols: int

    @property
    def num_reqs(self):
        return self.q.shape[0]

    @property
    def dql(self):
        return self.q.shape[1]


def pages_for(ctx: int, page_size: int) -> int:
    """Pages allocated for a context of ctx tokens: enough rows for every
    4-token group that has started (a page may hold a partial group's row,
    which the cache never writes; here it holds noise)."""
    rows = -(-ctx // TOKENS_PER_ROW)
    return -(-rows // page_size)


def decode_inputs(ctx_lens, dql: int, page_size: int, table_cols: int, spare_pages: int,
                  out_cols: int, seed: int, shuffle: bool = True) -> DecodeInputs:
    """Paged decode batch.  Every page (used, spare, tails) holds N(0,1) bf16
    noise, so reading a wrong page or row changes a score.  Page tables give
    each request distinct physical pages, shuffled over one pool, and -1 after
    the request's last page."""
    rng = np.random.default_rng(seed)
    ctx_lens = [int(c) for c in ctx_lens]
    num_reqs = len(ctx_lens)
    need = [pages_for(c, page_size) for c in ctx_lens]
    assert max(need + [0]) <= table_cols, "page table too narrow for the longest context"
    num_pages = sum(need) + spare_pages
    q = normal_bf16(rng, (num_reqs, dql, HEADS, DIM))
    k_pool = normal_bf16(rng, (num_pages, page_size, 1, DIM))
    phys = rng.permutation(num_pages) if shuffle else np.arange(num_pages)
    table = np.full((num_reqs, table_cols), -1, np.int32)
    at = 0
    for r, n in enumerate(need):
        table[r, :n] = phys[at:at + n]
        at += n
    seq_lens = np.asarray(ctx_lens, np.int32)
    qsl = np.arange(num_reqs + 1, dtype=np.int32) * dql
    return DecodeInputs(q, k_pool, table, seq_lens, qsl, page_size, out_cols)


# ----------------------------------------------------------------------------
# Prefill inputs: packed queries, packed per-request keys


@dataclass
class PrefillInputs:
    q: np.ndarray            # uint16 [T, 4, 128]
    k: np.ndarray            # uint16 [NK, 128], request r's keys at key_offsets[r]
    seq_lens: np.ndarray     # int32 [R]: prefix + query tokens
    query_start_loc: np.ndarray  # int32 [R+1]
    key_offsets: np.ndarray  # int32 [R]
    out_cols: int


def prefill_inputs(num_reqs: int, query_len: int, prefix: int, seed: int) -> PrefillInputs:
    """num_reqs requests, each with query_len new tokens after `prefix` cached
    tokens.  Each request owns one compressed-key row per complete 4-token
    group of its whole context, packed one request after another."""
    rng = np.random.default_rng(seed)
    seq = prefix + query_len
    rows = seq // TOKENS_PER_ROW
    q = normal_bf16(rng, (num_reqs * query_len, HEADS, DIM))
    k = normal_bf16(rng, (num_reqs * rows, DIM))
    seq_lens = np.full(num_reqs, seq, np.int32)
    qsl = np.arange(num_reqs + 1, dtype=np.int32) * query_len
    key_offsets = np.arange(num_reqs, dtype=np.int32) * rows
    return PrefillInputs(q, k, seq_lens, qsl, key_offsets, rows)


# ----------------------------------------------------------------------------
# The workloads


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str          # "decode" or "prefill"
    seed: int
    description: str
    params: dict = field(default_factory=dict)

    def make(self):
        p = self.params
        if self.kind == "decode":
            ctx = p["ctx"] if isinstance(p["ctx"], list) else [p["ctx"]] * p["num_reqs"]
            return decode_inputs(ctx, p["dql"], p["page_size"], p["table_cols"],
                                 p["spare_pages"], p["out_cols"], self.seed)
        return prefill_inputs(p["num_reqs"], p["query_len"], p["prefix"], self.seed)


C3_CONTEXTS = lognormal_contexts(16, 3508, 51200, 102400, seed=1)

WORKLOADS = {
    "tiny_decode": Workload(
        "tiny_decode", "decode", 1,
        "1 request, DQL 1, context 256 (64 compressed keys), page_size 16, 4 pages",
        dict(ctx=256, num_reqs=1, dql=1, page_size=16, table_cols=4, spare_pages=0,
             out_cols=64)),
    "decode_100k": Workload(
        "decode_100k", "decode", 2,
        "1 request, DQL 1, context 100,000 (25,000 compressed keys), page_size 64",
        dict(ctx=100_000, num_reqs=1, dql=1, page_size=64, table_cols=400, spare_pages=32,
             out_cols=25_000)),
    "specdecode_16x51k": Workload(
        "specdecode_16x51k", "decode", 3,
        "16 requests, DQL 4, log-normal contexts 3,508/51,200/102,400 (min/mean/max), "
        "page_size 64",
        dict(ctx=C3_CONTEXTS, num_reqs=16, dql=4, page_size=64, table_cols=400,
             spare_pages=0, out_cols=25_600)),
    "prefill_1x8k_8k": Workload(
        "prefill_1x8k_8k", "prefill", 4,
        "1 request, 8,192 query tokens after an 8,192-token prefix (4,096 keys)",
        dict(num_reqs=1, query_len=8192, prefix=8192)),
    "prefill_4x4k_100k": Workload(
        "prefill_4x4k_100k", "prefill", 5,
        "4 requests x 4,096 query tokens over a 100,000-token prefix (26,024 keys each), "
        "then top-512 blocks per row",
        dict(num_reqs=4, query_len=4096, prefix=100_000, topk=512)),
    "prefill_1x8k_100k": Workload(
        "prefill_1x8k_100k", "prefill", 6,
        "1 request, 8,192 query tokens over a 100,000-token prefix (27,048 keys)",
        dict(num_reqs=1, query_len=8192, prefix=100_000, topk=512)),
}


@dataclass
class PrepareInputs:
    q: np.ndarray          # bf16 bits [T, H*128]
    positions: np.ndarray  # int64 [T], or [3, T] (temporal, height, width)
    cos_sin: np.ndarray    # [rows, 64]: 32 cos then 32 sin; bf16 bits (uint16) or float32
    weight: np.ndarray     # [128]: bf16 bits or float32
    eps: float = 1e-6


def rope_table(rows: int, fmt: str = "bf16", base: float = 10000.0) -> np.ndarray:
    """A NeoX rotary cos/sin table as the caller supplies it (rotary dim 64):
    row p holds cos(p * base^(-j/32)) for pairs j < 32, then the sines."""
    inv = base ** (-np.arange(32) / 32.0)
    ang = np.arange(rows, dtype=np.float64)[:, None] * inv[None, :]
    t = np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)
    return t if fmt == "fp32" else bf16_bits(t)


def prepare_inputs(num_tokens: int, num_heads: int, seed: int, first_pos: int = 0, table_rows: int | None = None,
                   table: str = "bf16", weight: str = "bf16", mrope: bool = False) -> PrepareInputs:
    """Query heads of one prefill chunk at positions first_pos, first_pos+1, ...
    q ~ N(0, 1) in bf16; the RMSNorm weight ~ N(0, 0.1) (a Gemma gain near 1).
    With mrope the height and width positions trail the temporal one by up
    to 31, as for image patches."""
    rng = np.random.default_rng(seed)
    q = normal_bf16(rng, (num_tokens, num_heads * DIM))
    t = first_pos + np.arange(num_tokens, dtype=np.int64)
    if mrope:
        h = np.maximum(t - rng.integers(0, 32, num_tokens), 0)
        w = np.maximum(t - rng.integers(0, 32, num_tokens), 0)
        positions = np.stack([t, h, w]).astype(np.int64)
    else:
        positions = t
    rows = table_rows if table_rows is not None else first_pos + num_tokens
    w_f = (rng.standard_normal(DIM) * 0.1).astype(np.float32)
    return PrepareInputs(q, positions, rope_table(rows, table), w_f if weight == "fp32" else bf16_bits(w_f))
