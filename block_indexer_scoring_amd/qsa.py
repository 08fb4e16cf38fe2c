"""Python binding of the C ABI in include/qsa.h (libqsa.so).

Argument marshalling only: shapes, dtypes and strides of torch tensors are
turned into the pointers and sizes of the C entry points, and every step of
the computation runs in the library's HIP kernels.  Tensors must live on the
GPU; there is no CPU path.  The functions keep the C names.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqsa.so")

QSA_OK = 0
QSA_ERR_INVALID_ARGUMENT = 1
QSA_ERR_UNSUPPORTED = 2
QSA_ERR_LAYOUT = 3
QSA_ERR_DEVICE = 4
ABI_VERSION = 11

SYMBOLS = ("qsa_abi_version", "qsa_last_error", "qsa_set_launch_events", "qsa_split_batch",
           "qsa_build_metadata", "qsa_mqa_decode", "qsa_mqa_prefill", "qsa_topk_blocks",
           "qsa_mqa_prefill_topk", "qsa_prefill_topk_workspace_bytes", "qsa_mqa_decode_typed",
           "qsa_mqa_prefill_typed", "qsa_build_cache_metadata", "qsa_gather_keys", "qsa_prepare_q",
           "qsa_decode_plan_bytes", "qsa_build_decode_plan", "qsa_mqa_decode_planned",
           "qsa_decode_visible_blocks", "qsa_mqa_decode_static_plan", "qsa_build_ring_slots",
           "qsa_write_keys", "qsa_mqa_prefill_topk_typed")

# enum qsa_dtype
QSA_DTYPE_BF16 = 0
QSA_DTYPE_FP16 = 1
QSA_DTYPE_FP8_E4M3 = 2
QSA_DTYPE_FP32 = 3
_DTYPES = {torch.bfloat16: QSA_DTYPE_BF16, torch.float16: QSA_DTYPE_FP16,
           torch.float8_e4m3fn: QSA_DTYPE_FP8_E4M3, torch.float32: QSA_DTYPE_FP32}

DEFAULT_SCALE = 1.0 / math.sqrt(128.0)


class QSAError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"[{code}] {message}")
        self.code = code


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libqsa.so.  Raises if it has not been built: there is no fallback."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with block_indexer_scoring_amd/build.py "
                           "(or __graft_entry__.build()); there is no CPU fallback")
    lib = ctypes.CDLL(path)
    P, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    lib.qsa_abi_version.argtypes = []
    lib.qsa_abi_version.restype = ctypes.c_int
    lib.qsa_last_error.argtypes = []
    lib.qsa_last_error.restype = ctypes.c_char_p
    lib.qsa_set_launch_events.argtypes = [P, P]
    lib.qsa_set_launch_events.restype = ctypes.c_int
    lib.qsa_split_batch.argtypes = [P, i32, i32, P, P]
    lib.qsa_split_batch.restype = ctypes.c_int
    lib.qsa_build_metadata.argtypes = [P, P, i32, i32, i32, P, P, P, P, P, P, P, P]
    lib.qsa_build_metadata.restype = ctypes.c_int
    lib.qsa_mqa_decode.argtypes = [P, i64, i64, i64, P, i64, i32, P, i64, i32, P, P, i32, i32,
                                   i32, i32, f32, P, i64, i32, P]
    lib.qsa_mqa_decode.restype = ctypes.c_int
    lib.qsa_build_cache_metadata.argtypes = [P, P, i32, i32, i32, P, i64, i32, i32, P, P, P, i32, P]
    lib.qsa_build_cache_metadata.restype = ctypes.c_int
    lib.qsa_gather_keys.argtypes = [P, i32, i64, i32, P, i64, i32, P, P, i32, i32, P, i32, i64, i64, P]
    lib.qsa_gather_keys.restype = ctypes.c_int
    lib.qsa_mqa_decode_typed.argtypes = [P, i32, i64, i64, i64, P, i32, f32, i64, i32, P, i64, i32, P, P,
                                         i32, i32, i32, i32, f32, P, i64, i32, P]
    lib.qsa_mqa_decode_typed.restype = ctypes.c_int
    lib.qsa_mqa_prefill_typed.argtypes = [P, i64, i64, P, i64, i64, i32, P, P, i32, i32, i32, f32, P,
                                          i64, i32, P]
    lib.qsa_mqa_prefill_typed.restype = ctypes.c_int
    lib.qsa_mqa_prefill.argtypes = [P, i64, i64, P, i64, i64, P, P, i32, i32, i32, f32, P, i64,
                                    i32, P]
    lib.qsa_mqa_prefill.restype = ctypes.c_int
    lib.qsa_topk_blocks.argtypes = [P, i64, i32, i32, i32, P, i64, P]
    lib.qsa_topk_blocks.restype = ctypes.c_int
    lib.qsa_mqa_prefill_topk.argtypes = [P, i64, i64, P, i64, i64, P, P, i32, i32, i32, f32, i32, i32,
                                         P, i64, P, i64, P]
    lib.qsa_mqa_prefill_topk.restype = ctypes.c_int
    lib.qsa_mqa_prefill_topk_typed.argtypes = [P, i64, i64, P, i64, i64, i32, P, P, i32, i32, i32, f32, i32,
                                               i32, P, i64, P, i64, P]
    lib.qsa_mqa_prefill_topk_typed.restype = ctypes.c_int
    lib.qsa_prefill_topk_workspace_bytes.argtypes = [i32, i32, i32, P]
    lib.qsa_prefill_topk_workspace_bytes.restype = ctypes.c_int
    lib.qsa_prepare_q.argtypes = [P, i64, i32, i32, P, i64, i64, P, i32, i64, P, i32, f32, P, P, i32, f32,
                                  i64, i64, P]
    lib.qsa_prepare_q.restype = ctypes.c_int
    lib.qsa_decode_visible_blocks.argtypes = [P, i32, i32, P, P, P]
    lib.qsa_decode_visible_blocks.restype = ctypes.c_int
    lib.qsa_mqa_decode_static_plan.argtypes = [P, i32, i64, i64, i64, P, i32, f32, i64, i32, P, i64, i32, P, P,
                                               i32, i32, i32, i32, f32, P, i64, i32, P]
    lib.qsa_mqa_decode_static_plan.restype = ctypes.c_int
    lib.qsa_build_ring_slots.argtypes = [P, P, i32, i32, P, i64, i32, i32, P, P]
    lib.qsa_build_ring_slots.restype = ctypes.c_int
    lib.qsa_write_keys.argtypes = [P, i64, i32, P, P, i32, i64, i64, f32, P, i64, i64, P]
    lib.qsa_write_keys.restype = ctypes.c_int
    lib.qsa_decode_plan_bytes.argtypes = [i32, i32, P]
    lib.qsa_decode_plan_bytes.restype = ctypes.c_int
    lib.qsa_build_decode_plan.argtypes = [P, P, i64, i32, i64, i32, i32, i32, P, i64, P]
    lib.qsa_build_decode_plan.restype = ctypes.c_int
    lib.qsa_mqa_decode_planned.argtypes = [P, i64, P, i32, i64, i64, i64, P, i32, f32, i64, i32, P, i64, i32,
                                           P, i32, i32, i32, i32, f32, P, i64, i32, P]
    lib.qsa_mqa_decode_planned.restype = ctypes.c_int
    if lib.qsa_abi_version() != ABI_VERSION:
        raise RuntimeError(f"libqsa ABI {lib.qsa_abi_version()} != binding ABI {ABI_VERSION}")
    _lib = lib
    return lib


def _check(rc: int) -> None:
    if rc != QSA_OK:
        raise QSAError(rc, _lib.qsa_last_error().decode())


def _stream_handle(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if isinstance(stream, torch.cuda.Stream) else int(stream)


def _gpu(name: str, t: torch.Tensor, dtype: torch.dtype) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device}); there is no CPU path")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _ptr(t: torch.Tensor | None):
    return None if t is None else t.data_ptr()


def _gpu_format(name: str, t: torch.Tensor, allowed) -> int:
    """The enum qsa_dtype of a GPU tensor whose dtype is one of `allowed`."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device}); there is no CPU path")
    if t.dtype not in allowed:
        raise TypeError(f"{name} must be one of {[str(d) for d in allowed]}, got {t.dtype}")
    return _DTYPES[t.dtype]


# ----------------------------------------------------------------------------


def qsa_set_launch_events(start_event: int | None, stop_event: int | None) -> None:
    """Attach caller-owned hipEvent_t handles (as integers) to every kernel the
    library launches from this thread; None, None stops it."""
    _check(load_library().qsa_set_launch_events(start_event, stop_event))


def qsa_split_batch(query_start_loc, decode_threshold: int, reorder: bool = False):
    """Host-side decode/prefill split.  query_start_loc: host int sequence.
    Returns (order list or None, num_decodes, num_decode_tokens, num_prefills,
    num_prefill_tokens, dql)."""
    lib = load_library()
    qsl = (ctypes.c_int32 * len(query_start_loc))(*[int(x) for x in query_start_loc])
    num_reqs = len(query_start_loc) - 1
    order = (ctypes.c_int32 * max(num_reqs, 1))() if reorder else None
    counts = (ctypes.c_int32 * 5)()
    _check(lib.qsa_split_batch(ctypes.addressof(qsl), num_reqs, int(decode_threshold),
                               ctypes.addressof(order) if order is not None else None,
                               ctypes.addressof(counts)))
    return ((list(order[:num_reqs]) if reorder else None),) + tuple(int(c) for c in counts)


def qsa_build_metadata(query_start_loc: torch.Tensor, seq_lens: torch.Tensor, num_tokens: int,
                       compress_ratio: int = 4, key_offsets: torch.Tensor | None = None,
                       stream=None):
    """Per-token metadata on the GPU.  Returns a dict of device tensors:
    token_to_req, positions (int64), visible, comp_lens, and with key_offsets
    row_k_start / row_k_end."""
    lib = load_library()
    _gpu("query_start_loc", query_start_loc, torch.int32)
    _gpu("seq_lens", seq_lens, torch.int32)
    assert query_start_loc.is_contiguous() and seq_lens.is_contiguous()
    num_reqs = seq_lens.numel()
    assert query_start_loc.numel() == num_reqs + 1
    dev = seq_lens.device
    res = {
        "token_to_req": torch.empty(num_tokens, dtype=torch.int32, device=dev),
        "positions": torch.empty(num_tokens, dtype=torch.int64, device=dev),
        "visible": torch.empty(num_tokens, dtype=torch.int32, device=dev),
        "comp_lens": torch.empty(num_reqs, dtype=torch.int32, device=dev),
    }
    if key_offsets is not None:
        _gpu("key_offsets", key_offsets, torch.int32)
        assert key_offsets.is_contiguous() and key_offsets.numel() == num_reqs
        res["row_k_start"] = torch.empty(num_tokens, dtype=torch.int32, device=dev)
        res["row_k_end"] = torch.empty(num_tokens, dtype=torch.int32, device=dev)
    _check(lib.qsa_build_metadata(
        _ptr(query_start_loc), _ptr(seq_lens), num_reqs, int(num_tokens), int(compress_ratio),
        _ptr(key_offsets), _ptr(res["token_to_req"]), _ptr(res["positions"]),
        _ptr(res["visible"]), _ptr(res["comp_lens"]), _ptr(res.get("row_k_start")),
        _ptr(res.get("row_k_end")), _stream_handle(stream)))
    return res


def qsa_decode_visible_blocks(seq_lens: torch.Tensor, dql: int, stream=None):
    """Compressed lengths (int32 [R]) and visible blocks per decode row
    (int32 [R*dql]) of a batch of uniform decodes, on the GPU."""
    lib = load_library()
    _gpu("seq_lens", seq_lens, torch.int32)
    assert seq_lens.is_contiguous()
    num_reqs = seq_lens.numel()
    comp = torch.empty(num_reqs, dtype=torch.int32, device=seq_lens.device)
    vis = torch.empty(num_reqs * int(dql), dtype=torch.int32, device=seq_lens.device)
    _check(lib.qsa_decode_visible_blocks(_ptr(seq_lens), num_reqs, int(dql), _ptr(comp), _ptr(vis),
                                         _stream_handle(stream)))
    return comp, vis


def qsa_mqa_decode(q: torch.Tensor, k_cache: torch.Tensor, page_table: torch.Tensor,
                   comp_lens: torch.Tensor, visible: torch.Tensor | None = None,
                   out_cols: int | None = None, scale: float = DEFAULT_SCALE,
                   out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Decode scores.  q: bf16 [R, DQL, 4, 128] (unit feature stride, any other
    strides); k_cache: bf16 [P, page_size, 1, 128] contiguous; page_table:
    int32 [R, W] (unit column stride); comp_lens: int32 [R]; visible: int32
    [R*DQL] or None.  Returns fp32 [R*DQL, out_cols] (written into `out` if
    given; `out` may be a row-strided view)."""
    lib = load_library()
    _gpu("q", q, torch.bfloat16)
    _gpu("k_cache", k_cache, torch.bfloat16)
    _gpu("page_table", page_table, torch.int32)
    _gpu("comp_lens", comp_lens, torch.int32)
    if q.dim() != 4 or k_cache.dim() != 4 or page_table.dim() != 2:
        raise ValueError("q must be [R, DQL, H, D], k_cache [P, page_size, 1, D], page_table [R, W]")
    num_reqs, dql, heads, dim = q.shape
    if q.stride(3) != 1 and dim > 1:
        raise QSAError(QSA_ERR_LAYOUT, "q needs unit feature stride")
    if k_cache.shape[2] != 1 or k_cache.shape[3] != dim or not k_cache.is_contiguous():
        raise ValueError("k_cache must be a contiguous [P, page_size, 1, 128] tensor")
    if page_table.shape[0] != num_reqs or (page_table.shape[1] > 1 and page_table.stride(1) != 1):
        raise ValueError("page_table must be [R, W] with unit column stride")
    if comp_lens.numel() != num_reqs or not comp_lens.is_contiguous():
        raise ValueError("comp_lens must be a contiguous [R] tensor")
    if visible is not None:
        _gpu("visible", visible, torch.int32)
        if visible.numel() != num_reqs * dql or not visible.is_contiguous():
            raise ValueError("visible must be a contiguous [R*DQL] tensor")
    if out is None:
        if out_cols is None:
            raise ValueError("give out_cols or out")
        out = torch.empty((num_reqs * dql, out_cols), dtype=torch.float32, device=q.device)
    _gpu("out", out, torch.float32)
    if out.dim() != 2 or out.shape[0] != num_reqs * dql or (out.shape[1] > 1 and out.stride(1) != 1):
        raise ValueError("out must be [R*DQL, out_cols] with unit column stride")
    _check(lib.qsa_mqa_decode(
        _ptr(q), q.stride(0), q.stride(1), q.stride(2), _ptr(k_cache), k_cache.shape[0],
        k_cache.shape[1], _ptr(page_table), page_table.stride(0), page_table.shape[1],
        _ptr(comp_lens), _ptr(visible), num_reqs, dql, heads, dim, float(scale), _ptr(out),
        out.stride(0), out.shape[1], _stream_handle(stream)))
    return out


def qsa_mqa_prefill(q: torch.Tensor, k: torch.Tensor, row_k_start: torch.Tensor,
                    row_k_end: torch.Tensor, out_cols: int | None = None,
                    scale: float = DEFAULT_SCALE, out: torch.Tensor | None = None,
                    stream=None) -> torch.Tensor:
    """Prefill scores.  q: bf16 [T, 4, 128]; k: bf16 [NK, 128] (both unit
    feature stride, 16-byte aligned, outer strides multiples of 8); row_k_start,
    row_k_end: int32 [T].  Returns fp32 [T, out_cols]."""
    lib = load_library()
    _gpu("q", q, torch.bfloat16)
    _gpu("k", k, torch.bfloat16)
    _gpu("row_k_start", row_k_start, torch.int32)
    _gpu("row_k_end", row_k_end, torch.int32)
    if q.dim() != 3 or k.dim() != 2:
        raise ValueError("q must be [T, H, D] and k [NK, D]")
    num_rows, heads, dim = q.shape
    if (q.stride(2) != 1 and dim > 1) or (k.stride(1) != 1 and k.shape[1] > 1):
        raise QSAError(QSA_ERR_LAYOUT, "q and k need unit feature stride")
    if k.shape[1] != dim:
        raise ValueError("q and k head_dim differ")
    for name, t in (("row_k_start", row_k_start), ("row_k_end", row_k_end)):
        if t.numel() != num_rows or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [T] tensor")
    if out is None:
        if out_cols is None:
            raise ValueError("give out_cols or out")
        out = torch.empty((num_rows, out_cols), dtype=torch.float32, device=q.device)
    _gpu("out", out, torch.float32)
    if out.dim() != 2 or out.shape[0] != num_rows or (out.shape[1] > 1 and out.stride(1) != 1):
        raise ValueError("out must be [T, out_cols] with unit column stride")
    _check(lib.qsa_mqa_prefill(
        _ptr(q), q.stride(0), q.stride(1), _ptr(k), k.stride(0), k.shape[0], _ptr(row_k_start),
        _ptr(row_k_end), num_rows, heads, dim, float(scale), _ptr(out), out.stride(0),
        out.shape[1], _stream_handle(stream)))
    return out


def qsa_build_cache_metadata(query_start_loc: torch.Tensor, seq_lens: torch.Tensor, num_tokens: int,
                             block_table: torch.Tensor, storage_block_size: int, compress_ratio: int = 4,
                             common_slot_mapping: torch.Tensor | None = None, max_num_work: int = 0,
                             slot_mapping: torch.Tensor | None = None, k_work: torch.Tensor | None = None,
                             stream=None):
    """Compressed-cache slot of each token (int64 [num_tokens], -1 = none) and
    the cache writer's work items (int32 [max_num_work, 2], (-1, -1) past the
    last; None when max_num_work is 0).  block_table: int32 [R, cols] with unit
    column stride."""
    lib = load_library()
    _gpu("query_start_loc", query_start_loc, torch.int32)
    _gpu("seq_lens", seq_lens, torch.int32)
    _gpu("block_table", block_table, torch.int32)
    num_reqs = seq_lens.numel()
    if query_start_loc.numel() != num_reqs + 1 or not query_start_loc.is_contiguous() or not seq_lens.is_contiguous():
        raise ValueError("query_start_loc must be a contiguous [R+1] and seq_lens a contiguous [R] tensor")
    if block_table.dim() != 2 or block_table.shape[0] != num_reqs or (block_table.shape[1] > 1 and block_table.stride(1) != 1):
        raise ValueError("block_table must be [R, cols] with unit column stride")
    dev = query_start_loc.device
    if common_slot_mapping is not None:
        _gpu("common_slot_mapping", common_slot_mapping, torch.int64)
        if common_slot_mapping.numel() < num_tokens or not common_slot_mapping.is_contiguous():
            raise ValueError("common_slot_mapping must be a contiguous [num_tokens] tensor")
    if slot_mapping is None:
        slot_mapping = torch.empty(num_tokens, dtype=torch.int64, device=dev)
    _gpu("slot_mapping", slot_mapping, torch.int64)
    if slot_mapping.numel() < num_tokens or not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be a contiguous [num_tokens] tensor")
    if max_num_work > 0:
        if k_work is None:
            k_work = torch.empty((max_num_work, 2), dtype=torch.int32, device=dev)
        _gpu("k_work", k_work, torch.int32)
        if k_work.numel() < 2 * max_num_work or not k_work.is_contiguous():
            raise ValueError("k_work must be a contiguous [max_num_work, 2] tensor")
    else:
        k_work = None
    _check(lib.qsa_build_cache_metadata(
        _ptr(query_start_loc), _ptr(seq_lens), num_reqs, num_tokens, compress_ratio, _ptr(block_table),
        block_table.stride(0), block_table.shape[1], storage_block_size, _ptr(common_slot_mapping),
        _ptr(slot_mapping), _ptr(k_work), max_num_work if k_work is not None else 0, _stream_handle(stream)))
    return slot_mapping, k_work


def qsa_build_ring_slots(query_start_loc: torch.Tensor, seq_lens: torch.Tensor, num_tokens: int,
                         block_table: torch.Tensor, ring_size: int, stream=None) -> torch.Tensor:
    """int64 [num_tokens]: the raw-key ring slot of each query token, or -1."""
    lib = load_library()
    _gpu("query_start_loc", query_start_loc, torch.int32)
    _gpu("seq_lens", seq_lens, torch.int32)
    _gpu("block_table", block_table, torch.int32)
    assert query_start_loc.is_contiguous() and seq_lens.is_contiguous()
    if block_table.dim() != 2 or (block_table.shape[1] > 1 and block_table.stride(1) != 1):
        raise ValueError("block_table must be [R, W] with unit column stride")
    num_reqs = seq_lens.numel()
    out = torch.empty(int(num_tokens), dtype=torch.int64, device=seq_lens.device)
    _check(lib.qsa_build_ring_slots(_ptr(query_start_loc), _ptr(seq_lens), num_reqs, int(num_tokens),
                                    _ptr(block_table), block_table.stride(0), block_table.shape[1], int(ring_size),
                                    _ptr(out), _stream_handle(stream)))
    return out


def qsa_write_keys(keys: torch.Tensor, slots: torch.Tensor, cache: torch.Tensor, scale: float = 1.0,
                   positions: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Write bf16 key rows [T, >=128] to the rows of `cache` ([..., W]: bf16,
    or float8_e4m3fn for an e4m3 cache; contiguous) named by int64 slots [T];
    positions: int64 [3, T] (bf16 caches with W >= 140) or None.  In place;
    returns cache."""
    lib = load_library()
    _gpu("keys", keys, torch.bfloat16)
    _gpu("slots", slots, torch.int64)
    fmt = _gpu_format("cache", cache, (torch.bfloat16, torch.float8_e4m3fn))
    if keys.dim() != 2 or keys.stride(1) != 1 or not slots.is_contiguous() or slots.numel() != keys.shape[0]:
        raise ValueError("keys must be [T, >=128] with unit feature stride and slots a contiguous [T] tensor")
    if not cache.is_contiguous():
        raise ValueError("cache must be contiguous")
    width = cache.shape[-1]
    pa, pt = 0, 0
    if positions is not None:
        _gpu("positions", positions, torch.int64)
        if positions.dim() != 2 or positions.shape != (3, keys.shape[0]):
            raise ValueError("positions must be [3, T]")
        pa, pt = positions.stride(0), positions.stride(1)
    _check(lib.qsa_write_keys(_ptr(keys), keys.stride(0), keys.shape[0], _ptr(slots), _ptr(cache), fmt, width,
                              cache.numel() // max(width, 1), float(scale), _ptr(positions), pa, pt,
                              _stream_handle(stream)))
    return cache


def qsa_gather_keys(k_cache: torch.Tensor, page_table: torch.Tensor, key_counts: torch.Tensor,
                    key_offsets: torch.Tensor, max_keys: int, out: torch.Tensor | None = None,
                    out_rows: int | None = None, stream=None) -> torch.Tensor:
    """Request r's compressed keys 0 .. key_counts[r]-1 from the paged cache
    (bf16, fp16 or float8_e4m3fn [P, page_size, 1, 128], contiguous) into rows
    key_offsets[r] .. of `out` ([rows, 128], unit feature stride; the cache's
    dtype, or bf16/fp16 for an e4m3 cache, whose codes are then widened
    exactly); a missing page gives a zero row."""
    lib = load_library()
    fmt = _gpu_format("k_cache", k_cache, (torch.bfloat16, torch.float16, torch.float8_e4m3fn))
    _gpu("page_table", page_table, torch.int32)
    _gpu("key_counts", key_counts, torch.int32)
    _gpu("key_offsets", key_offsets, torch.int32)
    if k_cache.dim() != 4 or k_cache.shape[2] != 1 or k_cache.shape[3] != 128 or not k_cache.is_contiguous():
        raise ValueError("k_cache must be a contiguous [P, page_size, 1, 128] tensor")
    num_reqs = key_counts.numel()
    if page_table.dim() != 2 or page_table.shape[0] != num_reqs or (page_table.shape[1] > 1 and page_table.stride(1) != 1):
        raise ValueError("page_table must be [R, W] with unit column stride")
    if key_offsets.numel() != num_reqs or not key_offsets.is_contiguous() or not key_counts.is_contiguous():
        raise ValueError("key_counts and key_offsets must be contiguous [R] tensors")
    if out is None:
        if out_rows is None:
            raise ValueError("give out_rows or out")
        out = torch.zeros((out_rows, 128), dtype=k_cache.dtype, device=k_cache.device)
    widen_ok = k_cache.dtype == torch.float8_e4m3fn and out.dtype in (torch.bfloat16, torch.float16)
    if (out.dtype != k_cache.dtype and not widen_ok) or out.dim() != 2 or out.shape[1] != 128 or out.stride(1) != 1:
        raise ValueError("out must be a [rows, 128] tensor of k_cache's dtype (or bf16/fp16 for an e4m3 cache) "
                         "with unit feature stride")
    _check(lib.qsa_gather_keys(
        _ptr(k_cache), fmt, k_cache.shape[0], k_cache.shape[1], _ptr(page_table), page_table.stride(0),
        page_table.shape[1], _ptr(key_counts), _ptr(key_offsets), num_reqs, int(max_keys), _ptr(out),
        _DTYPES[out.dtype], out.stride(0), out.shape[0], _stream_handle(stream)))
    return out


def qsa_mqa_decode_typed(q: torch.Tensor, k_cache: torch.Tensor, page_table: torch.Tensor,
                         comp_lens: torch.Tensor, visible: torch.Tensor | None = None,
                         out_cols: int | None = None, k_scale: float = 1.0,
                         scale: float = DEFAULT_SCALE, out: torch.Tensor | None = None,
                         stream=None) -> torch.Tensor:
    """qsa_mqa_decode with typed elements: q bf16 or fp16; k_cache the same
    dtype as q, or float8_e4m3fn (an e4m3 cache whose elements stand for their
    value times k_scale).  Shapes and the rest as qsa_mqa_decode."""
    lib = load_library()
    q_fmt = _gpu_format("q", q, (torch.bfloat16, torch.float16))
    k_fmt = _gpu_format("k_cache", k_cache, (torch.bfloat16, torch.float16, torch.float8_e4m3fn))
    _gpu("page_table", page_table, torch.int32)
    _gpu("comp_lens", comp_lens, torch.int32)
    if q.dim() != 4 or k_cache.dim() != 4 or page_table.dim() != 2:
        raise ValueError("q must be [R, DQL, H, D], k_cache [P, page_size, 1, D], page_table [R, W]")
    num_reqs, dql, heads, dim = q.shape
    if q.stride(3) != 1 and dim > 1:
        raise QSAError(QSA_ERR_LAYOUT, "q needs unit feature stride")
    if k_cache.shape[2] != 1 or k_cache.shape[3] != dim or not k_cache.is_contiguous():
        raise ValueError("k_cache must be a contiguous [P, page_size, 1, 128] tensor")
    if page_table.shape[0] != num_reqs or (page_table.shape[1] > 1 and page_table.stride(1) != 1):
        raise ValueError("page_table must be [R, W] with unit column stride")
    if comp_lens.numel() != num_reqs or not comp_lens.is_contiguous():
        raise ValueError("comp_lens must be a contiguous [R] tensor")
    if visible is not None:
        _gpu("visible", visible, torch.int32)
        if visible.numel() != num_reqs * dql or not visible.is_contiguous():
            raise ValueError("visible must be a contiguous [R*DQL] tensor")
    if out is None:
        if out_cols is None:
            raise ValueError("give out_cols or out")
        out = torch.empty((num_reqs * dql, out_cols), dtype=torch.float32, device=q.device)
    _gpu("out", out, torch.float32)
    if out.dim() != 2 or out.shape[0] != num_reqs * dql or (out.shape[1] > 1 and out.stride(1) != 1):
        raise ValueError("out must be [R*DQL, out_cols] with unit column stride")
    _check(lib.qsa_mqa_decode_typed(
        _ptr(q), q_fmt, q.stride(0), q.stride(1), q.stride(2), _ptr(k_cache), k_fmt, float(k_scale),
        k_cache.shape[0], k_cache.shape[1], _ptr(page_table), page_table.stride(0), page_table.shape[1],
        _ptr(comp_lens), _ptr(visible), num_reqs, dql, heads, dim, float(scale), _ptr(out),
        out.stride(0), out.shape[1], _stream_handle(stream)))
    return out


def qsa_mqa_decode_static_plan(q: torch.Tensor, k_cache: torch.Tensor, page_table: torch.Tensor,
                               comp_lens: torch.Tensor, visible: torch.Tensor | None = None,
                               out_cols: int | None = None, k_scale: float = 1.0,
                               scale: float = DEFAULT_SCALE, out: torch.Tensor | None = None,
                               stream=None) -> torch.Tensor:
    """The planned decode with the task table in the library's own device
    memory (no allocation inside the call).  Arguments as
    qsa_mqa_decode_typed; pass `out` to keep the call itself free of
    allocations."""
    lib = load_library()
    q_fmt = _gpu_format("q", q, (torch.bfloat16, torch.float16))
    k_fmt = _gpu_format("k_cache", k_cache, (torch.bfloat16, torch.float16, torch.float8_e4m3fn))
    _gpu("page_table", page_table, torch.int32)
    _gpu("comp_lens", comp_lens, torch.int32)
    if q.dim() != 4 or k_cache.dim() != 4 or page_table.dim() != 2:
        raise ValueError("q must be [R, DQL, H, D], k_cache [P, page_size, 1, D], page_table [R, W]")
    num_reqs, dql, heads, dim = q.shape
    if q.stride(3) != 1 and dim > 1:
        raise QSAError(QSA_ERR_LAYOUT, "q needs unit feature stride")
    if k_cache.shape[2] != 1 or k_cache.shape[3] != dim or not k_cache.is_contiguous():
        raise ValueError("k_cache must be a contiguous [P, page_size, 1, 128] tensor")
    if page_table.shape[0] != num_reqs or (page_table.shape[1] > 1 and page_table.stride(1) != 1):
        raise ValueError("page_table must be [R, W] with unit column stride")
    if comp_lens.numel() != num_reqs or not comp_lens.is_contiguous():
        raise ValueError("comp_lens must be a contiguous [R] tensor")
    if visible is not None:
        _gpu("visible", visible, torch.int32)
        if visible.numel() != num_reqs * dql or not visible.is_contiguous():
            raise ValueError("visible must be a contiguous [R*DQL] tensor")
    if out is None:
        if out_cols is None:
            raise ValueError("give out_cols or out")
        out = torch.empty((num_reqs * dql, out_cols), dtype=torch.float32, device=q.device)
    _gpu("out", out, torch.float32)
    if out.dim() != 2 or out.shape[0] != num_reqs * dql or (out.shape[1] > 1 and out.stride(1) != 1):
        raise ValueError("out must be [R*DQL, out_cols] with unit column stride")
    _check(lib.qsa_mqa_decode_static_plan(
        _ptr(q), q_fmt, q.stride(0), q.stride(1), q.stride(2), _ptr(k_cache), k_fmt, float(k_scale),
        k_cache.shape[0], k_cache.shape[1], _ptr(page_table), page_table.stride(0), page_table.shape[1],
        _ptr(comp_lens), _ptr(visible), num_reqs, dql, heads, dim, float(scale), _ptr(out),
        out.stride(0), out.shape[1], _stream_handle(stream)))
    return out


def qsa_decode_plan_bytes(num_reqs: int, out_cols: int) -> int:
    """Bytes of the decode task table for num_reqs requests x out_cols columns."""
    n = ctypes.c_int64(0)
    _check(load_library().qsa_decode_plan_bytes(int(num_reqs), int(out_cols), ctypes.byref(n)))
    return int(n.value)


def qsa_build_decode_plan(comp_lens: torch.Tensor, page_table: torch.Tensor, num_pages: int, page_size: int,
                          out_cols: int, plan: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Decode task table (uint8 device tensor of qsa_decode_plan_bytes bytes,
    written into `plan` if given) for comp_lens int32 [R] and page_table int32
    [R, W] (unit column stride)."""
    lib = load_library()
    _gpu("comp_lens", comp_lens, torch.int32)
    _gpu("page_table", page_table, torch.int32)
    if page_table.dim() != 2 or (page_table.shape[1] > 1 and page_table.stride(1) != 1):
        raise ValueError("page_table must be [R, W] with unit column stride")
    num_reqs = comp_lens.numel()
    if page_table.shape[0] != num_reqs or not comp_lens.is_contiguous():
        raise ValueError("comp_lens must be a contiguous [R] tensor and page_table [R, W]")
    nbytes = qsa_decode_plan_bytes(num_reqs, out_cols)
    if plan is None:
        plan = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=comp_lens.device)
    _gpu("plan", plan, torch.uint8)
    _check(lib.qsa_build_decode_plan(
        _ptr(comp_lens), _ptr(page_table), page_table.stride(0), page_table.shape[1], int(num_pages),
        int(page_size), num_reqs, int(out_cols), _ptr(plan), plan.numel(), _stream_handle(stream)))
    return plan


def qsa_mqa_decode_planned(plan: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor,
                           page_table: torch.Tensor | None, visible: torch.Tensor | None = None,
                           out_cols: int | None = None, k_scale: float = 1.0,
                           scale: float = DEFAULT_SCALE, out: torch.Tensor | None = None,
                           stream=None) -> torch.Tensor:
    """qsa_mqa_decode_typed driven by a task table from qsa_build_decode_plan
    (built for the same requests, columns, page table and lengths).  The
    page table is read only for page sizes that are not multiples of 64."""
    lib = load_library()
    _gpu("plan", plan, torch.uint8)
    q_fmt = _gpu_format("q", q, (torch.bfloat16, torch.float16))
    k_fmt = _gpu_format("k_cache", k_cache, (torch.bfloat16, torch.float16, torch.float8_e4m3fn))
    if q.dim() != 4 or k_cache.dim() != 4:
        raise ValueError("q must be [R, DQL, H, D], k_cache [P, page_size, 1, D]")
    num_reqs, dql, heads, dim = q.shape
    if q.stride(3) != 1 and dim > 1:
        raise QSAError(QSA_ERR_LAYOUT, "q needs unit feature stride")
    if k_cache.shape[2] != 1 or k_cache.shape[3] != dim or not k_cache.is_contiguous():
        raise ValueError("k_cache must be a contiguous [P, page_size, 1, 128] tensor")
    pt_stride, pt_cols = 0, 0
    if page_table is not None:
        _gpu("page_table", page_table, torch.int32)
        if page_table.dim() != 2 or page_table.shape[0] != num_reqs or (
                page_table.shape[1] > 1 and page_table.stride(1) != 1):
            raise ValueError("page_table must be [R, W] with unit column stride")
        pt_stride, pt_cols = page_table.stride(0), page_table.shape[1]
    if visible is not None:
        _gpu("visible", visible, torch.int32)
        if visible.numel() != num_reqs * dql or not visible.is_contiguous():
            raise ValueError("visible must be a contiguous [R*DQL] tensor")
    if out is None:
        if out_cols is None:
            raise ValueError("give out_cols or out")
        out = torch.empty((num_reqs * dql, out_cols), dtype=torch.float32, device=q.device)
    _gpu("out", out, torch.float32)
    if out.dim() != 2 or out.shape[0] != num_reqs * dql or (out.shape[1] > 1 and out.stride(1) != 1):
        raise ValueError("out must be [R*DQL, out_cols] with unit column stride")
    _check(lib.qsa_mqa_decode_planned(
        _ptr(plan), plan.numel(), _ptr(q), q_fmt, q.stride(0), q.stride(1), q.stride(2), _ptr(k_cache), k_fmt,
        float(k_scale), k_cache.shape[0], k_cache.shape[1], _ptr(page_table), pt_stride, pt_cols, _ptr(visible),
        num_reqs, dql, heads, dim, float(scale), _ptr(out), out.stride(0), out.shape[1], _stream_handle(stream)))
    return out


def qsa_mqa_prefill_typed(q: torch.Tensor, k: torch.Tensor, row_k_start: torch.Tensor,
                          row_k_end: torch.Tensor, out_cols: int | None = None,
                          scale: float = DEFAULT_SCALE, out: torch.Tensor | None = None,
                          stream=None) -> torch.Tensor:
    """qsa_mqa_prefill with q and k both bf16 or both fp16."""
    lib = load_library()
    fmt = _gpu_format("q", q, (torch.bfloat16, torch.float16))
    if _gpu_format("k", k, (torch.bfloat16, torch.float16)) != fmt:
        raise TypeError("q and k must share their dtype")
    _gpu("row_k_start", row_k_start, torch.int32)
    _gpu("row_k_end", row_k_end, torch.int32)
    if q.dim() != 3 or k.dim() != 2:
        raise ValueError("q must be [T, H, D] and k [NK, D]")
    num_rows, heads, dim = q.shape
    if (q.stride(2) != 1 and dim > 1) or (k.stride(1) != 1 and k.shape[1] > 1):
        raise QSAError(QSA_ERR_LAYOUT, "q and k need unit feature stride")
    if k.shape[1] != dim:
        raise ValueError("q and k head_dim differ")
    for name, t in (("row_k_start", row_k_start), ("row_k_end", row_k_end)):
        if t.numel() != num_rows or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [T] tensor")
    if out is None:
        if out_cols is None:
            raise ValueError("give out_cols or out")
        out = torch.empty((num_rows, out_cols), dtype=torch.float32, device=q.device)
    _gpu("out", out, torch.float32)
    if out.dim() != 2 or out.shape[0] != num_rows or (out.shape[1] > 1 and out.stride(1) != 1):
        raise ValueError("out must be [T, out_cols] with unit column stride")
    _check(lib.qsa_mqa_prefill_typed(
        _ptr(q), q.stride(0), q.stride(1), _ptr(k), k.stride(0), k.shape[0], fmt, _ptr(row_k_start),
        _ptr(row_k_end), num_rows, heads, dim, float(scale), _ptr(out), out.stride(0),
        out.shape[1], _stream_handle(stream)))
    return out


def qsa_topk_blocks(logits: torch.Tensor, k: int, out: torch.Tensor | None = None,
                    stream=None) -> torch.Tensor:
    """Per-row top-k column indices of fp32 logits [T, C]: int32 [T, k],
    ascending, -1 padded."""
    lib = load_library()
    _gpu("logits", logits, torch.float32)
    if logits.dim() != 2 or (logits.shape[1] > 1 and logits.stride(1) != 1):
        raise ValueError("logits must be [T, C] with unit column stride")
    rows, cols = logits.shape
    if out is None:
        out = torch.empty((rows, k), dtype=torch.int32, device=logits.device)
    _gpu("out", out, torch.int32)
    if out.dim() != 2 or out.shape[0] != rows or out.shape[1] != k or (k > 1 and out.stride(1) != 1):
        raise ValueError("out must be [T, k] with unit column stride")
    _check(lib.qsa_topk_blocks(_ptr(logits), logits.stride(0), rows, cols, int(k), _ptr(out),
                               out.stride(0), _stream_handle(stream)))
    return out


def qsa_prefill_topk_workspace_bytes(num_rows: int, out_cols: int, topk: int) -> int:
    """Workspace bytes qsa_mqa_prefill_topk needs on the current device."""
    lib = load_library()
    n = ctypes.c_int64(0)
    _check(lib.qsa_prefill_topk_workspace_bytes(int(num_rows), int(out_cols), int(topk), ctypes.byref(n)))
    return int(n.value)


def qsa_mqa_prefill_topk(q: torch.Tensor, k: torch.Tensor, row_k_start: torch.Tensor,
                         row_k_end: torch.Tensor, out_cols: int, topk: int,
                         scale: float = DEFAULT_SCALE, out: torch.Tensor | None = None,
                         workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Prefill scores and per-row top-k in one call, without the score matrix:
    int32 [T, topk], equal to qsa_topk_blocks(qsa_mqa_prefill(...), topk)
    (qsa_mqa_prefill_typed for fp16 q and k).  workspace: uint8 device tensor
    of at least qsa_prefill_topk_workspace_bytes bytes (allocated here when
    not given)."""
    lib = load_library()
    fmt = _gpu_format("q", q, (torch.bfloat16, torch.float16))
    if _gpu_format("k", k, (torch.bfloat16, torch.float16)) != fmt:
        raise TypeError("q and k must share their dtype")
    _gpu("row_k_start", row_k_start, torch.int32)
    _gpu("row_k_end", row_k_end, torch.int32)
    if q.dim() != 3 or k.dim() != 2:
        raise ValueError("q must be [T, H, D] and k [NK, D]")
    num_rows, heads, dim = q.shape
    if (q.stride(2) != 1 and dim > 1) or (k.stride(1) != 1 and k.shape[1] > 1):
        raise QSAError(QSA_ERR_LAYOUT, "q and k need unit feature stride")
    if k.shape[1] != dim:
        raise ValueError("q and k head_dim differ")
    for name, t in (("row_k_start", row_k_start), ("row_k_end", row_k_end)):
        if t.numel() != num_rows or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [T] tensor")
    if out is None:
        out = torch.empty((num_rows, topk), dtype=torch.int32, device=q.device)
    _gpu("out", out, torch.int32)
    if out.dim() != 2 or out.shape[0] != num_rows or out.shape[1] != topk or (topk > 1 and out.stride(1) != 1):
        raise ValueError("out must be [T, topk] with unit column stride")
    need = qsa_prefill_topk_workspace_bytes(num_rows, out_cols, topk)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _gpu("workspace", workspace, torch.uint8)
    args = (_ptr(row_k_start), _ptr(row_k_end), num_rows, heads, dim, float(scale), int(out_cols), int(topk),
            _ptr(out), out.stride(0), _ptr(workspace), workspace.numel(), _stream_handle(stream))
    if fmt == QSA_DTYPE_BF16:
        _check(lib.qsa_mqa_prefill_topk(_ptr(q), q.stride(0), q.stride(1), _ptr(k), k.stride(0), k.shape[0], *args))
    else:
        _check(lib.qsa_mqa_prefill_topk_typed(_ptr(q), q.stride(0), q.stride(1), _ptr(k), k.stride(0),
                                              k.shape[0], fmt, *args))
    return out


def qsa_prepare_q(q: torch.Tensor, positions: torch.Tensor, cos_sin: torch.Tensor, norm_weight: torch.Tensor,
                  eps: float, mrope_section=None, out: torch.Tensor | None = None,
                  out_dtype: torch.dtype = torch.bfloat16, out_scale: float = 1.0, stream=None) -> torch.Tensor:
    """Gemma RMSNorm and NeoX rotary embedding of the indexer's query heads
    (qsa_prepare_q in include/qsa.h).  q: bf16 [T, H*128] or [T, H, 128]
    with contiguous heads; positions: int64 [T], or [3, T] (temporal, height,
    width) with mrope_section (t, h, w) summing to 32; cos_sin: bf16 or fp32
    [rows, 64] (32 cos, then 32 sin); norm_weight: bf16 or fp32 [128].
    Returns (or fills) out [T, H, 128] of bf16, or of float8_e4m3fn holding
    the bf16 result divided by out_scale."""
    lib = load_library()
    _gpu("q", q, torch.bfloat16)
    _gpu("positions", positions, torch.int64)
    cs_fmt = _gpu_format("cos_sin", cos_sin, (torch.bfloat16, torch.float32))
    w_fmt = _gpu_format("norm_weight", norm_weight, (torch.bfloat16, torch.float32))
    T = q.shape[0]
    if q.dim() == 3:
        if q.shape[2] != 128 or q.stride(2) != 1 or q.stride(1) != 128:
            raise ValueError("q [T, H, 128] needs contiguous heads")
        H = q.shape[1]
    elif q.dim() == 2 and q.shape[1] % 128 == 0 and q.stride(1) == 1:
        H = q.shape[1] // 128
    else:
        raise ValueError("q must be [T, H*128] or [T, H, 128] with contiguous heads")
    if positions.dim() == 1:
        if positions.shape[0] != T:
            raise ValueError("positions must be [T] or [3, T]")
        pos_axis, pos_tok = 0, positions.stride(0)
    elif positions.dim() == 2 and positions.shape == (3, T):
        if mrope_section is None:
            raise ValueError("[3, T] positions need an mrope_section")
        pos_axis, pos_tok = positions.stride(0), positions.stride(1)
    else:
        raise ValueError("positions must be [T] or [3, T]")
    if cos_sin.dim() != 2 or cos_sin.shape[1] != 64 or not cos_sin.is_contiguous():
        raise ValueError("cos_sin must be a contiguous [rows, 64] tensor")
    if norm_weight.numel() != 128 or not norm_weight.is_contiguous():
        raise ValueError("norm_weight must be a contiguous [128] tensor")
    if out is None:
        out = torch.empty((T, H, 128), dtype=out_dtype, device=q.device)
    out_fmt = _gpu_format("out", out, (torch.bfloat16, torch.float8_e4m3fn))
    if out.dim() != 3 or out.shape != (T, H, 128) or out.stride(2) != 1:
        raise ValueError("out must be [T, H, 128] with unit feature stride")
    sec = None
    if mrope_section is not None:
        sec = (ctypes.c_int32 * 3)(*[int(v) for v in mrope_section])
    _check(lib.qsa_prepare_q(
        _ptr(q), q.stride(0), T, H, _ptr(positions), pos_axis, pos_tok, _ptr(cos_sin), cs_fmt, cos_sin.shape[0],
        _ptr(norm_weight), w_fmt, float(eps), None if sec is None else ctypes.addressof(sec), _ptr(out), out_fmt,
        float(out_scale), out.stride(0), out.stride(1), _stream_handle(stream)))
    return out
