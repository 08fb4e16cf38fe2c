"""MI355X (gfx950) QSA lightweight MQA indexer: paged decode scores, packed
prefill scores, per-row top-k block selection, fused prefill top-k and
per-step metadata, as HIP kernels behind the C ABI in include/qsa.h
(libqsa.so).  Queries and keys are bf16 or fp16; decode also reads an fp8
e4m3 key cache.  The query heads' RMSNorm and rotary embedding (qsa_prepare_q)
precede scoring.  PyTorch supplies device memory and streams only."""
from .qsa import (DEFAULT_SCALE, QSA_DTYPE_BF16, QSA_DTYPE_FP16, QSA_DTYPE_FP8_E4M3, QSA_DTYPE_FP32, QSAError,
                  load_library, qsa_build_cache_metadata, qsa_build_decode_plan, qsa_build_metadata, qsa_build_ring_slots,
                  qsa_decode_plan_bytes, qsa_decode_visible_blocks, qsa_gather_keys, qsa_mqa_decode, qsa_mqa_decode_planned, qsa_mqa_decode_static_plan,
                  qsa_mqa_decode_typed,
                  qsa_mqa_prefill, qsa_mqa_prefill_topk, qsa_mqa_prefill_typed,
                  qsa_prefill_topk_workspace_bytes, qsa_prepare_q, qsa_set_launch_events, qsa_split_batch,
                  qsa_topk_blocks, qsa_write_keys)

__all__ = ["DEFAULT_SCALE", "QSA_DTYPE_BF16", "QSA_DTYPE_FP16", "QSA_DTYPE_FP8_E4M3", "QSA_DTYPE_FP32", "QSAError",
           "load_library", "qsa_build_cache_metadata", "qsa_build_decode_plan", "qsa_build_metadata", "qsa_build_ring_slots",
           "qsa_decode_plan_bytes", "qsa_decode_visible_blocks", "qsa_gather_keys", "qsa_mqa_decode", "qsa_mqa_decode_planned", "qsa_mqa_decode_static_plan",
           "qsa_mqa_decode_typed",
           "qsa_mqa_prefill", "qsa_mqa_prefill_topk", "qsa_mqa_prefill_typed",
           "qsa_prefill_topk_workspace_bytes", "qsa_prepare_q", "qsa_set_launch_events", "qsa_split_batch",
           "qsa_topk_blocks", "qsa_write_keys"]
