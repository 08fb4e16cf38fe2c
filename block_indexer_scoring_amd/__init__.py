"""MI355X (gfx950) QSA lightweight MQA indexer: paged decode scores, packed
prefill scores, per-row top-k block selection, fused prefill top-k and
per-step metadata, as HIP kernels behind the C ABI in include/qsa.h
(libqsa.so).  PyTorch supplies device memory and streams only."""
from .qsa import (DEFAULT_SCALE, QSAError, load_library, qsa_build_metadata, qsa_mqa_decode,
                  qsa_mqa_prefill, qsa_mqa_prefill_topk, qsa_prefill_topk_workspace_bytes,
                  qsa_set_launch_events, qsa_split_batch, qsa_topk_blocks)

__all__ = ["DEFAULT_SCALE", "QSAError", "load_library", "qsa_build_metadata", "qsa_mqa_decode",
           "qsa_mqa_prefill", "qsa_mqa_prefill_topk", "qsa_prefill_topk_workspace_bytes",
           "qsa_set_launch_events", "qsa_split_batch", "qsa_topk_blocks"]
