"""Benchmark of the QSA MQA indexer hot path on one MI355X.

One step = one pass of the whole path over one mixed batch, as a serving step
would run it (decodes first, then prefills):
  1. qsa_build_metadata  per-token request, position, visible blocks, key
                         intervals for all 8,256 query tokens of the batch;
  2. qsa_build_decode_plan  the decode task table of the step (built once
                         per step and shared by every layer's decode);
  3. qsa_mqa_decode_planned  16 requests x DQL 4, log-normal contexts
                         3,508 / 51,200 / 102,400 tokens (min/mean/max),
                         page_size 64, keys read through the page table;
  4. qsa_mqa_prefill     1 request: 8,192 query tokens over a 100,000-token
                         prefix (27,048 compressed keys);
  5. qsa_topk_blocks     top-512 blocks of every decode row and every
                         prefill row.
Inputs are resident in HBM before timing.  The decode key cache rotates over
several independently generated pools (more bytes than the 256 MB Infinity
Cache), so every decode launch streams its keys from HBM.

Headline `value`: decode throughput in GB/s with the pages' accounting
(unique bf16 keys + bf16 queries + fp32 logits of visible blocks), from the
decode kernel's average duration.  Each kernel is timed by HIP events that
the library attaches to its launch (qsa_set_launch_events), which mark the
kernel's own begin and end on the stream it runs on.  Prefill is reported in
TFLOP/s (2*4*128 FLOPs per visible block per row, the pages' figure) and
against HBM (the score matrix it writes), which is the tighter bound at this
shape; top-k in GB/s (logits read + indices written).

Work accounting follows vLLM PR 54513 ("Separate prefill and decode paths for
QSA indexer", section "Microbenchmarks"); tests/test_bench_accounting.py pins
these formulas to the GB/s and TFLOP/s printed there.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode GB/s (% HBM peak) @16 req ~51K ctx; prefill TFLOP/s (% MFMA peak) 1x8K"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
PAGES_DECODE_GBPS = 3374.0      # GB300, 16 req x DQL 4, 3,508/51,200/102,400 (PR 54513)
HEAD_DIM = 128
HEADS = 4


# ----------------------------------------------------------------------------
# Work accounting (the pages' convention)


def decode_bytes(num_reqs: int, dql: int, comp_total: float) -> float:
    """Unique bf16 keys (read once per request) + bf16 queries + fp32 logits of
    the visible blocks.  comp_total = sum over requests of compressed keys."""
    keys = comp_total * HEAD_DIM * 2
    queries = num_reqs * dql * HEADS * HEAD_DIM * 2
    logits = dql * comp_total * 4
    return keys + queries + logits


def prefill_flops(visible_total: int) -> float:
    """2 * heads * head_dim FLOPs per visible (row, block) pair."""
    return 2.0 * HEADS * HEAD_DIM * visible_total


def prefill_bytes(rows: int, cols: int, num_keys: int) -> float:
    """fp32 score matrix written + bf16 queries + bf16 keys read once."""
    return rows * cols * 4.0 + rows * HEADS * HEAD_DIM * 2.0 + num_keys * HEAD_DIM * 2.0


def topk_bytes(rows: int, cols: int, k: int) -> float:
    """fp32 logits read + int32 indices written."""
    return rows * cols * 4.0 + rows * k * 4.0


# ----------------------------------------------------------------------------


def prepare_bytes(tokens: int, heads: int) -> float:
    """Algorithmic HBM bytes of qsa_prepare_q with bf16 input, table, weight
    and output: each (token, head) row read and written once (256 + 256 B),
    each token's table row (64 bf16) and position (int64) read once, the
    weight once."""
    return tokens * heads * 512.0 + tokens * (128.0 + 8.0) + 256.0


def source_digest(kernel_file: str) -> str:
    """First 16 hex digits of the SHA-256 of a kernel's source file followed
    by the device and launch headers it includes."""
    csrc = os.path.join(ROOT, "block_indexer_scoring_amd", "csrc")
    h = hashlib.sha256()
    for name in (kernel_file, "qsa_device.h", "qsa_internal.h"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(kernel_file: str, kernel: str):
    """HBM traffic per launch from a committed rocprofv3 PMC summary, or None
    when no summary exists or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"pmc_traffic_{kernel}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                vals[key.strip()] = val.strip()
    if vals.get("source_sha256_16") != source_digest(kernel_file):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class HipEvents:
    """Raw hipEvent_t handles for per-kernel timing.  The library attaches a
    (start, stop) pair to its next launch (qsa_set_launch_events, which
    launches through hipExtLaunchKernel), so the runtime marks the kernel's
    own begin and end: the same interval a kernel trace reports, without the
    dispatch latency of an event pair recorded on the stream around the call."""

    def __init__(self, count: int):
        import ctypes
        path = next((ln.split()[-1] for ln in open("/proc/self/maps") if "libamdhip64" in ln), None)
        if path is None:
            raise RuntimeError("the HIP runtime is not loaded in this process")
        hip = ctypes.CDLL(path)
        hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                            ctypes.c_void_p]
        hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip, self.ct = hip, ctypes
        self.ev = []
        for _ in range(count):
            h = ctypes.c_void_p()
            self._check(hip.hipEventCreate(ctypes.byref(h)), "hipEventCreate")
            self.ev.append(h.value)

    def _check(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed with HIP error {rc}")

    def elapsed_us(self, i: int, j: int) -> float:
        ms = self.ct.c_float()
        self._check(self.hip.hipEventElapsedTime(self.ct.byref(ms), self.ev[i], self.ev[j]),
                    "hipEventElapsedTime")
        return ms.value * 1e3

    def close(self):
        for h in self.ev:
            self.hip.hipEventDestroy(h)
        self.ev = []


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(dec_inp, dec_vis, pre_inp, pre_ks, pre_ke, min_cpu_seconds: float = 12.0,
                 max_passes: int = 64):
    """The oracle, as it stands, on this host's cores.

    Headline (value): full decode passes over the spec-decode batch on all
    the host's threads until about min_cpu_seconds of CPU work (wall x
    threads) have run, in GB/s under the pages' accounting.  Also: one decode
    pass on one thread, and the oracle prefill on a fixed subset of the
    1x8K-over-100K rows (GFLOP/s, 2*4*128 FLOP per visible block) on all
    threads and on one thread."""
    import numpy as np

    from oracle import oracle as O
    threads = O._threads(None)
    comp = O.comp_lens(dec_inp.seq_lens)

    def decode_pass(n_threads):
        t0 = time.perf_counter()
        O.decode(dec_inp.q, dec_inp.k_pool, dec_inp.page_table, comp, dec_vis, dec_inp.out_cols,
                 threads=n_threads)
        return time.perf_counter() - t0

    passes, wall = 0, 0.0
    while passes < max_passes and wall * threads < min_cpu_seconds:
        wall += decode_pass(threads)
        passes += 1
    nbytes = decode_bytes(dec_inp.num_reqs, dec_inp.dql, float(comp.sum()))
    one_wall = decode_pass(1)

    T = pre_inp.q.shape[0]
    rows_all = np.linspace(0, T - 1, 128).astype(np.int64)   # 128 rows spread over the chunk
    rows_one = rows_all[::8]                                 # 16 of them on one thread

    def prefill_rate(rows, n_threads):
        t0 = time.perf_counter()
        O.prefill(pre_inp.q, pre_inp.k, pre_ks, pre_ke, pre_inp.out_cols, rows=rows, threads=n_threads)
        dt = time.perf_counter() - t0
        vis = float(np.maximum(pre_ke[rows].astype(np.int64) - pre_ks[rows], 0).sum())
        return prefill_flops(vis) / dt / 1e9, dt

    pf_all, pf_all_s = prefill_rate(rows_all, threads)
    pf_one, pf_one_s = prefill_rate(rows_one, 1)
    return {
        "value": round(nbytes / (wall / passes) / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{passes} full pass(es) of the oracle decode over the 16-request DQL-4 batch "
                  f"(64 rows x {dec_inp.out_cols} columns, {int(comp.sum())} keys), "
                  f"{wall:.2f} s wall on {threads} threads",
        "cpu_model": cpu_model(),
        "decode_1_thread": {"value": round(nbytes / one_wall / 1e9, 4), "unit": "GB/s", "cores": 1,
                            "sample": f"1 full pass, {one_wall:.2f} s wall"},
        "prefill_all_threads": {"value": round(pf_all, 3), "unit": "GFLOP/s", "cores": threads,
                                "sample": f"oracle prefill on 128 of the {T} rows of the 1x8K-over-100K chunk "
                                          f"(every {T // 128}th), {pf_all_s:.2f} s wall"},
        "prefill_1_thread": {"value": round(pf_one, 3), "unit": "GFLOP/s", "cores": 1,
                             "sample": f"16 of those rows, {pf_one_s:.2f} s wall"},
    }


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--pools", type=int, default=8, help="decode key pools rotated across steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--lib", default=None, help="load this libqsa.so instead of the in-tree build")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (PMC calibration)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only (got --gpus {args.gpus}); "
              "the indexer path has no multi-GPU mode.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import block_indexer_scoring_amd as qsa
    from workloads import WORKLOADS, decode_inputs

    lib = qsa.load_library(args.lib) if args.lib else qsa.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    def to_i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    # --- inputs -------------------------------------------------------------
    dw = WORKLOADS["specdecode_16x51k"]
    dec = dw.make()
    pw = WORKLOADS["prefill_1x8k_100k"]
    pre = pw.make()
    R, DQL = dec.num_reqs, dec.dql
    T_dec = R * DQL
    T_pre = pre.q.shape[0]
    qlens = [DQL] * R + [T_pre]
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    seq = np.concatenate([dec.seq_lens, pre.seq_lens]).astype(np.int32)
    key_offsets = np.zeros(R + 1, np.int32)  # the prefill request's keys start at 0
    split = qsa.qsa_split_batch(qsl.tolist(), DQL)
    assert split[1:] == (R, T_dec, 1, T_pre, DQL), split

    q_dec = to_bf16(dec.q)
    page_table = to_i32(dec.page_table)
    pools = [to_bf16(dec.k_pool)]
    for i in range(1, args.pools):
        pool = decode_inputs([int(x) for x in dec.seq_lens], DQL, dec.page_size,
                             dec.page_table.shape[1], 0, dec.out_cols, seed=1000 + i,
                             shuffle=False).k_pool
        assert pool.shape == dec.k_pool.shape
        pools.append(to_bf16(pool))
    q_pre, k_pre = to_bf16(pre.q), to_bf16(pre.k)
    qsl_d, seq_d, off_d = to_i32(qsl), to_i32(seq), to_i32(key_offsets)

    T_all = T_dec + T_pre
    meta = {
        "token_to_req": torch.empty(T_all, dtype=torch.int32, device=dev),
        "positions": torch.empty(T_all, dtype=torch.int64, device=dev),
        "visible": torch.empty(T_all, dtype=torch.int32, device=dev),
        "comp_lens": torch.empty(R + 1, dtype=torch.int32, device=dev),
        "row_k_start": torch.empty(T_all, dtype=torch.int32, device=dev),
        "row_k_end": torch.empty(T_all, dtype=torch.int32, device=dev),
    }
    dec_out = torch.empty((T_dec, dec.out_cols), dtype=torch.float32, device=dev)
    # The score matrix's rows start on 128-byte lines (a row pitch rounded up
    # to 32 floats: 27,072 for 27,048 columns), a layout the caller chooses;
    # the padding is never written or read.  An unpadded pitch runs the
    # kernel's line-aligned store layout instead (`prefill_natural_pitch`).
    pre_pitch = (pre.out_cols + 31) // 32 * 32
    pre_out = torch.empty((T_pre, pre_pitch), dtype=torch.float32, device=dev)[:, :pre.out_cols]
    TOPK = 512
    dec_top = torch.empty((T_dec, TOPK), dtype=torch.int32, device=dev)
    pre_top = torch.empty((T_pre, TOPK), dtype=torch.int32, device=dev)
    stream = torch.cuda.Stream(device=dev)
    sh = stream.cuda_stream

    def check(rc):
        if rc != 0:
            raise RuntimeError(lib.qsa_last_error().decode())

    scale = qsa.DEFAULT_SCALE
    NAMES = ["metadata", "decode_plan", "decode", "prefill", "topk_decode", "topk_prefill"]
    plan_bytes = qsa.qsa_decode_plan_bytes(R, dec.out_cols)
    plan = torch.empty(plan_bytes, dtype=torch.uint8, device=dev)

    def step(i, events=None):
        pool = pools[i % len(pools)]

        def rec(j):  # kernel j of the step is timed into events 2j, 2j + 1
            if events:
                check(lib.qsa_set_launch_events(events.ev[2 * j], events.ev[2 * j + 1]))

        rec(0)
        check(lib.qsa_build_metadata(
            qsl_d.data_ptr(), seq_d.data_ptr(), R + 1, T_all, 4, off_d.data_ptr(),
            meta["token_to_req"].data_ptr(), meta["positions"].data_ptr(),
            meta["visible"].data_ptr(), meta["comp_lens"].data_ptr(),
            meta["row_k_start"].data_ptr(), meta["row_k_end"].data_ptr(), sh))
        rec(1)
        check(lib.qsa_build_decode_plan(
            meta["comp_lens"].data_ptr(), page_table.data_ptr(), page_table.stride(0), page_table.shape[1],
            pool.shape[0], pool.shape[1], R, dec_out.shape[1], plan.data_ptr(), plan_bytes, sh))
        rec(2)
        check(lib.qsa_mqa_decode_planned(
            plan.data_ptr(), plan_bytes, q_dec.data_ptr(), qsa.QSA_DTYPE_BF16, q_dec.stride(0), q_dec.stride(1),
            q_dec.stride(2), pool.data_ptr(), qsa.QSA_DTYPE_BF16, 1.0, pool.shape[0], pool.shape[1],
            page_table.data_ptr(), page_table.stride(0), page_table.shape[1], meta["visible"].data_ptr(), R,
            DQL, 4, 128, scale, dec_out.data_ptr(), dec_out.stride(0), dec_out.shape[1], sh))
        rec(3)
        check(lib.qsa_mqa_prefill(
            q_pre.data_ptr(), q_pre.stride(0), q_pre.stride(1), k_pre.data_ptr(), k_pre.stride(0),
            k_pre.shape[0], meta["row_k_start"].data_ptr() + 4 * T_dec,
            meta["row_k_end"].data_ptr() + 4 * T_dec, T_pre, 4, 128, scale, pre_out.data_ptr(),
            pre_out.stride(0), pre_out.shape[1], sh))
        rec(4)
        check(lib.qsa_topk_blocks(dec_out.data_ptr(), dec_out.stride(0), T_dec, dec_out.shape[1],
                                  TOPK, dec_top.data_ptr(), TOPK, sh))
        rec(5)
        check(lib.qsa_topk_blocks(pre_out.data_ptr(), pre_out.stride(0), T_pre, pre_out.shape[1],
                                  TOPK, pre_top.data_ptr(), TOPK, sh))
        if events:
            check(lib.qsa_set_launch_events(None, None))

    # --- warmup -------------------------------------------------------------
    torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    vis_host = meta["visible"].cpu().numpy()
    comp_host = meta["comp_lens"].cpu().numpy()

    # --- timed region -------------------------------------------------------
    evs = [HipEvents(2 * len(NAMES)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    per = {n: [] for n in NAMES}
    for e in evs:
        for j, n in enumerate(NAMES):
            per[n].append(e.elapsed_us(2 * j, 2 * j + 1))
        e.close()
    avg = {n: float(np.mean(v)) for n, v in per.items()}
    med = {n: float(np.median(v)) for n, v in per.items()}
    p10 = {n: float(np.percentile(v, 10)) for n, v in per.items()}
    p90 = {n: float(np.percentile(v, 90)) for n, v in per.items()}

    comp_total = float(comp_host[:R].sum())
    dbytes = decode_bytes(R, DQL, comp_total)
    decode_gbps = dbytes / (avg["decode"] * 1e-6) / 1e9
    vis_pre_total = int(vis_host[T_dec:].astype(np.int64).sum())
    pflops = prefill_flops(vis_pre_total)
    prefill_tflops = pflops / (avg["prefill"] * 1e-6) / 1e12
    pbytes = prefill_bytes(T_pre, pre.out_cols, int(pre.k.shape[0]))
    prefill_gbps = pbytes / (avg["prefill"] * 1e-6) / 1e9
    tk_bytes = topk_bytes(T_pre, pre.out_cols, TOPK)
    topk_gbps = tk_bytes / (avg["topk_prefill"] * 1e-6) / 1e9

    def roof(bound, achieved, peak, unit, traffic):
        return {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": traffic}

    result = {
        "metric": METRIC,
        "value": round(decode_gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(decode_gbps / PAGES_DECODE_GBPS, 4),
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "mixed batch: decode 16 req x DQL 4, contexts 3,508/51,200/102,400 "
                        "(min/mean/max), page_size 64 + prefill 1x8,192 queries over a 100,000-token "
                        "prefix; top-512 per row",
            "decode_requests": R, "decode_query_len": DQL, "decode_keys": int(comp_total),
            "page_size": dec.page_size, "decode_key_pools": len(pools),
            "prefill_rows": T_pre, "prefill_keys": int(pre.k.shape[0]), "topk": TOPK,
            "score_row_pitch": pre_pitch,
        },
        "roofline": roof("hbm", decode_gbps, HBM_PEAK_GBPS, "GB/s",
                         read_traffic("decode.hip", "decode")),
        "roofline_prefill": roof("hbm", prefill_gbps, HBM_PEAK_GBPS, "GB/s",
                                 read_traffic("prefill.hip", "prefill")),
        "prefill_mfma": roof("mfma", prefill_tflops, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s", None),
        "roofline_topk": roof("hbm", topk_gbps, HBM_PEAK_GBPS, "GB/s",
                              read_traffic("topk.hip", "topk")),
        "kernel_us_avg": {n: round(v, 3) for n, v in avg.items()},
        "kernel_us_median": {n: round(v, 3) for n, v in med.items()},
        "kernel_us_p10": {n: round(v, 3) for n, v in p10.items()},
        "kernel_us_p90": {n: round(v, 3) for n, v in p90.items()},
        "prefill_tflops": round(prefill_tflops, 2),
        "decode_bytes": dbytes, "prefill_bytes": pbytes, "prefill_flops": pflops,
        "topk_prefill_bytes": tk_bytes,
    }

    # The decode without a task table (qsa_mqa_decode: each wave finds its
    # span from the compressed lengths), for context: 20 launches over the
    # rotating pools, and a bitwise check that both forms score alike.
    un_ev = [HipEvents(2) for _ in range(20)]
    un_out = torch.empty_like(dec_out)

    def mapped_decode(pool, out):
        check(lib.qsa_mqa_decode(
            q_dec.data_ptr(), q_dec.stride(0), q_dec.stride(1), q_dec.stride(2), pool.data_ptr(),
            pool.shape[0], pool.shape[1], page_table.data_ptr(), page_table.stride(0),
            page_table.shape[1], meta["comp_lens"].data_ptr(), meta["visible"].data_ptr(), R, DQL,
            4, 128, scale, out.data_ptr(), out.stride(0), out.shape[1], sh))

    for j in range(24):
        if j >= 4:
            check(lib.qsa_set_launch_events(un_ev[j - 4].ev[0], un_ev[j - 4].ev[1]))
        mapped_decode(pools[j % len(pools)], un_out)
        check(lib.qsa_set_launch_events(None, None))
    torch.cuda.synchronize()
    un_us = float(np.mean([e.elapsed_us(0, 1) for e in un_ev]))
    for e in un_ev:
        e.close()
    last_pool = pools[(args.warmup + args.steps - 1) % len(pools)]
    mapped_decode(last_pool, un_out)
    torch.cuda.synchronize()
    result["decode_unplanned"] = {
        "us": round(un_us, 3), "gbps": round(dbytes / (un_us * 1e-6) / 1e9, 2),
        "frac_of_hbm": round(dbytes / (un_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        "matches_planned": bool(torch.equal(un_out.view(torch.int32), dec_out.view(torch.int32))),
    }
    del un_out

    # The fused prefill top-k on the same prefill rows, for context: its
    # time (first kernel's begin to last kernel's end), the unfused pair's,
    # and whether its picks equal the step's own top-k of the prefill rows.
    nws = ctypes.c_int64(0)
    check(lib.qsa_prefill_topk_workspace_bytes(T_pre, pre.out_cols, TOPK, ctypes.byref(nws)))
    fz_ws = torch.empty(nws.value, dtype=torch.uint8, device=dev)
    fz_top = torch.empty_like(pre_top)
    fz_ev = [HipEvents(2) for _ in range(5)]
    for j in range(6):
        if j > 0:
            check(lib.qsa_set_launch_events(fz_ev[j - 1].ev[0], fz_ev[j - 1].ev[1]))
        check(lib.qsa_mqa_prefill_topk(
            q_pre.data_ptr(), q_pre.stride(0), q_pre.stride(1), k_pre.data_ptr(), k_pre.stride(0),
            k_pre.shape[0], meta["row_k_start"].data_ptr() + 4 * T_dec,
            meta["row_k_end"].data_ptr() + 4 * T_dec, T_pre, 4, 128, scale, pre.out_cols, TOPK,
            fz_top.data_ptr(), TOPK, fz_ws.data_ptr(), nws.value, sh))
        check(lib.qsa_set_launch_events(None, None))
    torch.cuda.synchronize()
    fz_us = [e.elapsed_us(0, 1) for e in fz_ev]
    for e in fz_ev:
        e.close()
    result["prefill_topk_fused"] = {
        "us": round(float(np.mean(fz_us)), 3),
        "unfused_us": round(avg["prefill"] + avg["topk_prefill"], 3),
        "workspace_bytes": int(nws.value),
        "matches_unfused": bool(torch.equal(fz_top, pre_top)),
    }
    del fz_ws

    # The same prefill rows with an unpadded row pitch (27,048 floats, rows
    # not on 128-byte lines): the kernel's line-aligned (rotated) store
    # layout.  6 launches after 4 warmup ones, back to back; compared with
    # the step's own last scores (still in pre_out).
    nat_out = torch.empty((T_pre, pre.out_cols), dtype=torch.float32, device=dev)
    nat_ev = [HipEvents(2) for _ in range(6)]
    for j in range(6 + 4):
        if j >= 4:
            check(lib.qsa_set_launch_events(nat_ev[j - 4].ev[0], nat_ev[j - 4].ev[1]))
        check(lib.qsa_mqa_prefill(
            q_pre.data_ptr(), q_pre.stride(0), q_pre.stride(1), k_pre.data_ptr(), k_pre.stride(0),
            k_pre.shape[0], meta["row_k_start"].data_ptr() + 4 * T_dec,
            meta["row_k_end"].data_ptr() + 4 * T_dec, T_pre, 4, 128, scale, nat_out.data_ptr(),
            nat_out.stride(0), nat_out.shape[1], sh))
        check(lib.qsa_set_launch_events(None, None))
    torch.cuda.synchronize()
    nat_us = float(np.mean([e.elapsed_us(0, 1) for e in nat_ev]))
    result["prefill_natural_pitch"] = {
        "us": round(nat_us, 3), "row_pitch": pre.out_cols, "step_row_pitch": pre_pitch,
        "tflops": round(pflops / (nat_us * 1e-6) / 1e12, 2),
        "frac_of_mfma": round(pflops / (nat_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "matches_step": bool(torch.equal(nat_out, pre_out)),
    }
    for e in nat_ev:
        e.close()
    del nat_out

    # The typed entry points on the same workloads, for context.  Decode
    # reads the batch's key caches written as e4m3 codes (the fp8 cache write
    # rule of the shared input generator): the 8 pools' codes and their
    # sign-flipped copies, 16 caches of 26 MB, more than the Infinity Cache
    # holds, so each launch streams from HBM.  Prefill runs on the step's
    # prefill rows with queries and keys in fp16.
    from workloads import FP8_K_SCALE, fp8_e4m3_cache
    f8_pools = []
    for pool in pools:
        codes = fp8_e4m3_cache(pool.view(torch.int16).cpu().numpy().view(np.uint16))
        f8_pools.append(torch.from_numpy(codes).to(dev))
        f8_pools.append(torch.from_numpy(codes ^ np.uint8(0x80)).to(dev))
    n_typed = 20
    ty_ev = [HipEvents(2) for _ in range(n_typed)]
    f8_out = torch.empty_like(dec_out)
    for j in range(n_typed + 4):
        if j >= 4:
            check(lib.qsa_set_launch_events(ty_ev[j - 4].ev[0], ty_ev[j - 4].ev[1]))
        pool8 = f8_pools[j % len(f8_pools)]
        check(lib.qsa_mqa_decode_typed(
            q_dec.data_ptr(), qsa.QSA_DTYPE_BF16, q_dec.stride(0), q_dec.stride(1), q_dec.stride(2),
            pool8.data_ptr(), qsa.QSA_DTYPE_FP8_E4M3, FP8_K_SCALE, dec.k_pool.shape[0], dec.page_size,
            page_table.data_ptr(), page_table.stride(0), page_table.shape[1], meta["comp_lens"].data_ptr(),
            meta["visible"].data_ptr(), R, DQL, 4, 128, scale, f8_out.data_ptr(), f8_out.stride(0),
            f8_out.shape[1], sh))
        check(lib.qsa_set_launch_events(None, None))
    torch.cuda.synchronize()
    f8_us = float(np.mean([e.elapsed_us(0, 1) for e in ty_ev]))
    f8_bytes = dbytes - 128.0 * comp_total  # 128-byte keys instead of 256
    result["decode_fp8_e4m3"] = {
        "us": round(f8_us, 3), "gbps": round(f8_bytes / (f8_us * 1e-6) / 1e9, 2),
        "frac_of_hbm": round(f8_bytes / (f8_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        "bytes": f8_bytes, "key_caches": len(f8_pools), "k_scale": FP8_K_SCALE,
    }
    del f8_pools
    q16, k16 = q_pre.to(torch.float16), k_pre.to(torch.float16)
    for j in range(6 + 4):
        if j >= 4:
            check(lib.qsa_set_launch_events(ty_ev[j - 4].ev[0], ty_ev[j - 4].ev[1]))
        check(lib.qsa_mqa_prefill_typed(
            q16.data_ptr(), q16.stride(0), q16.stride(1), k16.data_ptr(), k16.stride(0), k16.shape[0],
            qsa.QSA_DTYPE_FP16, meta["row_k_start"].data_ptr() + 4 * T_dec,
            meta["row_k_end"].data_ptr() + 4 * T_dec, T_pre, 4, 128, scale, pre_out.data_ptr(),
            pre_out.stride(0), pre_out.shape[1], sh))
        check(lib.qsa_set_launch_events(None, None))
    torch.cuda.synchronize()
    f16_us = float(np.mean([e.elapsed_us(0, 1) for e in ty_ev[:6]]))
    result["prefill_fp16"] = {
        "us": round(f16_us, 3), "tflops": round(pflops / (f16_us * 1e-6) / 1e12, 2),
        "frac_of_mfma": round(pflops / (f16_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
    }
    for e in ty_ev:
        e.close()
    del q16, k16


    # The other workload configurations, for context: each timed over its own
    # launches with the same per-kernel events, inputs resident in HBM.
    #   tiny_decode (1 request, context 256, page size 16) and decode_100k
    #   (1 request, context 100,000, page size 64; 48 key pools rotated, more
    #   than the Infinity Cache holds): planned decode, us and GB/s;
    #   prefill_1x8k_8k and prefill_4x4k_100k: prefill us, TFLOP/s, fraction
    #   of dense bf16 MFMA peak; and the top-512 of the 4x4K rows, us and GB/s.
    def timed(n, warm, launch):
        evs = [HipEvents(2) for _ in range(n)]
        for j in range(n + warm):
            if j >= warm:
                check(lib.qsa_set_launch_events(evs[j - warm].ev[0], evs[j - warm].ev[1]))
            launch(j)
            check(lib.qsa_set_launch_events(None, None))
        torch.cuda.synchronize()
        us = [e.elapsed_us(0, 1) for e in evs]
        for e in evs:
            e.close()
        return float(np.mean(us)), float(np.median(us))

    configs = {}
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    for name, n_pools in (("tiny_decode", 1), ("decode_100k", 48)):
        w = WORKLOADS[name].make()
        c_pools = [to_bf16(w.k_pool)] + [
            torch.randn(w.k_pool.shape, generator=gen, device=dev).to(torch.bfloat16) for _ in range(n_pools - 1)]
        c_pt = to_i32(w.page_table)
        c_q = to_bf16(w.q)
        c_comp, c_vis = qsa.qsa_decode_visible_blocks(to_i32(w.seq_lens), w.dql)
        c_plan = qsa.qsa_build_decode_plan(c_comp, c_pt, c_pools[0].shape[0], w.page_size, w.out_cols)
        c_out = torch.empty((w.num_reqs * w.dql, w.out_cols), dtype=torch.float32, device=dev)

        def c_launch(j, c_pools=c_pools, c_pt=c_pt, c_q=c_q, c_vis=c_vis, c_plan=c_plan, c_out=c_out, w=w):
            pool = c_pools[j % len(c_pools)]
            check(lib.qsa_mqa_decode_planned(
                c_plan.data_ptr(), c_plan.numel(), c_q.data_ptr(), qsa.QSA_DTYPE_BF16, c_q.stride(0), c_q.stride(1),
                c_q.stride(2), pool.data_ptr(), qsa.QSA_DTYPE_BF16, 1.0, pool.shape[0], pool.shape[1],
                c_pt.data_ptr(), c_pt.stride(0), c_pt.shape[1], c_vis.data_ptr(), w.num_reqs, w.dql, 4, 128, scale,
                c_out.data_ptr(), c_out.stride(0), c_out.shape[1], sh))

        c_mean, c_med = timed(50, 5, c_launch)
        c_bytes = decode_bytes(w.num_reqs, w.dql, float(c_comp.sum().item()))
        configs[name] = {"kernel": "decode (planned)", "us": round(c_mean, 3), "us_median": round(c_med, 3),
                         "bytes": c_bytes, "gbps": round(c_bytes / (c_mean * 1e-6) / 1e9, 2),
                         "frac_of_hbm": round(c_bytes / (c_mean * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                         "key_pools": len(c_pools)}
        del c_pools, c_out
    for name, n_launch in (("prefill_1x8k_8k", 20), ("prefill_4x4k_100k", 6)):
        w = WORKLOADS[name].make()
        Tw = w.q.shape[0]
        w_q, w_k = to_bf16(w.q), to_bf16(w.k)
        w_meta = qsa.qsa_build_metadata(to_i32(w.query_start_loc), to_i32(w.seq_lens), Tw,
                                        key_offsets=to_i32(w.key_offsets))
        # Rows on 128-byte lines, as in the step.
        w_pitch = (w.out_cols + 31) // 32 * 32
        w_out = torch.empty((Tw, w_pitch), dtype=torch.float32, device=dev)[:, :w.out_cols]

        def p_launch(j, w_q=w_q, w_k=w_k, w_meta=w_meta, w_out=w_out, Tw=Tw):
            check(lib.qsa_mqa_prefill(
                w_q.data_ptr(), w_q.stride(0), w_q.stride(1), w_k.data_ptr(), w_k.stride(0), w_k.shape[0],
                w_meta["row_k_start"].data_ptr(), w_meta["row_k_end"].data_ptr(), Tw, 4, 128, scale,
                w_out.data_ptr(), w_out.stride(0), w_out.shape[1], sh))

        p_mean, p_med = timed(n_launch, 2, p_launch)
        w_flops = prefill_flops(int(w_meta["visible"].to(torch.int64).sum().item()))
        w_tflops = w_flops / (p_mean * 1e-6) / 1e12
        configs[name] = {"kernel": "prefill", "us": round(p_mean, 3), "us_median": round(p_med, 3),
                         "flops": w_flops, "tflops": round(w_tflops, 2),
                         "frac_of_mfma": round(w_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                         "out_bytes": float(Tw) * w.out_cols * 4, "row_pitch": w_pitch}
        if name == "prefill_4x4k_100k":
            w_top = torch.empty((Tw, TOPK), dtype=torch.int32, device=dev)

            def t_launch(j, w_out=w_out, w_top=w_top, Tw=Tw):
                check(lib.qsa_topk_blocks(w_out.data_ptr(), w_out.stride(0), Tw, w_out.shape[1], TOPK,
                                          w_top.data_ptr(), TOPK, sh))

            t_mean, t_med = timed(n_launch, 2, t_launch)
            t_bytes = topk_bytes(Tw, w.out_cols, TOPK)
            configs[name + "_topk512"] = {"kernel": "top-k", "us": round(t_mean, 3), "us_median": round(t_med, 3),
                                          "bytes": t_bytes, "gbps": round(t_bytes / (t_mean * 1e-6) / 1e9, 2),
                                          "frac_of_hbm": round(t_bytes / (t_mean * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}
            del w_top
        del w_out
    result["configs"] = configs

    # The compressed-cache metadata of the step's batch (the decode requests'
    # page tables and a block table for the prefill chunk, page size 64,
    # 4,096 work-item slots), and the paged-key gather of the decode batch's
    # whole key set into one packed K (the keys a prefill over those requests
    # would read), both timed over 20 launches; the gather rotates the pools.
    cols = max(dec.page_table.shape[1], int(seq[-1]) // 4 // dec.page_size + 1)
    bt_host = np.full((R + 1, cols), -1, np.int32)
    bt_host[:R, :dec.page_table.shape[1]] = dec.page_table
    bt_host[R] = np.random.default_rng(6).permutation(cols) + dec.k_pool.shape[0]
    bt = to_i32(bt_host)
    cm_slots = torch.empty(T_all, dtype=torch.int64, device=dev)
    cm_work = torch.empty((4096, 2), dtype=torch.int32, device=dev)
    comp_dec = to_i32(comp_host[:R])
    gk_off = to_i32(np.concatenate([[0], np.cumsum(comp_host[:R - 1])]))
    gk_out = torch.empty((int(comp_total), 128), dtype=torch.bfloat16, device=dev)
    cm_ev = [HipEvents(2) for _ in range(20)]
    gk_ev = [HipEvents(2) for _ in range(20)]
    for j in range(24):
        if j >= 4:
            check(lib.qsa_set_launch_events(cm_ev[j - 4].ev[0], cm_ev[j - 4].ev[1]))
        check(lib.qsa_build_cache_metadata(
            qsl_d.data_ptr(), seq_d.data_ptr(), R + 1, T_all, 4, bt.data_ptr(), bt.stride(0), bt.shape[1],
            dec.page_size, None, cm_slots.data_ptr(), cm_work.data_ptr(), 4096, sh))
        if j >= 4:
            check(lib.qsa_set_launch_events(gk_ev[j - 4].ev[0], gk_ev[j - 4].ev[1]))
        pool = pools[j % len(pools)]
        check(lib.qsa_gather_keys(
            pool.data_ptr(), qsa.QSA_DTYPE_BF16, pool.shape[0], pool.shape[1], page_table.data_ptr(),
            page_table.stride(0), page_table.shape[1], comp_dec.data_ptr(), gk_off.data_ptr(), R,
            int(comp_host[:R].max()), gk_out.data_ptr(), qsa.QSA_DTYPE_BF16, gk_out.stride(0), gk_out.shape[0], sh))
        check(lib.qsa_set_launch_events(None, None))
    torch.cuda.synchronize()
    # The cache-metadata call is two kernels; the events bracket the first
    # kernel's begin and the last one's end.
    cm_us = float(np.mean([e.elapsed_us(0, 1) for e in cm_ev]))
    gk_us = float(np.mean([e.elapsed_us(0, 1) for e in gk_ev]))
    gk_bytes = 2.0 * comp_total * 256
    result["cache_metadata"] = {"us": round(cm_us, 3), "tokens": T_all, "requests": R + 1, "work_items": 4096}
    result["gather_keys"] = {
        "us": round(gk_us, 3), "keys": int(comp_total), "bytes": gk_bytes,
        "gbps": round(gk_bytes / (gk_us * 1e-6) / 1e9, 2),
        "frac_of_hbm": round(gk_bytes / (gk_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
    }
    for e in cm_ev + gk_ev:
        e.close()
    del gk_out

    # Query preparation of the prefill chunk: 8,192 tokens x 4 indexer heads
    # at positions 100,000.. (a 131,072-row bf16 cos/sin table), bf16 out,
    # timed over 20 launches that rotate 32 input and output buffers
    # (537 MB, beyond the on-die caches).
    from workloads import prepare_inputs
    prep = prepare_inputs(T_pre, 4, seed=9, first_pos=int(pre.seq_lens[0]) - T_pre, table_rows=131_072)
    pq0 = to_bf16(prep.q)
    pqs = [pq0.clone() for _ in range(32)]
    pos_d = torch.from_numpy(prep.positions).to(dev)
    cs_d, w_d = to_bf16(prep.cos_sin), to_bf16(prep.weight)
    pouts = [torch.empty((T_pre, 4, 128), dtype=torch.bfloat16, device=dev) for _ in range(32)]
    pp_ev = [HipEvents(2) for _ in range(20)]
    for j in range(24):
        if j >= 4:
            check(lib.qsa_set_launch_events(pp_ev[j - 4].ev[0], pp_ev[j - 4].ev[1]))
        pq, po = pqs[j % 32], pouts[(j + 7) % 32]
        check(lib.qsa_prepare_q(
            pq.data_ptr(), pq.stride(0), T_pre, 4, pos_d.data_ptr(), 0, 1, cs_d.data_ptr(), qsa.QSA_DTYPE_BF16,
            cs_d.shape[0], w_d.data_ptr(), qsa.QSA_DTYPE_BF16, prep.eps, None, po.data_ptr(), qsa.QSA_DTYPE_BF16,
            1.0, po.stride(0), po.stride(1), sh))
        check(lib.qsa_set_launch_events(None, None))
    torch.cuda.synchronize()
    pp_us = float(np.mean([e.elapsed_us(0, 1) for e in pp_ev]))
    pp_bytes = prepare_bytes(T_pre, 4)
    result["prepare_q"] = {
        "us": round(pp_us, 3), "tokens": T_pre, "heads": 4, "bytes": pp_bytes,
        "gbps": round(pp_bytes / (pp_us * 1e-6) / 1e9, 2),
        "frac_of_hbm": round(pp_bytes / (pp_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        "traffic": read_traffic("prepare.hip", "prepare_q"),
    }
    for e in pp_ev:
        e.close()
    del pqs, pouts, pq0

    # A measured bandwidth for context: a plain 1 GiB device-to-device copy
    # (read + write bytes over its time), and each HBM-bound kernel's rate as
    # a fraction of it.
    n_copy = (1 << 30) // 4
    c_src = torch.ones(n_copy, dtype=torch.float32, device=dev)
    c_dst = torch.empty_like(c_src)
    c_dst.copy_(c_src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        c_dst.copy_(c_src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbps = 2.0 * n_copy * 4 * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del c_src, c_dst
    result["measured_copy_gbps"] = round(copy_gbps, 1)
    result["frac_of_measured_copy"] = {
        "decode": round(decode_gbps / copy_gbps, 4),
        "prefill": round(prefill_gbps / copy_gbps, 4),
        "topk_prefill": round(topk_gbps / copy_gbps, 4),
    }

    # A measured matrix-core rate for context: a large square bf16 GEMM
    # (8192^3, fp32 accumulate) through the vendor BLAS, and the prefill
    # kernel's rate as a fraction of it.
    g = 8192
    ga = torch.randn(g, g, device=dev).to(torch.bfloat16)
    gb = torch.randn(g, g, device=dev).to(torch.bfloat16)
    gc = torch.mm(ga, gb)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        torch.mm(ga, gb, out=gc)
    e1.record()
    torch.cuda.synchronize()
    gemm_tflops = 2.0 * g ** 3 * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del ga, gb, gc
    result["measured_gemm_tflops"] = round(gemm_tflops, 1)
    result["prefill_frac_of_measured_gemm"] = round(prefill_tflops / gemm_tflops, 4)

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = n * 4

    if not args.no_cpu_baseline:
        from oracle import oracle as O
        _, _, dec_vis = O.token_metadata(dec.query_start_loc, dec.seq_lens, T_dec)
        p_req, _, p_vis = O.token_metadata(pre.query_start_loc, pre.seq_lens, T_pre)
        p_ks, p_ke = O.prefill_intervals(p_req, p_vis, pre.key_offsets)
        result["cpu_baseline"] = cpu_baseline(dec, dec_vis, pre, p_ks, p_ke)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
