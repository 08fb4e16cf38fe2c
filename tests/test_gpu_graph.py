"""GPU: every entry point captured into one HIP graph and replayed.

Validation reads only host arguments and no entry point clears memory with a
memset, so the calls can be captured.  The graph is replayed several times,
with eager work and poisoned outputs between replays, and every replay must
reproduce the eager results bit for bit.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from tests.parity import bf16_to_device, i32_to_device
from workloads import FP8_K_SCALE, decode_inputs, fp8_e4m3_cache, normal_bf16, prepare_inputs

pytestmark = pytest.mark.gpu


def test_capture_and_replay_all_entry_points():
    import block_indexer_scoring_amd as qsa
    qsa.load_library()
    dev = "cuda"
    # Decode: 3 requests, DQL 2, page size 16.
    dec = decode_inputs([700, 1300, 90], 2, 16, 30, 3, 400, seed=61)
    _, _, vis = O.token_metadata(dec.query_start_loc, dec.seq_lens, dec.q.shape[0] * dec.q.shape[1])
    q_dec, pool = bf16_to_device(dec.q), bf16_to_device(dec.k_pool)
    pt, comp, visd = i32_to_device(dec.page_table), i32_to_device(O.comp_lens(dec.seq_lens)), i32_to_device(vis)
    # Prefill: 300 rows over 2,000 keys, 1,500 columns; top-64.
    rng = np.random.default_rng(62)
    T, NK, cols, K = 300, 2000, 1500, 64
    q_pre, k_pre = bf16_to_device(normal_bf16(rng, (T, 4, 128))), bf16_to_device(normal_bf16(rng, (NK, 128)))
    ks = i32_to_device(np.zeros(T, np.int32))
    ke = i32_to_device(rng.integers(0, NK + 1, T).astype(np.int32))

    # Metadata for the decode batch (raw entry point, preallocated outputs).
    lib = qsa.load_library()
    n_tok = int(dec.query_start_loc[-1])
    qsl, seq = i32_to_device(dec.query_start_loc), i32_to_device(dec.seq_lens)
    meta = [torch.empty(n_tok, dtype=torch.int32, device=dev), torch.empty(n_tok, dtype=torch.int64, device=dev),
            torch.empty(n_tok, dtype=torch.int32, device=dev), torch.empty(3, dtype=torch.int32, device=dev)]

    dec_out = torch.empty((q_dec.shape[0] * q_dec.shape[1], 400), dtype=torch.float32, device=dev)
    pre_out = torch.empty((T, cols), dtype=torch.float32, device=dev)
    top = torch.empty((T, K), dtype=torch.int32, device=dev)
    fused = torch.empty((T, K), dtype=torch.int32, device=dev)
    ws = torch.empty(qsa.qsa_prefill_topk_workspace_bytes(T, cols, K), dtype=torch.uint8, device=dev)
    # Typed decode over an e4m3 copy of the cache, the cache metadata and
    # the key gather of the decode batch.
    pool8 = torch.from_numpy(fp8_e4m3_cache(dec.k_pool)).cuda().view(torch.float8_e4m3fn)
    dec8 = torch.empty_like(dec_out)
    bt = pt
    slots = torch.empty(n_tok, dtype=torch.int64, device=dev)
    work = torch.empty((32, 2), dtype=torch.int32, device=dev)
    comp_np = O.comp_lens(dec.seq_lens).astype(np.int32)
    offs = i32_to_device(np.concatenate([[0], np.cumsum(comp_np[:-1])]))
    kg = torch.empty((int(comp_np.sum()), 128), dtype=torch.bfloat16, device=dev)
    # Query preparation (MRoPE, e4m3 store) of 200 tokens x 4 heads.
    prep = prepare_inputs(200, 4, seed=63, first_pos=300, table_rows=600, mrope=True)
    prep_q, prep_pos = bf16_to_device(prep.q), torch.from_numpy(prep.positions).cuda()
    prep_cs, prep_w = bf16_to_device(prep.cos_sin), bf16_to_device(prep.weight)
    prep_out = torch.empty((200, 4, 128), dtype=torch.float8_e4m3fn, device=dev)
    outs = (dec_out, pre_out, top, fused, meta[0], meta[1], meta[2], meta[3], dec8, slots, work, kg,
            prep_out.view(torch.uint8))

    def run():
        assert lib.qsa_build_metadata(qsl.data_ptr(), seq.data_ptr(), 3, n_tok, 4, None, meta[0].data_ptr(),
                                      meta[1].data_ptr(), meta[2].data_ptr(), meta[3].data_ptr(), None, None,
                                      torch.cuda.current_stream().cuda_stream) == 0
        qsa.qsa_mqa_decode(q_dec, pool, pt, comp, visd, out=dec_out)
        qsa.qsa_mqa_prefill(q_pre, k_pre, ks, ke, out=pre_out)
        qsa.qsa_topk_blocks(pre_out, K, out=top)
        qsa.qsa_mqa_prefill_topk(q_pre, k_pre, ks, ke, cols, K, out=fused, workspace=ws)
        qsa.qsa_mqa_decode_typed(q_dec, pool8, pt, comp, visd, k_scale=FP8_K_SCALE, out=dec8)
        qsa.qsa_build_cache_metadata(qsl, seq, n_tok, bt, 16, 4, max_num_work=32, slot_mapping=slots, k_work=work)
        qsa.qsa_gather_keys(pool, pt, comp, offs, int(comp_np.max()), out=kg)
        qsa.qsa_prepare_q(prep_q, prep_pos, prep_cs, prep_w, prep.eps, mrope_section=(16, 8, 8), out=prep_out,
                          out_scale=0.25)

    run()
    torch.cuda.synchronize()
    want = [o.clone() for o in outs]
    assert torch.equal(want[2], want[3])
    req, pos, vis_o = O.token_metadata(dec.query_start_loc, dec.seq_lens, n_tok)
    assert np.array_equal(want[4].cpu().numpy(), req) and np.array_equal(want[5].cpu().numpy(), pos)
    assert np.array_equal(want[6].cpu().numpy(), vis_o)
    assert np.array_equal(want[7].cpu().numpy(), O.comp_lens(dec.seq_lens))
    assert np.array_equal(want[9].cpu().numpy(), O.cache_slots(dec.query_start_loc, dec.seq_lens, n_tok,
                                                               dec.page_table, 16, 4))
    assert np.array_equal(want[10].cpu().numpy(), O.k_work(dec.query_start_loc, dec.seq_lens, 32, 4))
    assert np.array_equal(want[12].cpu().numpy(), O.prepare_q(prep.q, prep.positions, prep.cos_sin, prep.weight,
                                                              prep.eps, (16, 8, 8), "fp8_e4m3", 0.25))

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()  # warm the capture stream once
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for rep in range(4):
        for o in outs:
            (o if o.dtype == torch.uint8 else o.view(torch.int16)).fill_(0x7F - rep if o.dtype == torch.uint8
                                                                          else 0x7FC0 + rep)  # poison (eager)
        assert not torch.equal(outs[0], want[0])
        scratch = torch.empty_like(dec_out)
        qsa.qsa_mqa_decode(q_dec, pool, pt, comp, visd, out=scratch)  # eager library work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        names = ("decode", "prefill", "top-k", "fused top-k", "token_to_req", "positions", "visible", "comp_lens",
                 "fp8 decode", "cache slots", "work items", "gathered keys", "prepared q")
        for name, o, w in zip(names, outs, want):
            assert torch.equal(o, w), f"replay {rep}: {name} differs"
        assert torch.equal(scratch.view(torch.int32), want[0].view(torch.int32))
