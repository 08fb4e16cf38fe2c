"""The C ABI on a host without a GPU: the library loads, exports every entry
point include/qsa.h declares, and rejects bad arguments before touching the
device.  No compute call runs here."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qsa.h")


@pytest.fixture(scope="module")
def lib():
    from block_indexer_scoring_amd import qsa
    if not os.path.exists(qsa.LIB_PATH):
        from block_indexer_scoring_amd import build
        build.build()
    return qsa.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qsa_\w+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    names = declared_functions()
    for n in ("qsa_mqa_decode", "qsa_mqa_prefill", "qsa_topk_blocks", "qsa_build_metadata",
              "qsa_split_batch", "qsa_last_error", "qsa_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"libqsa.so does not export {name}"
    from block_indexer_scoring_amd import qsa
    assert set(qsa.SYMBOLS) == set(declared_functions())


def test_abi_version(lib):
    from block_indexer_scoring_amd import qsa
    m = re.search(r"#define QSA_ABI_VERSION (\d+)", open(HEADER).read())
    assert lib.qsa_abi_version() == int(m.group(1)) == qsa.ABI_VERSION


def test_launch_events_set_and_clear_without_device(lib):
    assert lib.qsa_set_launch_events(None, None) == 0


def _err(lib):
    return lib.qsa_last_error().decode()


FAKE = 0x100000  # never dereferenced: every call below fails its checks first


def _decode(lib, **kw):
    a = dict(q=FAKE, sr=512, sj=512, sh=128, k=FAKE, num_pages=4, page_size=16, pt=FAKE,
             pt_stride=4, pt_cols=4, comp=FAKE, vis=None, num_reqs=1, dql=1, heads=4, dim=128,
             scale=0.088, out=FAKE, out_stride=64, out_cols=64)
    a.update(kw)
    return lib.qsa_mqa_decode(a["q"], a["sr"], a["sj"], a["sh"], a["k"], a["num_pages"],
                              a["page_size"], a["pt"], a["pt_stride"], a["pt_cols"], a["comp"],
                              a["vis"], a["num_reqs"], a["dql"], a["heads"], a["dim"], a["scale"],
                              a["out"], a["out_stride"], a["out_cols"], None)


@pytest.mark.parametrize("kw,code,text", [
    (dict(heads=8), 2, "(4, 128)"),
    (dict(dim=64), 2, "(4, 128)"),
    (dict(scale=0.0), 1, "scale"),
    (dict(scale=float("nan")), 1, "scale"),
    (dict(scale=float("inf")), 1, "scale"),
    (dict(scale=-1.0), 1, "scale"),
    (dict(dql=0), 1, "dql"),
    (dict(dql=17), 1, "dql"),
    (dict(page_size=0), 1, "page_size"),
    (dict(page_size=(1 << 20) + 1), 1, "page_size"),
    (dict(out_stride=10), 1, "out_stride"),
    (dict(num_reqs=-1), 1, "negative"),
    (dict(out_cols=-5, out_stride=0), 1, "negative"),
    (dict(num_reqs=2, pt_stride=2), 1, "page_table_stride"),
    (dict(q=None), 1, "NULL"),
    (dict(comp=None), 1, "NULL"),
    (dict(out=None), 1, "NULL"),
    (dict(k=None), 1, "k_cache"),
    (dict(pt=None), 1, "page_table"),
    (dict(k=FAKE + 8), 3, "aligned"),
    (dict(out=FAKE + 2), 3, "aligned"),
])
def test_decode_rejects(lib, kw, code, text):
    assert _decode(lib, **kw) == code
    assert text in _err(lib)


def _decode_typed(lib, q_dtype=0, k_dtype=0, k_scale=1.0, **kw):
    a = dict(q=FAKE, sr=512, sj=512, sh=128, k=FAKE, num_pages=4, page_size=16, pt=FAKE,
             pt_stride=4, pt_cols=4, comp=FAKE, vis=None, num_reqs=1, dql=1, heads=4, dim=128,
             scale=0.088, out=FAKE, out_stride=64, out_cols=64)
    a.update(kw)
    return lib.qsa_mqa_decode_typed(a["q"], q_dtype, a["sr"], a["sj"], a["sh"], a["k"], k_dtype, k_scale,
                                    a["num_pages"], a["page_size"], a["pt"], a["pt_stride"], a["pt_cols"],
                                    a["comp"], a["vis"], a["num_reqs"], a["dql"], a["heads"], a["dim"],
                                    a["scale"], a["out"], a["out_stride"], a["out_cols"], None)


@pytest.mark.parametrize("kw,code,text", [
    (dict(q_dtype=2, k_dtype=2), 2, "query format"),
    (dict(q_dtype=5), 2, "query format"),
    (dict(q_dtype=0, k_dtype=1), 2, "key format"),
    (dict(q_dtype=1, k_dtype=0), 2, "key format"),
    (dict(k_dtype=3), 2, "key format"),
    (dict(k_dtype=2, k_scale=0.0), 1, "k_scale"),
    (dict(k_dtype=2, k_scale=-1.0), 1, "k_scale"),
    (dict(k_dtype=2, k_scale=float("nan")), 1, "k_scale"),
    (dict(k_dtype=2, k_scale=float("inf")), 1, "k_scale"),
    (dict(k_dtype=2, k_scale=1e30, scale=1e30), 1, "scale * k_scale"),
    (dict(k_dtype=2, k_scale=1e-30, scale=1e-30), 1, "scale * k_scale"),
    (dict(k_dtype=2, k_scale=0.5, heads=8), 2, "(4, 128)"),
    (dict(k_dtype=2, k_scale=0.5, k=FAKE + 8), 3, "aligned"),
    (dict(q_dtype=1, k_dtype=1, dql=0), 1, "dql"),
])
def test_decode_typed_rejects(lib, kw, code, text):
    assert _decode_typed(lib, **kw) == code
    assert text in _err(lib)
    assert "qsa_mqa_decode_typed" in _err(lib)


def test_decode_typed_zero_work_and_ignored_scale(lib):
    # 16-bit keys ignore k_scale; zero work returns OK with no device call.
    assert _decode_typed(lib, q_dtype=1, k_dtype=1, k_scale=float("nan"), num_reqs=0, q=None) == 0
    assert _decode_typed(lib, q_dtype=0, k_dtype=2, k_scale=0.0125, out_cols=0, out_stride=0) == 0
    assert _err(lib) == ""


def _prefill_typed(lib, dtype, **kw):
    a = dict(q=FAKE, sq=512, sh=128, k=FAKE, sk=128, nk=100, ks=FAKE, ke=FAKE, rows=10, heads=4,
             dim=128, scale=0.088, out=FAKE, out_stride=100, out_cols=100)
    a.update(kw)
    return lib.qsa_mqa_prefill_typed(a["q"], a["sq"], a["sh"], a["k"], a["sk"], a["nk"], dtype, a["ks"],
                                     a["ke"], a["rows"], a["heads"], a["dim"], a["scale"], a["out"],
                                     a["out_stride"], a["out_cols"], None)


@pytest.mark.parametrize("dtype,kw,code,text", [
    (2, {}, 2, "format 2"),
    (-1, {}, 2, "format -1"),
    (1, dict(heads=2), 2, "(4, 128)"),
    (1, dict(out_stride=99), 1, "out_stride"),
    (1, dict(q=FAKE + 2), 3, "16-byte"),
])
def test_prefill_typed_rejects(lib, dtype, kw, code, text):
    assert _prefill_typed(lib, dtype, **kw) == code
    assert text in _err(lib)
    assert "qsa_mqa_prefill_typed" in _err(lib)


def _cache_meta(lib, **kw):
    a = dict(qsl=FAKE, seq=FAKE, num_reqs=3, num_tokens=10, cr=4, bt=FAKE, bt_stride=8, bt_cols=8, sbs=64,
             common=None, slots=FAKE, work=FAKE, max_work=16)
    a.update(kw)
    return lib.qsa_build_cache_metadata(a["qsl"], a["seq"], a["num_reqs"], a["num_tokens"], a["cr"], a["bt"],
                                        a["bt_stride"], a["bt_cols"], a["sbs"], a["common"], a["slots"], a["work"],
                                        a["max_work"], None)


@pytest.mark.parametrize("kw,code,text", [
    (dict(num_reqs=-1), 1, "negative"),
    (dict(max_work=-1), 1, "negative"),
    (dict(cr=0), 1, "compress_ratio"),
    (dict(sbs=0), 1, "storage_block_size"),
    (dict(bt_stride=4), 1, "block_table_stride"),
    (dict(qsl=None), 1, "query_start_loc"),
    (dict(seq=None), 1, "seq_lens"),
    (dict(bt=None), 1, "block_table"),
    (dict(num_reqs=9000), 2, "8192"),
])
def test_cache_metadata_rejects(lib, kw, code, text):
    assert _cache_meta(lib, **kw) == code
    assert text in _err(lib)


def test_cache_metadata_nothing_to_do(lib):
    assert _cache_meta(lib, slots=None, work=None, qsl=None) == 0
    assert _cache_meta(lib, num_tokens=0, max_work=0, qsl=None) == 0
    assert _err(lib) == ""


def _gather(lib, **kw):
    a = dict(k=FAKE, fmt=0, pages=8, ps=64, pt=FAKE, pt_stride=4, pt_cols=4, counts=FAKE, offs=FAKE, num_reqs=2,
             max_keys=256, out=FAKE, out_fmt=None, out_stride=128, out_rows=512)
    a.update(kw)
    out_fmt = a["fmt"] if a["out_fmt"] is None else a["out_fmt"]
    return lib.qsa_gather_keys(a["k"], a["fmt"], a["pages"], a["ps"], a["pt"], a["pt_stride"], a["pt_cols"],
                               a["counts"], a["offs"], a["num_reqs"], a["max_keys"], a["out"], out_fmt,
                               a["out_stride"], a["out_rows"], None)


@pytest.mark.parametrize("kw,code,text", [
    (dict(fmt=3), 2, "key format"),
    (dict(num_reqs=-1), 1, "negative"),
    (dict(ps=0), 1, "page_size"),
    (dict(max_keys=(1 << 30) + 1), 1, "max_keys"),
    (dict(out_stride=100), 1, "k_out_stride"),
    (dict(pt_stride=2), 1, "page_table_stride"),
    (dict(counts=None), 1, "NULL"),
    (dict(out=None), 1, "NULL"),
    (dict(k=None), 1, "k_cache"),
    (dict(pt=None), 1, "page_table"),
    (dict(k=FAKE + 8), 3, "aligned"),
    (dict(out=FAKE + 4), 3, "aligned"),
    (dict(out_stride=132), 3, "aligned"),
    (dict(fmt=2, out_stride=136), 3, "aligned"),
    (dict(fmt=0, out_fmt=1), 2, "output format"),
    (dict(fmt=1, out_fmt=2), 2, "output format"),
    (dict(fmt=2, out_fmt=7), 2, "output format"),
    (dict(fmt=2, out_fmt=0, out_stride=132), 3, "aligned"),
])
def test_gather_rejects(lib, kw, code, text):
    assert _gather(lib, **kw) == code
    assert text in _err(lib)


def test_gather_nothing_to_do(lib):
    assert _gather(lib, num_reqs=0, counts=None, out=None) == 0
    assert _gather(lib, max_keys=0, counts=None) == 0
    assert _gather(lib, fmt=2, out_stride=144, out_rows=0) == 0
    assert _err(lib) == ""


def _prepare(lib, **kw):
    import ctypes
    a = dict(q=FAKE, qs=512, T=64, H=4, pos=FAKE, pa=0, pt=1, cs=FAKE, csf=0, rows=1000, w=FAKE, wf=0,
             eps=1e-6, sec=None, out=FAKE, outf=0, scale=1.0, ost=512, osh=128)
    a.update(kw)
    sec = None
    if a["sec"] is not None:
        sec = (ctypes.c_int32 * 3)(*a["sec"])
    return lib.qsa_prepare_q(a["q"], a["qs"], a["T"], a["H"], a["pos"], a["pa"], a["pt"], a["cs"], a["csf"],
                             a["rows"], a["w"], a["wf"], a["eps"], None if sec is None else ctypes.addressof(sec),
                             a["out"], a["outf"], a["scale"], a["ost"], a["osh"], None)


@pytest.mark.parametrize("kw,code,text", [
    (dict(csf=1), 2, "cos/sin table format"),
    (dict(csf=2), 2, "cos/sin table format"),
    (dict(wf=2), 2, "norm weight format"),
    (dict(outf=1), 2, "output format"),
    (dict(outf=3), 2, "output format"),
    (dict(T=-1), 1, "negative"),
    (dict(rows=-1), 1, "negative"),
    (dict(cs=None, rows=-1), 1, "negative"),
    (dict(rows=1 << 24), 1, "table above"),
    (dict(csf=3, rows=1 << 23), 1, "table above"),
    (dict(T=1 << 29, H=4), 1, "too large"),
    (dict(H=0), 1, "num_heads"),
    (dict(H=1025), 1, "num_heads"),
    (dict(eps=float("nan")), 1, "eps"),
    (dict(eps=float("inf")), 1, "eps"),
    (dict(outf=2, scale=0.0), 1, "out_scale"),
    (dict(outf=2, scale=float("inf")), 1, "out_scale"),
    (dict(sec=(16, 8, 9)), 1, "MRoPE section"),
    (dict(sec=(34, -1, -1)), 1, "MRoPE section"),
    (dict(qs=256), 1, "q_stride_token"),
    (dict(q=None), 1, "NULL"),
    (dict(pos=None), 1, "NULL"),
    (dict(cs=None), 1, "NULL"),
    (dict(w=None), 1, "NULL"),
    (dict(out=None), 1, "NULL"),
    (dict(q=FAKE + 8), 3, "aligned"),
    (dict(qs=516), 3, "aligned"),
    (dict(cs=FAKE + 4), 3, "aligned"),
    (dict(w=FAKE + 8), 3, "aligned"),
    (dict(pos=FAKE + 4), 3, "aligned"),
    (dict(out=FAKE + 8), 3, "aligned"),
    (dict(outf=2, out=FAKE + 4), 3, "aligned"),
    (dict(ost=516), 3, "aligned"),
    (dict(osh=132), 3, "aligned"),
])
def test_prepare_q_rejects(lib, kw, code, text):
    assert _prepare(lib, **kw) == code
    assert text in _err(lib)


def test_prepare_q_nothing_to_do(lib):
    assert _prepare(lib, T=0, q=None, pos=None, cs=None, w=None, out=None) == 0
    assert _prepare(lib, T=0, sec=(16, 8, 8), pa=1) == 0
    assert _err(lib) == ""


def _planned(lib, plan=FAKE, plan_bytes=1 << 20, q_dtype=0, k_dtype=0, k_scale=1.0, **kw):
    a = dict(q=FAKE, sr=512, sj=512, sh=128, k=FAKE, num_pages=4, page_size=64, pt=None,
             pt_stride=0, pt_cols=0, vis=None, num_reqs=2, dql=4, heads=4, dim=128,
             scale=0.088, out=FAKE, out_stride=200, out_cols=200)
    a.update(kw)
    return lib.qsa_mqa_decode_planned(plan, plan_bytes, a["q"], q_dtype, a["sr"], a["sj"], a["sh"], a["k"],
                                      k_dtype, k_scale, a["num_pages"], a["page_size"], a["pt"], a["pt_stride"],
                                      a["pt_cols"], a["vis"], a["num_reqs"], a["dql"], a["heads"], a["dim"],
                                      a["scale"], a["out"], a["out_stride"], a["out_cols"], None)


@pytest.mark.parametrize("kw,code,text", [
    (dict(plan=None), 1, "NULL plan"),
    (dict(plan_bytes=2 * 4 * 16 - 1), 1, "needed"),
    (dict(plan=FAKE + 4), 3, "plan must be 16-byte aligned"),
    (dict(heads=8), 2, "(4, 128)"),
    (dict(dql=0), 1, "dql"),
    (dict(q_dtype=2, k_dtype=2), 2, "query format"),
    (dict(k_dtype=2, k_scale=0.0), 1, "k_scale"),
    (dict(out=None), 1, "NULL q or out"),
    (dict(pt_cols=3), 1, "page_table"),
])
def test_decode_planned_rejects(lib, kw, code, text):
    assert _planned(lib, **kw) == code
    assert text in _err(lib)
    assert "qsa_mqa_decode_planned" in _err(lib)


def test_decode_static_plan_capacity_checked_on_the_host(lib):
    """Beyond the library's 262,144-entry table the call is refused before
    any device work (the pointers here are never dereferenced)."""
    def call(num_reqs, out_cols):
        return lib.qsa_mqa_decode_static_plan(FAKE, 0, 512, 512, 128, FAKE, 0, 1.0, 4, 64, FAKE, 4, 4, FAKE,
                                              None, num_reqs, 1, 4, 128, 0.088, FAKE, out_cols, out_cols, None)
    assert call(1025, 256 * 64) == 2
    assert "262144" in _err(lib) and "qsa_mqa_decode_static_plan" in _err(lib)
    assert call(4097, 64) == 2 and "4096" in _err(lib)
    assert call(0, 64) == 0


def test_decode_planned_zero_work_and_plan_size(lib):
    assert _planned(lib, num_reqs=0, plan=None, q=None, out=None) == 0
    assert _planned(lib, out_cols=0, out_stride=0, plan=None) == 0
    n = ctypes.c_int64(-1)
    assert lib.qsa_decode_plan_bytes(16, 25600, ctypes.byref(n)) == 0 and n.value == 16 * 400 * 16
    assert lib.qsa_decode_plan_bytes(3, 65, ctypes.byref(n)) == 0 and n.value == 3 * 2 * 16
    assert lib.qsa_decode_plan_bytes(0, 100, ctypes.byref(n)) == 0 and n.value == 0
    assert lib.qsa_decode_plan_bytes(-1, 100, ctypes.byref(n)) == 1
    assert lib.qsa_decode_plan_bytes(1, 100, None) == 1


def _build_plan(lib, **kw):
    a = dict(comp=FAKE, pt=FAKE, pt_stride=8, pt_cols=8, num_pages=100, page_size=64, num_reqs=2, out_cols=200,
             plan=FAKE, plan_bytes=1 << 20)
    a.update(kw)
    return lib.qsa_build_decode_plan(a["comp"], a["pt"], a["pt_stride"], a["pt_cols"], a["num_pages"],
                                     a["page_size"], a["num_reqs"], a["out_cols"], a["plan"], a["plan_bytes"], None)


@pytest.mark.parametrize("kw,code,text", [
    (dict(num_reqs=-1), 1, "negative"),
    (dict(page_size=0), 1, "page_size"),
    (dict(num_reqs=3, pt_stride=4), 1, "page_table_stride"),
    (dict(num_reqs=4097), 2, "4096"),
    (dict(comp=None), 1, "NULL"),
    (dict(plan=None), 1, "NULL"),
    (dict(pt=None), 1, "page_table"),
    (dict(plan=FAKE + 8), 3, "aligned"),
    (dict(plan_bytes=2 * 4 * 16 - 16), 1, "needed"),
])
def test_build_decode_plan_rejects(lib, kw, code, text):
    assert _build_plan(lib, **kw) == code
    assert text in _err(lib)


def test_build_decode_plan_nothing_to_do(lib):
    assert _build_plan(lib, num_reqs=0, comp=None, plan=None) == 0
    assert _build_plan(lib, out_cols=0, comp=None, plan=None) == 0


@pytest.mark.parametrize("args,code,text", [
    ((FAKE, -1, 4), 1, "num_reqs"),
    ((FAKE, 3, 0), 1, "dql"),
    ((FAKE, 3, 17), 1, "dql"),
    ((None, 3, 4), 1, "NULL seq_lens"),
])
def test_decode_visible_blocks_rejects(lib, args, code, text):
    assert lib.qsa_decode_visible_blocks(args[0], args[1], args[2], FAKE, FAKE, None) == code
    assert text in _err(lib)


def test_decode_visible_blocks_nothing_to_do(lib):
    assert lib.qsa_decode_visible_blocks(None, 0, 4, FAKE, FAKE, None) == 0
    assert lib.qsa_decode_visible_blocks(None, 5, 4, None, None, None) == 0


def _write_keys(lib, **kw):
    a = dict(keys=FAKE, ks=128, T=10, slots=FAKE, cache=FAKE, dtype=0, rs=128, ns=100, scale=1.0, pos=None, pa=0, pt=0)
    a.update(kw)
    return lib.qsa_write_keys(a["keys"], a["ks"], a["T"], a["slots"], a["cache"], a["dtype"], a["rs"], a["ns"],
                              a["scale"], a["pos"], a["pa"], a["pt"], None)


@pytest.mark.parametrize("kw,code,text", [
    (dict(dtype=1), 2, "cache format"),
    (dict(dtype=3), 2, "cache format"),
    (dict(dtype=2, pos=FAKE, rs=140), 2, "positions"),
    (dict(dtype=2, scale=0.0), 1, "scale"),
    (dict(dtype=2, scale=float("nan")), 1, "scale"),
    (dict(T=-1), 1, "negative"),
    (dict(ns=-1), 1, "negative"),
    (dict(rs=120), 1, "row_stride"),
    (dict(rs=136, pos=FAKE), 1, "row_stride"),
    (dict(ks=64), 1, "key_stride"),
    (dict(keys=None), 1, "NULL"),
    (dict(slots=None), 1, "NULL"),
    (dict(cache=None), 1, "NULL"),
    (dict(keys=FAKE + 4), 3, "aligned"),
    (dict(ks=130), 3, "aligned"),
    (dict(rs=130), 3, "aligned"),
    (dict(cache=FAKE + 2), 3, "aligned"),
])
def test_write_keys_rejects(lib, kw, code, text):
    assert _write_keys(lib, **kw) == code
    assert text in _err(lib)


def test_write_keys_and_ring_slots_nothing_to_do(lib):
    assert _write_keys(lib, T=0, keys=None, slots=None, cache=None) == 0
    assert _write_keys(lib, ns=0, keys=None, slots=None, cache=None) == 0
    assert lib.qsa_build_ring_slots(None, None, 0, 0, None, 0, 0, 8, None, None) == 0


@pytest.mark.parametrize("args,code,text", [
    ((FAKE, FAKE, -1, 4, FAKE, 2, 2, 8, FAKE), 1, "negative"),
    ((FAKE, FAKE, 2, 4, FAKE, 2, 2, 0, FAKE), 1, "ring_size"),
    ((FAKE, FAKE, 2, 4, FAKE, 1, 2, 8, FAKE), 1, "block_table_stride"),
    ((None, FAKE, 2, 4, FAKE, 2, 2, 8, FAKE), 1, "NULL"),
    ((FAKE, FAKE, 2, 4, FAKE, 2, 2, 8, None), 1, "NULL"),
    ((FAKE, None, 2, 4, FAKE, 2, 2, 8, FAKE), 1, "NULL seq_lens"),
    ((FAKE, FAKE, 2, 4, None, 2, 2, 8, FAKE), 1, "NULL block_table"),
])
def test_ring_slots_rejects(lib, args, code, text):
    assert lib.qsa_build_ring_slots(*args, None) == code
    assert text in _err(lib)


def test_decode_zero_work_is_ok_without_device(lib):
    assert _decode(lib, num_reqs=0, q=None, comp=None, out=None) == 0
    assert _decode(lib, out_cols=0, out_stride=0, q=None, out=None) == 0
    assert _err(lib) == ""


def _prefill(lib, **kw):
    a = dict(q=FAKE, sq=512, sh=128, k=FAKE, sk=128, nk=100, ks=FAKE, ke=FAKE, rows=10, heads=4,
             dim=128, scale=0.088, out=FAKE, out_stride=100, out_cols=100)
    a.update(kw)
    return lib.qsa_mqa_prefill(a["q"], a["sq"], a["sh"], a["k"], a["sk"], a["nk"], a["ks"], a["ke"],
                               a["rows"], a["heads"], a["dim"], a["scale"], a["out"],
                               a["out_stride"], a["out_cols"], None)


@pytest.mark.parametrize("kw,code,text", [
    (dict(heads=2), 2, "(4, 128)"),
    (dict(scale=0.0), 1, "scale"),
    (dict(out_stride=99), 1, "out_stride"),
    (dict(rows=-1), 1, "negative"),
    (dict(nk=-1), 1, "negative"),
    (dict(q=None), 1, "NULL"),
    (dict(ks=None), 1, "NULL"),
    (dict(k=None), 1, "NULL k"),
    (dict(q=FAKE + 2), 3, "16-byte"),
    (dict(k=FAKE + 4), 3, "16-byte"),
    (dict(sq=516), 3, "multiples"),
    (dict(sq=0), 3, "multiples"),
    (dict(sh=130), 3, "multiples"),
    (dict(sh=0), 3, "multiples"),
    (dict(sk=132), 3, "multiples"),
    (dict(sk=-128), 3, "multiples"),
    (dict(out=FAKE + 1), 3, "aligned"),
    # Key offsets inside the kernel are 32-bit: strides past 2^22 elements
    # (8 MiB per key row) are refused before any launch.
    (dict(sk=(1 << 22) + 8), 2, "k_stride"),
])
def test_prefill_rejects(lib, kw, code, text):
    assert _prefill(lib, **kw) == code
    assert text in _err(lib)


def _fused(lib, **kw):
    a = dict(q=FAKE, sq=512, sh=128, k=FAKE, sk=128, nk=100, ks=FAKE, ke=FAKE, rows=10, heads=4,
             dim=128, scale=0.088, out_cols=100, topk=16, out=FAKE, out_stride=16, ws=FAKE, ws_bytes=1 << 40)
    a.update(kw)
    return lib.qsa_mqa_prefill_topk(a["q"], a["sq"], a["sh"], a["k"], a["sk"], a["nk"], a["ks"], a["ke"],
                                    a["rows"], a["heads"], a["dim"], a["scale"], a["out_cols"], a["topk"],
                                    a["out"], a["out_stride"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code,text", [
    (dict(heads=2), 2, "(4, 128)"),
    (dict(scale=float("nan")), 1, "scale"),
    (dict(topk=0), 1, "topk"),
    (dict(topk=2049, out_stride=4096), 1, "topk"),
    (dict(out_stride=15), 1, "out_stride"),
    (dict(rows=-1), 1, "negative"),
    (dict(out=None), 1, "NULL"),
    (dict(ws=None), 1, "NULL"),
    (dict(out=FAKE + 2), 3, "aligned"),
    (dict(ws=FAKE + 16), 3, "256-byte"),
    (dict(ws_bytes=1000), 1, "needed"),
    (dict(q=None), 1, "NULL"),
    (dict(k=FAKE + 4), 3, "16-byte"),
    # Rows of at most 32,768 columns take the score-key path, whose key
    # offsets are the prefill's; wider rows take the group-maximum path,
    # whose chunks hold at most 2^14-element key strides.
    (dict(sk=(1 << 22) + 8), 2, "k_stride"),
    (dict(out_cols=40000, sk=(1 << 14) + 8), 2, "k_stride"),
])
def test_fused_prefill_topk_rejects(lib, kw, code, text):
    assert _fused(lib, **kw) == code
    assert text in _err(lib)


def _fused_typed(lib, dtype, **kw):
    a = dict(q=FAKE, sq=512, sh=128, k=FAKE, sk=128, nk=100, ks=FAKE, ke=FAKE, rows=10, heads=4,
             dim=128, scale=0.088, out_cols=100, topk=16, out=FAKE, out_stride=16, ws=FAKE, ws_bytes=1 << 40)
    a.update(kw)
    return lib.qsa_mqa_prefill_topk_typed(a["q"], a["sq"], a["sh"], a["k"], a["sk"], a["nk"], dtype, a["ks"],
                                          a["ke"], a["rows"], a["heads"], a["dim"], a["scale"], a["out_cols"],
                                          a["topk"], a["out"], a["out_stride"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("dtype,kw,code,text", [
    (2, {}, 2, "format"),                                   # e4m3 queries and keys: not a prefill format
    (3, {}, 2, "format"),
    (1, dict(out_cols=40000), 2, "fp16 rows wider"),        # fp16 takes the key-prefix path only
    (1, dict(topk=0), 1, "topk"),
    (1, dict(ws_bytes=1000), 1, "needed"),
    (1, dict(rows=0, q=None, out=None, ws=None), 0, ""),
])
def test_fused_prefill_topk_typed_rejects(lib, dtype, kw, code, text):
    assert _fused_typed(lib, dtype, **kw) == code
    if code:
        assert text in _err(lib)


def test_fused_prefill_topk_zero_rows_and_workspace_size(lib):
    assert _fused(lib, rows=0, q=None, out=None, ws=None) == 0
    n = ctypes.c_int64(-1)
    assert lib.qsa_prefill_topk_workspace_bytes(8192, 27048, 512, ctypes.byref(n)) == 0
    # The cells' 16-bit key prefixes on rows padded to 64 columns, plus the
    # fallback's 64 fp32 scratch rows: half the 886 MB score matrix, under
    # the 512 MiB logits workspace.
    assert 8192 * 27072 * 2 + 64 * 27072 * 4 <= n.value < 8192 * 27072 * 2 + 8 * 2**20
    assert n.value < 512 * 2**20
    w = ctypes.c_int64(-1)
    # Wider rows: group maxima of 8-key groups (4 B each) and a candidate
    # pool of 8 (k - 1) + chunks * k 8-byte entries per row.
    assert lib.qsa_prefill_topk_workspace_bytes(1024, 40000, 512, ctypes.byref(w)) == 0
    assert 1024 * 8 * (8 * 511 + 512) < w.value
    m = ctypes.c_int64(-1)
    assert lib.qsa_prefill_topk_workspace_bytes(100, 27048, 512, ctypes.byref(m)) == 0
    assert 0 < m.value < n.value
    assert lib.qsa_prefill_topk_workspace_bytes(100, 1000, 0, ctypes.byref(m)) == 1
    assert lib.qsa_prefill_topk_workspace_bytes(100, 1000, 16, None) == 1
    assert lib.qsa_prefill_topk_workspace_bytes(-1, 1000, 16, ctypes.byref(m)) == 1


def test_prefill_layout_exemptions_for_single_element_axes(lib):
    # An axis of one element is exempt from the stride rule; nothing to
    # compute (out_cols 0) so no launch happens.
    assert _prefill(lib, rows=1, sq=3, out_cols=0, out_stride=0) == 0
    assert _prefill(lib, rows=0, q=None) == 0


@pytest.mark.parametrize("args,code,text", [
    ((FAKE, 10, 2, 10, 0, FAKE, 4), 1, "k must"),
    ((FAKE, 10, 2, 10, (1 << 20) + 1, FAKE, 1 << 21), 1, "k must"),
    ((FAKE, 9, 2, 10, 4, FAKE, 4), 1, "logits_stride"),
    ((FAKE, 10, 2, 10, 4, FAKE, 3), 1, "out_stride"),
    ((FAKE, 10, -2, 10, 4, FAKE, 4), 1, "negative"),
    ((None, 10, 2, 10, 4, FAKE, 4), 1, "NULL"),
    ((FAKE, 10, 2, 10, 4, None, 4), 1, "NULL"),
    ((FAKE + 2, 10, 2, 10, 4, FAKE, 4), 3, "aligned"),
])
def test_topk_rejects(lib, args, code, text):
    assert lib.qsa_topk_blocks(*args, None) == code
    assert text in _err(lib)


def test_metadata_rejects(lib):
    assert lib.qsa_build_metadata(FAKE, FAKE, -1, 4, 4, None, None, None, None, None, None, None, None) == 1
    assert lib.qsa_build_metadata(FAKE, FAKE, 1, 4, 0, None, None, None, None, None, None, None, None) == 1
    assert "compress_ratio" in _err(lib)
    assert lib.qsa_build_metadata(None, FAKE, 1, 4, 4, None, None, None, None, None, None, None, None) == 1
    assert lib.qsa_build_metadata(FAKE, FAKE, 1, 4, 4, FAKE, None, None, None, None, None, None, None) == 1
    assert "key_offsets" in _err(lib)
    assert lib.qsa_build_metadata(FAKE, FAKE, 1, 4, 4, None, None, None, None, None, FAKE, None, None) == 1
    assert lib.qsa_build_metadata(FAKE, None, 0, 0, 4, None, None, None, None, None, None, None, None) == 0


def test_split_batch_matches_oracle(lib):
    from block_indexer_scoring_amd import qsa
    rng = np.random.default_rng(1)
    for _ in range(300):
        R = int(rng.integers(0, 12))
        lens = rng.choice([0, 1, 2, 3, 4, 5, 9, 40], size=R, p=[.1, .2, .1, .05, .3, .05, .1, .1])
        qsl = [0] + np.cumsum(lens).tolist()
        thr = int(rng.integers(1, 6))
        for reorder in (False, True):
            assert qsa.qsa_split_batch(qsl, thr, reorder) == O.split_batch(qsl, thr, reorder), (qsl, thr)


def test_split_batch_rejects(lib):
    counts = (ctypes.c_int32 * 5)()
    bad = (ctypes.c_int32 * 3)(0, 5, 4)
    assert lib.qsa_split_batch(ctypes.addressof(bad), 2, 4, None, ctypes.addressof(counts)) == 1
    assert "decreases" in _err(lib)
    good = (ctypes.c_int32 * 3)(0, 4, 8)
    assert lib.qsa_split_batch(ctypes.addressof(good), 2, 0, None, ctypes.addressof(counts)) == 1
    assert lib.qsa_split_batch(None, 2, 4, None, ctypes.addressof(counts)) == 1
    assert lib.qsa_split_batch(ctypes.addressof(good), 2, 4, None, ctypes.addressof(counts)) == 0
    assert list(counts) == [2, 8, 0, 0, 4]


def test_binding_refuses_cpu_tensors(lib):
    import torch
    from block_indexer_scoring_amd import qsa
    q = torch.zeros((1, 1, 4, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        qsa.qsa_mqa_decode(q, q, torch.zeros((1, 1), dtype=torch.int32),
                           torch.zeros(1, dtype=torch.int32), out_cols=4)
    with pytest.raises(ValueError, match="GPU"):
        qsa.qsa_topk_blocks(torch.zeros((2, 3)), 1)


def test_bench_direct_calls_match_the_abi(lib):
    """bench.py calls the library directly (to time launches without Python
    wrappers); each such call must pass as many arguments as the declared
    signature has."""
    import ast
    src = open(os.path.join(ROOT, "bench.py")).read()
    calls = [n for n in ast.walk(ast.parse(src)) if isinstance(n, ast.Call) and isinstance(n.func, ast.Attribute)
             and isinstance(n.func.value, ast.Name) and n.func.value.id == "lib" and n.func.attr.startswith("qsa_")]
    assert len(calls) >= 8
    for c in calls:
        want = len(getattr(lib, c.func.attr).argtypes)
        assert len(c.args) == want, f"bench.py line {c.lineno}: {c.func.attr} takes {want} arguments, given {len(c.args)}"


def test_error_text_is_per_thread(lib):
    """The last-error text is thread-local: threads that fail different checks
    at the same time each read back their own message."""
    import threading
    results, barrier = {}, threading.Barrier(8)

    def worker(i):
        barrier.wait()
        for _ in range(200):
            if i % 2:
                rc = _decode(lib, dql=0)
                ok = rc == 1 and "dql" in _err(lib)
            else:
                rc = _prefill(lib, heads=2)
                ok = rc == 2 and "(4, 128)" in _err(lib)
            if not ok:
                results[i] = False
                return
        results[i] = True

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert all(results.get(i) for i in range(8)), results
