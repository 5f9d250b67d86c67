"""The C-ABI library loads, exports every function include/csa_attn.h
declares, and rejects bad arguments on the host before any HIP call (CPU
only: every call here fails validation, so no kernel is launched)."""
import ctypes as C
import os
import re

import pytest

from long_context_attention_23_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = C.c_void_p(4096)          # never dereferenced: validation fails first


def header_functions():
    text = open(os.path.join(ROOT, "include", "csa_attn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:csa_status|size_t|const char\*)\s+(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    return api.lib()


def test_exports_every_declared_symbol(L):
    names = header_functions()
    assert len(names) == 10
    assert sorted(names) == sorted(api.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_record_bytes(L):
    assert L.csa_kv_record_bytes(api.FP8_E4M3, 512, 64) == 592
    assert L.csa_kv_record_bytes(api.BF16, 512, 64) == 1024
    assert L.csa_kv_record_bytes(api.F32, 128, 64) == 512
    assert L.csa_kv_record_bytes(api.FP8_E4M3, 128, 64) == 64 + 128 + 4 + 12
    assert L.csa_kv_record_bytes(api.FP4_E2M1, 64, 0) == 0
    assert L.csa_kv_record_bytes(api.F32, 8, 10) == 0


def kv(fmt=api.FP8_E4M3, d=512, dr=64, ring=0, cap=16, rec=FAKE.value):
    return api.KVCacheT(rec, fmt, d, dr, ring, cap)


def idx(fmt=api.FP4_E2M1, di=64, cap=16, codes=FAKE.value, scales=FAKE.value):
    return api.IdxCacheT(codes, scales, fmt, di, cap)


def status_and_msg(L, st):
    return st, L.csa_last_error().decode()


def compress(L, **over):
    a = dict(x=FAKE, x_dtype=api.BF16, B=2, T=8, d=512, tok=FAKE, m=4, bias=FAKE, proj=None, gamma=None,
             eps=1e-6, dr=64, base=10000.0, kv_out=C.byref(kv()), idx_out=None)
    a.update(over)
    return status_and_msg(L, L.csa_compress_kv(a["x"], a["x_dtype"], a["B"], a["T"], a["d"], a["tok"], a["m"],
                                               a["bias"], a["proj"], a["gamma"], a["eps"], a["dr"], a["base"],
                                               a["kv_out"], a["idx_out"], None))


@pytest.mark.parametrize("over,code,frag", [
    (dict(d=513), 1, "even"),
    (dict(d=2048), 1, "[2, 1024]"),
    (dict(m=0), 1, "m 0"),
    (dict(B=-1), 1, "bad sizes"),
    (dict(dr=3), 1, "rope_dim"),
    (dict(x_dtype=api.FP8_E4M3), 2, "x dtype"),
    (dict(kv_out=None), 1, "exactly one"),
    (dict(idx_out="both"), 1, "exactly one"),
    (dict(kv_out="fp4"), 2, "kv_out fmt"),
    (dict(kv_out="wrong_d"), 1, "differ"),
    (dict(x=None), 1, "is null"),
    (dict(bias=None), 1, "is null"),
])
def test_compress_validation(L, over, code, frag):
    if over.get("idx_out") == "both":
        over["idx_out"] = C.byref(idx())
    if over.get("kv_out") == "fp4":
        over["kv_out"] = C.byref(kv(fmt=api.FP4_E2M1))
    if over.get("kv_out") == "wrong_d":
        over["kv_out"] = C.byref(kv(d=256))
    st, msg = compress(L, **over)
    assert st == code and frag in msg, (st, msg)


def test_compress_idx_validation(L):
    st, msg = compress(L, d=48, dr=0, kv_out=None, idx_out=C.byref(idx(di=48)))
    assert st == 2 and "FP4" in msg
    st, msg = compress(L, d=64, dr=0, kv_out=None, idx_out=C.byref(idx(scales=None)))
    assert st == 1 and "FP4" in msg
    st, msg = compress(L, d=64, dr=0, kv_out=None, idx_out=C.byref(idx(di=32)))
    assert st == 1 and "differs" in msg


def test_compress_empty_is_ok(L):
    st, msg = compress(L, T=3)          # T < m: no complete block, nothing launched
    assert st == 0 and msg == ""


def job(**over):
    kvs = over.pop("kv_struct", kv())
    a = dict(x=FAKE.value, B=2, T=8, d=512, tok_start=FAKE.value, m=4, score_bias=FAKE.value, score_proj=None,
             gamma=None, eps=1e-6, rope_dim=64, rope_base=10000.0, kv_out=C.pointer(kvs), idx_out=None)
    a.update(over)
    return api.CompressJobT(**a), kvs


def test_compress_batch_validation(L):
    st, msg = status_and_msg(L, L.csa_compress_kv_batch(None, 2, api.BF16, None))
    assert st == 1 and "njobs" in msg
    st, msg = status_and_msg(L, L.csa_compress_kv_batch(None, -1, api.BF16, None))
    assert st == 1 and "njobs" in msg
    st, msg = status_and_msg(L, L.csa_compress_kv_batch(None, 0, api.BF16, None))
    assert st == 0
    # one bad job among good ones: the whole call fails before any launch
    good, k0 = job()
    bad, k1 = job(d=513, kv_struct=kv(d=513))
    arr = (api.CompressJobT * 2)(good, bad)
    st, msg = status_and_msg(L, L.csa_compress_kv_batch(arr, 2, api.BF16, None))
    assert st == 1 and "even" in msg
    bad, k2 = job(m=0)
    arr = (api.CompressJobT * 2)(good, bad)
    st, msg = status_and_msg(L, L.csa_compress_kv_batch(arr, 2, api.BF16, None))
    assert st == 1 and "m 0" in msg
    arr = (api.CompressJobT * 1)(good)
    st, msg = status_and_msg(L, L.csa_compress_kv_batch(arr, 1, api.FP8_E4M3, None))
    assert st == 2 and "x dtype" in msg
    empty, k3 = job(T=3)                # T < m: nothing to launch
    arr = (api.CompressJobT * 2)(empty, empty)
    st, msg = status_and_msg(L, L.csa_compress_kv_batch(arr, 2, api.BF16, None))
    assert st == 0


def indexer(L, **over):
    a = dict(q=FAKE, qs=FAKE, qd=api.FP4_E2M1, w=FAKE, keys=idx(cap=100000), pos=FAKE, B=4, Tq=1, Hi=4, m=4,
             topk=1024, out=FAKE, ws=None, wsb=0)
    a.update(over)
    return status_and_msg(L, L.csa_indexer_topk(a["q"], a["qs"], a["qd"], a["w"], C.byref(a["keys"]), a["pos"],
                                                a["B"], a["Tq"], a["Hi"], a["m"], a["topk"], a["out"], a["ws"],
                                                a["wsb"], None))


@pytest.mark.parametrize("over,code,frag", [
    (dict(Hi=0), 1, "Hi"),
    (dict(Hi=17), 2, "Hi"),
    (dict(topk=0), 1, "topk"),
    (dict(topk=4096), 2, "topk"),
    (dict(keys=idx(di=48)), 2, "di"),
    (dict(keys=idx(di=512)), 2, "di"),
    (dict(qd=7), 2, "q dtype"),
    (dict(keys=idx(fmt=api.FP8_E4M3)), 2, "key fmt"),
    (dict(qs=None), 1, "q_idx_scales"),
    (dict(keys=idx(scales=None, cap=100000)), 1, "scales"),
    (dict(q=C.c_void_p(4097)), 1, "aligned"),
    (dict(out=None), 1, "is null"),
    (dict(), 4, "workspace"),
    (dict(ws=FAKE, wsb=100), 4, "workspace"),
])
def test_indexer_validation(L, over, code, frag):
    st, msg = indexer(L, **over)
    assert st == code and frag in msg, (st, msg)


def test_indexer_workspace_sizes(L):
    assert L.csa_indexer_topk_workspace_size(4, 1, 4096, 64) == 0          # small path: none
    n = L.csa_indexer_topk_workspace_size(4, 1, 262144, 1024)
    assert n >= 4 * 262144 * 12
    assert L.csa_indexer_topk_workspace_size(0, 1, 262144, 1024) == 0


def attn(L, sparse=True, **over):
    p = api.AttnParamsT(512, 64, 128, 4, 10000.0, 512 ** -0.5, 1e-6)
    a = dict(q=FAKE, qd=api.BF16, pos=FAKE, topk=FAKE, k=1024, comp=kv(cap=1 << 18), win=kv(ring=1, cap=128),
             gq=None, sink=FAKE, p=p, B=4, Tq=1, H=64, out=FAKE, od=api.BF16, ws=None, wsb=0)
    a.update(over)
    win = None if a["win"] is None else C.byref(a["win"])
    if sparse:
        st = L.csa_sparse_mqa_attn(a["q"], a["qd"], a["pos"], a["topk"], a["k"], C.byref(a["comp"]), win, a["gq"],
                                   a["sink"], C.byref(a["p"]), a["B"], a["Tq"], a["H"], a["out"], a["od"], a["ws"],
                                   a["wsb"], None)
    else:
        st = L.hca_dense_mqa_attn(a["q"], a["qd"], a["pos"], C.byref(a["comp"]), win, a["gq"], a["sink"],
                                  C.byref(a["p"]), a["B"], a["Tq"], a["H"], a["out"], a["od"], a["ws"], a["wsb"], None)
    return status_and_msg(L, st)


@pytest.mark.parametrize("sparse", [True, False])
@pytest.mark.parametrize("over,code,frag", [
    (dict(H=0), 1, "bad sizes"),
    (dict(H=512), 2, "H=512"),
    (dict(B=70000), 2, "query rows"),
    (dict(qd=api.FP8_E4M3), 2, "q dtype"),
    (dict(od=api.FP4_E2M1), 2, "out dtype"),
    (dict(comp=kv(d=256)), 1, "differ"),
    (dict(comp=kv(ring=1)), 1, "linear"),
    (dict(win=kv(ring=0, cap=128)), 1, "ring"),
    (dict(win=kv(ring=1, cap=100)), 3, "window ring cap"),
    (dict(win=None), 1, "window cache"),
    (dict(comp=kv(fmt=api.FP4_E2M1)), 2, "comp fmt"),
    (dict(sink=None), 1, "is null"),
    (dict(p=api.AttnParamsT(512, 63, 128, 4, 1e4, 0.1, 1e-6)), 1, "rope_dim"),
    (dict(), 4, "workspace"),
])
def test_attention_validation(L, sparse, over, code, frag):
    if not sparse and frag == "workspace":
        over = dict(over, comp=kv(cap=8192))
    st, msg = attn(L, sparse, **over)
    assert st == code and frag in msg, (st, msg)


def test_attention_sparse_specific(L):
    st, msg = attn(L, True, k=0)
    assert st == 1 and "topk" in msg
    st, msg = attn(L, True, topk=None)
    assert st == 1 and "topk_idx" in msg
    st, msg = attn(L, False, comp=kv(cap=1 << 20))
    assert st == 2 and "262144" in msg


def test_attention_window_ring_for_prefill(L):
    # a chunk of Tq queries needs window + Tq - 1 ring slots
    st, msg = attn(L, True, B=1, Tq=64, win=kv(ring=1, cap=128 + 62))
    assert st == 3, msg


@pytest.mark.parametrize("args,code,frag", [
    ((FAKE, 1, FAKE, 1, 4, 32768, 7168, 7, FAKE, 1), 1, "multiples"),
    ((FAKE, 1, FAKE, 0, 4, 32768, 7168, 8, FAKE, 1), 2, "dtypes"),
    ((FAKE, 2, FAKE, 2, 4, 32768, 7168, 8, FAKE, 1), 2, "dtypes"),
    ((FAKE, 1, FAKE, 1, 4, 32768, 7168, 8, FAKE, 3), 2, "y dtype"),
    ((None, 1, FAKE, 1, 4, 32768, 7168, 8, FAKE, 1), 1, "is null"),
    ((FAKE, 1, FAKE, 1, -1, 32768, 7168, 8, FAKE, 1), 1, "bad sizes"),
])
def test_projection_validation(L, args, code, frag):
    st, msg = status_and_msg(L, L.attn_out_proj_grouped(*args, None))
    assert st == code and frag in msg, (st, msg)


def test_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(api, "_lib", None)
    monkeypatch.setattr(api, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        api.lib()
