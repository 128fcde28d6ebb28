"""The C-ABI library loads, exports what include/dsa.h declares, and rejects
invalid arguments on the host with the documented status codes (CPU only:
validation runs before any HIP call, so no GPU is touched)."""
import ctypes
import os
import re
import subprocess

import pytest

import sparse_attention_11_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")
P = ctypes.c_void_p(4096)  # never dereferenced: every call below fails validation


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


@pytest.mark.parametrize("path", [dsa.LIB_PATH, dsa.DEBUG_LIB_PATH], ids=["release", "debug"])
def test_library_exports_every_declared_symbol(path):
    names = declared_functions()
    assert set(names) == set(dsa._EXPORTS), names
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for n in names:
        assert n in exported, n
        assert hasattr(dsa.lib(), n)


def test_debug_build_flag_and_validation():
    """libdsa_debug.so reports itself as the debug build and validates
    arguments exactly as the release build does (before any HIP call)."""
    rel, dbg = ctypes.CDLL(dsa.LIB_PATH), ctypes.CDLL(dsa.DEBUG_LIB_PATH)
    assert rel.dsa_debug_build() == 0 and dbg.dsa_debug_build() == 1
    for L in (rel, dbg):
        L.dsa_topk.argtypes = [ctypes.c_void_p] * 2 + [ctypes.c_int] * 4 + [ctypes.c_void_p,
                                                                           ctypes.c_size_t,
                                                                           ctypes.c_void_p]
        assert L.dsa_topk(P, P, 1, 4, 100, 0, None, 0, None) == 1      # topk < 1
        assert L.dsa_topk(P, P, 1, 4, 5000, 4096, None, 0, None) == 2  # topk > DSA_MAX_TOPK
        assert L.dsa_topk(P, P, 1, 4, 50000, 2048, None, 0, None) == 3  # no workspace
    dbg.dsa_status_string.restype = ctypes.c_char_p
    assert dbg.dsa_status_string(5) == b"DSA_ERR_CHECK"


def test_status_strings():
    L = dsa.lib()
    assert L.dsa_status_string(0) == b"DSA_OK"
    assert L.dsa_status_string(1) == b"DSA_ERR_INVALID_ARG"
    assert L.dsa_status_string(2) == b"DSA_ERR_UNSUPPORTED"
    assert L.dsa_status_string(3) == b"DSA_ERR_WORKSPACE"
    assert L.dsa_status_string(4) == b"DSA_ERR_HIP"
    assert L.dsa_status_string(5) == b"DSA_ERR_CHECK"


def idx(**kw):
    a = dict(q=P, k=P, w=P, s=P, B=1, S=4, T=8, past=0, HI=2, DI=64, scale=0.125, relu=0, dt=1)
    a.update(kw)
    return dsa.lib().dsa_index_scores(a["q"], a["k"], a["w"], a["s"], a["B"], a["S"], a["T"],
                                      a["past"], a["HI"], a["DI"], a["scale"], a["relu"], a["dt"],
                                      None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(s=None), 1), (dict(B=0), 1), (dict(S=0), 1), (dict(HI=0), 1),
    (dict(past=-1), 1), (dict(T=3), 1), (dict(past=5), 1), (dict(scale=0.0), 1),
    (dict(scale=float("inf")), 1), (dict(scale=float("nan")), 1), (dict(relu=3), 1),
    (dict(dt=2), 1), (dict(DI=48), 2), (dict(DI=256), 2),
])
def test_index_scores_validation(kw, code):
    assert idx(**kw) == code
    assert dsa.dsa_last_error().startswith("dsa_index_scores")


def topk(fn="dsa_topk", **kw):
    a = dict(s=P, i=P, B=1, S=2, T=100, k=10, ws=None, nb=0)
    a.update(kw)
    return getattr(dsa.lib(), fn)(a["s"], a["i"], a["B"], a["S"], a["T"], a["k"], a["ws"], a["nb"],
                                  None)


@pytest.mark.parametrize("fn", ["dsa_topk", "dsa_topk_unsorted"])
@pytest.mark.parametrize("kw,code", [
    (dict(s=None), 1), (dict(i=None), 1), (dict(k=0), 1), (dict(k=101), 1), (dict(T=0), 1),
    (dict(T=5000, k=2049), 2),
])
def test_topk_validation(fn, kw, code):
    assert topk(fn, **kw) == code
    assert dsa.dsa_last_error().startswith(fn + ":")


def index_topk(**kw):
    a = dict(q=P, k=P, w=P, i=P, B=1, S=4, T=8, past=0, HI=2, DI=64, scale=0.125, relu=0, dt=1,
             topk=4, sorted=1, ws=None, nb=0)
    a.update(kw)
    return dsa.lib().dsa_index_topk(a["q"], a["k"], a["w"], a["i"], a["B"], a["S"], a["T"],
                                    a["past"], a["HI"], a["DI"], a["scale"], a["relu"], a["dt"],
                                    a["topk"], a["sorted"], a["ws"], a["nb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(i=None), 1), (dict(T=3), 1), (dict(past=5), 1), (dict(DI=48), 2),
    (dict(topk=0), 1), (dict(topk=9), 1), (dict(T=5000, topk=4096), 2), (dict(sorted=2), 1),
    (dict(scale=0.0), 1), (dict(relu=3), 1), (dict(dt=2), 1),
    (dict(), 3),                                     # scores need a workspace
    (dict(ws=P, nb=8 * 4 * 4 - 1), 3),               # one byte short of B*S*T fp32 scores
])
def test_index_topk_validation(kw, code):
    assert index_topk(**kw) == code
    assert dsa.dsa_last_error().startswith("dsa_index_topk:")


def test_index_topk_workspace_size():
    # B*S*T fp32 scores, 256-byte aligned, then the top-k's own workspace
    assert dsa.dsa_index_topk_workspace_size(1, 4, 8, 4) == 256
    assert dsa.dsa_index_topk_workspace_size(2, 100, 40000, 512) == \
        (2 * 100 * 40000 * 4 + 255) // 256 * 256 + dsa.dsa_topk_workspace_size(2, 100, 40000, 512)
    for bad in ((0, 4, 8, 4), (1, 4, 8, 9), (1, 4, 8, 0), (1, 4, 5000, 4096)):
        assert dsa.dsa_index_topk_workspace_size(*bad) == 0


def prefill(**kw):
    a = dict(q=P, k=P, v=P, i=P, g=P, o=P, B=1, S=32, T=64, past=0, H=2, nope=64, rope=64, v_dim=128,
             topk=16, sc=0.1, gd=1, dt=1, ws=None, nb=0)
    a.update(kw)
    return dsa.lib().dsa_sparse_attn_prefill(a["q"], a["k"], a["v"], a["i"], a["g"], a["o"], a["B"],
                                             a["S"], a["T"], a["past"], a["H"], a["nope"],
                                             a["rope"], a["v_dim"], a["topk"], a["sc"], a["gd"],
                                             a["dt"], a["ws"], a["nb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(i=None), 1), (dict(g=None), 1), (dict(gd=7), 1), (dict(sc=-1.0), 1),
    (dict(past=40), 1), (dict(topk=0), 1), (dict(topk=65), 1), (dict(dt=5), 1), (dict(H=0), 1),
    (dict(nope=60), 2), (dict(v_dim=300), 2), (dict(T=5000, topk=4096), 2),
    (dict(), 3),  # a workspace (selection bitmap) is required and none is given
    (dict(nb=1, ws=P), 3),
])
def test_prefill_validation(kw, code):
    assert prefill(**kw) == code


def test_prefill_without_gate_is_valid_until_workspace():
    # gate may be NULL with gate_dim 0; the next failing check is the workspace
    assert prefill(g=None, gd=0) == 3


def test_workspace_sizes():
    L = dsa.lib()
    # bf16, many queries: one bit per (query, key) in 32-bit words, plus partial softmax
    # states when the grid is small enough that long query tiles are split
    bitmap = 4096 * 128 * 4
    assert L.dsa_sparse_attn_prefill_workspace_size(1, 4096, 4096, 20, 128, 128, 512, 1) > bitmap
    assert L.dsa_sparse_attn_prefill_workspace_size(1, 32768, 32768, 128, 192, 128, 2048, 1) == 32768 * 1024 * 4
    assert L.dsa_sparse_attn_decode_workspace_size(8, 128, 128, 2048) > 0
    assert L.dsa_topk_workspace_size(1, 1, 100, 10) == 0
    assert L.swa_attn_workspace_size(1, 4096, 32, 192, 128, 512, 1) == 0
    assert L.swa_attn_workspace_size(1, 1, 32, 192, 128, 512, 1) > 0


def swa(**kw):
    a = dict(q=P, k=P, v=P, g=P, o=P, B=1, S=10, Tb=10, past=0, off=0, H=2, nope=64, rope=64, v_dim=128,
             W=4, sc=0.1, gd=1, dt=1, ws=None, nb=0)
    a.update(kw)
    return dsa.lib().swa_attn(a["q"], a["k"], a["v"], a["g"], a["o"], a["B"], a["S"], a["Tb"], a["past"],
                              a["off"], a["H"], a["nope"], a["rope"], a["v_dim"], a["W"], a["sc"],
                              a["gd"], a["dt"], a["ws"], a["nb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(W=0), 1), (dict(off=-1), 1), (dict(past=100, Tb=110, off=98), 1),
    (dict(past=100, Tb=50, off=97), 1), (dict(Tb=11), 1), (dict(nope=8, rope=0), 2),
])
def test_swa_validation(kw, code):
    assert swa(**kw) == code


def decode(**kw):
    a = dict(q=P, k=P, v=P, i=P, g=P, o=P, B=2, T=100, H=2, nope=64, rope=64, v_dim=128, topk=16,
             sc=0.1, gd=1, dt=1, ws=None, nb=0)
    a.update(kw)
    return dsa.lib().dsa_sparse_attn_decode(a["q"], a["k"], a["v"], a["i"], a["g"], a["o"], a["B"],
                                            a["T"], a["H"], a["nope"], a["rope"], a["v_dim"],
                                            a["topk"], a["sc"], a["gd"], a["dt"], a["ws"], a["nb"],
                                            None)


@pytest.mark.parametrize("kw,code", [
    (dict(i=None), 1), (dict(topk=101), 1), (dict(B=0), 1), (dict(), 3),
])
def test_decode_validation(kw, code):
    assert decode(**kw) == code


# ---------------------------------------------------- attention sinks (PAS)
def prefill_pas(**kw):
    a = dict(q=P, k=P, v=P, sk=P, sv=P, ns=128, i=P, g=P, o=P, B=1, S=32, T=64, past=0, H=2,
             nope=64, rope=64, v_dim=128, topk=16, sc=0.1, gd=1, dt=1, ws=None, nb=0)
    a.update(kw)
    return dsa.lib().dsa_sparse_attn_prefill_pas(
        a["q"], a["k"], a["v"], a["sk"], a["sv"], a["ns"], a["i"], a["g"], a["o"], a["B"],
        a["S"], a["T"], a["past"], a["H"], a["nope"], a["rope"], a["v_dim"], a["topk"], a["sc"],
        a["gd"], a["dt"], a["ws"], a["nb"], None)


def decode_pas(**kw):
    a = dict(q=P, k=P, v=P, sk=P, sv=P, ns=128, i=P, g=P, o=P, B=2, T=100, H=2, nope=64, rope=64,
             v_dim=128, topk=16, sc=0.1, gd=1, dt=1, ws=None, nb=0)
    a.update(kw)
    return dsa.lib().dsa_sparse_attn_decode_pas(
        a["q"], a["k"], a["v"], a["sk"], a["sv"], a["ns"], a["i"], a["g"], a["o"], a["B"], a["T"],
        a["H"], a["nope"], a["rope"], a["v_dim"], a["topk"], a["sc"], a["gd"], a["dt"], a["ws"],
        a["nb"], None)


def swa_pas(**kw):
    a = dict(q=P, k=P, v=P, sk=P, sv=P, ns=128, g=P, o=P, B=1, S=10, Tb=10, past=0, off=0, H=2,
             nope=64, rope=64, v_dim=128, W=4, sc=0.1, gd=1, dt=1, ws=None, nb=0)
    a.update(kw)
    return dsa.lib().swa_attn_pas(
        a["q"], a["k"], a["v"], a["sk"], a["sv"], a["ns"], a["g"], a["o"], a["B"], a["S"], a["Tb"],
        a["past"], a["off"], a["H"], a["nope"], a["rope"], a["v_dim"], a["W"], a["sc"], a["gd"],
        a["dt"], a["ws"], a["nb"], None)


@pytest.mark.parametrize("fn", [prefill_pas, decode_pas, swa_pas])
@pytest.mark.parametrize("kw,code", [
    (dict(sk=None), 1), (dict(sv=None), 1), (dict(ns=-1), 1), (dict(ns=257), 1),
    (dict(ns=0, sk=None, sv=None, q=None), 1),  # no sinks: NULL sink pointers are fine
])
def test_sink_validation(fn, kw, code):
    assert fn(**kw) == code


def test_sink_workspace_sizes():
    L = dsa.lib()
    # MFMA path: sinks are extra key blocks and need no workspace of their own
    assert (L.dsa_sparse_attn_prefill_pas_workspace_size(1, 4096, 4096, 20, 128, 128, 512, 128, 1)
            == L.dsa_sparse_attn_prefill_workspace_size(1, 4096, 4096, 20, 128, 128, 512, 1))
    assert L.swa_attn_pas_workspace_size(1, 4096, 32, 192, 128, 512, 128, 1) == 0
    # gather path: sinks are extra entries (more splits may need more partial states)
    assert (L.dsa_sparse_attn_decode_pas_workspace_size(8, 128, 128, 2048, 0)
            == L.dsa_sparse_attn_decode_workspace_size(8, 128, 128, 2048))
    assert (L.dsa_sparse_attn_decode_pas_workspace_size(1, 4, 128, 16, 128)
            > L.dsa_sparse_attn_decode_workspace_size(1, 4, 128, 16))


def swa_gqa(**kw):
    a = dict(q=P, k=P, v=P, g=P, o=P, B=1, S=10, Tb=10, past=0, off=0, H=8, Hkv=2, nope=128,
             rope=128, v_dim=256, W=4, sc=0.1, gd=1, dt=1, ws=None, nb=0)
    a.update(kw)
    return dsa.lib().swa_attn_gqa(a["q"], a["k"], a["v"], a["g"], a["o"], a["B"], a["S"], a["Tb"],
                                  a["past"], a["off"], a["H"], a["Hkv"], a["nope"], a["rope"],
                                  a["v_dim"], a["W"], a["sc"], a["gd"], a["dt"], a["ws"], a["nb"],
                                  None)


@pytest.mark.parametrize("kw,code", [
    (dict(Hkv=0), 1), (dict(Hkv=3), 1), (dict(Hkv=16), 1), (dict(H=6, Hkv=4), 1),
    (dict(W=0), 1), (dict(Tb=11), 1), (dict(k=None), 1), (dict(nope=8, rope=0), 2),
    (dict(S=1, Tb=10, past=9), 3),  # gather path (decode) without a workspace
])
def test_swa_gqa_validation(kw, code):
    assert swa_gqa(**kw) == code
    assert dsa.dsa_last_error().startswith("swa_attn_gqa")


def test_swa_gqa_workspace_sizes():
    L = dsa.lib()
    # same partial states as plain SWA: they are kept per query head
    for args in [(1, 4096, 8, 256, 256, 512, 1), (1, 1, 8, 256, 256, 512, 1),
                 (2, 5, 4, 48, 32, 16, 0)]:
        assert L.swa_attn_gqa_workspace_size(*args) == L.swa_attn_workspace_size(*args)
    assert L.swa_attn_gqa_workspace_size(1, 4096, 8, 256, 256, 512, 1) == 0


def test_noalloc_decode_rejects_calls_beyond_the_static_scratch():
    # 300 sequences x 128 heads x (256 + 4) floats of partial state > 32 MiB:
    # rejected on the host before any HIP call
    L = dsa.lib()
    need = dsa.dsa_sparse_attn_decode_workspace_size(300, 128, 256, 2048)
    assert need > dsa.STATIC_SCRATCH_BYTES
    st = L.dsa_sparse_attn_decode_noalloc(P, P, P, P, P, P, 300, 4096, 128, 128, 64, 256, 2048,
                                          0.07, 1, 1, None)
    assert st == dsa.DSA_ERR_UNSUPPORTED
    assert "static scratch" in dsa.dsa_last_error()
    # invalid arguments are still INVALID_ARG
    assert L.dsa_sparse_attn_decode_noalloc(None, P, P, P, P, P, 1, 4096, 8, 128, 64, 128, 64,
                                            0.07, 1, 1, None) == dsa.DSA_ERR_INVALID_ARG


def mla(**kw):
    a = dict(qr=P, qc=P, hd=P, wq=P, wa=P, wb=P, cos=P, sin=P, q=P, g=P, kc=P, vc=P, B=1, S=4,
             T=8, past=0, Qr=64, Qc=32, Hd=96, L=64, H=2, N=64, R=32, Dv=64, dt=1, ws=P,
             wsb=1 << 30)
    a.update(kw)
    return dsa.lib().dsa_mla_prologue(a["qr"], a["qc"], a["hd"], a["wq"], a["wa"], a["wb"],
                                      a["cos"], a["sin"], a["q"], a["g"], a["kc"], a["vc"], a["B"],
                                      a["S"], a["T"], a["past"], a["Qr"], a["Qc"], a["Hd"], a["L"],
                                      a["H"], a["N"], a["R"], a["Dv"], a["dt"], a["ws"], a["wsb"],
                                      None)


@pytest.mark.parametrize("kw,code", [
    (dict(qr=None), 1), (dict(wb=None), 1), (dict(kc=None), 1), (dict(cos=None), 1),
    (dict(B=0), 1), (dict(T=3), 1), (dict(past=-1), 1), (dict(N=0, R=0), 1), (dict(dt=2), 1),
    (dict(dt=0), 2), (dict(Qr=48), 2), (dict(L=40), 2), (dict(N=24), 2), (dict(R=8), 2),
    (dict(N=192, R=128), 2), (dict(Dv=272), 2), (dict(ws=None), 3), (dict(wsb=100), 3),
])
def test_mla_prologue_validation(kw, code):
    assert mla(**kw) == code
    assert dsa.dsa_last_error().startswith("dsa_mla_prologue")


def test_mla_prologue_rope_tables_optional_without_rope():
    # R = 0: no rotation, the tables may be NULL; the call then fails only on the
    # workspace (checked last), so validation passed
    assert mla(R=0, cos=None, sin=None, wsb=0) == dsa.DSA_ERR_WORKSPACE
    assert dsa.dsa_mla_prologue_workspace_size(2, 5, 64) == 2 * 5 * 64 * 2
    assert dsa.dsa_mla_prologue_workspace_size(2, 5, 40) == 0
