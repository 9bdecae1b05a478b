"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every entry point declared in include/pa.h, and rejects bad arguments before
anything is launched."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "pa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(pa_[a-z_0-9]+)\s*\(", text)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    from paged_attention_flat_amd import _lib
    return _lib.LIB


def test_header_declares_the_boundary():
    names = header_functions()
    for required in ("pa_kv_write", "pa_attention_fwd", "pa_split_combine"):
        assert required in names


def test_every_declared_symbol_is_exported(lib):
    from paged_attention_flat_amd import _lib
    for name in header_functions():
        assert hasattr(lib, name), name
        assert name in _lib.PROTOTYPES, f"{name} has no Python prototype"


def test_status_strings(lib):
    for s in range(6):
        assert lib.pa_status_string(s)
    assert lib.pa_status_string(99) == b"unknown status"
    assert lib.pa_version() >= 100


def test_kv_write_validation(lib):
    P = ctypes.c_void_p(16)  # never dereferenced: every call below fails validation
    assert lib.pa_kv_write(P, P, P, P, P, 4, 0, 128, 16, 8, 1, None) == 2   # no KV heads
    assert lib.pa_kv_write(P, P, P, P, P, 4, 2, 96, 16, 8, 1, None) == 3    # head_dim
    assert lib.pa_kv_write(P, P, P, P, P, 4, 2, 128, 32, 8, 1, None) == 3   # block size
    assert lib.pa_kv_write(P, P, P, P, P, 4, 2, 128, 16, 8, 7, None) == 2   # dtype
    assert lib.pa_kv_write(None, P, P, P, P, 4, 2, 128, 16, 8, 1, None) == 1
    assert lib.pa_kv_write(None, None, None, None, None, 0, 2, 128, 16, 8, 1, None) == 0
    assert lib.pa_kv_write(ctypes.c_void_p(18), P, P, P, P, 4, 2, 128, 16, 8, 1, None) == 2


def _fwd(lib, **kw):
    P = ctypes.c_void_p(256)
    a = dict(q=P, kc=P, vc=P, qsl=P, sl=P, bt=P, ns=2, nt=3, mq=2, ms=40, hq=8, hkv=2, d=128,
             bs=16, stride=3, nb=10, scale=0.1, splits=1, out=P, lse=None, ws=P,
             wsb=1 << 20, dtype=1)
    a.update(kw)
    return lib.pa_attention_fwd(a["q"], a["kc"], a["vc"], a["qsl"], a["sl"], a["bt"], a["ns"],
                                a["nt"], a["mq"], a["ms"], a["hq"], a["hkv"], a["d"], a["bs"],
                                a["stride"], a["nb"], a["scale"], a["splits"], a["out"],
                                a["lse"], a["ws"], a["wsb"], a["dtype"], None)


def test_attention_validation(lib):
    assert _fwd(lib, hq=6, hkv=4) == 2                # Hq % Hkv != 0
    assert _fwd(lib, hq=6, hkv=2) == 3                # group 3 not implemented
    assert _fwd(lib, hq=64, hkv=2) == 3               # group 32 not implemented
    assert _fwd(lib, d=80) == 3
    assert _fwd(lib, bs=8) == 3
    assert _fwd(lib, splits=-1) == 2
    assert _fwd(lib, splits=257) == 2
    assert _fwd(lib, scale=float("nan")) == 2
    assert _fwd(lib, scale=0.0) == 2
    assert _fwd(lib, scale=-0.5) == 2
    assert _fwd(lib, dtype=5) == 2
    assert _fwd(lib, mq=4) == 2                       # max_query_len > num_tokens
    assert _fwd(lib, ms=1) == 2                       # max_seq_len < max_query_len
    assert _fwd(lib, stride=2) == 2                   # table narrower than max_seq_len
    assert _fwd(lib, qsl=None) == 1
    assert _fwd(lib, out=None) == 1
    assert _fwd(lib, ws=None) == 4
    assert _fwd(lib, wsb=16) == 4
    need = lib.pa_attention_workspace_size(2, 3, 8, 128, 4)
    assert _fwd(lib, splits=4, wsb=need - 1) == 4
    assert _fwd(lib, ns=0) == 0 and _fwd(lib, nt=0) == 0


def test_split_combine_validation(lib):
    P = ctypes.c_void_p(256)
    assert lib.pa_split_combine(P, P, 0, 4, 8, 128, P, None, 1, None) == 2
    assert lib.pa_split_combine(P, P, 300, 4, 8, 128, P, None, 1, None) == 2
    assert lib.pa_split_combine(P, P, 4, 4, 8, 100, P, None, 1, None) == 3
    assert lib.pa_split_combine(None, P, 4, 4, 8, 128, P, None, 1, None) == 1
    assert lib.pa_split_combine(None, None, 4, 0, 8, 128, None, None, 1, None) == 0


def test_workspace_size_grows_with_splits(lib):
    one = lib.pa_attention_workspace_size(1, 1, 32, 128, 1)
    many = lib.pa_attention_workspace_size(1, 1, 32, 128, 64)
    assert many - one >= 64 * 32 * 129 * 4
    assert lib.pa_attention_workspace_size(1, 1, 32, 128, 0) == 0


def test_split_heuristic_crossover(lib):
    f = lib.pa_choose_num_splits
    assert f(1, 1, 32768, 32, 8, 256) == 32          # long single decode: a split per CU
    assert f(256, 1, 8192, 32, 8, 256) == 1          # batch fills the grid: no split
    assert f(4, 8192, 8192, 32, 8, 256) == 1         # prefill rows present
    assert f(4098, 2048, 18432, 32, 8, 256) == 1
    assert f(1, 1, 64, 32, 8, 256) == 1              # too few blocks to split
    # one KV head (a tensor-parallel shard): a split per CU would be 256, but
    # the in-launch merge of that many partials costs more than it gains
    assert f(1, 1, 32768, 4, 1, 256) == 64
    assert f(1, 1, 4096, 4, 1, 256) == 32            # >= 8 blocks per split
    assert 1 < f(2, 1, 4096, 32, 8, 256) <= 256
    assert f(1, 4, 4096, 32, 8, 256) > 1             # 4 new tokens still pack (G = 4)
    assert f(1, 5, 4096, 32, 8, 256) == 1


def test_capture_size_matches_printed_ladder(lib):
    # "Model execution", section "Code": the printed padding table and ladder
    from conftest import read_golden
    g = read_golden("capture_ladder_printed.txt")
    for tokens, used, padded in g["pad"]:
        got = lib.pa_capture_size(tokens, 512)
        assert got == used, (tokens, got, used)
        if used > 0:
            assert got - tokens == padded
    sizes = sorted({lib.pa_capture_size(n, 512) for n in range(1, 513)})
    assert len(sizes) == g["count"][0][0]
    assert sizes[:6] == g["first"][0] and sizes[-3:] == g["last"][0]
    assert lib.pa_capture_size(0, 512) == -1 and lib.pa_capture_size(-3, 512) == -1
    # a smaller top size cuts the ladder there
    assert lib.pa_capture_size(200, 128) == -1 and lib.pa_capture_size(128, 128) == 128


# ---- the entry points beyond the core three: host validation and empty steps ----

P = ctypes.c_void_p(256)


def test_kv_write_fp8_validation(lib):
    f = lib.pa_kv_write_fp8
    assert f(P, P, P, P, P, P, P, 4, 2, 96, 16, 8, 1, None) == 3        # head_dim
    assert f(P, P, P, P, P, P, P, 4, 2, 128, 32, 8, 1, None) == 3       # block size
    assert f(P, P, P, P, P, P, P, 4, 2, 128, 16, 8, 9, None) == 2       # dtype
    assert f(P, P, P, P, P, None, P, 4, 2, 128, 16, 8, 1, None) == 1    # no K scales
    assert f(P, P, P, P, P, P, P, 4, 0, 128, 16, 8, 1, None) == 2       # no KV heads
    assert f(None, None, None, None, None, None, None, 0, 2, 128, 16, 8, 1, None) == 0


def test_rope_kv_write_validation(lib):
    def rope(**kw):
        a = dict(q=P, k=P, v=P, kc=P, vc=P, sm=P, pos=P, cs=P, maxp=64, nt=4, hq=8, hkv=2,
                 d=128, bs=16, nb=8, dtype=1)
        a.update(kw)
        return lib.pa_rope_kv_write(a["q"], a["k"], a["v"], a["kc"], a["vc"], a["sm"], a["pos"],
                                    a["cs"], a["maxp"], a["nt"], a["hq"], a["hkv"], a["d"],
                                    a["bs"], a["nb"], a["dtype"], None)
    assert rope(hq=6, hkv=4) == 2
    assert rope(d=96) == 3
    assert rope(bs=8) == 3
    assert rope(dtype=4) == 2
    assert rope(pos=None) == 1
    assert rope(cs=None) == 1
    assert rope(q=None, k=None, v=None, kc=None, vc=None, sm=None, pos=None, cs=None, nt=0) == 0


def _fwd_fp8(lib, **kw):
    a = dict(q=P, kc=P, vc=P, ks=P, vs=P, qsl=P, sl=P, bt=P, ns=2, nt=3, mq=2, ms=40, hq=8,
             hkv=2, d=128, bs=16, stride=3, nb=10, scale=0.1, splits=1, out=P, lse=None, ws=P,
             wsb=1 << 20)
    a.update(kw)
    return lib.pa_attention_fwd_fp8(a["q"], a["kc"], a["vc"], a["ks"], a["vs"], a["qsl"],
                                    a["sl"], a["bt"], a["ns"], a["nt"], a["mq"], a["ms"],
                                    a["hq"], a["hkv"], a["d"], a["bs"], a["stride"], a["nb"],
                                    a["scale"], a["splits"], a["out"], a["lse"], a["ws"],
                                    a["wsb"], None)


def test_attention_fp8_validation(lib):
    assert _fwd_fp8(lib, hq=6, hkv=2) == 3
    assert _fwd_fp8(lib, d=80) == 3
    assert _fwd_fp8(lib, scale=0.0) == 2
    assert _fwd_fp8(lib, ks=None) == 1
    assert _fwd_fp8(lib, vs=None) == 1
    assert _fwd_fp8(lib, ws=None) == 4
    assert _fwd_fp8(lib, ns=0) == 0 and _fwd_fp8(lib, nt=0) == 0


def _cascade(lib, **kw):
    a = dict(q=P, kc=P, vc=P, qsl=P, sl=P, bt=P, ns=2, nt=2, mq=1, ms=40, hq=8, hkv=2, d=128,
             bs=16, stride=3, nb=10, scale=0.1, splits=1, sh=P, nsh=2, pb=P, npb=2, out=P,
             lse=None, ws=P, wsb=1 << 20)
    a.update(kw)
    return lib.pa_attention_fwd_cascade(a["q"], a["kc"], a["vc"], a["qsl"], a["sl"], a["bt"],
                                        a["ns"], a["nt"], a["mq"], a["ms"], a["hq"], a["hkv"],
                                        a["d"], a["bs"], a["stride"], a["nb"], a["scale"],
                                        a["splits"], a["sh"], a["nsh"], a["pb"], a["npb"],
                                        a["out"], a["lse"], a["ws"], a["wsb"], None)


def test_cascade_validation(lib):
    assert _cascade(lib, nsh=-1) == 2
    assert _cascade(lib, npb=-3) == 2
    assert _cascade(lib, sh=None) == 1
    assert _cascade(lib, pb=None) == 1
    assert _cascade(lib, d=96) == 3
    assert _cascade(lib, hq=6, hkv=4) == 2
    assert _cascade(lib, ns=0) == 0


def _step_cascade(lib, **kw):
    a = dict(k=P, v=P, kc=P, vc=P, sm=P, q=P, qsl=P, sl=P, bt=P, ns=2, nt=2, mq=1, ms=40, hq=8,
             hkv=2, d=128, bs=16, stride=3, nb=10, scale=0.1, splits=1, sh=P, nsh=2, pb=P, npb=2,
             out=P, lse=None, ws=P, wsb=1 << 20)
    a.update(kw)
    return lib.pa_decode_step_cascade(a["k"], a["v"], a["kc"], a["vc"], a["sm"], a["q"],
                                      a["qsl"], a["sl"], a["bt"], a["ns"], a["nt"], a["mq"],
                                      a["ms"], a["hq"], a["hkv"], a["d"], a["bs"], a["stride"],
                                      a["nb"], a["scale"], a["splits"], a["sh"], a["nsh"],
                                      a["pb"], a["npb"], a["out"], a["lse"], a["ws"], a["wsb"],
                                      None)


def test_decode_step_cascade_validation(lib):
    assert _step_cascade(lib, nsh=-1) == 2
    assert _step_cascade(lib, npb=-1) == 2
    assert _step_cascade(lib, sh=None) == 1
    assert _step_cascade(lib, pb=None) == 1
    assert _step_cascade(lib, k=None) == 1                  # the write needs the new K
    assert _step_cascade(lib, sm=None) == 1
    assert _step_cascade(lib, v=ctypes.c_void_p(258)) == 2  # misaligned new V
    assert _step_cascade(lib, d=96) == 3
    assert _step_cascade(lib, hq=6, hkv=4) == 2
    assert _step_cascade(lib, bs=32) == 3
    assert _step_cascade(lib, nt=0) == 0                    # empty step


def _step(lib, fp8=False, **kw):
    a = dict(k=P, v=P, kc=P, vc=P, sm=P, ks=P, vs=P, q=P, qsl=P, sl=P, bt=P, ns=2, nt=2, mq=1,
             ms=40, hq=8, hkv=2, d=128, bs=16, stride=3, nb=10, scale=0.1, splits=1, out=P,
             lse=None, ws=P, wsb=1 << 20, dtype=1)
    a.update(kw)
    head = [a["k"], a["v"], a["kc"], a["vc"], a["sm"]]
    if fp8:
        head += [a["ks"], a["vs"]]
    rest = [a["q"], a["qsl"], a["sl"], a["bt"], a["ns"], a["nt"], a["mq"], a["ms"], a["hq"],
            a["hkv"], a["d"], a["bs"], a["stride"], a["nb"], a["scale"], a["splits"], a["out"],
            a["lse"], a["ws"], a["wsb"], a["dtype"], None]
    f = lib.pa_decode_step_fp8 if fp8 else lib.pa_decode_step
    return f(*head, *rest)


def test_decode_step_validation(lib):
    for fp8 in (False, True):
        assert _step(lib, fp8, hq=6, hkv=4) == 2          # heads
        assert _step(lib, fp8, d=96) == 3                 # one launch: the kernel's check
        assert _step(lib, fp8, k=None) == 1               # one launch needs the new K
        assert _step(lib, fp8, k=ctypes.c_void_p(258)) == 2   # misaligned new K
        assert _step(lib, fp8, mq=5, nt=5, d=96) == 3     # two calls: the KV write's check
        assert _step(lib, fp8, dtype=0, d=96) == 3        # fp32: two calls as well
        assert _step(lib, fp8, nt=0) == 0                 # empty step
    assert _step(lib, True, ks=None) == 1


def test_workspace_init_validation(lib):
    assert lib.pa_attention_workspace_init(None, 0, None) == 0
    assert lib.pa_attention_workspace_init(None, 64, None) == 1
    assert lib.pa_attention_workspace_init(ctypes.c_void_p(260), 64, None) == 2


def test_unshared_blocks_hint(lib):
    # a host-side setting: returns the previous mode; positive means 1,
    # negative -1, zero the automatic default
    before = lib.pa_set_unshared_blocks(0)
    try:
        assert lib.pa_set_unshared_blocks(1) == 0
        assert lib.pa_set_unshared_blocks(7) == 1
        assert lib.pa_set_unshared_blocks(-5) == 1
        assert lib.pa_set_unshared_blocks(0) == -1
        assert lib.pa_set_unshared_blocks(0) == 0
    finally:
        lib.pa_set_unshared_blocks(before)
