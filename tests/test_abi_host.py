"""Host-side checks of the C ABI (no GPU): the library loads, exports every
function include/*.h declares, and rejects bad arguments with the documented
status codes before any launch."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))


@pytest.fixture(scope="module")
def lib():
    import position_agnostic_kv_amd as pak
    if not os.path.exists(pak.lib_path()):
        from position_agnostic_kv_amd import build
        build.build()
    return pak.load_library()


def declared_functions():
    names = []
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("kvcache_append", "lazyattn_decode", "lazyattn_prefill", "lazyattn_cache_acquire"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} is declared in include/ but not exported"


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert lib.lazyattn_status_string(code)
    assert lib.lazyattn_version() >= 100


NULL = ctypes.c_void_p(0)
P = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def decode(lib, **kw):
    a = dict(out=P, q=P, q_pos=P, k=P, v=P, table=P, max_blocks=4, fill=NULL, seq_lens=P, batch=2, hq=8, hkv=2,
             d=128, nb=16, dtype=1, scale=0.088, theta=1e4, split=0, ws=P, ws_bytes=1 << 30, stream=NULL)
    a.update(kw)
    fn = lib.lazyattn_decode_eager if a.pop("eager", False) else lib.lazyattn_decode
    return fn(a["out"], a["q"], a["q_pos"], a["k"], a["v"], a["table"], a["max_blocks"], a["fill"],
              a["seq_lens"], a["batch"], a["hq"], a["hkv"], a["d"], a["nb"], a["dtype"],
              a["scale"], a["theta"], a["split"], a["ws"], a["ws_bytes"], a["stream"])


def test_eager_baseline_checks_arguments_alike(lib):
    for kw in ({"dtype": 7}, {"hq": 6, "hkv": 4}, {"d": 96}, {"split": 2}, {"q": NULL},
               {"batch": 0, "q": NULL}, {"ws": NULL, "max_blocks": 4000}):
        assert decode(lib, eager=True, **kw) == decode(lib, **kw)
    f, g, h = lib.lazyattn_prefill, lib.lazyattn_prefill_eager, lib.lazyattn_prefill_precise
    ok = [P, P, 4096, P, P, P, P, P, 8, NULL, P, 2, 128, 32, 8, 128, 64, 1, 0.088, 5e5, NULL]
    for idx, val in ((17, 0), (15, 256), (2, -1), (1, NULL), (14, 3), (19, 1.0)):
        bad = list(ok)
        bad[idx] = val
        assert g(*bad) == f(*bad) == h(*bad) != 0
    empty = list(ok)
    empty[11] = 0
    empty[1] = NULL
    assert h(*empty) == 0


def test_decode_argument_errors(lib):
    assert decode(lib, dtype=7) == -2
    assert decode(lib, hq=6, hkv=4) == -3          # not a multiple
    assert decode(lib, hq=24, hkv=2) == -3         # group 12 not offered
    assert decode(lib, hq=128, hkv=1) == -3        # groups beyond 64 not offered
    assert decode(lib, d=96) == -3
    assert decode(lib, d=16) == -3                 # bf16 needs 64/128
    assert decode(lib, nb=65537) == -3
    assert decode(lib, split=2) == -3
    assert decode(lib, theta=1.0) == -3
    assert decode(lib, q=NULL) == -1
    assert decode(lib, batch=0, q=NULL) == 0       # empty batch: no-op before pointer checks
    assert decode(lib, ws=NULL, max_blocks=4000) == -4
    assert decode(lib, ws_bytes=16, max_blocks=4000) == -4
    assert decode(lib, ws=ctypes.c_void_p(0x1008), max_blocks=4000) == -4   # partials are read 16 bytes at a time


def planned(lib, **kw):
    a = dict(out=P, q=P, q_pos=P, k=P, v=P, table=P, max_blocks=4, fill=NULL, seq_lens=P, batch=2, hq=8, hkv=2,
             d=128, nb=16, dtype=1, scale=0.088, theta=1e4, plan=P, items=4, max_items=2, ws=P, ws_bytes=1 << 30,
             stream=NULL)
    a.update(kw)
    return lib.lazyattn_decode_planned(*a.values())


def test_planned_decode_argument_errors(lib):
    """Every argument error returns before any launch (the pointers are never
    dereferenced)."""
    assert planned(lib, dtype=0) == -2             # bf16 pools only
    assert planned(lib, dtype=7) == -2
    assert planned(lib, d=64) == -3                # head_dim 128 only
    assert planned(lib, hq=64, hkv=2) == -3        # groups up to 16
    assert planned(lib, hq=6, hkv=4) == -3
    assert planned(lib, hq=6, hkv=2) == -3         # group 3
    assert planned(lib, items=0) == -3
    assert planned(lib, max_items=0) == -3
    assert planned(lib, plan=NULL) == -1
    assert planned(lib, plan=ctypes.c_void_p(0x1008)) == -3   # items are read 16 bytes at a time
    assert planned(lib, q=NULL) == -1
    assert planned(lib, nb=65537) == -3
    assert planned(lib, ws=NULL) == -4
    assert planned(lib, ws_bytes=16) == -4
    assert planned(lib, ws=ctypes.c_void_p(0x1008)) == -4
    assert planned(lib, batch=0, q=NULL) == 0      # empty batch: no-op
    assert lib.lazyattn_decode_planned_workspace_size(2, 8, 2, 128, 1) == 0
    # 2 x 2 (sequence, KV head) units, 3 slots, 4 heads: (max, sum) pairs padded to 256 B, then outputs
    assert lib.lazyattn_decode_planned_workspace_size(2, 8, 2, 128, 3) == 512 + 4 * 3 * 4 * 128 * 4
    assert lib.lazyattn_decode_planned_workspace_size(2, 8, 2, 128, 0) == 0


def test_alibi_entry_points_check_arguments(lib):
    fd, fp = lib.lazyattn_decode_alibi, lib.lazyattn_prefill_alibi
    ok_d = [P, P, P, P, P, P, 4, NULL, P, P, 2, 8, 2, 128, 16, 1, 0.088, 0, P, 1 << 30, NULL]
    assert fd(*[NULL if i == 9 else x for i, x in enumerate(ok_d)]) == -1     # slopes NULL
    assert fd(*[7 if i == 15 else x for i, x in enumerate(ok_d)]) == -2      # dtype
    assert fd(*[96 if i == 13 else x for i, x in enumerate(ok_d)]) == -3     # head_dim
    assert fd(*[0 if i == 10 else (NULL if i == 9 else x) for i, x in enumerate(ok_d)]) == 0  # empty batch
    ok_p = [P, P, 4096, P, P, P, P, P, 8, NULL, P, P, 2, 128, 32, 8, 128, 64, 1, 0.088, NULL]
    assert fp(*[NULL if i == 11 else x for i, x in enumerate(ok_p)]) == -1
    assert fp(*[0 if i == 18 else x for i, x in enumerate(ok_p)]) == -2      # fp32 prefill not offered
    assert fp(*[96 if i == 16 else x for i, x in enumerate(ok_p)]) == -3


def test_workspace_size(lib):
    ws = lib.lazyattn_decode_workspace_size
    assert ws(1, 4, 4, 16, 3, 0) == 0                   # one split: no partials
    small = ws(64, 32, 8, 128, 513, 64)
    big = ws(64, 32, 8, 128, 513, 16)
    splits = -(-513 // 64)
    assert small >= 64 * 8 * splits * 4 * (128 * 4 + 8)
    assert big > small
    assert ws(0, 4, 4, 16, 3, 0) == 0


def test_prefill_and_append_argument_errors(lib):
    f = lib.lazyattn_prefill
    ok = [P, P, 4096, P, P, P, P, P, 8, NULL, P, 2, 128, 32, 8, 128, 64, 1, 0.088, 5e5, NULL]
    bad_dtype = list(ok)
    bad_dtype[17] = 0
    assert f(*bad_dtype) == -2                      # fp32 prefill not offered
    bad_d = list(ok)
    bad_d[15] = 256
    assert f(*bad_d) == -3
    bad_tq = list(ok)
    bad_tq[2] = -1
    assert f(*bad_tq) == -3
    null_q = list(ok)
    null_q[1] = NULL
    assert f(*null_q) == -1
    empty = list(ok)
    empty[11] = 0
    empty[1] = NULL
    assert f(*empty) == 0
    a = lib.kvcache_append
    assert a(P, P, 3, 16, 8, 128, P, P, P, 4, NULL) == -2
    assert a(P, P, 1, 16, 8, 100, P, P, P, 4, NULL) == -3
    assert a(P, P, 1, 16, 8, 128, P, P, NULL, 4, NULL) == -1
    assert a(NULL, NULL, 1, 16, 8, 128, NULL, NULL, NULL, 0, NULL) == 0


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_fp8_entry_points_check_arguments(lib, fmt):
    """The E4M3 and int8 pools' calls check their arguments alike."""
    a = getattr(lib, f"kvcache_append_{fmt}")
    ok = [P, P, 1, 16, 8, 128, P, P, P, 4, 0.5, 0.5, NULL]

    def with_(args, **kw):
        idx = {"dtype": 2, "d": 5, "k_new": 6, "tokens": 9, "ks": 10, "vs": 11}
        out = list(args)
        for k, v in kw.items():
            out[idx[k]] = v
        return out
    assert a(*with_(ok, dtype=7)) == -2
    assert a(*with_(ok, d=100)) == -3
    assert a(*with_(ok, ks=0.0)) == -3
    assert a(*with_(ok, vs=float("nan"))) == -3
    assert a(*with_(ok, vs=float("inf"))) == -3
    assert a(*with_(ok, k_new=NULL)) == -1
    assert a(*with_(ok, tokens=0, k_new=NULL)) == 0
    d = getattr(lib, f"lazyattn_decode_{fmt}")
    ok_d = [P, P, P, P, P, P, 4, NULL, P, 2, 8, 2, 128, 16, 0.088, 1e4, 0.5, 0.5, 0, P, 1 << 30, NULL]

    def dwith(**kw):
        idx = {"q": 1, "max_blocks": 6, "batch": 9, "hq": 10, "hkv": 11, "d": 12, "ks": 16, "vs": 17,
               "split": 18, "ws": 19}
        out = list(ok_d)
        for k, v in kw.items():
            out[idx[k]] = v
        return d(*out)
    p = getattr(lib, f"lazyattn_prefill_{fmt}")
    ok_p = [P, P, 8, P, P, P, P, P, 4, NULL, P, 1, 8, 8, 2, 128, 16, 0.088, 1e4, 0.5, 0.5, P, 1 << 30, NULL]

    def pwith(**kw):
        idx = {"q": 1, "total_q": 2, "batch": 11, "max_q": 12, "hq": 13, "hkv": 14, "d": 15, "ks": 19, "vs": 20,
               "ws": 21, "wsb": 22}
        out = list(ok_p)
        for k, v in kw.items():
            out[idx[k]] = v
        return p(*out)
    assert pwith(d=64) == -3                        # 8-bit pools: head_dim 128 only
    assert pwith(ks=0.0) == -3
    assert pwith(vs=float("inf")) == -3
    assert pwith(hq=6, hkv=4) == -3
    assert pwith(q=NULL) == -1
    assert pwith(batch=0, q=NULL) == 0
    assert pwith(ws=NULL) == -4
    pp = getattr(lib, f"lazyattn_prefill_{fmt}_precise")   # the precise variant checks alike
    for kw in ({"d": 64}, {"ks": 0.0}, {"vs": float("inf")}, {"hq": 6, "hkv": 4}, {"q": NULL},
               {"batch": 0, "q": NULL}, {"ws": NULL}):
        args = list(ok_p)
        for k, v in kw.items():
            args[{"q": 1, "batch": 11, "hq": 13, "hkv": 14, "d": 15, "ks": 19, "vs": 20, "ws": 21}[k]] = v
        assert pp(*args) == pwith(**kw)
    need = lib.lazyattn_prefill_fp8_workspace_size(1, 4, 2, 128)
    assert need == 2 * 1 * 4 * 2 * 16 * 128 * 2     # K and V, bf16, every block slot
    assert lib.lazyattn_prefill_fp8_workspace_size(1, 4, 2, 64) == 0
    assert pwith(ws=NULL) == -4                     # the widened copy needs a workspace
    assert pwith(wsb=need - 1) == -4
    assert dwith(d=64) == -3                        # 8-bit pools: head_dim 128 only
    assert dwith(ks=-1.0) == -3
    assert dwith(vs=0.0) == -3
    assert dwith(hq=6, hkv=4) == -3
    assert dwith(split=2) == -3
    assert dwith(q=NULL) == -1
    assert dwith(batch=0, q=NULL) == 0
    assert dwith(ws=NULL, max_blocks=4000) == -4
