"""The C-ABI library loads, exports every symbol its header declares, and
validates arguments on the host (no GPU needed: every case here returns an
error before any HIP call)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "basiskv.h")
LIB = os.path.join(ROOT, "routed_decode_attention_amd", "libbasiskv.so")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from routed_decode_attention_amd import build
        build.build()
    import routed_decode_attention_amd as rda
    return rda


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(basiskv_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 13
    raw = C.CDLL(LIB)
    for n in names:
        assert hasattr(raw, n), n
    assert set(names) == set(lib.EXPORTS)


def test_exports_nothing_but_the_declared_api(lib):
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    syms = {l.split()[-1] for l in out.splitlines() if l.strip()}
    syms = {x for x in syms if not x.startswith("__hip_cuid")}
    assert syms == set(declared_functions())


def test_version_matches_header(lib):
    m = re.search(r"#define BASISKV_VERSION (\d+)", open(HEADER).read())
    assert lib.basiskv_version() == int(m.group(1))


def _dims(lib, **kw):
    base = dict(batch=2, n_q_heads=4, n_kv_heads=1, head_dim=128, rank_v=32, rank_k=16,
                page_size=64, d_model=512, top_k=4, max_pages_per_seq=16, num_phys_pages=32,
                dtype=1, softmax_scale=0.0)
    base.update(kw)
    return lib.Dims(**base)


FAKE = C.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def _route(lib, d, **ptrs):
    raw = lib.basiskv._lib
    f = lib.basiskv.basiskv_factors(FAKE.value, FAKE.value, FAKE.value, FAKE.value, FAKE.value)
    c = lib.basiskv.basiskv_cache(FAKE.value, FAKE.value, FAKE.value, FAKE.value, FAKE.value)
    args = dict(seq_lens=FAKE, q=FAKE, sel=FAKE, n_sel=FAKE, scores=FAKE)
    args.update(ptrs)
    return raw.basiskv_route(C.byref(d.c()), C.byref(f), C.byref(c), args["seq_lens"], args["q"],
                             args["sel"], args["n_sel"], args["scores"], None, None)


def _decode(lib, d, ws_bytes):
    raw = lib.basiskv._lib
    f = lib.basiskv.basiskv_factors(FAKE.value, FAKE.value, FAKE.value, FAKE.value, FAKE.value)
    c = lib.basiskv.basiskv_cache(FAKE.value, FAKE.value, FAKE.value, FAKE.value, FAKE.value)
    return raw.basiskv_decode(C.byref(d.c()), C.byref(f), C.byref(c), FAKE, FAKE, FAKE, FAKE, None, FAKE,
                              ws_bytes, None, FAKE, None)


@pytest.mark.parametrize("kw,code", [
    (dict(n_q_heads=6, n_kv_heads=4), -2),
    (dict(top_k=17), -2),
    (dict(batch=0), -2),
    (dict(rank_v=256), -2),
    (dict(dtype=7), -2),
    (dict(softmax_scale=-1.0), -2),
    (dict(sink_pages=-1), -2),
    (dict(local_pages=-3), -2),
    (dict(group_mean=2), -2),
    (dict(head_select=-1), -2),
    (dict(head_dim=96, rank_v=32), -3),
    (dict(page_size=48), -3),
    (dict(rank_v=24), -3),
    (dict(rank_k=6), -3),
    (dict(n_q_heads=32, n_kv_heads=1), -3),
    (dict(max_pages_per_seq=9000, top_k=4), -3),
])
def test_route_rejects_bad_dims(lib, kw, code):
    assert _route(lib, _dims(lib, **kw)) == code
    assert lib.basiskv._lib.basiskv_last_error().decode() != ""


def test_null_pointers_and_small_workspace(lib):
    assert _route(lib, _dims(lib), sel=None) == -1  # sel and n_sel: both or neither
    assert _route(lib, _dims(lib), n_sel=None) == -1
    assert _route(lib, _dims(lib), scores=None) == -1
    assert _decode(lib, _dims(lib), 0) == -4
    assert _decode(lib, _dims(lib), lib.workspace_bytes(_dims(lib)) - 1) == -4
    raw = lib.basiskv._lib
    assert raw.basiskv_route(None, None, None, None, None, None, None, None, None, None) == -1


def test_workspace_bytes(lib):
    d = _dims(lib)
    n = lib.workspace_bytes(d)
    assert n > 0 and n % 256 == 0
    assert lib.workspace_bytes(d, 2048) > n
    raw = lib.basiskv._lib
    assert raw.basiskv_workspace_bytes(C.byref(_dims(lib, batch=0).c()), 0) == 0


def test_strerror(lib):
    raw = lib.basiskv._lib
    assert raw.basiskv_strerror(-4).decode() == "workspace too small"
    assert raw.basiskv_strerror(0).decode() == "ok"


def test_product_path_never_touches_the_oracle():
    """The library sources, header and binding name no oracle module."""
    pkg = os.path.join(ROOT, "routed_decode_attention_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "liboracle" not in text, f
                assert "ora_" not in text, f


def test_stream_read_validates_on_the_host(lib):
    raw = C.CDLL(LIB)
    f = raw.basiskv_stream_read
    f.argtypes = [C.c_void_p, C.c_size_t, C.c_void_p, C.c_int32, C.c_void_p]
    f.restype = C.c_int
    assert f(None, 64, FAKE, 4, None) == lib.E_NULL
    assert f(FAKE, 64, None, 4, None) == lib.E_NULL
    assert f(FAKE, 62, FAKE, 4, None) == lib.E_DIMS           # not whole words
    assert f(FAKE, 64, FAKE, 0, None) == lib.E_DIMS           # no workgroup
    assert f(C.c_void_p(0x1004), 64, FAKE, 4, None) == lib.E_DIMS  # misaligned
