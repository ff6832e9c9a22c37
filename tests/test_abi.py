"""C-ABI checks that need no GPU: the library loads, exports every function
include/gdr.h declares, and validates descriptors / arguments before touching
the device (every call below returns from the host-side checks)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdr.h")

gdr = pytest.importorskip("chunked_gated_delta_gdr_amd")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gdr.library_path()):
        import chunked_gated_delta_gdr_amd.build as b
        b.build()
    return gdr._load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdr_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"gdr_bwd", "gdr_bwd_workspace_bytes", "gdr_strerror"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in gdr.h but not exported"


def test_version_and_strerror(lib):
    assert lib.gdr_version().decode().count(".") == 2
    for code in (0, -1, -2, -3, -4, 7):
        assert isinstance(lib.gdr_strerror(code), bytes)


def desc(**kw):
    base = dict(B=2, T=4096, H=16, Hg=16, K=128, V=128, chunk=64, n_seqs=0, gate=0,
                io_dtype=1, scale=0.0, sub_chunk=16)
    base.update(kw)
    return gdr.Desc(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(), 0),
    (dict(H=32, Hg=16, chunk=32, io_dtype=2, gate=1), 0),
    (dict(K=64, V=64, io_dtype=0, T=256, B=1, H=2, Hg=2), 0),
    (dict(B=1, T=32768, n_seqs=24), 0),
    (dict(H=16, Hg=5), -1),
    (dict(B=0), -1),
    (dict(T=-1), -1),
    (dict(gate=2), -1),
    (dict(io_dtype=7), -1),
    (dict(n_seqs=3), -1),            # varlen needs B == 1
    (dict(K=96, V=96), -2),
    (dict(K=128, V=64), -2),
    (dict(chunk=16), -2),
    (dict(sub_chunk=8), -2),
    (dict(io_dtype=0), -2),          # fp32 io is built for K = 64 only
])
def test_check_codes(lib, kw, code):
    assert gdr.check(desc(**kw)) == code


def test_workspace_bytes(lib):
    d = desc()
    n = gdr.workspace_bytes(d)
    offs = gdr.workspace_offsets(d)
    assert offs["total"] == n
    order = [offs[k] for k in gdr.WS_NAMES]
    assert order == sorted(order) and all(o % 256 == 0 for o in order)
    # the per-chunk states: 128 chunks x 16 heads x 128 x 128 bf16
    assert offs["X"] - offs["h"] >= 128 * 16 * 128 * 128 * 2
    assert lib.gdr_bwd_workspace_bytes(ctypes.byref(desc(K=96, V=96))) == 0
    # varlen capacity: floor(T / C) + n_seqs chunks
    dv = desc(B=1, T=1000, n_seqs=7)
    o = gdr.workspace_offsets(dv)
    assert o["seq_off"] - o["ctab"] >= (1000 // 64 + 7) * 16


def _call(lib, d, ptrs=None, ws=None, wsb=0, **over):
    names = ["q", "k", "v", "g", "beta", "h0", "do", "dht", "cu", "dq", "dk", "dv", "dg", "db", "dh0"]
    p = {n: ctypes.c_void_p(0x100000 * (i + 1)) for i, n in enumerate(names)}
    p["h0"] = p["dht"] = p["cu"] = None
    if ptrs:
        p.update(ptrs)
    return lib.gdr_bwd(ctypes.byref(d), *[p[n] for n in names],
                       ws, ctypes.c_size_t(wsb), None)


def test_bwd_argument_errors_before_any_launch(lib):
    d = desc()
    need = gdr.workspace_bytes(d)
    big = ctypes.c_void_p(0x7F0000000000)
    assert _call(lib, desc(K=96, V=96)) == -2
    assert _call(lib, d, {"q": None}, big, need) == -1            # null input
    assert _call(lib, d, {"dg": ctypes.c_void_p(0x100008)}, big, need) == -1  # misaligned
    assert _call(lib, d, None, None, need) == -3                  # no workspace
    assert _call(lib, d, None, big, need - 1) == -3               # too small
    assert _call(lib, d, None, ctypes.c_void_p(0x7F0000000010), need) == -1  # not 256-aligned
    dvl = desc(B=1, T=1000, n_seqs=4)
    assert _call(lib, dvl, None, big, gdr.workspace_bytes(dvl)) == -1  # varlen without cu_seqlens
    assert _call(lib, d, {"cu": ctypes.c_void_p(0x200000)}, big, need) == -1  # cu without varlen


def test_fwd_argument_errors(lib):
    """gdr_fwd rejects bad arguments before touching the GPU."""
    d = desc()
    P = ctypes.c_void_p
    ptrs = [P(0x100000 * (i + 1)) for i in range(6)]   # q, k, v, g, beta, o
    ws = P(0x1000000)
    n = lib.gdr_bwd_workspace_bytes(ctypes.byref(d))
    def call(q=ptrs[0], o=ptrs[5], wsp=ws, wsb=n, cu=None, dd=d):
        return lib.gdr_fwd(ctypes.byref(dd), q, ptrs[1], ptrs[2], ptrs[3], ptrs[4], None, cu, o, None,
                           wsp, ctypes.c_size_t(wsb), None)
    assert call(q=None) == -1                      # required input missing
    assert call(o=None) == -1                      # output missing
    assert call(q=P(0x100001)) == -1               # misaligned
    assert call(wsb=n - 1) == -3                   # workspace too small
    assert call(wsp=None) == -3
    assert call(cu=P(0x2000000)) == -1             # cu_seqlens without n_seqs
    assert call(dd=desc(K=96, V=96)) == -2         # unsupported


def test_bwd_after_fwd_argument_errors(lib):
    """gdr_bwd_after_fwd rejects bad arguments before touching the GPU."""
    d = desc()
    P = ctypes.c_void_p
    ptrs = [P(0x100000 * (i + 1)) for i in range(12)]   # q k v g beta do dq dk dv dg db dh0
    ws = P(0x1000000)
    n = lib.gdr_bwd_workspace_bytes(ctypes.byref(d))
    def call(over=None, wsp=ws, wsb=n, cu=None, dd=d):
        a = list(ptrs)
        for i, v in (over or {}).items():
            a[i] = v
        return lib.gdr_bwd_after_fwd(ctypes.byref(dd), *a[:6], None, cu, *a[6:],
                                     wsp, ctypes.c_size_t(wsb), None)
    assert call({0: None}) == -1                   # q missing
    assert call({11: None}) == -1                  # dh0 missing (always written)
    assert call({9: P(0x100004)}) == -1            # misaligned dg
    assert call(wsb=n - 1) == -3                   # workspace too small
    assert call(wsp=None) == -3
    assert call(wsp=P(0x1000010)) == -1            # workspace not 256-aligned
    assert call(cu=P(0x2000000)) == -1             # cu_seqlens without n_seqs
    assert call(dd=desc(K=96, V=96)) == -2         # unsupported


def test_static_entry_rejects_problems_over_its_scratch(lib):
    """gdr_bwd_static returns GDR_ESCRATCH for a descriptor whose workspace
    exceeds GDR_STATIC_SCRATCH_BYTES, before touching the device (so NULL
    buffers are fine here); invalid descriptors keep their own codes."""
    P = [None] * 15
    big = desc()   # the full-size headline workload: several hundred MB of workspace
    assert gdr.workspace_bytes(big) > gdr.STATIC_SCRATCH_BYTES
    assert lib.gdr_bwd_static(ctypes.byref(big), *P, None) == -5
    assert b"scratch" in lib.gdr_strerror(-5)
    assert lib.gdr_bwd_static(ctypes.byref(desc(K=96, V=96)), *P, None) == -2
    assert lib.gdr_bwd_static(ctypes.byref(desc(H=16, Hg=5)), *P, None) == -1
    with open(HEADER) as f:
        assert f"((size_t){gdr.STATIC_SCRATCH_BYTES >> 20} << 20)" in f.read()


def test_from_states_argument_checks(lib):
    """gdr_bwd_from_states validates on the host before touching the device:
    the descriptor (state_v_first in {0, 1}), the per-chunk state count (fixed
    length: exactly B ceil(T / chunk)) and the required pointers."""
    P = ctypes.c_void_p
    fake = P(0x10000)   # never dereferenced: every call below fails its host checks
    bufs = [fake] * 8   # q, k, v, g, beta, do, dht, cu_seqlens
    outs = [fake] * 6
    d = desc(B=1, T=130, H=2, Hg=2)   # 3 chunks of 64
    call = lambda dd, cu, h, n: lib.gdr_bwd_from_states(ctypes.byref(dd), *bufs[:7], cu, h, ctypes.c_int64(n),
                                                        *outs, fake, ctypes.c_size_t(0), None)
    assert gdr.check(desc(state_v_first=2)) == -1
    assert call(d, None, fake, 2) == -1          # fixed length needs exactly 3 states
    assert call(d, None, fake, 4) == -1
    assert call(d, None, None, 3) == -1          # h required when there are tokens
    assert call(d, None, fake, 3) == -3          # right count: then the (missing) workspace is the error
    assert call(desc(state_v_first=3), None, fake, 3) == -1
