"""The C ABI without a GPU: the library loads, exports every function include/gdn.h declares, and
rejects bad arguments on the host before any HIP call (so these run on a CPU-only machine)."""
import ctypes
import os
import re

import pytest

import linear_attention_sequence_rule_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gdn.lib_path()):
        import __graft_entry__
        __graft_entry__.build()
    return gdn.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|const char\*|void)\s+(gdn_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == ["gdn_chunk_fwd", "gdn_chunk_fwd_noalloc", "gdn_chunk_workspace_size",
                                    "gdn_recurrent_step", "gdn_status_string"]


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    assert gdn.gdn_status_string(0) == "GDN_OK"
    assert gdn.gdn_status_string(3) == "GDN_ERR_WORKSPACE"
    assert gdn.gdn_status_string(5) == "GDN_ERR_SCRATCH"
    assert gdn.gdn_status_string(99) == "GDN_ERR_UNKNOWN"


FAKE = 0x10000  # 16-byte aligned, never dereferenced: every case below fails validation first


def chunk(lib, **kw):
    a = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, g=FAKE * 4, beta=FAKE * 5, gp=None, s0=None, cu=None, conv=None,
             cst=None, z=None, nw=None, o=FAKE * 6, sf=None, ws=None, wsb=None, N=1, T=64, H=1, Hk=None, dk=32,
             dv=32, dtype=1, chunk=64, scale=1.0, eps=1e-3, flags=1)
    a.update(kw)
    if a["Hk"] is None:
        a["Hk"] = a["H"]
    return lib.gdn_chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["gp"], a["s0"], a["cu"], a["conv"],
                             a["cst"], a["z"], a["nw"], a["o"], a["sf"], a["ws"], a["wsb"], a["N"], a["T"], a["H"],
                             a["Hk"], a["dk"], a["dv"], a["dtype"], a["chunk"], a["scale"], a["eps"], a["flags"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dk=48), gdn.GDN_ERR_UNSUPPORTED),
    (dict(dv=256), gdn.GDN_ERR_UNSUPPORTED),
    (dict(dtype=7), gdn.GDN_ERR_UNSUPPORTED),
    (dict(chunk=32), gdn.GDN_ERR_UNSUPPORTED),
    (dict(q=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(o=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(N=0), gdn.GDN_ERR_INVALID_ARG),
    (dict(H=0), gdn.GDN_ERR_INVALID_ARG),
    (dict(T=-1), gdn.GDN_ERR_INVALID_ARG),
    (dict(N=3, T=64), gdn.GDN_ERR_INVALID_ARG),          # T_tot not divisible without cu_seqlens
    (dict(flags=8), gdn.GDN_ERR_INVALID_ARG),
    (dict(scale=float("nan")), gdn.GDN_ERR_INVALID_ARG),
    (dict(q=FAKE + 4), gdn.GDN_ERR_INVALID_ARG),          # misaligned
    (dict(o=FAKE), gdn.GDN_ERR_INVALID_ARG),              # o aliases q
    (dict(sf=FAKE * 3), gdn.GDN_ERR_INVALID_ARG),         # final state overlaps v
    (dict(s0=FAKE * 20, sf=FAKE * 20 + 16), gdn.GDN_ERR_INVALID_ARG),  # partial state overlap
    (dict(gp=FAKE * 7 + 8), gdn.GDN_ERR_INVALID_ARG),     # misaligned gate parameters
    (dict(gp=FAKE * 6 + 64), gdn.GDN_ERR_INVALID_ARG),    # o overlaps the gate parameters
    (dict(cst=FAKE * 8), gdn.GDN_ERR_INVALID_ARG),        # conv state without conv weights
    (dict(conv=FAKE * 7, cst=FAKE + 256), gdn.GDN_ERR_INVALID_ARG),    # conv state inside q
    (dict(conv=FAKE * 7, cst=FAKE * 7 + 64), gdn.GDN_ERR_INVALID_ARG),  # conv state overlaps conv_w
    (dict(conv=FAKE * 7, cst=FAKE * 8 + 4), gdn.GDN_ERR_INVALID_ARG),   # misaligned conv state
    (dict(H=4, Hk=3), gdn.GDN_ERR_INVALID_ARG),           # value heads not a multiple of query/key heads
    (dict(H=2, Hk=0), gdn.GDN_ERR_INVALID_ARG),
    (dict(H=2, Hk=4), gdn.GDN_ERR_INVALID_ARG),
    (dict(z=FAKE * 9), gdn.GDN_ERR_INVALID_ARG),                      # output gate without norm weight
    (dict(nw=FAKE * 9), gdn.GDN_ERR_INVALID_ARG),                     # norm weight without output gate
    (dict(z=FAKE * 9, nw=FAKE * 10, eps=-1.0), gdn.GDN_ERR_INVALID_ARG),
    (dict(z=FAKE * 9, nw=FAKE * 10, eps=float("inf")), gdn.GDN_ERR_INVALID_ARG),
    (dict(z=FAKE * 6 + 512, nw=FAKE * 10), gdn.GDN_ERR_INVALID_ARG),  # output gate overlaps o
    (dict(z=FAKE * 9, nw=FAKE * 6 + 64), gdn.GDN_ERR_INVALID_ARG),    # norm weight inside o
    (dict(z=FAKE * 9 + 8, nw=FAKE * 10), gdn.GDN_ERR_INVALID_ARG),    # misaligned
])
def test_chunk_validation(lib, kw, status):
    assert chunk(lib, **kw) == status


def test_workspace_query(lib):
    n = ctypes.c_size_t(0)
    # one long sequence, 16 heads: too few (head, row block) units for the device -> segments
    assert lib.gdn_chunk_workspace_size(1, 262144, 16, 16, 128, 128, gdn.GDN_BF16, 64, 0, 0, 1, ctypes.byref(n)) == 0
    need = n.value
    assert need > 0
    wsb = ctypes.c_size_t(0)
    big = 1 << 32  # disjoint fake ranges, never dereferenced (the call fails before any launch)
    st = chunk(lib, N=1, T=262144, H=16, dk=128, dv=128, q=big, k=2 * big, v=3 * big, g=4 * big, beta=5 * big,
               o=6 * big, ws=None, wsb=ctypes.byref(wsb))
    assert st == gdn.GDN_ERR_WORKSPACE and wsb.value == need
    # a workspace overlapping an input is rejected
    wsb = ctypes.c_size_t(need)
    st = chunk(lib, N=1, T=262144, H=16, dk=128, dv=128, q=big, k=2 * big, v=3 * big, g=4 * big, beta=5 * big,
               o=6 * big, ws=3 * big + 64, wsb=ctypes.byref(wsb))
    assert st == gdn.GDN_ERR_INVALID_ARG


def test_workspace_segments_flag(lib):
    n = ctypes.c_size_t(0)
    seg = lambda p: (p & 0xFF) << 8
    # explicit single segment: no workspace; explicit 4 segments on a short input: workspace
    assert lib.gdn_chunk_workspace_size(1, 262144, 16, 16, 128, 128, 1, 64, 0, 0, 1 | seg(1), ctypes.byref(n)) == 0
    assert n.value == 0
    assert lib.gdn_chunk_workspace_size(2, 256, 2, 2, 64, 32, 1, 64, 0, 0, 1 | seg(4), ctypes.byref(n)) == 0
    units = 2 * 4 * 2
    assert n.value >= units * (32 * 64 + 64 * 64 + 1) * 4
    # many (sequence, head) units: automatic single pass
    assert lib.gdn_chunk_workspace_size(64, 64 * 4096, 32, 32, 128, 128, 1, 64, 1, 0, 1, ctypes.byref(n)) == 0
    assert n.value == 0
    # segments need the bf16 path (with or without conv)
    assert lib.gdn_chunk_workspace_size(1, 4096, 1, 1, 32, 32, 0, 64, 0, 0, 1 | seg(2), ctypes.byref(n)) == \
        gdn.GDN_ERR_UNSUPPORTED
    assert lib.gdn_chunk_workspace_size(1, 4096, 1, 1, 32, 32, 1, 64, 0, 1, 1 | seg(2), ctypes.byref(n)) == 0
    assert n.value > 0


def test_workspace_segments_layout(lib):
    """The segmented path's workspace: per (sequence, segment, head) the end state B_p, the
    transition A_p, its mark, the first chunk's kept operands (19,776 bytes) and the chained
    entering state, each region rounded up to 256 bytes."""
    n = ctypes.c_size_t(0)
    seg = lambda p: (p & 0xFF) << 8
    a256 = lambda x: (x + 255) // 256 * 256
    for N, H, dk, dv, P in ((2, 2, 64, 32, 4), (1, 16, 128, 128, 16), (3, 5, 32, 64, 3)):
        assert lib.gdn_chunk_workspace_size(N, N * 64 * P, H, H, dk, dv, 1, 64, 0, 0, 1 | seg(P), ctypes.byref(n)) == 0
        units = N * P * H
        want = (a256(units * dv * dk * 4) + a256(units * dk * dk * 4) + a256(units * 4) + a256(units * 19776)
                + a256(units * dv * dk * 4))
        assert n.value == want, (N, H, dk, dv, P, n.value, want)


def test_workspace_size_validation(lib):
    n = ctypes.c_size_t(0)
    assert lib.gdn_chunk_workspace_size(1, 64, 1, 1, 33, 32, 1, 64, 0, 0, 1, ctypes.byref(n)) == gdn.GDN_ERR_UNSUPPORTED
    assert lib.gdn_chunk_workspace_size(3, 64, 1, 1, 32, 32, 1, 64, 0, 0, 1, ctypes.byref(n)) == gdn.GDN_ERR_INVALID_ARG
    assert lib.gdn_chunk_workspace_size(1, 64, 1, 1, 32, 32, 1, 64, 0, 0, 1, None) == gdn.GDN_ERR_INVALID_ARG
    assert lib.gdn_chunk_workspace_size(1, 64, 1, 1, 32, 32, 1, 64, 0, 0, 1 << 20, ctypes.byref(n)) == \
        gdn.GDN_ERR_INVALID_ARG


@pytest.mark.parametrize("kw,status", [
    (dict(dk=16), gdn.GDN_ERR_UNSUPPORTED),
    (dict(state=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(N=-1), gdn.GDN_ERR_INVALID_ARG),
    (dict(o=FAKE * 6 + 64), gdn.GDN_ERR_INVALID_ARG),   # o inside the state
    (dict(flags=2), gdn.GDN_ERR_INVALID_ARG),
    (dict(flags=1 | (2 << 8)), gdn.GDN_ERR_INVALID_ARG),  # segments are a prefill option
    (dict(N=0), gdn.GDN_OK),                        # empty batch: no-op, no launch
    (dict(conv=FAKE * 7), gdn.GDN_ERR_INVALID_ARG),         # conv weights without a conv state
    (dict(cst=FAKE * 8), gdn.GDN_ERR_INVALID_ARG),          # conv state without conv weights
    (dict(conv=FAKE * 7, cst=FAKE * 6 + 128), gdn.GDN_ERR_INVALID_ARG),  # conv state inside the state
    (dict(conv=FAKE * 7, cst=FAKE * 2 + 32), gdn.GDN_ERR_INVALID_ARG),   # conv state overlaps k
    (dict(conv=FAKE * 7, cst=FAKE * 8 + 2), gdn.GDN_ERR_INVALID_ARG),    # misaligned
    (dict(gp=FAKE * 100 + 16), gdn.GDN_ERR_INVALID_ARG),    # gate parameters inside o
    (dict(gp=FAKE * 9 + 4), gdn.GDN_ERR_INVALID_ARG),       # misaligned gate parameters
    (dict(H=3, Hk=2), gdn.GDN_ERR_INVALID_ARG),             # value heads not a multiple of query/key heads
    (dict(Hk=0), gdn.GDN_ERR_INVALID_ARG),
    (dict(z=FAKE * 9), gdn.GDN_ERR_INVALID_ARG),                      # output gate without norm weight
    (dict(z=FAKE * 9, nw=FAKE * 10, eps=float("nan")), gdn.GDN_ERR_INVALID_ARG),
    (dict(z=FAKE * 100 + 64, nw=FAKE * 10), gdn.GDN_ERR_INVALID_ARG),  # output gate overlaps o
    (dict(z=FAKE * 9, nw=FAKE * 6 + 256), gdn.GDN_ERR_INVALID_ARG),   # norm weight inside the state
])
def test_step_validation(lib, kw, status):
    a = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, g=FAKE * 4, beta=FAKE * 5, gp=None, state=FAKE * 6, conv=None, cst=None,
             z=None, nw=None, o=FAKE * 100, N=2, H=1, Hk=None, dk=32, dv=32, dtype=1, scale=1.0, eps=1e-3, flags=1)
    a.update(kw)
    if a["Hk"] is None:
        a["Hk"] = a["H"]
    assert lib.gdn_recurrent_step(a["q"], a["k"], a["v"], a["g"], a["beta"], a["gp"], a["state"], a["conv"],
                                  a["cst"], a["z"], a["nw"], a["o"], a["N"], a["H"], a["Hk"], a["dk"], a["dv"],
                                  a["dtype"], a["scale"], a["eps"], a["flags"], None) == status


def test_python_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(gdn, "_lib", None)
    monkeypatch.setattr(gdn, "_LIB_PATH", "/nonexistent/libgdn.so")
    with pytest.raises(RuntimeError, match="not built"):
        gdn.load_library()


def test_workspace_conv_pass(lib):
    """A bf16 call with conv weights needs room for the convolved q, k and v (the conv pass), unless
    the conv runs inside the chunk kernel (GDN_CONV_FUSED, or dk = 128 with dv a multiple of 128);
    the fp32 path never does."""
    n = ctypes.c_size_t(0)
    a256 = lambda x: (x + 255) // 256 * 256
    N, T, H, Hk, dk, dv = 2, 1000, 4, 2, 64, 32
    one_seg = 1 | (1 << 8)
    assert lib.gdn_chunk_workspace_size(N, T, H, Hk, dk, dv, 1, 64, 1, 1, one_seg, ctypes.byref(n)) == 0
    assert n.value == 2 * a256(T * Hk * dk * 2) + a256(T * H * dv * 2)
    assert lib.gdn_chunk_workspace_size(N, T, H, Hk, dk, dv, 1, 64, 1, 1, one_seg | gdn.GDN_CONV_FUSED,
                                        ctypes.byref(n)) == 0
    assert n.value == 0
    assert lib.gdn_chunk_workspace_size(N, T, H, Hk, dk, dv, 0, 64, 1, 1, one_seg, ctypes.byref(n)) == 0
    assert n.value == 0
    assert lib.gdn_chunk_workspace_size(N, T, H, Hk, dk, dv, 1, 64, 1, 0, one_seg, ctypes.byref(n)) == 0
    assert n.value == 0
    # dk = dv = 128 (128-row workgroups): the conv runs inside the chunk kernel, no conv workspace
    assert lib.gdn_chunk_workspace_size(64, 64 * 4096, 32, 32, 128, 128, 1, 64, 1, 1, one_seg, ctypes.byref(n)) == 0
    assert n.value == 0
    # a bf16 conv call without that workspace reports the size and launches nothing
    big = 1 << 32
    wsb = ctypes.c_size_t(0)
    st = chunk(lib, N=N, T=T, H=H, Hk=Hk, dk=dk, dv=dv, q=big, k=2 * big, v=3 * big, g=4 * big, beta=5 * big,
               o=6 * big, conv=7 * big, cu=8 * big, flags=one_seg, wsb=ctypes.byref(wsb))
    assert st == gdn.GDN_ERR_WORKSPACE and wsb.value == 2 * a256(T * Hk * dk * 2) + a256(T * H * dv * 2)
    # Hk must divide H here too
    assert lib.gdn_chunk_workspace_size(N, T, 3, 2, dk, dv, 1, 64, 1, 1, 1, ctypes.byref(n)) == gdn.GDN_ERR_INVALID_ARG


def test_noalloc_rejects_calls_beyond_its_scratch(lib):
    """gdn_chunk_fwd_noalloc: a call whose workspace exceeds the static scratch (here the separate
    conv pass of a long 64-wide input: T_tot (2 Hk dk + H dv) 2 bytes) returns GDN_ERR_SCRATCH on the
    host, before any launch; argument errors come first, as for gdn_chunk_fwd."""
    big = 1 << 36
    T, H, dk, dv = 1 << 20, 32, 64, 64
    n = ctypes.c_size_t(0)
    assert lib.gdn_chunk_workspace_size(1, T, H, H, dk, dv, 1, 64, 1, 1, 1 | (1 << 8), ctypes.byref(n)) == 0
    assert n.value > gdn.GDN_NOALLOC_SCRATCH_BYTES
    args = [big, 2 * big, 3 * big, 4 * big, 5 * big, None, None, 6 * big, 7 * big, None, None, None, 8 * big, None]
    st = lib.gdn_chunk_fwd_noalloc(*args, 1, T, H, H, dk, dv, 1, 64, 1.0, 1e-3, 1 | (1 << 8), None)
    assert st == gdn.GDN_ERR_SCRATCH
    st = lib.gdn_chunk_fwd_noalloc(*args, 1, T, H, H, 48, dv, 1, 64, 1.0, 1e-3, 1 | (1 << 8), None)
    assert st == gdn.GDN_ERR_UNSUPPORTED
