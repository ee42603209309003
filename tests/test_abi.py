"""The C ABI library loads, exports every symbol the header declares, and rejects bad arguments
on the host before touching the device (these checks run without a GPU: every call below fails
validation, so nothing is ever enqueued)."""
import ctypes
import os
import re

import pytest

import chunked_weight_sequence_amd as ttt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ttt_mi355x.h")

OK, E_NULL, E_SHAPE, E_DTYPE, E_ALIGN, E_WS, E_UNSUP, E_LAUNCH, E_ALIAS = range(9)
A = 0x7F0000000000          # fake, 16-byte aligned device addresses (never dereferenced)
MB = 1 << 20


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ttt_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert set(names) == set(ttt.EXPORTED), names
    lib = ctypes.CDLL(ttt.library_path)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_status_strings():
    m = re.search(r"#define TTT_ABI_VERSION (\d+)", open(HEADER).read())
    assert ttt.abi_version() == int(m.group(1))
    for code in range(9):
        s = ttt.status_string(code)
        assert s.startswith("TTT_"), s
    assert "unknown" in ttt.status_string(99)


def scan(**kw):
    a = dict(Z=A, V=A + 64 * MB, ind=1, W0=A + 128 * MB, shared=1, O=A + 192 * MB, outd=1,
             Wf=A + 256 * MB, B=1, T=1024, F=256, D=64, C=64, eta=1e-3, ws=A + 512 * MB,
             wsb=1 << 40, stream=None)
    a.update(kw)
    return ttt.lib().ttt_chunk_scan(a["Z"], a["V"], a["ind"], a["W0"], a["shared"], a["O"],
                                    a["outd"], a["Wf"], a["B"], a["T"], a["F"], a["D"], a["C"],
                                    a["eta"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(Z=None), E_NULL), (dict(V=None), E_NULL), (dict(W0=None), E_NULL),
    (dict(O=None), E_NULL),
    (dict(ind=7), E_DTYPE), (dict(outd=-1), E_DTYPE),
    (dict(F=24), E_SHAPE), (dict(D=8), E_SHAPE), (dict(C=0), E_SHAPE), (dict(T=0), E_SHAPE),
    (dict(B=0), E_SHAPE), (dict(eta=float("nan")), E_SHAPE),
    (dict(eta=1e-20), E_UNSUP), (dict(eta=-3e18), E_UNSUP),      # bf16 state is W / eta
    (dict(Z=A + 8), E_ALIGN), (dict(Wf=A + 256 * MB + 4), E_ALIGN),
    (dict(wsb=16), E_WS), (dict(ws=None), E_WS),
    (dict(Wf=A + 1024), E_ALIAS),                          # W_final inside Z
    (dict(O=A + 64 * MB + 4096), E_ALIAS),                 # O inside V_hat
    (dict(B=2, Wf=A + 128 * MB), E_ALIAS),                 # in place on a shared W0, B > 1
    (dict(Wf=A + 128 * MB + 4096), E_ALIAS),               # partial overlap with W0
    (dict(ws=A + 192 * MB), E_ALIAS),                      # workspace on top of O
])
def test_scan_rejects_bad_arguments(kw, code):
    assert scan(**kw) == code


def test_scan_workspace_query():
    lib = ttt.lib()
    assert lib.ttt_chunk_scan_workspace(1, 1024, 24, 64, 64, 1) == 0          # invalid
    assert lib.ttt_chunk_scan_workspace(1, 1024, 256, 64, 64, 5) == 0         # bad dtype
    small = lib.ttt_chunk_scan_workspace(1, 1024, 256, 64, 64, 0)
    assert small == 64 * 256 * 4                                             # fp32 working W
    big = lib.ttt_chunk_scan_workspace(1, 32768, 9728, 2560, 512, 1)
    assert big > 2 * 32768 * (9728 + 2560)                                   # staged operands


def linear(**kw):
    a = dict(Q=A, K=A + 64 * MB, V=A + 128 * MB, ind=1, W0=None, O=A + 192 * MB, outd=1,
             Wf=None, loss=None, B=1, T=256, H=4, dh=64, b=16, eta=0.1, stream=None)
    a.update(kw)
    return ttt.lib().ttt_linear_minibatch(a["Q"], a["K"], a["V"], a["ind"], a["W0"], a["O"],
                                          a["outd"], a["Wf"], a["loss"], a["B"], a["T"], a["H"],
                                          a["dh"], a["b"], a["eta"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(Q=None), E_NULL), (dict(O=None), E_NULL), (dict(ind=3), E_DTYPE),
    (dict(dh=32), E_UNSUP), (dict(b=0), E_SHAPE), (dict(T=250, b=16), E_SHAPE),
    (dict(H=0), E_SHAPE), (dict(K=A + 64 * MB + 2), E_ALIGN),
    (dict(O=A + 4096), E_ALIAS), (dict(loss=A + 128 * MB + 4096), E_ALIAS),
    (dict(W0=A + 256 * MB, Wf=A + 256 * MB + 64), E_ALIAS),
])
def test_linear_rejects_bad_arguments(kw, code):
    assert linear(**kw) == code


def route(**kw):
    a = dict(loss=A, K=A + 64 * MB, V=A + 128 * MB, kvd=1, B=4, T=2048, H=16, dh=64, C=64,
             pct=0.95, ema=0.9, ratio=0.8, cap=256, tau=A + 192 * MB, mask=A + 200 * MB,
             idx=A + 208 * MB, ck=A + 216 * MB, cv=A + 232 * MB, cnt=A + 248 * MB,
             tot=A + 249 * MB, stream=None)
    a.update(kw)
    return ttt.lib().ttt_surprisal_route(a["loss"], a["K"], a["V"], a["kvd"], a["B"], a["T"],
                                         a["H"], a["dh"], a["C"], a["pct"], a["ema"],
                                         a["ratio"], a["cap"], a["tau"], a["mask"], a["idx"],
                                         a["ck"], a["cv"], a["cnt"], a["tot"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(loss=None), E_NULL), (dict(idx=None), E_NULL), (dict(K=None), E_NULL),
    (dict(kvd=9), E_DTYPE), (dict(C=60), E_SHAPE), (dict(C=2048), E_SHAPE),
    (dict(T=(1 << 22) + 64, C=64), E_SHAPE), (dict(pct=0.0), E_SHAPE), (dict(pct=1.5), E_SHAPE),
    (dict(ema=-0.1), E_SHAPE), (dict(cap=0), E_SHAPE), (dict(cap=5000), E_SHAPE),
    (dict(H=1, dh=3), E_SHAPE), (dict(tau=A + 192 * MB + 2), E_ALIGN),
    (dict(idx=A + 64 * MB), E_ALIAS), (dict(cnt=A + 208 * MB), E_ALIAS),
])
def test_route_rejects_bad_arguments(kw, code):
    assert route(**kw) == code


def test_binding_refuses_cpu_tensors():
    import torch
    z = torch.zeros(64, 256, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ttt.chunk_scan(z, torch.zeros(64, 64, dtype=torch.bfloat16),
                       torch.zeros(64, 256), 16, 0.0)


def target(**kw):
    a = dict(X=A, ind=1, cw=A + 64 * MB, width=4, W=A + 128 * MB, V=A + 192 * MB, outd=1, B=1,
             T=1024, din=128, dout=96, C=64, ws=A + 512 * MB, wsb=1 << 40, stream=None)
    a.update(kw)
    return ttt.lib().ttt_lm_target(a["X"], a["ind"], a["cw"], a["width"], a["W"], a["V"],
                                   a["outd"], a["B"], a["T"], a["din"], a["dout"], a["C"],
                                   a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(X=None), E_NULL), (dict(cw=None), E_NULL), (dict(W=None), E_NULL), (dict(V=None), E_NULL),
    (dict(ind=3), E_DTYPE), (dict(outd=9), E_DTYPE),
    (dict(din=96), E_SHAPE), (dict(dout=40), E_SHAPE), (dict(width=0), E_SHAPE),
    (dict(width=17), E_SHAPE), (dict(C=0), E_SHAPE), (dict(T=0), E_SHAPE), (dict(B=0), E_SHAPE),
    (dict(ind=0), E_UNSUP),                                 # fp32 X0: not implemented
    (dict(V=A + 192 * MB + 8), E_ALIGN), (dict(ws=A + 8), E_ALIGN),
    (dict(wsb=100), E_WS), (dict(ws=None), E_WS),
    (dict(V=A + 4096), E_ALIAS),                            # V_hat inside X0
    (dict(ws=A + 128 * MB), E_ALIAS),                       # workspace on W_target
])
def test_lm_target_rejects_bad_arguments(kw, code):
    assert target(**kw) == code


def test_lm_target_workspace_query():
    lib = ttt.lib()
    a = (2 * 1000 * 128 * 2 + 255) // 256 * 256
    assert lib.ttt_lm_target_workspace(2, 1000, 128, 96) == a + 128 * 96 * 2
    assert lib.ttt_lm_target_workspace(1, 1000, 100, 96) == 0
    assert lib.ttt_lm_target_workspace(0, 1000, 128, 96) == 0
    assert lib.ttt_lm_target_workspace(1, 1000, 128, 40) == 0


def gz(**kw):
    a = dict(X=A, ind=1, W=A + 64 * MB, Z=A + 128 * MB, outd=1, B=2, T=1000, dm=128, dff=96,
             stream=None)
    a.update(kw)
    return ttt.lib().ttt_gated_z(a["X"], a["ind"], a["W"], a["Z"], a["outd"], a["B"], a["T"],
                                 a["dm"], a["dff"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(X=None), E_NULL), (dict(W=None), E_NULL), (dict(Z=None), E_NULL),
    (dict(ind=3), E_DTYPE), (dict(outd=-1), E_DTYPE),
    (dict(dm=96), E_SHAPE), (dict(dm=0), E_SHAPE), (dict(dff=100), E_SHAPE), (dict(dff=0), E_SHAPE),
    (dict(T=0), E_SHAPE), (dict(B=0), E_SHAPE), (dict(B=70000), E_SHAPE),
    (dict(dm=1 << 16, dff=1 << 15), E_SHAPE),                # weight offsets past 32 bits
    (dict(ind=0), E_UNSUP),                                  # fp32 X: not implemented
    (dict(X=A + 8), E_ALIGN), (dict(W=A + 64 * MB + 4), E_ALIGN), (dict(Z=A + 128 * MB + 2), E_ALIGN),
    (dict(Z=A + 4096), E_ALIAS),                             # Z inside X
    (dict(Z=A + 64 * MB + 16), E_ALIAS),                     # Z on W_gu
    (dict(Z=A + 64 * MB - 16), E_ALIAS),                     # Z's tail reaches W_gu
])
def test_gated_z_rejects_bad_arguments(kw, code):
    assert gz(**kw) == code


def readout(**kw):
    a = dict(Q=A, K=A + 16 * MB, V=A + 32 * MB, qd=1, mask=A + 48 * MB, O=A + 64 * MB,
             out=A + 80 * MB, outd=1, alpha=A + 96 * MB, B=4, T=2048, H=16, dh=64, C=64, cap=256,
             scale=0.125, stream=None)
    a.update(kw)
    return ttt.lib().ttt_cache_readout(a["Q"], a["K"], a["V"], a["qd"], a["mask"], a["O"],
                                       a["out"], a["outd"], a["alpha"], a["B"], a["T"], a["H"],
                                       a["dh"], a["C"], a["cap"], a["scale"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(Q=None), E_NULL), (dict(mask=None), E_NULL), (dict(alpha=None), E_NULL),
    (dict(out=None), E_NULL), (dict(qd=5), E_DTYPE), (dict(outd=7), E_DTYPE),
    (dict(T=0), E_SHAPE), (dict(B=0), E_SHAPE), (dict(H=0), E_SHAPE), (dict(C=0), E_SHAPE),
    (dict(C=96), E_SHAPE),                                   # T % chunk != 0
    (dict(cap=0), E_SHAPE), (dict(scale=float("nan")), E_SHAPE),
    (dict(qd=0), E_UNSUP), (dict(dh=128, H=8), E_UNSUP), (dict(C=32), E_UNSUP),
    (dict(cap=257), E_UNSUP),
    (dict(out=A + 80 * MB + 8), E_ALIGN), (dict(alpha=A + 96 * MB + 4), E_ALIGN),
    (dict(mask=A + 48 * MB + 1), E_ALIGN),
    (dict(out=A + 4096), E_ALIAS),                           # out inside Q
    (dict(out=A + 64 * MB + 64), E_ALIAS),                   # partial overlap with ttt_out
    (dict(out=A + 96 * MB - 1024), E_ALIAS),                 # out's tail reaches alpha
])
def test_cache_readout_rejects_bad_arguments(kw, code):
    assert readout(**kw) == code



def docs(**kw):
    import ctypes
    a = dict(Z=A, V=A + 64 * MB, ind=1, W0=A + 128 * MB, sh=1, O=A + 192 * MB, outd=1,
             Wf=A + 256 * MB, B=2, T=1024, F=256, D=128, C=64, eta=0.01, starts=None, counts=None,
             tau=0.5, ws=A + 512 * MB, wsb=1 << 40, stream=None)
    a.update(kw)
    keep = []

    def arr(x):
        if x is None:
            return None
        c = (ctypes.c_int * max(1, len(x)))(*x)
        keep.append(c)
        return ctypes.addressof(c)

    return ttt.lib().ttt_chunk_scan_docs(a["Z"], a["V"], a["ind"], a["W0"], a["sh"], a["O"],
                                         a["outd"], a["Wf"], a["B"], a["T"], a["F"], a["D"],
                                         a["C"], a["eta"], arr(a["starts"]), arr(a["counts"]),
                                         a["tau"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(Z=None), E_NULL), (dict(ind=4), E_DTYPE), (dict(F=100), E_SHAPE),
    (dict(tau=float("nan")), E_SHAPE),
    (dict(starts=[100], counts=[1, 0]), E_SHAPE),            # not a multiple of the chunk
    (dict(starts=[0], counts=[1, 0]), E_SHAPE),              # must lie inside (0, T)
    (dict(starts=[1024], counts=[1, 0]), E_SHAPE),
    (dict(starts=[256, 128], counts=[2, 0]), E_SHAPE),       # not increasing
    (dict(starts=[128], counts=[-1, 2]), E_SHAPE),
    (dict(starts=None, counts=[1, 0]), E_NULL),
    (dict(wsb=100), E_WS), (dict(ws=None), E_WS),
    (dict(ws=A + 4096), E_ALIAS),                            # workspace on Z
    (dict(O=A + 64 * MB), E_ALIAS),
    (dict(Wf=A + 128 * MB), E_ALIAS),                        # shared W0 with B = 2 in place
])
def test_chunk_scan_docs_rejects_bad_arguments(kw, code):
    assert docs(**kw) == code


def test_chunk_scan_docs_workspace_grows_with_clipping():
    lib = ttt.lib()
    plain = lib.ttt_chunk_scan_workspace(2, 1024, 256, 128, 64, 1)
    assert lib.ttt_chunk_scan_docs_workspace(2, 1024, 256, 128, 64, 1, 0.0) >= plain
    with_clip = lib.ttt_chunk_scan_docs_workspace(2, 1024, 256, 128, 64, 1, 0.5)
    assert with_clip >= plain + 2 * 1024 * 128 * 2
    assert lib.ttt_chunk_scan_docs_workspace(2, 1024, 100, 128, 64, 1, 0.5) == 0
    assert lib.ttt_chunk_scan_docs_workspace(2, 1024, 256, 128, 64, 1, float("nan")) == 0


def timeouts(**kw):
    a = dict(B=1, T=4096, F=512, D=256, C=512, dt=1, ws=A, wsb=1 << 40, count=A + 1024 * MB,
             stream=None)
    a.update(kw)
    return ttt.lib().ttt_chunk_scan_handover_timeouts(a["B"], a["T"], a["F"], a["D"], a["C"],
                                                      a["dt"], a["ws"], a["wsb"], a["count"],
                                                      a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(count=None), E_NULL), (dict(dt=4), E_DTYPE), (dict(F=24), E_SHAPE),
    (dict(ws=None), E_WS), (dict(wsb=64), E_WS),
    (dict(count=A + 1024 * MB + 4), E_ALIGN),
    (dict(count=A + 256), E_ALIAS),                      # the count word inside the workspace
])
def test_handover_timeouts_rejects_bad_arguments(kw, code):
    assert timeouts(**kw) == code


def test_schedule_knobs_come_only_from_the_test_entry_point(monkeypatch):
    """The environment no longer steers the scan: only ttt_scan_test_overrides does, and its
    defaults come back with (0, -1, -1)."""
    lib = ttt.lib()
    shape = (1, 32768, 9728, 2560, 512, 1)
    base = lib.ttt_chunk_scan_workspace(*shape)
    monkeypatch.setenv("TTT_SCAN_GROUP_TOKENS", "4096")
    monkeypatch.setenv("TTT_SCAN_SPLIT", "0")
    assert lib.ttt_chunk_scan_workspace(*shape) == base
    try:
        assert lib.ttt_scan_test_overrides(4096, -1, -1) == OK
        # four times fewer groups: fewer bf16 snapshots (49.8 MB each at this shape)
        assert lib.ttt_chunk_scan_workspace(*shape) < base - 10 * 9728 * 2560 * 2
        assert lib.ttt_scan_test_overrides(0, 0, -1) == OK
        # no token split: no hand-over states (99.6 MB of fp32 state tiles)
        assert lib.ttt_chunk_scan_workspace(*shape) < base - 9728 * 2560 * 4 + 1
    finally:
        lib.ttt_scan_test_overrides(0, -1, -1)
    assert lib.ttt_chunk_scan_workspace(*shape) == base


def test_noalloc_refuses_a_workspace_beyond_its_scratch():
    """ttt_chunk_scan_noalloc refuses, on the sizes alone and before any HIP call, a shape whose
    workspace exceeds the static scratch (the benchmark shape needs about 2 GB), and applies
    ttt_chunk_scan's other checks first."""
    lib = ttt.lib()
    big = (1, 32768, 9728, 2560, 512)
    assert lib.ttt_chunk_scan_workspace(*big, 1) > 64 << 20
    def call(**kw):
        a = dict(Z=A, V=A + 1024 * MB, W0=A + 2048 * MB, O=A + 3072 * MB, Wf=None, B=big[0],
                 T=big[1], F=big[2], D=big[3], C=big[4], eta=1e-4)
        a.update(kw)
        return lib.ttt_chunk_scan_noalloc(a["Z"], a["V"], 1, a["W0"], 1, a["O"], 1, a["Wf"],
                                          a["B"], a["T"], a["F"], a["D"], a["C"], a["eta"], None)
    assert call() == E_WS
    assert call(Z=None) == E_NULL
    assert call(F=24) == E_SHAPE
    assert call(O=A + 1024 * MB + 64) == E_ALIAS      # O inside V_hat


def test_scan_workspace_minimum_bounds_the_long_context_memory():
    """With bf16 inputs the scan accepts any workspace from ttt_chunk_scan_workspace_min up (it
    then runs in segments); the minimum does not grow with T, and below it the call is refused
    before anything is enqueued."""
    lib = ttt.lib()
    full32 = lib.ttt_chunk_scan_workspace(1, 32768, 9728, 2560, 512, 1)
    min32 = lib.ttt_chunk_scan_workspace_min(1, 32768, 9728, 2560, 512, 1)
    min128 = lib.ttt_chunk_scan_workspace_min(1, 131072, 9728, 2560, 512, 1)
    full128 = lib.ttt_chunk_scan_workspace(1, 131072, 9728, 2560, 512, 1)
    assert min32 < full32 / 10 and min128 == min32 and full128 > 3 * full32
    # the minimum holds one group's operands and snapshot plus the fp32 state
    assert min32 >= 2560 * 9728 * 4
    assert lib.ttt_chunk_scan_workspace_min(1, 1024, 256, 64, 64, 0) == \
        lib.ttt_chunk_scan_workspace(1, 1024, 256, 64, 64, 0)            # fp32: no segments
    assert lib.ttt_chunk_scan_workspace_min(1, 1024, 24, 64, 64, 1) == 0  # rejected shape
    GB = 1 << 30
    big = dict(B=1, T=32768, F=9728, D=2560, C=512, Z=A, V=A + GB, W0=A + 2 * GB, O=A + 3 * GB,
               Wf=None, ws=A + 5 * GB)   # no W_final: the state lives in the workspace
    assert scan(wsb=min32 - 256, **big) == E_WS
