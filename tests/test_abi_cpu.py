"""The C ABI without a GPU: the library loads, exports every declared symbol, and rejects bad
arguments on the host (every rejected call returns before anything is enqueued)."""
import ctypes
import os
import re

import pytest

from test_ridge_regression_amd import gka

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gka.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gka.LIB_PATH):
        from test_ridge_regression_amd.build import build_library
        build_library()
    return gka.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gka_\w+)\s*\(", text)))


def test_header_declares_the_bound_functions():
    assert declared_functions() == sorted(gka.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert lib.gka_abi_version() == 8


def test_status_strings(lib):
    for code in range(9):
        assert lib.gka_status_str(code)
    assert lib.gka_status_str(99) == b"unknown status"


# fake, 256-byte-aligned device addresses: never dereferenced because every case below fails a
# host-side check before any launch
ADDR = [0x7F0000000000 + i * (1 << 32) for i in range(12)]
VP = [ctypes.c_void_p(x) for x in ADDR]


def params(**kw):
    base = dict(B=2, T=128, H=2, D=64, chunk=64, iters=8, a=0.1, dtype_code=gka.GKA_BF16)
    base.update(kw)
    seg = base.pop("segments", 0)
    return gka.make_params(base["B"], base["T"], base["H"], base["D"], base["chunk"],
                           base["iters"], base["a"], base["dtype_code"], seg)


def fwd(lib, p, q=VP[0], k=VP[1], v=VP[2], g=VP[3], o=VP[4], h=None, u=None, n2=None, hn=None,
        ws=None, wsb=0):
    return lib.gka_fwd_chunked(ctypes.byref(p) if p is not None else None, q, k, v, g, o, h, u,
                               n2, hn, ws, ctypes.c_size_t(wsb), None, None)


def step(lib, p, q=VP[0], k=VP[1], v=VP[2], g=VP[3], o=VP[4], h=VP[5], u=VP[6], n2=VP[7]):
    return lib.gka_step(ctypes.byref(p) if p is not None else None, q, k, v, g, o, h, u, n2, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype_code=7), 4),
    (dict(D=48), 2), (dict(D=256), 2), (dict(dtype_code=gka.GKA_FP32, D=128), 2),
    (dict(chunk=48), 2), (dict(chunk=8), 2), (dict(chunk=128), 2), (dict(D=16, chunk=16), 2),
    (dict(B=0), 2), (dict(H=0), 2), (dict(T=-1), 2), (dict(segments=-3), 2),
    (dict(a=0.0), 3), (dict(a=-0.1), 3), (dict(a=float("nan")), 3), (dict(a=float("inf")), 3),
    (dict(iters=0), 3), (dict(iters=65), 3),
])
def test_fwd_rejects_bad_params(lib, kw, code):
    assert fwd(lib, params(**kw)) == code
    assert lib.gka_fwd_workspace_bytes(ctypes.byref(params(**kw))) == 0


def test_fwd_null_and_mixed_state(lib):
    assert fwd(lib, None) == 1
    assert fwd(lib, params(), q=None) == 1
    assert fwd(lib, params(), g=None) == 1
    assert fwd(lib, params(), o=None) == 1
    assert fwd(lib, params(), h=VP[5]) == 1  # state pointers must be all NULL or all set
    assert fwd(lib, params(), h=VP[5], u=VP[6]) == 1


def test_fwd_alignment_alias_and_workspace(lib):
    assert fwd(lib, params(), q=ctypes.c_void_p(ADDR[0] + 2)) == 2
    assert fwd(lib, params(), h=ctypes.c_void_p(ADDR[5] + 4), u=VP[6], n2=VP[7]) == 2
    assert fwd(lib, params(), o=VP[0]) == 7  # o == q
    assert fwd(lib, params(), o=ctypes.c_void_p(ADDR[1] + 1024)) == 7  # o inside k
    p = params(B=1, H=1, T=64 * 32, segments=8)
    need = lib.gka_fwd_workspace_bytes(ctypes.byref(p))
    assert need > 0
    assert fwd(lib, p) == 5
    assert fwd(lib, p, ws=VP[8], wsb=need - 1) == 5
    assert fwd(lib, p, ws=ctypes.c_void_p(ADDR[8] + 8), wsb=need) == 5


def test_fwd_empty_sequence_is_a_noop(lib):
    # T = 0: valid, nothing is launched, the (absent or present) state is untouched
    assert fwd(lib, params(T=0), q=None, k=None, v=None, g=None, o=None) == 0


def seg_bytes(B, H, S, D):
    """Per-segment states, log2 gates and the start norm of an S-segment plan (0 for S = 1)."""
    return 0 if S == 1 else ((B * H * S * (2 * D * D + 1) + B * H) * 4 + 255) // 256 * 256


def test_workspace_plan(lib):
    D = 128
    P = ctypes.byref
    one = lib.gka_fwd_workspace_bytes(P(params(D=D, B=1, H=1, T=64, segments=0)))
    assert one == 0  # a single chunk: one segment, no workspace
    p = params(B=8, H=8, T=2048, D=D)  # 32 chunks per head -> four segments (one per CU)
    ws = lib.gka_fwd_workspace_bytes(P(p))
    assert ws == seg_bytes(8, 8, 4, D)
    # explicit segment counts are clamped to the number of chunks
    big = lib.gka_fwd_workspace_bytes(P(params(B=1, H=1, T=128, D=D, segments=50)))
    two = lib.gka_fwd_workspace_bytes(P(params(B=1, H=1, T=128, D=D, segments=2)))
    assert big == two == seg_bytes(1, 1, 2, D)
    assert lib.gka_fwd_workspace_bytes(P(params(B=1, H=1, T=128, D=D, segments=1))) == 0


def test_step_rejects_bad_arguments(lib):
    assert step(lib, None) == 1
    assert step(lib, params(), h=None) == 1
    assert step(lib, params(), n2=None) == 1
    assert step(lib, params(D=96)) == 2
    assert step(lib, params(iters=0)) == 3
    assert step(lib, params(a=0.0)) == 3
    assert step(lib, params(dtype_code=3)) == 4
    assert step(lib, params(), h=ctypes.c_void_p(ADDR[5] + 8)) == 2
    assert step(lib, params(), o=VP[2]) == 7


def fwd_beta(lib, p, beta, o=VP[4], q=VP[0], g=VP[3]):
    return lib.gka_fwd_chunked_beta(ctypes.byref(p) if p is not None else None, q, VP[1], VP[2],
                                    g, beta, o, None, None, None, None, None, ctypes.c_size_t(0),
                                    None, None)


def step_beta(lib, p, beta, o=VP[4]):
    return lib.gka_step_beta(ctypes.byref(p) if p is not None else None, VP[0], VP[1], VP[2],
                             VP[3], beta, o, VP[5], VP[6], VP[7], None)


def test_beta_entry_points_check_like_the_base_ones(lib):
    one = dict(B=1, H=1, T=64, segments=1)  # a single segment: no workspace needed
    # the base checks come first, in the same order
    assert fwd_beta(lib, None, VP[9]) == 1
    assert fwd_beta(lib, params(D=48, **one), VP[9]) == 2
    assert fwd_beta(lib, params(iters=0, **one), VP[9]) == 3
    assert fwd_beta(lib, params(**one), VP[9], q=None) == 1
    assert fwd_beta(lib, params(**one), VP[9], o=VP[0]) == 7
    assert step_beta(lib, params(dtype_code=3), VP[9]) == 4
    # the write gate itself: 4-byte aligned, not overlapping o
    assert fwd_beta(lib, params(**one), ctypes.c_void_p(ADDR[9] + 2)) == 2
    assert fwd_beta(lib, params(**one), ctypes.c_void_p(ADDR[4] + 64)) == 7  # beta inside o
    assert step_beta(lib, params(), ctypes.c_void_p(ADDR[9] + 1)) == 2
    assert step_beta(lib, params(), VP[4]) == 7  # beta == o
    # an empty sequence is a no-op with or without the gate
    assert fwd_beta(lib, params(T=0), None, q=None, g=None, o=None) == 0
    assert fwd_beta(lib, params(T=0), VP[9], q=None, g=None, o=None) == 0


def test_binding_checks_the_write_gate():
    import torch
    q = torch.zeros(1, 64, 1, 32, dtype=torch.bfloat16)
    g = torch.ones(1, 64, 1)
    for bad in (torch.ones(1, 64, 1, dtype=torch.float64), torch.ones(1, 64, 2),
                torch.ones(1, 64, 2)[:, :, :1]):
        with pytest.raises(ValueError):
            gka._require_beta(bad, (1, 64, 1))
    gka._require_beta(None, (1, 64, 1))
    gka._require_beta(g, (1, 64, 1))
    assert q.shape[:3] == g.shape


def test_residual_entry_points_check_their_output(lib):
    P = ctypes.byref
    one = params(B=1, H=1, T=64, segments=1)
    fwd_res = lambda p, r, o=VP[4]: lib.gka_fwd_chunked_residuals(
        P(p) if p is not None else None, VP[0], VP[1], VP[2], VP[3], None, o, None, None, None,
        None, r, None, ctypes.c_size_t(0), None)
    step_res = lambda p, r, o=VP[4]: lib.gka_step_residuals(
        P(p) if p is not None else None, VP[0], VP[1], VP[2], VP[3], None, o, VP[5], VP[6],
        VP[7], r, None)
    assert fwd_res(None, VP[10]) == 1
    assert fwd_res(params(D=48, B=1, H=1, T=64), VP[10]) == 2
    assert fwd_res(one, None) == 1  # the residual output is required
    assert fwd_res(one, ctypes.c_void_p(ADDR[10] + 2)) == 2
    assert fwd_res(one, ctypes.c_void_p(ADDR[4] + 4)) == 7  # overlaps o
    assert fwd_res(params(T=0), None) == 0  # an empty sequence writes nothing
    assert step_res(None, VP[10]) == 1
    assert step_res(params(iters=0), VP[10]) == 3
    assert step_res(params(), None) == 1
    assert step_res(params(), ctypes.c_void_p(ADDR[10] + 1)) == 2
    assert step_res(params(), VP[4]) == 7


def test_varlen_entry_point_checks(lib):
    P = ctypes.byref
    vl = lambda p, cu, total, q=VP[0], o=VP[4]: lib.gka_fwd_varlen(
        P(p) if p is not None else None, cu, ctypes.c_int64(total), q, VP[1], VP[2], VP[3], None,
        o, None, None, None, None, None, ctypes.c_size_t(0), None)
    one = params(B=4, H=1, T=64, segments=1)
    assert vl(one, VP[11], 10) == 5  # the dispatch order needs a workspace even for one segment
    ws = lib.gka_fwd_varlen_workspace_bytes(P(one))
    assert ws >= 4 * 4 and ws % 256 == 0
    vl = lambda p, cu, total, q=VP[0], o=VP[4], w=ctypes.c_void_p(ADDR[11] + (1 << 31)), wsb=1 << 30: lib.gka_fwd_varlen(
        P(p) if p is not None else None, cu, ctypes.c_int64(total), q, VP[1], VP[2], VP[3], None,
        o, None, None, None, None, w, ctypes.c_size_t(wsb), None)
    assert vl(None, VP[11], 10) == 1
    assert vl(params(D=48, B=4, T=64), VP[11], 10) == 2
    assert vl(one, None, 10) == 1  # the offsets are required
    assert vl(one, ctypes.c_void_p(ADDR[11] + 2), 10) == 2
    assert vl(one, VP[11], -1) == 2
    assert vl(one, VP[11], 4 * 64 + 1) == 2  # more rows than B sequences of T
    assert vl(one, VP[11], 0, q=None, o=None) == 0  # no rows: nothing to do
    assert vl(params(T=0, B=4), VP[11], 0, q=None, o=None) == 0
    assert vl(one, VP[11], 100, q=None) == 1
    assert vl(one, VP[11], 100, o=VP[0]) == 7
    # the alias check covers the packed rows: o starting inside the 100 rows of q is rejected
    p2 = params(B=4, H=1, T=64, D=64, segments=1)
    assert vl(p2, VP[11], 100, o=ctypes.c_void_p(ADDR[0] + 99 * 64 * 2)) == 7


def test_varlen_plan_and_workspace(lib):
    P = ctypes.byref
    # dense plans are unchanged by the packed-batch plan
    p = params(B=8, H=8, T=2048, D=128)
    assert lib.gka_fwd_workspace_bytes(P(p)) == lib.gka_fwd_workspace_bytes(P(params(B=8, H=8, T=2048, D=128)))
    # packed: about 12 chunks of T per segment by default, plus the order of the B sequences
    D, B, H = 128, 64, 8
    for T, S in ((64, 1), (768, 1), (832, 2), (2048, 3)):
        ws = lib.gka_fwd_varlen_workspace_bytes(P(params(B=B, H=H, T=T, D=D)))
        assert ws == seg_bytes(B, H, S, D) + 256, (T, S, ws)
    # more sequences than the order kernel takes: no order, no extra bytes
    big = params(B=5000, H=1, T=64, D=32)
    assert lib.gka_fwd_varlen_workspace_bytes(P(big)) == lib.gka_fwd_workspace_bytes(P(big))


def test_missing_library_fails_loudly(tmp_path):
    # no fallback path: without the built library the binding raises
    saved = gka._lib
    try:
        gka._lib = None
        with pytest.raises(FileNotFoundError):
            gka.load(str(tmp_path / "libgka.so"))
    finally:
        gka._lib = saved


def test_all_head_sizes_are_accepted(lib):
    P = ctypes.byref
    # multi-segment plans need a workspace: a nonzero size means the shape passed the checks
    for dt, D, C in ((gka.GKA_BF16, 16, 32), (gka.GKA_BF16, 16, 64), (gka.GKA_FP32, 128, 16),
                     (gka.GKA_BF16, 32, 16), (gka.GKA_BF16, 128, 16)):
        assert lib.gka_fwd_workspace_bytes(P(params(dtype_code=dt, D=D, chunk=C, T=4096))) > 0
    for C in (32, 64):  # float32 D = 128 only with chunks of 16
        assert lib.gka_fwd_workspace_bytes(P(params(dtype_code=gka.GKA_FP32, D=128, chunk=C,
                                                    T=4096))) == 0


def test_backward_entry_point_checks(lib):
    P = ctypes.byref
    p = params(B=1, H=1, T=64, D=32)
    need = lib.gka_bwd_workspace_bytes(P(p))
    up = lambda x: (x + 63) // 64 * 64
    n, D, N = 64, 32, 1  # one chunk of 64 tokens
    scans = 2 * (up(N * 2 * D * D) + up(N) + up(1))  # the forward and the reverse scan
    # bf16 (chunks of 64, matrix cores): x, y, 2 Gam E H0 k per token and 4 scalars, the segment
    # states of the chunk-state walk (one segment here), every chunk's start state in fp16 with
    # two exponents, the reverse scan (float32 inputs, fp16 outputs with row exponents); no
    # snapshots
    seg = up(2 * D * D) + up(1) + up(1)
    fs16 = up(N * D * D) + up(N * 2)
    rscan = up(N * D * D) + up(N * D * D // 32) + up(N) + up(1) + up(N * D * D) + up(N * 2 * D)
    assert need == 4 * (3 * up(n * D) + up(n * 4) + seg + fs16 + rscan)
    # float32 (vector sweeps): every H_t, U_t, then x, y, c
    need32 = lib.gka_bwd_workspace_bytes(P(params(B=1, H=1, T=64, D=32, dtype_code=gka.GKA_FP32)))
    assert need32 == 4 * (up(n * 2 * D * D) + 2 * up(n * D) + up(n) + scans)
    w = ctypes.c_void_p(ADDR[11] + (1 << 31))
    bw = lambda p, q=VP[0], dq=VP[5], dk=VP[6], dg=VP[8], ws=w, wsb=need: lib.gka_bwd(
        P(p) if p is not None else None, q, VP[1], VP[2], VP[3], None, VP[4], dq, dk, VP[7], dg,
        None, ws, ctypes.c_size_t(wsb), None)
    assert bw(None) == 1
    assert bw(params(D=48)) == 2
    assert bw(params(iters=0)) == 3
    assert bw(p, q=None) == 1
    assert bw(p, dg=None) == 1
    assert bw(p, dq=VP[0]) == 7  # dq == q
    assert bw(p, dk=VP[5]) == 7  # dk == dq
    assert bw(p, ws=None) == 5
    assert bw(p, wsb=need - 1) == 5
    assert bw(params(T=0), q=None, dq=None) == 0


class _NoGpuLib:
    """Stands in for libgka.so: the binding must reject the call before any entry point runs.
    Only the workspace queries (pure host functions) answer."""

    def gka_fwd_workspace_bytes(self, p):
        return 0

    def gka_fwd_varlen_workspace_bytes(self, p):
        return 0

    def gka_bwd_workspace_bytes(self, p):
        return 0

    def __getattr__(self, name):
        raise AssertionError(f"{name} reached with arguments the binding should have rejected")


@pytest.fixture
def stub_lib():
    saved = gka._lib
    gka._lib = _NoGpuLib()
    try:
        yield
    finally:
        gka._lib = saved


def test_binding_rejects_host_tensors_and_bad_shapes(stub_lib):
    """Host (CPU) tensors would hand host pointers to the kernels; a short gamma or state would
    be read (and the state written) past its end. The binding raises ValueError for each before
    any library call (the stub fails the test if one is reached)."""
    import torch
    B, T, H, D = 1, 64, 2, 32
    q = torch.zeros(B, T, H, D, dtype=torch.bfloat16)
    g = torch.ones(B, T, H)
    st = gka.GkaState(torch.zeros(B, H, D, D), torch.zeros(B, H, D, D), torch.zeros(B, H))
    with pytest.raises(ValueError, match="GPU"):  # right shapes, host memory
        gka.fwd_chunked(q, q, q, g, 0.1, 4, 64, state=st)
    with pytest.raises(ValueError, match="gamma"):
        gka.fwd_chunked(q, q, q, torch.ones(B, T, 1), 0.1, 4, 64)
    with pytest.raises(ValueError, match="state"):
        bad = gka.GkaState(torch.zeros(B, H, D, D), torch.zeros(B, H, D, D // 2), torch.zeros(B, H))
        gka.fwd_chunked(q, q, q, g, 0.1, 4, 64, state=bad)
    with pytest.raises(ValueError, match="state"):
        bad = gka.GkaState(torch.zeros(B, 1, D, D), torch.zeros(B, 1, D, D), torch.zeros(B, 1))
        gka.fwd_chunked(q, q, q, g, 0.1, 4, 64, state=bad)
    with pytest.raises(ValueError, match="state"):
        bad = gka.GkaState(torch.zeros(B, H, D, D), torch.zeros(B, H, D, D), torch.zeros(B, H, 1))
        gka.fwd_chunked_residuals(q, q, q, g, 0.1, 4, 64, state=bad)
    # decode: gamma [B, H] and the state
    q1 = torch.zeros(B, H, D, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        gka.step(q1, q1, q1, torch.ones(B, H), 0.1, 4, st)
    with pytest.raises(ValueError, match="gamma"):
        gka.step(q1, q1, q1, torch.ones(B, H, 1), 0.1, 4, st)
    with pytest.raises(ValueError, match="gamma"):
        gka.step_residuals(q1, q1, q1, torch.ones(B), 0.1, 4, st)
    # packed batches: gamma [total, H]; one state per sequence
    qp = torch.zeros(10, H, D, dtype=torch.bfloat16)
    cu = torch.tensor([0, 4, 10], dtype=torch.int32)
    with pytest.raises(ValueError, match="gamma"):
        gka.fwd_varlen(qp, qp, qp, torch.ones(9, H), cu, 6, 0.1, 4)
    with pytest.raises(ValueError, match="state"):
        gka.fwd_varlen(qp, qp, qp, torch.ones(10, H), cu, 6, 0.1, 4, state=st)  # B = 2 sequences
    with pytest.raises(ValueError, match="GPU"):
        gka.fwd_varlen(qp, qp, qp, torch.ones(10, H), cu, 6, 0.1, 4)
    # backward
    with pytest.raises(ValueError, match="gamma"):
        gka.bwd(q, q, q, torch.ones(B, T), q, 0.1, 4)
    with pytest.raises(ValueError, match="GPU"):
        gka.bwd(q, q, q, g, q, 0.1, 4)


def test_binding_device_check_names_the_foreign_tensor():
    import torch
    q = torch.zeros(2, 3)
    with pytest.raises(ValueError, match="GPU"):
        gka._require_device(q, [q])


def test_row_spans_past_32_bit_offsets_are_rejected(lib):
    """The kernels address one chunk's 64 token rows of every head with 32-bit byte offsets:
    head counts whose row span reaches 2^31 bytes are refused on the host."""
    P = ctypes.byref
    # bf16 D = 128: 64 * H * 256 bytes < 2^31  <=>  H < 131072
    ok, bad = params(B=1, H=131071, D=128, T=64), params(B=1, H=131072, D=128, T=64)
    assert fwd(lib, bad) == 2
    assert lib.gka_fwd_workspace_bytes(P(bad)) == 0
    assert step(lib, bad) == 2
    # (the accepted one passes the shape checks and stops at the missing gamma)
    assert fwd(lib, ok, g=None) == 1
    # float32 D = 128 (chunk 16): 64 * H * 512 bytes
    assert fwd(lib, params(B=1, H=65536, D=128, T=16, chunk=16, dtype_code=gka.GKA_FP32)) == 2
    # the residual rows: 64 * H * (iters + 1) * 4 bytes < 2^31; at iters = 64 that is
    # H <= 129055 (D = 16 keeps the q, k, v rows small)
    # (gamma NULL: a call that passes the shape checks stops at GKA_ERR_NULL, never launches)
    res = lambda p: lib.gka_fwd_chunked_residuals(P(p), VP[0], VP[1], VP[2], None, None, VP[4],
                                                  None, None, None, None, VP[8], None,
                                                  ctypes.c_size_t(0), None)
    sres = lambda p: lib.gka_step_residuals(P(p), VP[0], VP[1], VP[2], None, None, VP[4], VP[5],
                                            VP[6], VP[7], VP[8], None)
    assert res(params(B=1, H=129056, D=16, T=64, chunk=32, iters=64)) == 2
    assert sres(params(B=1, H=129056, D=16, iters=64)) == 2
    assert sres(params(B=1, H=129055, D=16, iters=64)) == 1
    assert res(params(B=1, H=129055, D=16, T=64, chunk=32, iters=64, segments=1)) == 1  # no gamma
    assert fwd(lib, params(B=1, H=129056, D=16, T=64, chunk=32, iters=64), g=None) == 1


def test_static_entry_point_checks_before_any_device_call(lib):
    """gka_fwd_chunked_static validates like gka_fwd_chunked_beta, and a plan whose segment
    states exceed the static scratch is GKA_ERR_SCRATCH -- all on the host, before the scratch
    address is looked up (no GPU here)."""
    def call(p, **kw):
        a = dict(q=VP[0], k=VP[1], v=VP[2], g=VP[3], b=None, o=VP[4], h=None, u=None, n2=None,
                 hn=None)
        a.update(kw)
        return lib.gka_fwd_chunked_static(ctypes.byref(p) if p is not None else None, a["q"],
                                          a["k"], a["v"], a["g"], a["b"], a["o"], a["h"], a["u"],
                                          a["n2"], a["hn"], None)
    assert call(None) == 1
    assert call(params(D=48)) == 2
    assert call(params(a=0.0)) == 3
    assert call(params(), q=None) == 1
    assert call(params(), o=VP[0]) == 7
    assert call(params(), h=VP[5]) == 1            # state pointers mixed NULL / non-NULL
    # T = 0: a no-op that needs no scratch
    assert call(params(T=0)) == 0
    # B 64 x H 8 heads of D = 128 in 32 segments: 64 * 8 * 32 * 2 * 64 KiB = 2 GiB of states
    big = params(B=64, T=4096, H=8, D=128, segments=32)
    assert lib.gka_fwd_workspace_bytes(ctypes.byref(big)) > gka.GKA_STATIC_SCRATCH_BYTES
    assert call(big) == 8
    # multi-segment plans that fit still fail their argument checks first
    mid = params(B=2, T=1024, H=2, D=128)
    assert 0 < lib.gka_fwd_workspace_bytes(ctypes.byref(mid)) <= gka.GKA_STATIC_SCRATCH_BYTES
    assert call(mid, g=None) == 1
    assert call(mid, o=VP[1]) == 7
    assert call(mid, q=ctypes.c_void_p(ADDR[0] + 8)) == 2
    assert b"static scratch" in lib.gka_status_str(8)
