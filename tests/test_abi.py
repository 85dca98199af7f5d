"""C-ABI checks that need no GPU: the library loads, exports every function
include/twell.h declares, sizes workspaces, and rejects bad arguments before
anything is enqueued (every call below fails validation on the host)."""

import ctypes

import pytest

import activation_sparse_ffn_gate_amd as tw
from activation_sparse_ffn_gate_amd._lib import _Packed

OK, E_ARG, E_UNSUP, E_WS = 0, -1, -2, -3
FAKE = ctypes.c_void_p(0x100000)  # never dereferenced: validation fails first


def test_exports_every_declared_function():
    L = tw.lib()
    names = tw.header_functions()
    assert "twell_gate_pack" in names and "twell_dense_ffn_forward" in names
    for n in names:
        assert hasattr(L, n), f"libtwell.so does not export {n}"


def test_abi_version_and_status_strings():
    L = tw.lib()
    assert L.twell_abi_version() == 7
    for s in (OK, E_ARG, E_UNSUP, E_WS, -4, -5):
        assert tw.status_string(s)
    assert tw.status_string(12345) == "unknown status"


@pytest.mark.parametrize("M,d,F,T,C", [(4096, 2048, 8192, 128, 16), (64, 256, 1024, 64, 8), (0, 256, 128, 64, 1)])
def test_workspace_sizes(M, d, F, T, C):
    nT = F // T
    g = tw.ctrl_bytes(M)
    assert tw.workspace_bytes(tw.OP_GATE_PACK, M, d, F, T, C) == 0
    f = tw.workspace_bytes(tw.OP_FFN_FORWARD, M, d, F, T, C)
    dn = tw.workspace_bytes(tw.OP_DENSE_FFN, M, d, F)
    fb = tw.workspace_bytes(tw.OP_DENSE_FALLBACK, M, d, F)
    assert g >= 256 + 4 * M + 4 * 256 and g % 256 == 0  # header, row flags, split counters
    assert f >= M * nT * C * 5 + M * nT * 2 + 4 * M + 4 * M * F
    assert dn >= 2 * M * F and fb >= 4 * M * F + 512 * 65536  # hidden pair + split partial tiles
    assert f % 256 == 0 and dn % 256 == 0
    sl = tw.workspace_bytes(tw.OP_SLICED_UPDOWN, M, d, F, T, C)
    assert sl >= 8 * M * nT * C * 4 and sl % 256 == 0
    # the forward's up/down kernels and its fallback run concurrently: disjoint regions
    assert f >= M * nT * C * 5 + M * nT * 2 + 4 * M + sl + 4 * M * F + 512 * 65536


@pytest.mark.parametrize("d,ok", [(256, True), (768, True), (2048, True), (2560, True), (4096, True),
                                  (7168, True), (8192, True), (2304, False), (4608, False), (7936, False)])
def test_sliced_supported_d(d, ok):
    """d / 64 must be 2^a * b with b in {1, 3, 5, 7} (b <= 2 at 2^a = 64)."""
    n = tw.workspace_bytes(tw.OP_SLICED_UPDOWN, 64, d, 1024, 64, 8)
    assert (n > 0) == ok
    assert tw.workspace_bytes(tw.OP_FFN_FORWARD, 64, d, 1024, 64, 8) > 0  # the fused form covers the rest


@pytest.mark.parametrize(
    "args,want",
    [
        ((4096, 2048, 8192, 100, 16), 0),  # T not 64/128
        ((4096, 2048, 8192, 128, 0), 0),  # C < 1
        ((4096, 2048, 8192, 128, 129), 0),  # C > T
        ((4096, 2048, 8000, 128, 16), 0),  # F % T
        ((4096, 2000, 8192, 128, 16), 0),  # d % 256
        ((-1, 2048, 8192, 128, 16), 0),  # M < 0
    ],
)
def test_workspace_bytes_rejects(args, want):
    assert tw.workspace_bytes(tw.OP_FFN_FORWARD, *args) == want


def _packed():
    return _Packed(FAKE.value, FAKE.value, FAKE.value, FAKE.value, FAKE.value)


def test_gate_pack_validation():
    L = tw.lib()
    pk = _packed()
    cb = tw.ctrl_bytes(256)
    assert cb >= 256 + 4 * 256 and tw.ctrl_bytes(-1) == 0
    call = L.twell_gate_pack
    assert call(None, FAKE, 256, 256, 1024, 64, 8, ctypes.byref(pk), None, FAKE, cb, None) == E_ARG
    assert call(FAKE, FAKE, 256, 256, 1024, 64, 8, None, None, FAKE, cb, None) == E_ARG
    bad = _Packed(FAKE.value, 0, FAKE.value, FAKE.value, FAKE.value)
    assert call(FAKE, FAKE, 256, 256, 1024, 64, 8, ctypes.byref(bad), None, FAKE, cb, None) == E_ARG
    no_n = _Packed(FAKE.value, FAKE.value, FAKE.value, FAKE.value, 0)
    assert call(FAKE, FAKE, 0, 256, 1024, 64, 8, ctypes.byref(no_n), None, FAKE, cb, None) == E_ARG
    assert call(FAKE, FAKE, -5, 256, 1024, 64, 8, ctypes.byref(pk), None, FAKE, cb, None) == E_ARG
    assert call(FAKE, FAKE, 256, 256, 1000, 64, 8, ctypes.byref(pk), None, FAKE, cb, None) == E_UNSUP
    assert call(FAKE, FAKE, 256, 256, 1024, 32, 8, ctypes.byref(pk), None, FAKE, cb, None) == E_UNSUP
    assert call(FAKE, FAKE, 256, 256, 1024, 64, 65, ctypes.byref(pk), None, FAKE, cb, None) == E_UNSUP
    assert call(FAKE, FAKE, 256, 300, 1024, 64, 8, ctypes.byref(pk), None, FAKE, cb, None) == E_UNSUP
    assert call(FAKE, FAKE, 256, 256, 1024, 64, 8, ctypes.byref(pk), None, None, cb, None) == E_WS
    assert call(FAKE, FAKE, 256, 256, 1024, 64, 8, ctypes.byref(pk), None, FAKE, cb - 1, None) == E_WS
    mis = ctypes.c_void_p(FAKE.value + 8)
    assert call(FAKE, FAKE, 256, 256, 1024, 64, 8, ctypes.byref(pk), None, mis, cb, None) == E_WS


def test_forward_validation():
    L = tw.lib()
    ws = tw.workspace_bytes(tw.OP_FFN_FORWARD, 256, 256, 1024, 64, 8)
    cb = tw.ctrl_bytes(256)
    f = L.twell_ffn_forward
    assert f(FAKE, FAKE, None, FAKE, 256, 256, 1024, 64, 8, FAKE, FAKE, cb, FAKE, ws, None) == E_ARG
    assert f(FAKE, FAKE, FAKE, FAKE, 256, 256, 1024, 64, 8, None, FAKE, cb, FAKE, ws, None) == E_ARG
    assert f(FAKE, FAKE, FAKE, FAKE, 256, 256, 1024, 96, 8, FAKE, FAKE, cb, FAKE, ws, None) == E_UNSUP
    assert f(FAKE, FAKE, FAKE, FAKE, 256, 256, 1024, 64, 8, FAKE, FAKE, cb, FAKE, ws - 256, None) == E_WS
    assert f(FAKE, FAKE, FAKE, FAKE, 256, 256, 1024, 64, 8, FAKE, FAKE, cb - 4, FAKE, ws, None) == E_WS
    assert f(FAKE, FAKE, FAKE, FAKE, 256, 256, 1024, 64, 8, FAKE, None, cb, FAKE, ws, None) == E_WS
    ft = L.twell_ffn_forward_timed  # both events required; then the forward's own checks, before any record
    assert ft(FAKE, FAKE, FAKE, FAKE, 256, 256, 1024, 64, 8, FAKE, FAKE, cb, FAKE, ws, None, FAKE, None) == E_ARG
    assert ft(FAKE, FAKE, FAKE, FAKE, 256, 256, 1024, 64, 8, FAKE, FAKE, cb, FAKE, ws, FAKE, None, None) == E_ARG
    assert ft(FAKE, FAKE, FAKE, FAKE, 256, 256, 1024, 96, 8, FAKE, FAKE, cb, FAKE, ws, FAKE, FAKE, None) == E_UNSUP
    assert ft(FAKE, FAKE, FAKE, FAKE, 256, 256, 1024, 64, 8, FAKE, FAKE, cb, FAKE, ws - 256, FAKE, FAKE, None) == E_WS
    d = L.twell_dense_ffn_forward
    dws = tw.workspace_bytes(tw.OP_DENSE_FFN, 256, 256, 1024)
    assert d(FAKE, FAKE, FAKE, FAKE, 256, 256, 1000, FAKE, FAKE, dws, None) == E_UNSUP
    assert d(FAKE, FAKE, FAKE, FAKE, 256, 256, 1024, FAKE, FAKE, dws - 1, None) == E_WS
    u = L.twell_fused_updown
    pk = _packed()
    assert u(FAKE, FAKE, FAKE, None, 256, 256, 1024, 64, 8, FAKE, None) == E_ARG
    assert u(FAKE, FAKE, FAKE, ctypes.byref(pk), 256, 256, 1024, 64, 0, FAKE, None) == E_UNSUP
    sl = L.twell_sliced_updown
    sws = tw.workspace_bytes(tw.OP_SLICED_UPDOWN, 256, 256, 1024, 64, 8)
    assert sl(FAKE, FAKE, FAKE, None, 256, 256, 1024, 64, 8, FAKE, FAKE, sws, None) == E_ARG
    assert sl(FAKE, FAKE, FAKE, ctypes.byref(pk), 256, 256, 1024, 64, 0, FAKE, FAKE, sws, None) == E_UNSUP
    assert sl(FAKE, FAKE, FAKE, ctypes.byref(pk), 256, 2304, 1024, 64, 8, FAKE, FAKE, sws, None) == E_UNSUP
    assert sl(FAKE, FAKE, FAKE, ctypes.byref(pk), 256, 256, 1024, 64, 8, FAKE, FAKE, sws - 1, None) == E_WS
    assert sl(FAKE, FAKE, FAKE, ctypes.byref(pk), 256, 256, 1024, 64, 8, FAKE, None, sws, None) == E_WS
    fb = L.twell_dense_fallback
    fws = tw.workspace_bytes(tw.OP_DENSE_FALLBACK, 256, 256, 1024)
    assert fb(FAKE, FAKE, FAKE, FAKE, ctypes.byref(pk), 256, 256, 1024, FAKE, FAKE, cb, FAKE, fws - 1, None) == E_WS
    assert fb(FAKE, FAKE, FAKE, FAKE, ctypes.byref(pk), 256, 256, 1024, FAKE, None, cb, FAKE, fws, None) == E_WS
    assert fb(FAKE, FAKE, FAKE, FAKE, ctypes.byref(pk), 256, 256, 1024, FAKE, FAKE, cb - 1, FAKE, fws, None) == E_WS
    assert fb(FAKE, FAKE, FAKE, FAKE, None, 256, 256, 1024, FAKE, FAKE, cb, FAKE, fws, None) == E_ARG


def test_packed_view_is_host_arithmetic():
    L = tw.lib()
    M, d, F, T, C = 256, 256, 1024, 64, 8
    ws = tw.workspace_bytes(tw.OP_FFN_FORWARD, M, d, F, T, C)
    base = 0x10000000
    pk = _Packed()
    assert L.twell_packed_view(ctypes.c_void_p(base), ws, M, d, F, T, C, ctypes.byref(pk)) == OK
    ptrs = [pk.vals, pk.idx, pk.counts, pk.ovf_rows, pk.n_ovf]
    assert all(p % 256 == 0 for p in ptrs)
    assert all(base <= p < base + ws for p in ptrs)
    nT = F // T
    assert pk.idx - pk.vals >= M * nT * C * 4 and pk.counts - pk.idx >= M * nT * C
    assert L.twell_packed_view(ctypes.c_void_p(base), ws - 1, M, d, F, T, C, ctypes.byref(pk)) == E_WS


# ------------------------------------------------------------- dead gate units
@pytest.mark.parametrize("F,T,density,seed", [(1024, 64, 0.7, 1), (8192, 128, 0.7, 2), (192, 64, 0.0, 3),
                                              (256, 128, 1.0, 4), (4096, 128, 0.01, 5), (96, 7, 0.5, 6)])
def test_live_layout_matches_oracle(F, T, density, seed):
    """twell_live_layout is host code: checked against the oracle's layout."""
    import numpy as np

    import oracle as O

    rng = np.random.default_rng(seed)
    active = rng.random(F) < density
    words = np.zeros(-(-F // 32), dtype=np.uint32)
    for j in np.flatnonzero(active):
        words[j // 32] |= np.uint32(1 << (j % 32))
    got = tw.live_layout(words, F, T)
    want = O.live_layout(active, T)
    assert got.dtype == np.int32 and np.array_equal(got.astype(np.int64), want)


def test_live_layout_validation():
    import numpy as np

    L = tw.lib()
    words = np.full(2, 0xFFFFFFFF, dtype=np.uint32)
    pw = words.ctypes.data_as(ctypes.c_void_p)
    width = ctypes.c_int64(-1)
    assert L.twell_live_layout(pw, 64, 64, None, 0, ctypes.byref(width)) == OK and width.value == 64
    assert L.twell_live_layout(pw, 60, 64, None, 0, ctypes.byref(width)) == OK and width.value == 64
    src = np.full(8, 7, dtype=np.int32)
    assert L.twell_live_layout(pw, 64, 64, src.ctypes.data_as(ctypes.c_void_p), 8, ctypes.byref(width)) == E_ARG
    assert (src == 7).all()  # nothing written when src is too short
    assert L.twell_live_layout(None, 64, 64, None, 0, ctypes.byref(width)) == E_ARG
    assert L.twell_live_layout(pw, 0, 64, None, 0, ctypes.byref(width)) == E_ARG
    assert L.twell_live_layout(pw, 64, 0, None, 0, ctypes.byref(width)) == E_ARG
    assert L.twell_live_layout(pw, 64, 64, None, 0, None) == E_ARG


def test_column_activity_and_gather_validation():
    L = tw.lib()
    M, d, F, T, C = 64, 256, 1024, 64, 8
    ws = tw.workspace_bytes(tw.OP_COLUMN_ACTIVITY, M, d, F, T, C)
    nT = F // T
    assert ws >= M * nT * C * 5 + M * nT * 2 + 4 * M
    g = tw.ctrl_bytes(M)
    ok = (FAKE, FAKE, M, d, F, T, C, FAKE, FAKE, g, FAKE, ws, None)
    f = L.twell_column_activity
    assert f(*ok[:7], None, *ok[8:]) == E_ARG  # no activity bits
    assert f(FAKE, FAKE, M, d, F, T, C, FAKE, FAKE, g, FAKE, ws - 256, None) == E_WS
    assert f(FAKE, FAKE, M, d, F, T, C, FAKE, FAKE, g - 256, FAKE, ws, None) == E_WS
    assert f(FAKE, FAKE, M, d, F, 96, C, FAKE, FAKE, g, FAKE, ws, None) == E_UNSUP
    assert f(FAKE, FAKE, M, 320, F, T, C, FAKE, FAKE, g, FAKE, ws, None) == E_UNSUP
    gr = L.twell_gather_rows
    assert gr(FAKE, F, d, FAKE, -1, FAKE, None) == E_ARG
    assert gr(None, F, d, None, 0, None, None) == OK  # nothing to do
    assert gr(None, F, d, FAKE, 4, FAKE, None) == E_ARG
    assert gr(FAKE, F, 100, FAKE, 4, FAKE, None) == E_UNSUP
    assert gr(FAKE, 0, d, FAKE, 4, FAKE, None) == E_ARG


# ------------------------------------------------------------ training side
def test_backward_validation():
    from activation_sparse_ffn_gate_amd._lib import _Hybrid, _Spill

    L = tw.lib()
    M, d, F, T, K, R = 64, 256, 1024, 64, 8, 4
    ws = tw.backward_workspace_bytes(M, d, F, K, R)
    assert ws >= 6 * 4 * (M * K + R * F)
    assert tw.backward_workspace_bytes(M, d, 32768, K, R) == 0  # F past the placement's LDS counters
    assert tw.backward_workspace_bytes(M, 320, F, K, R) == 0      # d not supported
    assert tw.backward_workspace_bytes(M, d, F, 0, R) == 0        # K >= 1
    assert tw.backward_workspace_bytes(M, d, F, K, M + 1) == 0    # R <= M
    assert tw.backward_workspace_bytes(1 << 24, d, F, 256, 0) == 0  # entry list past 2^31
    pk = _Packed(FAKE.value, FAKE.value, FAKE.value, FAKE.value, FAKE.value)
    hy = _Hybrid(*([FAKE.value] * 6))
    hp = L.twell_hybrid_pack
    assert hp(ctypes.byref(pk), None, M, F, T, 8, K, R, ctypes.byref(hy), None) == E_ARG  # C < T needs the spill
    sp = _Spill(FAKE.value, FAKE.value, FAKE.value, -1)
    assert hp(ctypes.byref(pk), ctypes.byref(sp), M, F, T, 8, K, R, ctypes.byref(hy), None) == E_ARG  # cap < 0
    assert hp(ctypes.byref(pk), None, M, F, T, T, 0, R, ctypes.byref(hy), None) == E_ARG
    assert hp(ctypes.byref(pk), None, M, F, T, T, K, M + 1, ctypes.byref(hy), None) == E_ARG
    assert hp(None, None, M, F, T, T, K, R, ctypes.byref(hy), None) == E_ARG
    gs = L.twell_gate_pack_spill
    g = tw.ctrl_bytes(M)
    ok_sp = _Spill(FAKE.value, FAKE.value, FAKE.value, 16)
    assert gs(FAKE, FAKE, M, d, F, T, 8, ctypes.byref(pk), None, None, FAKE, g, None) == E_ARG
    no_n = _Spill(FAKE.value, FAKE.value, 0, 16)
    assert gs(FAKE, FAKE, M, d, F, T, 8, ctypes.byref(pk), ctypes.byref(no_n), None, FAKE, g, None) == E_ARG
    big = _Spill(FAKE.value, FAKE.value, FAKE.value, (1 << 31) // T)
    assert gs(FAKE, FAKE, M, d, F, T, 8, ctypes.byref(pk), ctypes.byref(big), None, FAKE, g, None) == E_ARG
    assert gs(FAKE, FAKE, M, d, F, 96, 8, ctypes.byref(pk), ctypes.byref(ok_sp), None, FAKE, g, None) == E_UNSUP
    assert gs(FAKE, FAKE, M, d, F, T, 8, ctypes.byref(pk), ctypes.byref(ok_sp), None, FAKE, g - 256, None) == E_WS
    fb = L.twell_ffn_backward
    ok = [FAKE] * 5 + [ctypes.byref(hy), M, d, F, K, R] + [FAKE] * 4
    assert fb(*ok, FAKE, ws - 256, None) == E_WS
    assert fb(*ok, ctypes.c_void_p(FAKE.value + 8), ws, None) == E_WS  # misaligned
    bad_d = ok[:7] + [320] + ok[8:]
    assert fb(*bad_d, FAKE, ws, None) == E_UNSUP
    no_dx = ok[:11] + [None] + ok[12:]
    assert fb(*no_dx, FAKE, ws, None) == E_ARG


def test_gate_offset_limits():
    """Shapes whose x, Wg or packed values pass 2^31 bytes are refused before
    anything is enqueued (the gate kernels use 32-bit offsets)."""
    L = tw.lib()
    pk = _Packed(FAKE.value, FAKE.value, FAKE.value, FAKE.value, FAKE.value)
    g = tw.ctrl_bytes(1 << 20)
    # x: 2^20 rows of d = 1024 is 2^31 bytes
    assert L.twell_gate_pack(FAKE, FAKE, 1 << 20, 1024, 1024, 128, 16, ctypes.byref(pk), None, FAKE, g, None) == E_UNSUP
    # Wg: 2^20 units of d = 1024
    assert L.twell_gate_pack(FAKE, FAKE, 64, 1024, 1 << 20, 128, 16, ctypes.byref(pk), None, FAKE,
                             tw.ctrl_bytes(64), None) == E_UNSUP
    # packed values: M (F / T) C 4 = 2^31 with M = 2^17, F = 8192, T = 128, C = 64
    assert L.twell_gate_pack(FAKE, FAKE, 1 << 17, 256, 8192, 128, 64, ctypes.byref(pk), None, FAKE,
                             tw.ctrl_bytes(1 << 17), None) == E_UNSUP


def test_row_and_unit_limits():
    """The documented limits: M <= 2^30 and F <= 2^24 are accepted by the
    sizing calls, one past either is TWELL_E_INVALID_ARG (0 from the sizing
    calls)."""
    L = tw.lib()
    M_max, F_max = 1 << 30, 1 << 24
    assert tw.ctrl_bytes(M_max) > 0 and tw.ctrl_bytes(M_max + 1) == 0
    assert tw.workspace_bytes(tw.OP_DENSE_FFN, 64, 256, F_max) > 0
    assert tw.workspace_bytes(tw.OP_DENSE_FFN, 64, 256, F_max + 64) == 0
    assert tw.workspace_bytes(tw.OP_FFN_FORWARD, M_max, 256, 1024, 64, 8) > 0
    assert tw.workspace_bytes(tw.OP_FFN_FORWARD, M_max + 1, 256, 1024, 64, 8) == 0
    pk = _Packed(FAKE.value, FAKE.value, FAKE.value, FAKE.value, FAKE.value)
    g = tw.ctrl_bytes(64)
    assert L.twell_gate_pack(FAKE, FAKE, M_max + 1, 256, 1024, 64, 8, ctypes.byref(pk), None, FAKE, g,
                             None) == E_ARG
    assert L.twell_gate_pack(FAKE, FAKE, 64, 256, F_max + 128, 128, 8, ctypes.byref(pk), None, FAKE, g,
                             None) == E_ARG
    # at the limits themselves the gate's 32-bit offsets decide (not the row/unit limit)
    assert L.twell_gate_pack(FAKE, FAKE, M_max, 256, 1024, 64, 8, ctypes.byref(pk), None, FAKE,
                             tw.ctrl_bytes(M_max), None) == E_UNSUP
    assert L.twell_gate_pack(FAKE, FAKE, 64, 256, F_max, 128, 8, ctypes.byref(pk), None, FAKE, g, None) == E_UNSUP


def test_static_forward_validation():
    """twell_ffn_forward_static refuses, before any HIP call, more than 256
    rows, shapes whose scratch passes its static buffer, and bad arguments;
    M = 0 is a no-op."""
    L = tw.lib()
    f = L.twell_ffn_forward_static
    E_SCRATCH = -5
    assert "static buffer" in tw.status_string(E_SCRATCH)
    assert f(FAKE, FAKE, FAKE, FAKE, 257, 2048, 8192, 128, 16, FAKE, None) == E_UNSUP
    assert f(FAKE, FAKE, FAKE, FAKE, 256, 2048, 8192, 96, 16, FAKE, None) == E_UNSUP
    assert f(FAKE, FAKE, None, FAKE, 256, 2048, 8192, 128, 16, FAKE, None) == E_ARG
    assert f(FAKE, FAKE, FAKE, FAKE, 256, 2048, 8192, 128, 16, None, None) == E_ARG
    # 256 rows of F = 32768: the z spill alone is 32 MiB
    assert f(FAKE, FAKE, FAKE, FAKE, 256, 1024, 32768, 128, 16, FAKE, None) == E_SCRATCH
    assert f(None, FAKE, FAKE, FAKE, 0, 2048, 8192, 128, 16, None, None) == OK


def _a256(n):
    return (n + 255) // 256 * 256


def test_dense_ring_workspace():
    """Host sizing of the ring kernels' regions. The dense baseline holds h
    [M, F] bf16, Wd^T [d, F] bf16 and S - 1 fp32 partial outputs [M, d], where
    the down product's ceil(M / 256) * (d / 256) output tiles are split
    S = min(256 / tiles, F / 256) ways below 256 tiles. The forward, the
    gate-only forward and the standalone fallback gain exactly Wd^T once a
    batch can hold an overflow list of the ring fallback's length, the first
    row count whose down tiles reach 256."""
    def dense_expect(M, d, F):
        tiles = -(-M // 256) * (d // 256)
        S = 1 if tiles >= 256 else max(1, min(256 // tiles, (F // 32) // 8))
        return _a256(M * F * 2) + _a256(F * d * 2) + _a256((S - 1) * M * d * 4)

    for M, d, F in [(4096, 2048, 8192), (1, 512, 2048), (300, 256, 1088), (8192, 2048, 8192),
                    (16384, 2560, 10240), (300, 8192, 512)]:
        assert tw.workspace_bytes(tw.OP_DENSE_FFN, M, d, F) == dense_expect(M, d, F), (M, d, F)

    for d, F, first in [(2048, 8192, 7937), (8192, 512, 1793), (2560, 10240, 6401)]:
        wdt = F * d * 2
        for op, T, C in [(tw.OP_FFN_FORWARD, 128, 16), (tw.OP_FFN_FORWARD_GATEUP, 128, 16),
                         (tw.OP_DENSE_FALLBACK, 0, 0)]:
            w = [tw.workspace_bytes(op, M, d, F, T, C) for M in (first - 2, first - 1, first)]
            assert w[1] - w[0] < wdt // 2, (op, d)  # one more row: its own few KB
            assert wdt <= w[2] - w[1] < wdt + wdt // 2, (op, d)  # ... plus Wd^T
        fb = tw.workspace_bytes(tw.OP_DENSE_FALLBACK, first, d, F)
        assert fb == 2 * _a256(first * F * 2) + 512 * 64 * 1024 + _a256(wdt)
