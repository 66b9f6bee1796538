"""The C-ABI library loads, exports every declared entry point and rejects
bad arguments on the host before launching anything (CPU only: none of
these calls reaches a HIP API)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

import gated_deltanet_state_amd as gdn  # noqa: E402

OK, NULLP, SHAPE, UNSUP, ALIGN, WS = 0, 1, 2, 3, 4, 5
F32, BF16 = 0, 1


@pytest.fixture(scope="module")
def lib():
    # GDN_TEST_LIB names another build of the library to check (the
    # host-sanitized one, from tests/test_abi_asan.py); default: the product
    path = os.environ.get("GDN_TEST_LIB")
    return gdn.declare(ctypes.CDLL(path)) if path else gdn.library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert {"gdn_replay", "gdn_chunk_operator", "gdn_compose"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_status_strings(lib):
    assert lib.gdn_abi_version() == 4
    for code, name in [(0, b"GDN_OK"), (1, b"GDN_ERR_NULL_POINTER"), (2, b"GDN_ERR_BAD_SHAPE"),
                       (3, b"GDN_ERR_UNSUPPORTED"), (4, b"GDN_ERR_ALIGNMENT"),
                       (5, b"GDN_ERR_WORKSPACE"), (6, b"GDN_ERR_HIP")]:
        assert lib.gdn_status_string(code) == name


P = 0x10000  # a 16-byte aligned fake address; never dereferenced (checks fail first)


def replay(lib, q=P, k=P, v=P, a=P, b=P, S0=None, cu=P, N=1, T=10, H=2, dk=64, dv=64,
           dt=F32, o=P, odt=F32, S=P):
    return lib.gdn_replay(q, k, v, a, b, S0, cu, N, T, H, dk, dv, dt, o, odt, S, None, 0, None)


def test_replay_argument_checks(lib):
    assert replay(lib, k=None) == NULLP
    assert b"required" in lib.gdn_last_error()
    assert replay(lib, S=None) == NULLP
    assert replay(lib, cu=None) == NULLP
    assert replay(lib, q=None) == NULLP             # o requested without q
    assert replay(lib, N=0) == SHAPE
    assert replay(lib, T=-1) == SHAPE
    assert replay(lib, H=0) == SHAPE
    assert replay(lib, dk=96) == UNSUP
    assert replay(lib, dv=32) == UNSUP
    assert replay(lib, dt=7) == UNSUP
    assert replay(lib, odt=9) == UNSUP
    assert replay(lib, T=1 << 31) == UNSUP
    assert replay(lib, H=65537) == UNSUP            # in-chunk offsets are 32-bit
    assert replay(lib, k=P + 2) == ALIGN
    assert b"k is not 16-byte aligned" in lib.gdn_last_error()
    assert replay(lib, S0=P + 8) == ALIGN
    assert replay(lib, o=P + 4) == ALIGN


def test_segmented_replay_argument_checks(lib):
    lib.gdn_replay_segmented.argtypes = [ctypes.c_void_p] * 7 + [ctypes.c_int32, ctypes.c_int64] + \
        [ctypes.c_int32] * 3 + [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int32,
                                ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]

    def rs(segments, k=P, ws=None, nbytes=0):
        return lib.gdn_replay_segmented(P, k, P, P, P, None, P, 1, 10, 2, 64, 64, BF16, P, F32, P, segments, ws,
                                        nbytes, None)
    assert rs(-1) == SHAPE and b"segments" in lib.gdn_last_error()
    assert rs(65) == SHAPE
    assert rs(3, k=None) == NULLP
    assert rs(3) == WS                              # workspace checked before any launch
    assert b"gdn_replay_segmented" in lib.gdn_last_error()
    assert rs(0, k=P + 2) == ALIGN


def test_raw_replay_argument_checks(lib):
    def rr(dt=BF16, k=P, ws=None, nbytes=0):
        return lib.gdn_replay_raw(P, k, P, P, P, None, P, 1, 10, 2, 64, 64, dt, P, F32, P, ws, nbytes, None)
    assert rr(dt=F32) == UNSUP and b"GDN_BF16" in lib.gdn_last_error()
    assert rr(k=None) == NULLP
    assert rr() == WS and b"gdn_replay_raw" in lib.gdn_last_error()
    # the workspace adds 256 bytes of reciprocal key norms per chunk slot
    # and head to the replay's; a single long sequence over few heads takes
    # the time split (segment operators beyond the records and norms)
    slots = 4000 // 64 + 1 + 1
    assert lib.gdn_replay_raw_workspace_bytes(1, 4000, 4, 128, 128) == \
        lib.gdn_replay_workspace_bytes(1, 4000, 4, 128, 128) + slots * 4 * 256
    assert lib.gdn_replay_workspace_bytes(1, 4000, 4, 128, 128) > slots * 4 * 12288


def test_chunk_operator_argument_checks(lib):
    def co(k=P, v=P, a=P, b=P, cu=P, C=2, T=10, H=2, dk=64, dv=64, dt=BF16, TC=P, SL=P):
        return lib.gdn_chunk_operator(k, v, a, b, cu, C, T, H, dk, dv, dt, TC, SL, None, 0, None)
    assert co(TC=None) == NULLP
    assert co(v=None) == NULLP                      # v without S_local
    assert co(SL=None) == NULLP
    assert co(C=-1) == SHAPE
    assert co(dk=100) == UNSUP
    assert co(H=65537) == UNSUP
    assert co(b=P + 2) == ALIGN
    assert co(C=0) == OK                            # nothing to do, nothing launched


def test_compose_argument_checks(lib):
    def cp(Si=None, TC=P, SL=P, C=3, H=2, dk=128, dv=64, So=P):
        return lib.gdn_compose(Si, TC, SL, C, H, dk, dv, So, None, 0, None)
    assert cp(So=None) == NULLP
    assert cp(TC=None) == NULLP
    assert cp(C=-2) == SHAPE
    assert cp(dv=48) == UNSUP
    assert cp(C=1 << 30, H=4) == UNSUP           # operator-conversion grid beyond 32 bits
    assert cp(Si=P + 4) == ALIGN
    assert cp() == WS                             # the converted operators need a workspace


def test_decode_argument_checks(lib):
    def dc(q=P, k=P, v=P, a=P, b=P, Si=None, N=4, H=2, dk=128, dv=128, dt=BF16, o=P, odt=0, So=P):
        return lib.gdn_decode(q, k, v, a, b, Si, N, H, dk, dv, dt, o, odt, So, None)
    assert dc(So=None) == NULLP
    assert dc(k=None) == NULLP
    assert dc(q=None) == NULLP                    # o requested without q
    assert dc(N=-1) == SHAPE
    assert dc(H=0) == SHAPE
    assert dc(dk=96) == UNSUP
    assert dc(dt=7) == UNSUP
    assert dc(H=65537) == UNSUP
    assert dc(Si=P + 8) == ALIGN
    assert dc(N=0) == OK                          # nothing to do, nothing launched


def test_front_end_argument_checks(lib):
    def fe(qr=P, kr=P, g=P, b=P, T=8, H=2, dk=128, dt=BF16, q=P, k=P, a=P, be=P):
        return lib.gdn_front_end(qr, kr, g, b, T, H, dk, dt, q, k, a, be, None)
    assert fe(kr=None) == NULLP
    assert fe(be=None) == NULLP
    assert fe(q=None) == NULLP                    # q_raw without q
    assert fe(qr=None) == NULLP                   # q without q_raw
    assert fe(T=-1) == SHAPE
    assert fe(H=0) == SHAPE
    assert fe(dk=96) == UNSUP
    assert fe(dt=7) == UNSUP
    assert fe(H=65537) == UNSUP
    assert fe(T=(1 << 40) + 1) == UNSUP
    assert fe(g=P + 4) == ALIGN
    assert fe(T=0) == OK                          # nothing to do, nothing launched
    assert fe(qr=None, q=None, T=0) == OK


def test_scalar_decay_argument_checks(lib):
    def op(k=P, v=P, a=P, b=P, cu=P, C=4, T=100, H=2, dk=128, dv=128, dt=BF16, g=P, SL=P):
        return lib.gdn_scalar_chunk_operator(k, v, a, b, cu, C, T, H, dk, dv, dt, g, SL, None)
    assert op(g=None) == NULLP
    assert op(cu=None) == NULLP
    assert op(v=None) == NULLP                    # S_local without v
    assert op(C=-1) == SHAPE
    assert op(H=0) == SHAPE
    assert op(dv=96) == UNSUP
    assert op(dt=7) == UNSUP
    assert op(T=1 << 31) == UNSUP
    assert op(SL=P + 4) == ALIGN
    assert op(C=0) == OK
    assert op(v=None, SL=None, C=0) == OK

    def co(Si=None, g=P, SL=P, C=3, H=2, dk=64, dv=64, So=P):
        return lib.gdn_scalar_compose(Si, g, SL, C, H, dk, dv, So, None)
    assert co(So=None) == NULLP
    assert co(g=None) == NULLP
    assert co(C=-1) == SHAPE
    assert co(dk=32) == UNSUP
    assert co(H=65537) == UNSUP
    assert co(Si=P + 8) == ALIGN


def test_workspace_queries(lib):
    # one 12 KiB record of per-chunk factors ((I + A)^{-1} diag(beta) fragments) per chunk
    # slot and head; slots = n_tokens / 64 + n_seqs + 1 (sequence n's chunk j sits
    # in slot floor(cu[n] / 64) + n + j)
    lib.gdn_replay_segmented_workspace_bytes.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                                         ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
    lib.gdn_replay_segmented_workspace_bytes.restype = ctypes.c_size_t
    seg_ws = lib.gdn_replay_segmented_workspace_bytes
    tau = lambda n_seqs, n_tokens, H: (n_tokens // 64 + n_seqs + 1) * H * 12288
    # 16 sequences x 32 heads already fill the chip: no time split, and room
    # for the longest-first order of the 16 sequences (256 bytes)
    assert lib.gdn_replay_workspace_bytes(16, 30000, 32, 128, 128) == tau(16, 30000, 32) + 256
    assert lib.gdn_chunk_operator_workspace_bytes(64, 32768, 32, 128, 128) == tau(64, 32768, 32)
    # one long sequence: room for P segment operators (T_seg and S_seg per
    # head), 1 < P <= 16, or with outputs also the start states (3 <= P <= 9:
    # the lead segment and up to 8 more)
    extra = lib.gdn_replay_workspace_bytes(1, 3277, 32, 128, 128) - tau(1, 3277, 32)
    per_seg = 32 * (128 * 128 + 128 * 128) * 4
    per_seg_o = 32 * (128 * 128 + 2 * 128 * 128) * 4
    assert ((extra % per_seg == 0 and 2 <= extra // per_seg <= 16)
            or (extra % per_seg_o == 0 and 3 <= extra // per_seg_o <= 9)), extra
    # a forced segment count sets P directly
    # (room for the replay with outputs: segment operators, states and start states)
    assert seg_ws(2, 300, 4, 64, 128, 5) == tau(2, 300, 4) + 2 * 5 * 4 * (64 * 64 + 2 * 128 * 64) * 4
    assert seg_ws(1, 3277, 32, 128, 128, 1) == tau(1, 3277, 32)
    # 0 is the cost model, exactly gdn_replay's size; out-of-range counts give 0
    for args in [(1, 3277, 32, 128, 128), (16, 30000, 32, 128, 128), (2, 300, 4, 64, 128)]:
        assert seg_ws(*args, 0) == lib.gdn_replay_workspace_bytes(*args)
    assert seg_ws(1, 3277, 32, 128, 128, -1) == 0
    # gdn_compose: the operators converted to fragments, as many bytes as T_C
    assert lib.gdn_compose_workspace_bytes(64, 32, 128, 128) == 64 * 32 * 128 * 128 * 4
    assert lib.gdn_compose_workspace_bytes(0, 32, 128, 128) == 0
    # a missing workspace is reported before anything is launched
    assert replay(lib) == WS
    assert b"workspace" in lib.gdn_last_error()
    assert lib.gdn_chunk_operator(P, P, P, P, P, 2, 10, 2, 64, 64, BF16, P, P, None, 0, None) == WS


def test_chunk_slots_are_unique():
    """The slot rule floor(cu[n]/64) + n + j never collides and stays below
    n_tokens / 64 + n_seqs + 1 (checked exhaustively on random packings)."""
    import numpy as np
    rng = np.random.Generator(np.random.PCG64(3))
    for _ in range(300):
        lens = rng.integers(0, 300, size=rng.integers(1, 12))
        cu = np.concatenate([[0], np.cumsum(lens)])
        slots = []
        for n, L in enumerate(lens):
            slots += [cu[n] // 64 + n + j for j in range(-(-L // 64))]
        assert len(slots) == len(set(slots))
        assert all(0 <= s < cu[-1] // 64 + len(lens) + 1 for s in slots)
