"""C ABI checks that need no GPU: the library loads, exports every entry point
the header declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "loglin.h")
# LOGLIN_LIB points the checks at another build of the library (the host-sanitizer build)
LIB = os.environ.get("LOGLIN_LIB", os.path.join(ROOT, "log_linear_token_amd", "libloglin.so"))

EINVAL, EUNSUPPORTED, ENOMEM, ECAPACITY = 1, 2, 3, 4


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"LOGLIN_API\s+[\w\s\*]*?\b(loglin_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} missing: build it with python -m log_linear_token_amd.build")
    lib = ctypes.CDLL(LIB)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.loglin_fwd_workspace_bytes.argtypes = [i] * 7
    lib.loglin_fwd_workspace_bytes.restype = sz
    lib.loglin_fwd_chunked.argtypes = [vp] * 6 + [i] * 8 + [vp, sz, vp]
    lib.loglin_fwd_chunked.restype = i
    lib.loglin_fwd_plan.argtypes = [i] * 7 + [vp]
    lib.loglin_state_init.argtypes = [ctypes.POINTER(vp), i, i, i, i, i, vp]
    lib.loglin_state_free.argtypes = [vp]
    lib.loglin_state_load.argtypes = [vp, vp, vp, vp]
    lib.loglin_state_export.argtypes = [vp, vp, vp, vp]
    lib.loglin_decode_step.argtypes = [vp] * 7 + [i, vp]
    lib.loglin_debug_level_map.argtypes = [i, vp, vp]
    lib.loglin_prefill_workspace_bytes.argtypes = [i] * 6
    lib.loglin_prefill_workspace_bytes.restype = sz
    lib.loglin_prefill_states.argtypes = [vp] * 4 + [i] * 7 + [vp, sz, vp]
    lib.loglin_bwd_workspace_bytes.argtypes = [i] * 7
    lib.loglin_bwd_workspace_bytes.restype = sz
    lib.loglin_bwd_chunked.argtypes = [vp] * 11 + [i] * 8 + [vp, sz, vp]
    lib.loglin_last_error.restype = ctypes.c_char_p
    lib.loglin_status_string.restype = ctypes.c_char_p
    return lib


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ["loglin_fwd_chunked", "loglin_fwd_workspace_bytes", "loglin_decode_step",
              "loglin_state_init", "loglin_state_free", "loglin_state_load",
              "loglin_state_export", "loglin_debug_level_map", "loglin_last_error",
              "loglin_prefill_states", "loglin_prefill_workspace_bytes",
              "loglin_bwd_chunked", "loglin_bwd_workspace_bytes"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in _declared():
        assert hasattr(lib, n), n


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def _fwd(lib, B=1, H=1, T=64, dk=16, dv=16, L=8, C=16, dtype=1, ws=None, nws=0, ptrs=None):
    p = [FAKE] * 6 if ptrs is None else ptrs
    return lib.loglin_fwd_chunked(*p, B, H, T, dk, dv, L, C, dtype, ws, nws, None)


@pytest.mark.parametrize("C", [0, 8, 48, 256])
def test_unsupported_chunk(lib, C):
    assert _fwd(lib, C=C) == EUNSUPPORTED
    assert b"chunk" in lib.loglin_last_error()


@pytest.mark.parametrize("dk,dv", [(8, 16), (16, 24), (256, 64), (64, 0)])
def test_unsupported_head_dims(lib, dk, dv):
    assert _fwd(lib, dk=dk, dv=dv) == EUNSUPPORTED


def test_too_few_levels(lib):
    # T = 64 uses levels 0..6 -> L >= 7
    assert _fwd(lib, T=64, L=6, C=64) == EINVAL
    assert _fwd(lib, T=65, L=7, C=16, ws=None) == EINVAL  # 65 tokens need 8 levels
    assert _fwd(lib, T=64, L=65, C=64) == EINVAL


def test_null_pointer(lib):
    assert _fwd(lib, C=64, ptrs=[FAKE, None, FAKE, FAKE, FAKE, FAKE]) == EINVAL


def test_bad_dtype(lib):
    assert _fwd(lib, dtype=7) == EINVAL


def test_empty_is_noop(lib):
    assert _fwd(lib, B=0, ptrs=[None] * 6) == 0
    assert _fwd(lib, T=0, ptrs=[None] * 6) == 0
    assert _fwd(lib, B=-1) == EINVAL


def test_workspace_sizes(lib):
    w = lambda *a: lib.loglin_fwd_workspace_bytes(*a, 0)  # noqa: E731  (fp32: chunked path)
    assert w(1, 1, 64, 16, 16, 64) == 0           # one chunk: no inter-chunk state
    assert w(1, 1, 64, 16, 16, 16) > 4 * 16 * 16 * 4
    n = w(2, 3, 1000, 64, 32, 64)                   # 16 chunks, ragged
    assert n >= 6 * 16 * 64 * 32 * 4 and n % 256 == 0
    assert w(1, 1, 64, 16, 16, 12) == ctypes.c_size_t(-1).value
    assert lib.loglin_fwd_workspace_bytes(1, 1, 64, 16, 16, 16, 5) == ctypes.c_size_t(-1).value
    # bf16: fused path, one state per segment instead of one per chunk
    nb = lib.loglin_fwd_workspace_bytes(4, 16, 8192, 128, 64, 64, 1)
    nf = lib.loglin_fwd_workspace_bytes(4, 16, 8192, 128, 64, 64, 0)
    assert 0 < nb < nf


class Plan(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int), ("tile", ctypes.c_int), ("seg_tiles", ctypes.c_int),
                ("nseg", ctypes.c_int), ("col_block", ctypes.c_int),
                ("coarse_levels", ctypes.c_int), ("state_split", ctypes.c_int),
                ("workspace_bytes", ctypes.c_size_t)]


@pytest.mark.parametrize("B,H,T,dk,dv,C", [(4, 16, 8192, 128, 64, 64), (1, 16, 65536, 128, 128, 128),
                                           (2, 8, 2048, 64, 64, 64), (1, 1, 64, 16, 16, 16),
                                           (1, 1, 1, 16, 16, 16), (3, 5, 1000, 32, 16, 32)])
def test_plan(lib, B, H, T, dk, dv, C):
    pl = Plan()
    assert lib.loglin_fwd_plan(B, H, T, dk, dv, C, 1, ctypes.byref(pl)) == 0
    assert pl.path == 1 and pl.tile == 64
    ntiles = -(-T // 64)
    assert pl.nseg == -(-ntiles // pl.seg_tiles)
    assert (1 << pl.coarse_levels) >= pl.nseg > (1 << pl.coarse_levels) // 2 or pl.nseg == 1
    assert pl.col_block == min(dv, 64)
    assert pl.workspace_bytes == lib.loglin_fwd_workspace_bytes(B, H, T, dk, dv, C, 1)
    assert lib.loglin_fwd_plan(B, H, T, dk, dv, C, 0, ctypes.byref(pl)) == 0
    assert pl.path == 0 and pl.tile == C and pl.nseg == -(-T // C)


def test_plan_env_forces_chunked(lib, monkeypatch):
    monkeypatch.setenv("LOGLIN_FWD_PATH", "chunked")
    pl = Plan()
    assert lib.loglin_fwd_plan(4, 16, 8192, 128, 64, 64, 1, ctypes.byref(pl)) == 0
    assert pl.path == 0 and pl.nseg == 128


def test_workspace_too_small(lib):
    # fp32 inputs take the chunked path: 4 chunks of 16 need chunk states
    assert _fwd(lib, T=64, C=16, dtype=0, ws=None, nws=0) == EINVAL
    assert b"workspace" in lib.loglin_last_error()
    assert _fwd(lib, T=64, C=16, dtype=0, ws=FAKE * 256, nws=16) == EINVAL
    assert _fwd(lib, T=64, C=16, dtype=0, ws=FAKE + 16, nws=1 << 20) == EINVAL  # misaligned
    # bf16: 1024 tokens make 16 tiles; with 16 heads the fused path uses segments
    assert _fwd(lib, B=1, H=16, T=1024, dk=64, dv=64, L=11, C=64, dtype=1, ws=None) == EINVAL


def test_too_many_chunks(lib):
    assert _fwd(lib, T=16 * 65536 + 16, C=16, L=30) == EUNSUPPORTED


def test_state_init_validation(lib):
    h = ctypes.c_void_p()
    assert lib.loglin_state_init(None, 1, 1, 16, 16, 8, None) == EINVAL
    assert lib.loglin_state_init(ctypes.byref(h), 0, 1, 16, 16, 8, None) == EINVAL
    assert lib.loglin_state_init(ctypes.byref(h), 1, 1, 12, 16, 8, None) == EUNSUPPORTED
    assert lib.loglin_state_init(ctypes.byref(h), 1, 1, 16, 16, 0, None) == EINVAL
    assert lib.loglin_state_init(ctypes.byref(h), 1, 1, 16, 16, 49, None) == EINVAL
    assert not h.value


def test_state_init_allocation_failure_is_reported(lib, monkeypatch):
    monkeypatch.setenv("LOGLIN_TEST_FAIL_ALLOC", "1")
    h = ctypes.c_void_p()
    assert lib.loglin_state_init(ctypes.byref(h), 2, 2, 16, 16, 8, None) == ENOMEM
    assert not h.value
    assert b"injected" in lib.loglin_last_error()


def test_state_calls_reject_null_handle(lib):
    assert lib.loglin_state_free(None) == 0
    assert lib.loglin_state_load(None, FAKE, None, None) == EINVAL
    assert lib.loglin_state_export(None, None, None, None) == EINVAL
    assert lib.loglin_decode_step(None, *[FAKE] * 6, 1, None) == EINVAL


def test_level_map_validation(lib):
    assert lib.loglin_debug_level_map(0, FAKE, None) == EINVAL
    assert lib.loglin_debug_level_map(16385, FAKE, None) == EINVAL
    assert lib.loglin_debug_level_map(8, None, None) == EINVAL


def test_status_strings(lib):
    assert lib.loglin_status_string(0) == b"LOGLIN_OK"
    assert lib.loglin_status_string(4) == b"LOGLIN_ECAPACITY"


# ---------------------------------------------------------------- prefill -> decode

def _prefill_jobs(T):
    """Pieces of the prefix: whole 512-token pieces of the large buckets, one
    per smaller bucket (set bits of (T-1) mod 512), one for level 0."""
    if T <= 0:
        return 0
    n = T - 1
    return n // 512 + bin(n % 512).count("1") + 1


@pytest.mark.parametrize("B,H,T,dk,dv,Lmax", [(1, 1, 1, 16, 16, 1), (2, 3, 64, 64, 32, 8),
                                              (4, 16, 8192, 128, 64, 15), (1, 16, 65536, 128, 128, 18),
                                              (1, 1, 0, 16, 16, 4)])
def test_prefill_workspace_bytes(lib, B, H, T, dk, dv, Lmax):
    want = B * H * _prefill_jobs(T) * dk * dv * 4
    want = (want + 255) // 256 * 256
    assert lib.loglin_prefill_workspace_bytes(B, H, T, dk, dv, Lmax) == want


def _prefill(lib, B=1, H=1, T=64, dk=16, dv=16, Lmax=8, dtype=1, ws=FAKE, nws=1 << 30, ptrs=None):
    p = [FAKE] * 4 if ptrs is None else ptrs
    return lib.loglin_prefill_states(*p, B, H, T, dk, dv, Lmax, dtype, ws, nws, None)


def test_prefill_validation(lib):
    # T = 1000 needs bit_length(999) + 1 = 11 levels
    assert _prefill(lib, T=1000, Lmax=10) == ECAPACITY
    assert lib.loglin_prefill_workspace_bytes(1, 1, 1000, 16, 16, 10) == ctypes.c_size_t(-1).value
    assert _prefill(lib, dk=48) == EUNSUPPORTED
    assert _prefill(lib, Lmax=0) == EINVAL
    assert _prefill(lib, Lmax=49) == EINVAL
    assert _prefill(lib, dtype=7) == EINVAL
    assert _prefill(lib, ptrs=[FAKE, FAKE, FAKE, None]) == EINVAL
    assert _prefill(lib, ptrs=[None, FAKE, FAKE, FAKE]) == EINVAL
    assert _prefill(lib, ptrs=[FAKE, FAKE, FAKE, FAKE + 4]) == EINVAL  # states misaligned
    assert _prefill(lib, nws=16) == EINVAL                             # workspace too small
    assert _prefill(lib, ws=FAKE + 64) == EINVAL                       # workspace misaligned
    assert _prefill(lib, B=0) == 0                                      # no-op


# ---- backward pass: workspace sizes and argument checks (nothing launched)

def _align(x):
    return (x + 255) // 256 * 256


def _bwd_tail(BH, N, T, dk, dv, off):
    """R and R^T (when N > 1), then the two per-token dot products."""
    if N > 1:
        off = _align(_align(off + BH * N * dk * dv * 4) + BH * N * dk * dv * 4)
    return _align(_align(off + BH * T * 4) + BH * T * 4)


@pytest.mark.parametrize("B,H,T,dk,dv,C", [(1, 1, 1, 16, 16, 16), (1, 2, 37, 16, 32, 16),
                                           (4, 16, 8192, 128, 64, 64), (1, 16, 65536, 128, 128, 128)])
def test_bwd_workspace_bytes(lib, monkeypatch, B, H, T, dk, dv, C):
    """The chunk-state layout: nodes, chunk totals, fp64 chunk ends, then R,
    R^T and the dot products (fp32 inputs always; bf16 where the fused dq
    pass does not apply or is switched off)."""
    monkeypatch.setenv("LOGLIN_BWD_DQ", "chunked")
    BH, N = B * H, (T + C - 1) // C
    off = 0
    if N > 1:
        off = _align(_align(_align(BH * N * dk * dv * 4) + BH * N * 4) + BH * N * 8)
    want = _bwd_tail(BH, N, T, dk, dv, off)
    assert lib.loglin_bwd_workspace_bytes(B, H, T, dk, dv, C, 1) == want
    assert lib.loglin_bwd_workspace_bytes(B, H, T, dk, dv, C, 0) == want
    monkeypatch.delenv("LOGLIN_BWD_DQ")
    assert lib.loglin_bwd_workspace_bytes(B, H, T, dk, dv, C, 0) == want


def _fused_dq_layout(BH, N, T, dk, dv, nseg, LU, ncb, nsub):
    off = _align(_align(_align(BH * nseg * dk * dv * 4) + BH * nseg * 4) + BH * nseg * 8)
    off = _align(off + BH * nseg * dk * dv * 2)
    if nsub > 1:  # sub-range states and totals
        off = _align(_align(off + BH * nseg * nsub * dk * dv * 4) + BH * nseg * nsub * 4)
    off = _align(off + ncb * BH * T * LU * 4)
    off = _align(off + ncb * BH * T * 4)
    off = _align(off + BH * N * 8)
    return _bwd_tail(BH, N, T, dk, dv, off)


def test_bwd_workspace_bytes_fused_dq(lib, monkeypatch):
    """bf16, d_v = 64: the fused dq pass's layout at the 8K workload's shape.
    Its plan (swapped problem: d_k 64, d_v 128, 128 tiles, 64 (batch, head)
    pairs): segments of 32 tiles (every segment length costs the same serial
    tiles per compute unit; the longest wins), 4 segments, five register
    levels and two above the segment, so the 128 columns run as one block;
    with 64 pairs the segment states come in two sub-ranges (3 x 64 blocks
    would leave compute units idle).  Segment nodes fp32 [64][4][128][64],
    totals, fp64 ends, bf16 fragments, the sub-range states [64][4][2][128][64]
    and totals; the dlambda parts [1][64][14][8192] (positions
    below 8192 use levels 0..13) and the parts of q . dq [1][64][8192]; the
    fp64 chunk ends [64][128]; then R, R^T and the dot products.  With
    LOGLIN_BWD_DQ=fused64 the pass keeps two 64-column blocks: two parts
    of each, and the segment states in one sub-range (3 x 128 blocks)."""
    monkeypatch.delenv("LOGLIN_BWD_DQ", raising=False)
    B, H, T, dk, dv, C = 4, 16, 8192, 128, 64, 64
    BH, N, nseg, LU = B * H, T // C, 4, 14
    assert lib.loglin_bwd_workspace_bytes(B, H, T, dk, dv, C, 1) == _fused_dq_layout(BH, N, T, dk, dv, nseg, LU, 1, 2)
    monkeypatch.setenv("LOGLIN_BWD_DQ", "fused64")
    assert lib.loglin_bwd_workspace_bytes(B, H, T, dk, dv, C, 1) == _fused_dq_layout(BH, N, T, dk, dv, nseg, LU, 2, 1)


def _bwd(lib, B=1, H=1, T=64, dk=16, dv=16, L=8, C=16, dtype=1, ws=FAKE * 256, nws=1 << 30,
         ptrs=None):
    p = [FAKE] * 11 if ptrs is None else ptrs
    return lib.loglin_bwd_chunked(*p, B, H, T, dk, dv, L, C, dtype, ws, nws, None)


def test_bwd_validation(lib):
    assert lib.loglin_bwd_workspace_bytes(1, 1, 64, 48, 16, 16, 1) == ctypes.c_size_t(-1).value
    assert lib.loglin_bwd_workspace_bytes(1, 1, 64, 16, 16, 16, 9) == ctypes.c_size_t(-1).value
    assert _bwd(lib, C=8) == EUNSUPPORTED
    assert _bwd(lib, dv=24) == EUNSUPPORTED
    assert _bwd(lib, T=1000, L=10) == EINVAL          # needs 11 levels
    assert _bwd(lib, L=65) == EINVAL
    assert _bwd(lib, dtype=3) == EINVAL
    for k in range(11):
        p = [FAKE] * 11
        p[k] = None
        assert _bwd(lib, ptrs=p) == EINVAL, k
    p = [FAKE] * 11
    p[5] = FAKE + 8                                     # dout misaligned
    assert _bwd(lib, ptrs=p) == EINVAL
    assert _bwd(lib, nws=16) == EINVAL                  # workspace too small
    assert b"workspace" in lib.loglin_last_error()
    assert _bwd(lib, ws=None) == EINVAL
    assert _bwd(lib, ws=FAKE * 256 + 64) == EINVAL      # workspace misaligned
    assert _bwd(lib, B=0) == 0 and _bwd(lib, T=0, ws=None, nws=0) == 0


def test_noalloc_rejects_on_the_host(lib):
    """The allocation-free forward reports sizes its array cannot hold, and
    whatever the forward itself rejects, before touching a device."""
    f = lib.loglin_fwd_chunked_noalloc
    f.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_int] * 8 + [ctypes.c_void_p]
    f.restype = ctypes.c_int
    # fp32 inputs at B=4, H=16, T=8192: a 256 MiB workspace
    assert f(*([FAKE] * 6), 4, 16, 8192, 128, 64, 15, 64, 0, None) == EUNSUPPORTED
    assert b"workspace" in lib.loglin_last_error()
    assert f(*([FAKE] * 6), 1, 1, 64, 16, 16, 8, 48, 1, None) == EUNSUPPORTED  # chunk size
    assert f(*([FAKE] * 6), 1, 1, 64, 16, 16, 3, 16, 1, None) == EINVAL        # levels
    assert f(*([FAKE] * 6), 1, 1, 64, 16, 16, 8, 16, 7, None) == EINVAL        # dtype
