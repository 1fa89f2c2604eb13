"""The C-ABI library loads, exports every function include/sdm.h declares, and refuses bad
arguments on the host with the documented status codes (CPU only: nothing is launched)."""

import ctypes
import os
import re

import pytest

from sparse_delta_memory_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sdm.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libsdm_amd.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(sdm_\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_function():
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS), names
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), name


def shape(**kw):
    d = dict(N=4, C=64, W=4, R=4, P=1, key_bits=12, stream_offset=0, first_partial=4, valid_last=64, tile_len=128,
             g_lane_stride=0, idx_bytes=4, val_bytes=4, tiled=0, lds_budget=0, pair_walk=0)
    d.update(kw)
    return _lib.P1Shape(*[d[f] for f, _ in _lib.P1Shape._fields_])


FAKE = 0x10000  # never dereferenced: every check below fails before a launch


def io(**kw):
    o = _lib.P1IO()
    for f in _lib.P1_IO_FIELDS:
        setattr(o, f, FAKE)
    o.workspace = FAKE
    o.workspace_bytes = 1 << 40
    for k, v in kw.items():
        setattr(o, k, v)
    return o


def call_p1(s, o):
    lib = _lib.load()
    return lib.sdm_phase1(ctypes.byref(s) if s is not None else None, ctypes.byref(o) if o is not None else None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(C=0), _lib.SDM_ESHAPE), (dict(C=257), _lib.SDM_ESHAPE), (dict(W=0), _lib.SDM_ESHAPE),
    (dict(R=300), _lib.SDM_ESHAPE), (dict(P=0), _lib.SDM_ESHAPE), (dict(N=-1), _lib.SDM_ESHAPE),
    (dict(key_bits=0), _lib.SDM_EINVAL), (dict(key_bits=31), _lib.SDM_EINVAL),
    (dict(first_partial=5), _lib.SDM_EINVAL), (dict(valid_last=65), _lib.SDM_EINVAL),
    (dict(tile_len=0), _lib.SDM_EINVAL), (dict(stream_offset=-1), _lib.SDM_EINVAL),
    (dict(g_lane_stride=2), _lib.SDM_EINVAL), (dict(g_lane_stride=-1), _lib.SDM_EINVAL),
    (dict(idx_bytes=2), _lib.SDM_EINVAL), (dict(idx_bytes=16), _lib.SDM_EINVAL),
    (dict(val_bytes=1), _lib.SDM_EINVAL), (dict(val_bytes=8), _lib.SDM_EINVAL),
    (dict(tiled=2), _lib.SDM_EINVAL), (dict(tiled=-1), _lib.SDM_EINVAL),
])
def test_phase1_shape_refusals(kw, status):
    s = shape(**kw)
    assert call_p1(s, io()) == status
    assert _lib.load().sdm_phase1_workspace(ctypes.byref(s)) == 0
    assert len(_lib.load().sdm_last_error()) > 0


def test_long_rows_take_the_tiled_path():
    """Rows past 16384 entries (up to C (W + R) = 2^17) are accepted and sized with the tiled path's
    workspace: its sort buffers and reverse-scan results on top of the pair records and 32-bit
    entry-order words; tiled = 1 asks for the same layout at any size."""
    lib = _lib.load()
    up = lambda b: (b + 255) // 256 * 256  # noqa: E731
    for C, W, R, tiled in ((256, 256, 256, 0), (256, 48, 48, 0), (64, 4, 4, 1)):
        s = shape(N=2, C=C, W=W, R=R, first_partial=2, valid_last=C, tiled=tiled)
        n, N = C * (W + R), 2
        hot = C * W // 16
        want = (up(N * n * 16) + up(N * C * W * 4) + up(N * C * R * 4) + up(N * (hot + 1) * 8)
                + up(N * n * 16) + up(N * n * 12))
        assert lib.sdm_phase1_workspace(ctypes.byref(s)) == want
    s = shape(N=2, C=64, W=4, R=4, first_partial=2, valid_last=64)   # on chip: 16-bit words, no sort buffers
    n = 64 * 8
    assert lib.sdm_phase1_workspace(ctypes.byref(s)) == up(2 * n * 16) + 2 * up(2 * 64 * 4 * 2) + up(2 * 17 * 8)


def test_phase1_argument_refusals():
    s = shape()
    assert call_p1(None, io()) == _lib.SDM_EINVAL
    assert call_p1(s, None) == _lib.SDM_EINVAL
    for f in ("k_idx", "q_idx", "k_val", "q_val", "g", "spay_k", "krec", "tiles_k"):
        assert call_p1(s, io(**{f: None})) == _lib.SDM_EINVAL, f
    assert call_p1(s, io(krec=FAKE + 4)) == _lib.SDM_EALIGN
    assert call_p1(s, io(log_k=FAKE + 2)) == _lib.SDM_EALIGN
    need = _lib.load().sdm_phase1_workspace(ctypes.byref(s))
    assert need > 0
    assert call_p1(s, io(workspace_bytes=need - 1)) == _lib.SDM_EWORKSPACE
    assert call_p1(s, io(workspace=None)) == _lib.SDM_EWORKSPACE
    # N = 0 is a valid no-op: nothing to launch, no device needed.
    assert call_p1(shape(N=0, first_partial=0), io()) == _lib.SDM_OK


def dw(**kw):
    o = _lib.DwIO()
    d = dict(bank=FAKE, bank_dtype=_lib.SDM_BF16, rows=1 << 20, hd=128, dv=FAKE, dv_dtype=_lib.SDM_F32,
             dv_step_rows=64, dv_rows=256, krec=FAKE, P=1, C=64, W=4, N=4, snap_dtype=_lib.SDM_BF16)
    d.update(kw)
    for k, v in d.items():
        setattr(o, k, v)
    return o


@pytest.mark.parametrize("kw,ti,status", [
    (dict(), -1, _lib.SDM_ESHAPE), (dict(), 4, _lib.SDM_ESHAPE), (dict(P=2), 2, _lib.SDM_ESHAPE),
    (dict(C=0), 0, _lib.SDM_ESHAPE), (dict(W=257), 0, _lib.SDM_ESHAPE),
    (dict(bank_dtype=7), 0, _lib.SDM_EINVAL), (dict(dv_dtype=3), 0, _lib.SDM_EINVAL),
    (dict(hd=0), 0, _lib.SDM_ESHAPE), (dict(hd=8192), 0, _lib.SDM_ESHAPE),
    (dict(hd=1032), 0, _lib.SDM_EUNSUPPORTED), (dict(hd=2048), 0, _lib.SDM_EUNSUPPORTED),
    (dict(hd=126, bank=FAKE + 1), 0, _lib.SDM_EALIGN), (dict(hd=126, dv=FAKE + 2), 0, _lib.SDM_EALIGN),
    (dict(hd=37, snap=FAKE + 1, snap_rows=1 << 20), 0, _lib.SDM_EALIGN),   # (bf16 bank: 2-byte rows)
    (dict(snap=FAKE, snap_rows=1 << 20, snap_dtype=_lib.SDM_F32), 0, _lib.SDM_EINVAL),   # f32 rows of a bf16 bank
    (dict(snap=FAKE, snap_rows=1 << 20, snap_dtype=9), 0, _lib.SDM_EINVAL),
    (dict(snap=FAKE, snap_rows=1 << 20, snap_ord=FAKE + 2), 0, _lib.SDM_EALIGN),
    (dict(bank=None), 0, _lib.SDM_EINVAL), (dict(krec=None), 0, _lib.SDM_EINVAL),
    (dict(bank=FAKE + 8), 0, _lib.SDM_EALIGN), (dict(dv=FAKE + 4), 0, _lib.SDM_EALIGN),
    (dict(krec=FAKE + 8), 0, _lib.SDM_EALIGN), (dict(rows=0), 0, _lib.SDM_EINVAL),
    (dict(dv_rows=255), 3, _lib.SDM_EINVAL), (dict(dv_step_rows=-1), 0, _lib.SDM_EINVAL),
    (dict(workspace=FAKE, workspace_bytes=16), 0, _lib.SDM_EWORKSPACE),
    (dict(workspace=FAKE + 4, workspace_bytes=1 << 40), 0, _lib.SDM_EALIGN),
    (dict(snap=FAKE + 8, snap_rows=1 << 20), 0, _lib.SDM_EALIGN),
    (dict(snap=FAKE, snap_step_rows=256, snap_rows=511), 1, _lib.SDM_EINVAL),
    (dict(snap=FAKE, snap_step_rows=-1, snap_rows=1 << 20), 0, _lib.SDM_EINVAL),
])
def test_dw_refusals(kw, ti, status):
    lib = _lib.load()
    assert lib.sdm_dw_step(ctypes.byref(dw(**kw)), ti, None) == status
    assert len(lib.sdm_last_error()) > 0


def test_status_strings():
    lib = _lib.load()
    for s in range(-6, 1):
        assert len(lib.sdm_status_string(s)) > 0


def test_dw_workspace_size():
    lib = _lib.load()
    o = dw(P=2, C=64, W=4, hd=128)
    need = lib.sdm_dw_workspace(ctypes.byref(o))
    blocks = (2 * 64 * 4 + 31) // 32   # one counter, one metadata pair and two partial rows per 32 positions
    up = lambda b: (b + 255) // 256 * 256  # noqa: E731
    assert need == up(4 * blocks) + up(8 * blocks) + up(2 * blocks * 128 * 4)
    assert lib.sdm_dw_workspace(ctypes.byref(dw(P=0))) == 0


def read_io(**kw):
    o = _lib.ReadIO()
    for f, _ in _lib.ReadIO._fields_:
        if f not in ("events",):
            setattr(o, f, FAKE if _ == ctypes.c_void_p else 0)
    o.bank_dtype, o.rows, o.hd = _lib.SDM_BF16, 1 << 20, 128
    o.step_rows, o.out_rows = 512, 1 << 20
    o.P, o.C, o.W, o.R, o.N, o.first_partial, o.valid_last = 4, 128, 16, 16, 8, 8, 128
    for k, v in kw.items():
        setattr(o, k, v)
    return o


@pytest.mark.parametrize("kw,ti,status", [
    (dict(C=0), 0, _lib.SDM_ESHAPE), (dict(C=257), 0, _lib.SDM_ESHAPE), (dict(R=0), 0, _lib.SDM_ESHAPE),
    (dict(P=0), 0, _lib.SDM_ESHAPE), (dict(), 2, _lib.SDM_ESHAPE), (dict(), -1, _lib.SDM_ESHAPE),
    (dict(hd=0), 0, _lib.SDM_ESHAPE), (dict(hd=5000), 0, _lib.SDM_ESHAPE), (dict(bank_dtype=7), 0, _lib.SDM_EINVAL),
    (dict(hd=12, v=FAKE + 2), 0, _lib.SDM_EALIGN), (dict(hd=12, bank=FAKE + 1), 0, _lib.SDM_EALIGN),
    (dict(valid_last=129), 0, _lib.SDM_EINVAL), (dict(first_partial=9), 0, _lib.SDM_EINVAL),
    (dict(out_rows=100), 0, _lib.SDM_EINVAL), (dict(beta=None), 0, _lib.SDM_EINVAL),
    (dict(dv=FAKE + 4), 0, _lib.SDM_EALIGN), (dict(a=FAKE + 2), 0, _lib.SDM_EALIGN),
    (dict(idx_bytes=3), 0, _lib.SDM_EINVAL), (dict(idx_bytes=8, k_idx=FAKE + 4), 0, _lib.SDM_EALIGN),
    (dict(val_bytes=3), 0, _lib.SDM_EINVAL), (dict(k_eff=FAKE + 2), 0, _lib.SDM_EALIGN),
    (dict(val_bytes=2, q_w=FAKE + 1), 0, _lib.SDM_EALIGN), (dict(rows=0), 0, _lib.SDM_EINVAL),
])
def test_read_step_refusals(kw, ti, status):
    lib = _lib.load()
    o = read_io(**kw)
    assert lib.sdm_read_step(ctypes.byref(o), ti, None) == status
    assert len(lib.sdm_last_error()) > 0
    assert lib.sdm_read_step(None, 0, None) == _lib.SDM_EINVAL


def test_phase1_int64_ids_alignment():
    s = shape(idx_bytes=8)
    assert call_p1(s, io(k_idx=FAKE + 4)) == _lib.SDM_EALIGN


def test_phase1_value_alignment():
    """float32 values need 4-byte alignment, bfloat16 values 2-byte."""
    assert call_p1(shape(), io(k_val=FAKE + 2)) == _lib.SDM_EALIGN
    assert call_p1(shape(), io(cpe=FAKE + 2)) == _lib.SDM_EALIGN
    assert call_p1(shape(val_bytes=2), io(q_w=FAKE + 1)) == _lib.SDM_EALIGN
    assert call_p1(shape(), io(gord_k=FAKE + 2)) == _lib.SDM_EALIGN


def gds_io(**kw):
    o = _lib.GdsIO()
    d = dict(bank=FAKE, bank_dtype=_lib.SDM_BF16, rows=1 << 20, hd=128, q_idx=FAKE, q_w=FAKE, spay_q=FAKE, gr=FAKE,
             step_rows=512, gr_rows=1 << 20, d_q_w=FAKE, grad=FAKE, grad_dtype=_lib.SDM_F32, P=4, C=128, R=16, N=8,
             first_partial=8, valid_last=128, idx_bytes=4, val_bytes=4)
    d.update(kw)
    for k, v in d.items():
        setattr(o, k, v)
    return o


@pytest.mark.parametrize("kw,ti,status", [
    (dict(), 2, _lib.SDM_ESHAPE), (dict(), -1, _lib.SDM_ESHAPE), (dict(C=0), 0, _lib.SDM_ESHAPE),
    (dict(R=257), 0, _lib.SDM_ESHAPE), (dict(hd=126), 0, _lib.SDM_ESHAPE), (dict(bank_dtype=5), 0, _lib.SDM_EINVAL),
    (dict(grad_dtype=5), 0, _lib.SDM_EINVAL), (dict(idx_bytes=2), 0, _lib.SDM_EINVAL),
    (dict(val_bytes=8), 0, _lib.SDM_EINVAL), (dict(gr_rows=100), 0, _lib.SDM_EINVAL),
    (dict(spay_q=None), 0, _lib.SDM_EINVAL), (dict(gr=FAKE + 8), 0, _lib.SDM_EALIGN),
    (dict(bank=FAKE + 4), 0, _lib.SDM_EALIGN), (dict(grad=FAKE + 8), 0, _lib.SDM_EALIGN),
    (dict(q_w=FAKE + 2), 0, _lib.SDM_EALIGN), (dict(valid_last=129), 0, _lib.SDM_EINVAL),
    (dict(rows=0), 0, _lib.SDM_EINVAL),
])
def test_gds_refusals(kw, ti, status):
    lib = _lib.load()
    assert lib.sdm_gds_step(ctypes.byref(gds_io(**kw)), ti, None) == status
    assert len(lib.sdm_last_error()) > 0
    assert lib.sdm_gds_step(None, 0, None) == _lib.SDM_EINVAL


def gwr_io(**kw):
    o = _lib.GwrIO()
    d = dict(grad=FAKE, grad_dtype=_lib.SDM_BF16, rows=1 << 20, hd=128, k_idx=FAKE, w=FAKE, dv=FAKE, step_rows=512,
             dv_rows=1 << 20, d_dv=FAKE, d_k_pd=FAKE, P=4, C=128, W=16, N=8, first_partial=8, valid_last=128,
             idx_bytes=4)
    d.update(kw)
    for k, v in d.items():
        setattr(o, k, v)
    return o


@pytest.mark.parametrize("kw,ti,status", [
    (dict(), 2, _lib.SDM_ESHAPE), (dict(W=0), 0, _lib.SDM_ESHAPE), (dict(hd=1028), 0, _lib.SDM_ESHAPE),
    (dict(hd=6), 0, _lib.SDM_ESHAPE), (dict(grad_dtype=3), 0, _lib.SDM_EINVAL), (dict(idx_bytes=5), 0, _lib.SDM_EINVAL),
    (dict(dv_rows=100), 0, _lib.SDM_EINVAL), (dict(w=None), 0, _lib.SDM_EINVAL), (dict(dv=FAKE + 4), 0, _lib.SDM_EALIGN),
    (dict(d_dv=FAKE + 8), 0, _lib.SDM_EALIGN), (dict(grad=FAKE + 4), 0, _lib.SDM_EALIGN),
    (dict(d_k_pd=FAKE + 2), 0, _lib.SDM_EALIGN), (dict(first_partial=9), 0, _lib.SDM_EINVAL),
    (dict(rows=0), 0, _lib.SDM_EINVAL),
])
def test_gwr_refusals(kw, ti, status):
    lib = _lib.load()
    assert lib.sdm_gwr_step(ctypes.byref(gwr_io(**kw)), ti, None) == status
    assert len(lib.sdm_last_error()) > 0
    assert lib.sdm_gwr_step(None, 0, None) == _lib.SDM_EINVAL


def pa_io(**kw):
    o = _lib.PaIO()
    d = dict(grad=FAKE, grad_dtype=_lib.SDM_F32, bank=FAKE, bank_dtype=_lib.SDM_BF16, rows=1 << 20, hd=128, snap=FAKE,
             snap_step_rows=0, snap_rows=1 << 16, krec=FAKE, k_eff=FAKE, beta=FAKE, d_dva=FAKE, step_rows=512,
             dva_rows=1 << 20, g_decay=FAKE, d_k_eff=FAKE, P=4, C=128, W=16, N=8, val_bytes=4)
    d.update(kw)
    for k, v in d.items():
        setattr(o, k, v)
    return o


@pytest.mark.parametrize("kw,ti,status", [
    (dict(), 2, _lib.SDM_ESHAPE), (dict(C=300), 0, _lib.SDM_ESHAPE), (dict(hd=2048), 0, _lib.SDM_ESHAPE),
    (dict(grad_dtype=4), 0, _lib.SDM_EINVAL), (dict(bank_dtype=4), 0, _lib.SDM_EINVAL), (dict(val_bytes=3), 0, _lib.SDM_EINVAL),
    (dict(snap_rows=100), 0, _lib.SDM_EINVAL), (dict(dva_rows=100), 0, _lib.SDM_EINVAL), (dict(beta=None), 0, _lib.SDM_EINVAL),
    (dict(snap=FAKE + 4), 0, _lib.SDM_EALIGN), (dict(krec=FAKE + 8), 0, _lib.SDM_EALIGN),
    (dict(d_k_eff=FAKE + 2), 0, _lib.SDM_EALIGN),
    (dict(workspace=FAKE, workspace_bytes=16), 0, _lib.SDM_EWORKSPACE),
    (dict(workspace=FAKE + 4, workspace_bytes=1 << 40), 0, _lib.SDM_EALIGN), (dict(rows=0), 0, _lib.SDM_EINVAL),
])
def test_pa_refusals(kw, ti, status):
    lib = _lib.load()
    assert lib.sdm_pa_step(ctypes.byref(pa_io(**kw)), ti, None) == status
    assert len(lib.sdm_last_error()) > 0
    assert lib.sdm_pa_step(None, 0, None) == _lib.SDM_EINVAL


def test_pa_workspace_size():
    lib = _lib.load()
    o = pa_io(P=2, C=64, W=4, hd=96)
    need = lib.sdm_pa_workspace(ctypes.byref(o))
    blocks = (2 * 64 * 4 + 31) // 32   # one counter, one segment count and two partial rows per 32 positions
    up = lambda b: (b + 255) // 256 * 256  # noqa: E731
    assert need == up(4 * blocks) + up(4 * blocks) + up(2 * blocks * 96 * 4)
    assert lib.sdm_pa_workspace(ctypes.byref(pa_io(P=0))) == 0


def gds_io(**kw):
    o = _lib.GdsIO()
    d = dict(bank=FAKE, bank_dtype=_lib.SDM_BF16, rows=1 << 20, hd=128, q_idx=FAKE, q_w=FAKE, spay_q=FAKE, gr=FAKE,
             step_rows=512, gr_rows=1 << 20, d_q_w=FAKE, grad=FAKE, grad_dtype=_lib.SDM_F32, P=4, C=128, R=16, N=8,
             first_partial=8, valid_last=128, idx_bytes=4, val_bytes=4)
    d.update(kw)
    for k, v in d.items():
        setattr(o, k, v)
    return o


@pytest.mark.parametrize("kw,status", [
    (dict(workspace=FAKE, workspace_bytes=16), _lib.SDM_EWORKSPACE),
    (dict(workspace=FAKE + 4, workspace_bytes=1 << 40), _lib.SDM_EALIGN),
    (dict(hd=6), _lib.SDM_ESHAPE),
])
def test_gds_workspace_refusals(kw, status):
    assert _lib.load().sdm_gds_step(ctypes.byref(gds_io(**kw)), 0, None) == status


def test_gds_workspace_size():
    lib = _lib.load()
    need = lib.sdm_gds_workspace(ctypes.byref(gds_io(P=2, C=64, R=4, hd=96)))
    blocks = (2 * 64 * 4 + 31) // 32   # one counter, one segment count and two partial rows per 32 positions
    up = lambda b: (b + 255) // 256 * 256  # noqa: E731
    assert need == up(4 * blocks) + up(4 * blocks) + up(2 * blocks * 96 * 4)
    assert lib.sdm_gds_workspace(ctypes.byref(gds_io(R=0))) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(lds_budget=1000), _lib.SDM_EINVAL), (dict(lds_budget=200000), _lib.SDM_EINVAL),
    (dict(lds_budget=-1), _lib.SDM_EINVAL), (dict(pair_walk=2), _lib.SDM_EINVAL),
])
def test_phase1_knob_refusals(kw, status):
    assert call_p1(shape(**kw), io()) == status
    assert len(_lib.load().sdm_last_error()) > 0


def test_phase1_lds_budget_too_small_is_refused_before_any_device_call():
    """A budget the sort/scan kernel's plan cannot fit in (a 16384-entry row needs its 64 KB of keys
    and more) is refused on the host, without touching the device."""
    s = shape(N=2, C=256, W=32, R=32, first_partial=2, valid_last=256, lds_budget=65536)
    need = _lib.load().sdm_phase1_workspace(ctypes.byref(s))
    assert call_p1(s, io(workspace_bytes=need)) == _lib.SDM_EUNSUPPORTED
    assert b"budget" in _lib.load().sdm_last_error()


def call_pairs(s, o):
    lib = _lib.load()
    return lib.sdm_phase1_pairs(ctypes.byref(s) if s is not None else None, ctypes.byref(o) if o is not None else None,
                                None)


def test_deferred_pair_refusals():
    """defer_pairs is 0 or 1 and defers something (a or qk set); sdm_phase1_pairs refuses a bad
    shape, a missing io, no pair output, misaligned outputs and a short workspace, all on the host."""
    s = shape()
    assert call_p1(s, io(defer_pairs=2)) == _lib.SDM_EINVAL
    assert call_p1(s, io(defer_pairs=-1)) == _lib.SDM_EINVAL
    assert call_p1(s, io(defer_pairs=1, a=None, qk=None)) == _lib.SDM_EINVAL
    assert call_pairs(None, io()) == _lib.SDM_EINVAL
    assert call_pairs(shape(C=0), io()) == _lib.SDM_ESHAPE
    assert call_pairs(s, None) == _lib.SDM_EINVAL
    assert call_pairs(s, io(a=None, qk=None)) == _lib.SDM_EINVAL
    assert call_pairs(s, io(a=FAKE + 2)) == _lib.SDM_EALIGN
    need = _lib.load().sdm_phase1_workspace(ctypes.byref(s))
    assert call_pairs(s, io(workspace_bytes=need - 1)) == _lib.SDM_EWORKSPACE
    assert call_pairs(s, io(workspace=None)) == _lib.SDM_EWORKSPACE
    assert call_pairs(s, io(workspace=FAKE + 8)) == _lib.SDM_EALIGN
    assert call_pairs(shape(N=0, first_partial=0), io()) == _lib.SDM_OK   # nothing to launch
