"""Host-side checks of the C ABI (include/mosaic_bsa.h): no GPU needed.

Only argument sets that the library rejects during validation are passed, so
no call here reaches the HIP runtime (validation completes before any HIP
call; the fake pointers below are never dereferenced).  Every case that
expects a shape or support error also carries a workspace (or saved state)
that is too small, which validation checks later: should the shape become
valid, the call still stops at MOSAIC_ERR_WORKSPACE (and the test fails)
instead of launching kernels on the fake pointers.  Host-only by design: the
module is skipped when a GPU is visible.

MOSAIC_ABI_TEST_LIB, when set, names the library to load instead of the
package's own (the host-only sanitizer build of tests/test_abi_sanitized.py).
"""

import ctypes
import os
import re
import subprocess

import pytest

from spherical_block_sparse_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mosaic_bsa.h")

if os.environ.get("MOSAIC_ABI_TEST_LIB"):
    _lib.LIB_PATH = os.environ["MOSAIC_ABI_TEST_LIB"]


def _gpu_visible() -> bool:
    import torch
    return torch.cuda.device_count() > 0   # counts devices without initialising one


pytestmark = [
    pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libmosaic_bsa.so not built"),
    pytest.mark.skipif(_gpu_visible(), reason="host-only checks with fake device pointers: not run where a GPU is visible"),
]

FAKE = 0x10000          # 256-byte aligned, never dereferenced
OK, NULL, SHAPE, UNSUP, MISAL, WS, HIP = range(7)


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(mosaic_[a-z_]+)\s*\(", text)))


def test_header_declares_and_library_exports_the_same_symbols():
    declared = declared_functions()
    assert set(declared) == set(_lib.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (mosaic_[a-z_]+)\b", out))
    assert set(declared) <= exported, set(declared) - exported
    L = _lib.lib()
    for name in declared:
        assert hasattr(L, name)


def test_probe_header_declares_and_library_exports_the_same_symbols():
    """libmosaic_probe.so (the measurement probes) exports what include/mosaic_probe.h
    declares, and rejects bad arguments before any launch."""
    from spherical_block_sparse_amd import probe
    L = probe.lib()
    with open(os.path.join(ROOT, "include", "mosaic_probe.h")) as f:
        declared = set(re.findall(r"^int (mosaic_probe_\w+)\(", f.read(), flags=re.M))
    assert declared == set(probe.EXPORTED)
    for name in declared:
        assert hasattr(L, name)
    INVALID = 1   # hipErrorInvalidValue
    assert L.mosaic_probe_read(None, 1024, FAKE, 4, None) == INVALID
    assert L.mosaic_probe_read(FAKE + 8, 1024, FAKE, 4, None) == INVALID
    assert L.mosaic_probe_read(FAKE, 1024, FAKE, 0, None) == INVALID
    assert L.mosaic_probe_mfma(None, 4, 4, None, None) == INVALID
    assert L.mosaic_probe_mfma(FAKE, 4, 0, None, None) == INVALID
    assert L.mosaic_probe_overlap(None, 4, 4, 0, None, None, None) == INVALID
    assert L.mosaic_probe_overlap(FAKE, 4, 4, 6, None, None, None) == INVALID
    assert L.mosaic_probe_overlap(FAKE, 4, 4, -1, None, None, None) == INVALID
    assert L.mosaic_probe_overlap(FAKE, 0, 4, 0, None, None, None) == INVALID


def test_version_and_status_strings():
    L = _lib.lib()
    hdr = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "mosaic_bsa.h")
    with open(hdr) as f:
        want = int(re.search(r"#define MOSAIC_BSA_ABI_VERSION (\d+)", f.read()).group(1))
    assert L.mosaic_bsa_abi_version() == want
    for code, name in _lib.STATUS_NAMES.items():
        assert L.mosaic_status_string(code).decode() == name
    assert L.mosaic_status_string(99).decode() == "MOSAIC_ERR_UNKNOWN"


def test_workspace_bytes_layout():
    L = _lib.lib()
    # ns128: S = 192, m = 3072, d = 64 -> two float64 and two float32 [S][m][d] sections, the
    # float32 [S][m] largest key norm per block, the bf16 [S][m][2][d] pieces of k̄, the
    # float32 [S][m] |k̄_j|^2 and the float32 [S][m] selected-block bound per query block
    e = 192 * 3072 * 64
    assert L.mosaic_bsa_workspace_bytes(24, 8, 64, 128, 64, 16) == e * (8 + 8 + 4 + 4 + 4) + 192 * 3072 * 4 * 3
    # tiny: S = 2, m = 48, d = 32 -> sections rounded up to 256 bytes
    e = 2 * 48 * 32
    r = lambda x: (x + 255) // 256 * 256
    assert L.mosaic_bsa_workspace_bytes(1, 2, 32, 8, 16, 4) == 2 * r(8 * e) + 3 * r(4 * e) + 3 * r(4 * 2 * 48)
    assert L.mosaic_bsa_workspace_bytes(1, 2, 32, 8, 16, 0) == 0      # invalid -> 0
    assert L.mosaic_bsa_workspace_bytes(1, 2, 48, 8, 16, 4) == 0      # unsupported -> 0


def fwd(q=FAKE, k=FAKE, v=FAKE, gates=FAKE, batch=1, heads=2, d=32, nside=8, block=16, topn=4,
        window=32, out=FAKE, sel=FAKE, ws=FAKE, ws_bytes=16):
    L = _lib.lib()
    return L.mosaic_bsa_forward(q, k, v, gates, batch, heads, d, nside, block, topn, window, out, sel,
                                ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(k=None), NULL), (dict(v=None), NULL), (dict(gates=None), NULL),
    (dict(out=None), NULL), (dict(sel=None), NULL), (dict(ws=None), NULL),
    (dict(q=FAKE + 8), MISAL), (dict(out=FAKE + 4), MISAL), (dict(ws=FAKE + 16), MISAL),
    (dict(gates=FAKE + 2), MISAL),
    (dict(batch=0), SHAPE), (dict(heads=-1), SHAPE),
    (dict(nside=3), SHAPE), (dict(nside=0), SHAPE),
    (dict(block=8), SHAPE), (dict(block=32), SHAPE), (dict(block=256), SHAPE),   # 256 > nside^2 = 64
    (dict(topn=0), SHAPE), (dict(topn=49), SHAPE), (dict(window=0), SHAPE),
    (dict(d=48), UNSUP), (dict(d=128), UNSUP), (dict(nside=16384), UNSUP),
    (dict(nside=4096, block=1, heads=1), UNSUP),    # 2^26 queries: too many for the one-wave-per-query kernel
    (dict(nside=4096, block=16, heads=85), UNSUP),  # batch*heads*N >= 2^31
    # valid shapes that only the too-small workspace stops (blocks of 1 and 4, top-n above 64)
    (dict(block=4), WS), (dict(block=1), WS), (dict(nside=16, block=16, topn=65), WS), (dict(topn=48), WS),
    (dict(ws_bytes=100), WS),
])
def test_forward_validation(kw, code):
    # the default workspace (16 bytes) is too small for every shape: a case
    # that validation let through would stop there, not launch
    assert fwd(**kw) == code
    assert _lib.lib().mosaic_last_error().decode() != ""


def test_stage_entry_points_validate():
    L = _lib.lib()
    pool = lambda *a: L.mosaic_bsa_pool(FAKE, FAKE, *a, None)
    assert pool(None, 1, 2, 32, 8, 16, FAKE, FAKE, FAKE, None, None, None) == NULL
    assert pool(FAKE, 1, 2, 32, 8, 12, FAKE, FAKE, FAKE, None, None, None) == SHAPE
    assert pool(FAKE, 1, 2, 32, 8, 16, FAKE + 8, FAKE, FAKE, None, None, None) == MISAL
    assert pool(FAKE, 1, 2, 32, 8, 16, FAKE, FAKE, FAKE, FAKE + 2, None, None) == MISAL
    assert pool(FAKE, 1, 2, 32, 8, 16, FAKE, FAKE, FAKE, None, FAKE + 8, FAKE) == MISAL     # kpieces
    assert pool(FAKE, 1, 2, 32, 8, 16, FAKE, FAKE, FAKE, None, FAKE, FAKE + 2) == MISAL     # kbn2
    assert pool(FAKE, 1, 2, 32, 8, 16, FAKE, FAKE, FAKE, None, FAKE, None) == NULL          # pieces alone
    assert pool(FAKE, 1, 2, 32, 8, 16, FAKE, FAKE, FAKE, None, None, FAKE) == NULL          # norms alone
    cs = lambda *a: L.mosaic_bsa_compress_select(FAKE, FAKE, FAKE, *a, None)
    assert cs(1, 2, 32, 8, 16, 0, None, None, FAKE, FAKE) == SHAPE
    assert cs(1, 2, 32, 8, 16, 4, None, None, None, FAKE) == NULL
    assert cs(1, 2, 32, 8, 16, 4, FAKE, None, FAKE, FAKE) == NULL
    assert cs(1, 2, 32, 8, 16, 4, None, FAKE, FAKE, FAKE) == NULL
    assert cs(1, 2, 32, 8, 16, 4, FAKE + 8, FAKE, FAKE, FAKE) == MISAL
    fine = lambda *a: L.mosaic_bsa_fine(FAKE, FAKE, FAKE, FAKE, FAKE, *a, None)
    assert fine(FAKE, None, None, 1, 2, 32, 8, 16, 4, 0, FAKE) == SHAPE
    assert fine(None, None, None, 1, 2, 32, 8, 16, 4, 32, FAKE) == NULL
    assert fine(FAKE, None, None, 1, 2, 48, 8, 16, 4, 32, FAKE) == UNSUP
    assert fine(FAKE, FAKE + 2, None, 1, 2, 32, 8, 16, 4, 32, FAKE) == MISAL
    assert fine(FAKE, FAKE, FAKE + 2, 1, 2, 32, 8, 16, 4, 32, FAKE) == MISAL
    assert fine(FAKE, None, FAKE, 1, 2, 32, 8, 16, 4, 32, FAKE) == NULL          # a bound without knorm
    bound = lambda *a: L.mosaic_bsa_select_bound(*a, None)
    assert bound(FAKE, FAKE, 1, 2, 32, 8, 16, 0, FAKE) == SHAPE                   # topn 0
    assert bound(FAKE, FAKE, 1, 2, 32, 8, 16, 49, FAKE) == SHAPE                  # topn above m = 48
    assert bound(None, FAKE, 1, 2, 32, 8, 16, 4, FAKE) == NULL
    assert bound(FAKE, None, 1, 2, 32, 8, 16, 4, FAKE) == NULL
    assert bound(FAKE, FAKE, 1, 2, 32, 8, 16, 4, None) == NULL
    assert bound(FAKE, FAKE, 1, 2, 32, 8, 16, 4, FAKE + 2) == MISAL
    assert bound(FAKE, FAKE, 1, 2, 32, 12, 16, 4, FAKE) == SHAPE                  # nside not a power of two


def test_python_binding_rejects_bad_tensors_without_launch():
    import torch
    q = torch.zeros(1, 2, 768, 32, dtype=torch.float32)
    with pytest.raises((TypeError, ValueError)):
        _lib.mosaic_bsa_forward(q, q, q, torch.zeros(1, 2, 768, 3), 8, 16, 4, 32,
                                out=torch.zeros(1), sel_idx=torch.zeros(1), workspace=torch.zeros(1, dtype=torch.uint8))
    with pytest.raises(ValueError):
        _lib.mosaic_bsa_forward(q[:, :, :700], q, q, q, 8, 16, 4, 32)
    # the selection bound's tensors are checked against m = 12*nside^2/block (48 here), not
    # taken from their own shapes: a call that names nside 16 for nside-8 selections never launches
    sel = torch.zeros(1, 2, 48, 4, dtype=torch.int32)
    kn = torch.zeros(1, 2, 48)
    with pytest.raises(ValueError, match="shape"):
        _lib.mosaic_bsa_select_bound(sel, kn, 16, 16, 4, 32)
    with pytest.raises(ValueError, match="shape"):
        _lib.mosaic_bsa_select_bound(sel, kn, 8, 16, 8, 32)
    with pytest.raises(ValueError, match="device"):
        _lib.mosaic_bsa_select_bound(sel, kn, 8, 16, 4, 32)


def bwd(q=FAKE, k=FAKE, v=FAKE, gates=FAKE, sel=FAKE, dout=FAKE, batch=1, heads=2, d=64, nside=32, block=64,
        topn=16, window=256, saved=None, saved_bytes=0, dq=FAKE, dk=FAKE, dv=FAKE, dg=FAKE, ws=FAKE,
        ws_bytes=16):
    L = _lib.lib()
    return L.mosaic_bsa_backward(q, k, v, gates, sel, dout, batch, heads, d, nside, block, topn, window,
                                 saved, saved_bytes, dq, dk, dv, dg, ws, ws_bytes, None)


def fwd_train(q=FAKE, k=FAKE, v=FAKE, gates=FAKE, batch=1, heads=2, d=64, nside=32, block=64, topn=16,
              window=256, out=FAKE, sel=FAKE, saved=FAKE, saved_bytes=16):
    L = _lib.lib()
    return L.mosaic_bsa_forward_train(q, k, v, gates, batch, heads, d, nside, block, topn, window, out, sel,
                                      saved, saved_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(sel=None), NULL), (dict(dout=None), NULL), (dict(dq=None), NULL),
    (dict(dk=None), NULL), (dict(dv=None), NULL), (dict(dg=None), NULL), (dict(ws=None), NULL),
    (dict(dout=FAKE + 8), MISAL), (dict(dq=FAKE + 4), MISAL), (dict(sel=FAKE + 2), MISAL),
    (dict(ws=FAKE + 16), MISAL),
    (dict(batch=0), SHAPE), (dict(topn=0), SHAPE), (dict(window=0), SHAPE), (dict(block=32), SHAPE),
    (dict(block=16), UNSUP),                     # backward needs block >= 64
    (dict(topn=65), UNSUP),                      # and topn <= 64
    (dict(nside=16, block=64), UNSUP),           # m = 48, not a multiple of 64
    (dict(d=48), UNSUP),
    (dict(ws_bytes=1000), WS),
    (dict(saved=FAKE + 16, saved_bytes=1 << 40), MISAL),
    (dict(saved=FAKE, saved_bytes=1000, ws_bytes=1 << 40), WS),   # a saved state smaller than needed
])
def test_backward_validation(kw, code):
    assert bwd(**kw) == code
    assert _lib.lib().mosaic_last_error().decode() != ""


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(gates=None), NULL), (dict(out=None), NULL), (dict(sel=None), NULL),
    (dict(saved=None), NULL), (dict(saved=FAKE + 64), MISAL), (dict(out=FAKE + 4), MISAL),
    (dict(saved_bytes=4096), WS), (dict(window=0), SHAPE), (dict(topn=0), SHAPE), (dict(d=16), UNSUP),
])
def test_forward_train_validation(kw, code):
    assert fwd_train(**kw) == code
    assert _lib.lib().mosaic_last_error().decode() != ""


def test_saved_bytes():
    L = _lib.lib()
    b, h, d, nside, block = 1, 2, 64, 32, 64
    n, m, s = 12 * nside * nside, 12 * nside * nside // block, b * h
    got = L.mosaic_bsa_saved_bytes(b, h, d, nside, block)
    # float32 branch outputs + float32 log-sum-exps + the forward workspace, in 256-byte sections
    assert got >= s * n * 2 * d * 4 + s * n * 2 * 4 + L.mosaic_bsa_workspace_bytes(b, h, d, nside, block, 1)
    assert got < s * n * 2 * d * 4 + s * n * 2 * 4 + L.mosaic_bsa_workspace_bytes(b, h, d, nside, block, 1) + 1024
    assert L.mosaic_bsa_saved_bytes(b, h, d, nside, 32) == 0      # not a power of four
    assert L.mosaic_bsa_saved_bytes(b, h, 48, nside, block) == 0  # head_dim


def test_backward_workspace_bytes():
    L = _lib.lib()
    assert L.mosaic_bsa_backward_workspace_bytes(1, 2, 64, 32, 64, 16) > 0
    assert L.mosaic_bsa_backward_workspace_bytes(1, 2, 64, 32, 16, 16) == 0   # block < 64
    assert L.mosaic_bsa_backward_workspace_bytes(1, 2, 64, 16, 64, 16) == 0   # m = 48
    assert L.mosaic_bsa_backward_workspace_bytes(1, 1, 64, 256, 64, 16) > 0   # m = 12288
    assert L.mosaic_bsa_backward_workspace_bytes(1, 1, 64, 512, 64, 16) == 0  # m = 49152 > 16384
    # the largest section is the bf16 copy of dout plus the per-query statistics
    n, s = 12 * 32 * 32, 2
    assert L.mosaic_bsa_backward_workspace_bytes(1, 2, 64, 32, 64, 16) >= s * n * 64 * 2 + 2 * s * n * 12


def layer(x=FAKE, w_in=FAKE, w_out=FAKE, batch=1, heads=2, d=64, channels=128, nside=32, block=64, topn=16,
          window=256, y=FAKE + 4096, sel=FAKE, ws=FAKE, ws_bytes=16):
    L = _lib.lib()
    return L.mosaic_bsa_layer_forward(x, w_in, w_out, batch, heads, d, channels, nside, block, topn, window,
                                      y, sel, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), NULL), (dict(w_in=None), NULL), (dict(w_out=None), NULL), (dict(y=None), NULL),
    (dict(sel=None), NULL), (dict(ws=None), NULL),
    (dict(x=FAKE + 8), MISAL), (dict(w_in=FAKE + 2), MISAL), (dict(y=FAKE + 4), MISAL), (dict(ws=FAKE + 64), MISAL),
    (dict(channels=96), UNSUP), (dict(channels=32), UNSUP), (dict(channels=16384 + 64), UNSUP),
    (dict(heads=1, d=32), UNSUP),                # H*d = 32 is not a multiple of 64
    (dict(topn=0), SHAPE), (dict(window=0), SHAPE), (dict(block=32), SHAPE),
    (dict(ws_bytes=4096), WS),
    (dict(y=FAKE), SHAPE),                       # y aliases x
])
def test_layer_validation(kw, code):
    assert layer(**kw) == code
    assert _lib.lib().mosaic_last_error().decode() != ""


def test_layer_stage_validation():
    L = _lib.lib()
    assert L.mosaic_bsa_layer_in(None, FAKE, 1, 2, 64, 128, 32, FAKE, FAKE, FAKE, FAKE, None) == NULL
    assert L.mosaic_bsa_layer_in(FAKE, FAKE, 1, 2, 64, 100, 32, FAKE, FAKE, FAKE, FAKE, None) == UNSUP
    assert L.mosaic_bsa_layer_in(FAKE, FAKE, 1, 2, 64, 128, 32, FAKE + 8, FAKE, FAKE, FAKE, None) == MISAL
    assert L.mosaic_bsa_layer_in(FAKE, FAKE, 1, 2, 64, 128, 3, FAKE, FAKE, FAKE, FAKE, None) == SHAPE
    assert L.mosaic_bsa_layer_out(FAKE, FAKE, None, 1, 2, 64, 128, 32, FAKE, None) == NULL
    assert L.mosaic_bsa_layer_out(FAKE, FAKE, FAKE, 1, 2, 64, 128, 32, FAKE + 2, None) == MISAL
    assert L.mosaic_bsa_layer_out(FAKE, FAKE, FAKE, 1, 1, 32, 128, 32, FAKE, None) == UNSUP
    assert L.mosaic_bsa_layer_out_merged(None, FAKE, FAKE, 1, 2, 64, 128, 32, FAKE, None) == NULL
    assert L.mosaic_bsa_layer_out_merged(FAKE, FAKE, FAKE, 1, 2, 64, 128, 32, FAKE + 2, None) == MISAL
    assert L.mosaic_bsa_layer_out_merged(FAKE, FAKE, FAKE, 1, 1, 32, 128, 32, FAKE, None) == UNSUP
    assert L.mosaic_bsa_layer_out_merged(FAKE, FAKE, FAKE, 1, 2, 64, 128, 3, FAKE, None) == SHAPE


def test_layer_workspace_bytes():
    L = _lib.lib()
    b, h, d, c, nside, block, topn = 1, 2, 64, 128, 32, 64, 16
    n = 12 * nside * nside
    got = L.mosaic_bsa_layer_workspace_bytes(b, h, d, c, nside, block, topn)
    # q, k, v bf16 + gates + bf16 attention output + the forward workspace
    floor = 3 * b * h * n * d * 2 + b * h * n * 3 * 4 + b * h * n * d * 2 + \
        L.mosaic_bsa_workspace_bytes(b, h, d, nside, block, topn)
    assert floor <= got < floor + 8 * 256
    assert L.mosaic_bsa_layer_workspace_bytes(b, h, d, 100, nside, block, topn) == 0


def test_coarsen_validation():
    L = _lib.lib()
    f = L.mosaic_healpix_coarsen
    assert f(None, 1, 64, 32, 1, FAKE, None) == NULL
    assert f(FAKE, 1, 64, 32, 1, None, None) == NULL
    assert f(FAKE + 8, 1, 64, 32, 1, FAKE, None) == MISAL
    assert f(FAKE, 1, 64, 32, 1, FAKE + 4, None) == MISAL
    assert f(FAKE, 0, 64, 32, 1, FAKE, None) == SHAPE
    assert f(FAKE, 1, 64, 24, 1, FAKE, None) == SHAPE      # nside not a power of two
    assert f(FAKE, 1, 64, 32, 0, FAKE, None) == SHAPE      # levels < 1
    assert f(FAKE, 1, 64, 32, 6, FAKE, None) == SHAPE      # nside / 2^6 < 1
    assert f(FAKE, 1, 60, 32, 1, FAKE, None) == UNSUP      # channels not a multiple of 8
    assert _lib.lib().mosaic_last_error().decode() != ""


def test_interp_validation():
    L = _lib.lib()
    f = L.mosaic_interp_attention

    def call(k=FAKE, v=FAKE, w=FAKE, nbr=FAKE, rel=FAKE, s=2, n_src=1000, n_dst=500, K=16, d=64, dv=64,
             out=FAKE, ws=FAKE, ws_bytes=16):
        return f(k, v, w, nbr, rel, s, n_src, n_dst, K, d, dv, out, ws, ws_bytes, None)
    assert call(k=None) == NULL
    assert call(rel=None) == NULL
    assert call(ws=None) == NULL
    assert call(k=FAKE + 8) == MISAL
    assert call(out=FAKE + 4) == MISAL
    assert call(ws=FAKE + 128) == MISAL
    assert call(s=0) == SHAPE
    assert call(n_dst=0) == SHAPE
    assert call(K=0) == UNSUP
    assert call(K=17) == UNSUP
    assert call(d=60) == UNSUP
    assert call(dv=32) == UNSUP
    assert call(ws_bytes=100) == WS
    assert L.mosaic_interp_workspace_bytes(2, 1000) >= 2 * 1000 * 16
    assert L.mosaic_interp_workspace_bytes(0, 1000) == 0


def test_forward_noalloc_validation():
    L = _lib.lib()

    def call(q=FAKE, gates=FAKE, batch=1, heads=2, d=32, nside=8, block=16, topn=4, window=32, out=FAKE, sel=FAKE):
        return L.mosaic_bsa_forward_noalloc(q, FAKE, FAKE, gates, batch, heads, d, nside, block, topn, window,
                                            out, sel, None)
    assert call(q=None) == NULL
    assert call(sel=None) == NULL
    assert call(out=FAKE + 4) == MISAL
    assert call(gates=FAKE + 2) == MISAL
    assert call(topn=0) == SHAPE
    assert call(block=8) == SHAPE
    assert call(d=48) == UNSUP
    # a valid shape whose workspace exceeds the 256 MiB static scratch: rejected before any HIP call
    # (batch 24 x 8 heads at nside 128 needs 1.06 GB)
    assert call(batch=24, heads=8, d=64, nside=128, block=64, topn=16, window=512) == UNSUP
    assert "static scratch" in L.mosaic_last_error().decode()
    assert L.mosaic_bsa_workspace_bytes(24, 8, 64, 128, 64, 16) > 256 << 20
    assert L.mosaic_bsa_workspace_bytes(2, 16, 64, 256, 256, 8) <= 256 << 20
