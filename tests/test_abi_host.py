"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/moe_fp4.h declares, and rejects invalid arguments with
the documented status codes before launching anything. No call here passes
validation, so nothing is ever enqueued."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "moe_fp4.h")).read()
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def moe():
    import block_scaled_fp4_top_amd as m
    return m


def test_exports_every_declared_symbol(moe):
    lib = ctypes.CDLL(moe.lib_path())
    names = _declared()
    assert "moe_forward" in names and "moe_prepare_weights" in names and "moe_finalize" in names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(moe.EXPORTS)


def _dims(moe, E=8, H=256, I=128, act="swiglu", wfmt="nvfp4"):
    return moe._Dims(E, H, I, moe.ACTS[act], moe.WFMTS[wfmt])


FAKE = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: validation fails first


def test_sizes_and_dims_validation(moe):
    L = moe._lib
    assert L.moe_prepared_bytes(ctypes.byref(_dims(moe))) > 0
    assert L.moe_prepared_bytes(ctypes.byref(_dims(moe, H=200))) == 0
    assert "multiples of 128" in L.moe_last_error().decode()
    assert L.moe_prepared_bytes(ctypes.byref(_dims(moe, E=0))) == 0
    assert L.moe_prepared_bytes(ctypes.byref(_dims(moe, E=2000))) == 0
    assert L.moe_workspace_bytes(ctypes.byref(_dims(moe)), 16, 2, 0) > 0
    assert L.moe_workspace_bytes(ctypes.byref(_dims(moe)), 16, 9, 0) == 0      # K > E
    assert L.moe_workspace_bytes(ctypes.byref(_dims(moe)), 0, 2, 0) == 0       # T = 0
    assert L.moe_workspace_bytes(ctypes.byref(_dims(moe)), 16, 2, 3) == 0      # MXFP8 on NVFP4
    assert L.moe_workspace_bytes(ctypes.byref(_dims(moe, wfmt="mxfp8")), 16, 2, 3) > 0


def test_workspace_grows_with_tokens(moe):
    L = moe._lib
    d = ctypes.byref(_dims(moe, E=64, H=2048, I=1024))
    a = L.moe_workspace_bytes(d, 16, 6, 2)
    b = L.moe_workspace_bytes(d, 256, 6, 2)
    assert 0 < a < b


def _fwd(moe, d, prepared=FAKE, pb=1 << 40, x=FAKE, logits=FAKE, T=16, K=2, mode=0, act=0, oni=0,
         det=1, ws=FAKE, wsb=1 << 40, y=FAKE):
    return moe._lib.moe_forward(ctypes.byref(d), prepared, pb, x, logits, T, K, mode, act, oni,
                                det, ws, wsb, y, None)


def test_forward_rejects_before_launch(moe):
    d = _dims(moe)
    assert _fwd(moe, d, prepared=None) == 1
    assert _fwd(moe, d, x=None) == 1
    assert _fwd(moe, d, y=None) == 1
    assert _fwd(moe, d, mode=3) == 1                       # blob format/mode mismatch
    assert _fwd(moe, d, act=1) == 1                        # act differs from prepared
    assert _fwd(moe, d, K=9) == 1
    assert _fwd(moe, d, T=0) == 1
    assert _fwd(moe, d, oni=2) == 1
    assert _fwd(moe, d, det=5) == 1
    assert _fwd(moe, d, x=ctypes.c_void_p((1 << 20) + 2)) == 1   # misaligned
    assert _fwd(moe, d, ws=ctypes.c_void_p((1 << 20) + 16)) == 1  # workspace not 256-aligned
    assert _fwd(moe, d, wsb=1024) == 3                     # MOE_ERR_WORKSPACE
    assert "workspace" in moe._lib.moe_last_error().decode()
    # a prepared blob smaller than these dimensions need (e.g. prepared for a
    # smaller layer) is refused before anything could read past its end
    need = moe._lib.moe_prepared_bytes(ctypes.byref(d))
    assert _fwd(moe, d, pb=need - 1) == 3
    assert "prepared blob" in moe._lib.moe_last_error().decode()
    assert moe._lib.moe_forward_status(None, ctypes.byref(ctypes.c_int32()), None) == 1
    assert _fwd(moe, _dims(moe, H=200)) == 2               # MOE_ERR_UNSUPPORTED
    big = _dims(moe, E=64, H=8192, I=2048)
    assert _fwd(moe, big, T=1 << 15, K=8) == 2              # activations of 4 GiB or more
    assert "4 GiB" in moe._lib.moe_last_error().decode()


def test_finalize_and_quantize_reject(moe):
    L = moe._lib
    assert L.moe_finalize(None, 0, FAKE, None, 4, 2, 256, FAKE, None) == 1
    assert L.moe_finalize(FAKE, 0, FAKE, None, 4, 65, 256, FAKE, None) == 1   # K > 64
    assert L.moe_finalize(FAKE, 0, FAKE, None, 4, 2, 250, FAKE, None) == 2    # H % 4
    assert L.moe_finalize(FAKE, 3, FAKE, None, 4, 2, 256, FAKE, None) == 1
    assert L.moe_quantize(FAKE, 4, 48, 0, FAKE, FAKE, FAKE, FAKE, None) == 2  # cols % 32
    assert L.moe_quantize(FAKE, 4, 64, 7, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert L.moe_quantize(FAKE, 4, 64, 0, FAKE, FAKE, None, FAKE, None) == 1  # g missing


def test_prepare_rejects(moe):
    L = moe._lib
    d = _dims(moe)
    n = L.moe_prepared_bytes(ctypes.byref(d))
    assert L.moe_prepare_weights(ctypes.byref(d), None, FAKE, FAKE, n, None) == 1
    assert L.moe_prepare_weights(ctypes.byref(d), FAKE, FAKE, ctypes.c_void_p((1 << 20) + 64), n, None) == 1
    assert L.moe_prepare_weights(ctypes.byref(d), FAKE, FAKE, FAKE, n - 1, None) == 3


def test_workspace_views(moe):
    L = moe._lib
    d = _dims(moe)
    off, nb = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.moe_workspace_view(ctypes.byref(d), 16, 2, 0, 0, ctypes.byref(off), ctypes.byref(nb)) == 0
    assert nb.value == 16 * 2 * 4
    # W4A16 produces no FC1-input codes
    assert L.moe_workspace_view(ctypes.byref(d), 16, 2, 2, 6, ctypes.byref(off), ctypes.byref(nb)) == 1
    assert L.moe_workspace_view(ctypes.byref(d), 16, 2, 0, 99, ctypes.byref(off), ctypes.byref(nb)) == 1


@pytest.mark.parametrize("E,K", [(64, 6), (256, 8), (8, 2)])
def test_workspace_never_shrinks_as_tokens_grow(moe, E, K):
    """moe_workspace_bytes(T_max) must cover every forward with T <= T_max,
    also across the small-batch permutation threshold (4096 routes)."""
    L = moe._lib
    d = ctypes.byref(_dims(moe, E=E, H=512, I=256))
    prev = 0
    for T in list(range(1, 40)) + list(range(4096 // K - 20, 4096 // K + 20)):
        b = L.moe_workspace_bytes(d, T, K, moe.MODES["w4a16"])
        assert b >= prev, (T, b, prev)
        prev = b


@pytest.mark.parametrize("unit,S", [(1, 64), (4, 128)])
def test_weight_scale_layout_round_trip(unit, S):
    """The test unpackers' view of the stored weight-scale layout: byte b of
    unit u of strip nt at K step kt lives at ((nt // 4) * KT + kt) * 4 S +
    u * 4 unit + (nt % 4) * unit + b (group of four strips per step, the
    strips' units side by side); tile_scales restores micro-tile order."""
    from tests.helpers import tile_scales
    import numpy as np
    NT, KT = 8, 3
    tiles = np.arange(NT * KT * S, dtype=np.int64).reshape(NT, KT, S) % 251
    stored = np.zeros(NT * KT * S, np.int64)
    for nt in range(NT):
        for kt in range(KT):
            for u in range(S // unit):
                for b in range(unit):
                    off = ((nt // 4) * KT + kt) * 4 * S + u * 4 * unit + (nt % 4) * unit + b
                    stored[off] = tiles[nt, kt, u * unit + b]
    assert np.array_equal(tile_scales(stored, NT, KT, unit).reshape(NT, KT, S), tiles)
