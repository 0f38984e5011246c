"""Host-side tests of the C ABI (no GPU needed, no kernel is launched).

- the built library loads and exports every function include/qlora.h declares;
- the compiled-in NF4 table equals the oracle's table bit for bit;
- status strings, workspace queries and argument validation (errors are
  returned before anything is enqueued).
"""
import ctypes
import os
import re

import numpy as np
import pytest

from qlora_fine_tuning_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlora.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qlora_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        from qlora_fine_tuning_amd import build
        build.build(verbose=False)
    return _lib.lib()


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert len(names) >= 11
    for n in names:
        assert hasattr(L, n), n
    assert sorted(_lib.EXPORTED) == names


def test_nf4_table_matches_oracle(L):
    from oracle import nf4
    buf = (ctypes.c_float * 16)()
    L.qlora_nf4_levels(buf)
    got = np.array(list(buf), dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), nf4.nf4_levels().view(np.uint32))


def test_status_strings_and_version(L):
    for code in (0, -1, -2, -3, -4, -5):
        assert L.qlora_status_string(code)
    assert L.qlora_status_string(12345) == b"unknown status"
    assert b"gfx950" in L.qlora_version()


def test_workspace_queries(L):
    for mode in (0, 1, 2):
        assert L.qlora_linear_workspace_bytes(8192, 4096, 4096, 16, mode) > 0
        assert L.qlora_mlp_workspace_bytes(8192, 4096, 11008, 16, mode) > 0
    # invalid shapes / ranks / modes give 0
    assert L.qlora_linear_workspace_bytes(8, 100, 64, 16, 0) == 0
    assert L.qlora_linear_workspace_bytes(8, 64, 64, 0, 0) == 0
    assert L.qlora_linear_workspace_bytes(8, 64, 64, 65, 0) == 0
    assert L.qlora_linear_workspace_bytes(8, 64, 64, 8, 7) == 0
    assert L.qlora_mlp_workspace_bytes(8, 64, 64, 65, 0) == 0
    assert L.qlora_mlp_workspace_bytes(8, 64, 64, 64, 0) > 0
    # staged keeps a bf16 copy of the weight, fused does not
    assert L.qlora_mlp_workspace_bytes(8192, 4096, 11008, 16, 2) >= L.qlora_mlp_workspace_bytes(
        8192, 4096, 11008, 16, 1)


def test_gemm_split_count(L):
    """K splits: none at 256 or more output tiles or below 16 k-steps of 64; otherwise
    enough ranges to reach about 256 tiles, each at least 8 k-steps, at most 8."""
    f = L.qlora_gemm_split_count
    assert f(8192, 4096, 11008) == 1        # 512 tiles
    assert f(4096, 4096, 4096) == 1         # exactly 256 tiles
    assert f(8192, 1024, 4096) == 2         # 128 tiles
    assert f(1024, 4096, 11008) == 4        # 64 tiles
    assert f(1024, 4096, 22016) == 4
    assert f(129, 1024, 4160) == 8          # 4 tiles, capped at 8
    assert f(300, 320, 2368) == 4           # 37 k-steps: 8 per split at most 4 ranges
    assert f(300, 2368, 960) == 1           # 15 k-steps
    assert f(1, 64, 1536) == 3
    assert f(0, 64, 4096) == 1
    assert f(-1, 64, 64) == -1
    # the fp32 partials are part of the workspace: the staged linear (which
    # splits) needs at least 2 x m x n x 4 bytes more than the fused one
    assert L.qlora_linear_workspace_bytes(129, 4160, 1024, 8, 2) - L.qlora_linear_workspace_bytes(
        129, 4160, 1024, 8, 1) >= 2 * 129 * 1024 * 4


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


def _nf4(n, k, ok=True):
    return _lib.Nf4(0x1000 if ok else 0, 0x2000 if ok else 0, n, k)


def test_linear_validation_errors(L):
    ws = ctypes.c_void_p(0x100000)
    big = 1 << 40
    f = L.qlora_linear_fwd
    # null pointer
    assert f(None, 8, _nf4(64, 64), FAKE, FAKE, 8, 1.0, FAKE, None, 0, ws, big, None) == -1
    assert f(FAKE, 8, _nf4(64, 64, ok=False), FAKE, FAKE, 8, 1.0, FAKE, None, 0, ws, big, None) == -1
    # rank / scale / mode
    assert f(FAKE, 8, _nf4(64, 64), FAKE, FAKE, 0, 1.0, FAKE, None, 0, ws, big, None) == -1
    assert f(FAKE, 8, _nf4(64, 64), FAKE, FAKE, 65, 1.0, FAKE, None, 0, ws, big, None) == -1
    assert f(FAKE, 8, _nf4(64, 64), FAKE, FAKE, 8, float("nan"), FAKE, None, 0, ws, big, None) == -1
    assert f(FAKE, 8, _nf4(64, 64), FAKE, FAKE, 8, 1.0, FAKE, None, 9, ws, big, None) == -1
    # shapes: k, n multiples of 64; m >= 0
    assert f(FAKE, 8, _nf4(64, 96), FAKE, FAKE, 8, 1.0, FAKE, None, 0, ws, big, None) == -2
    assert f(FAKE, 8, _nf4(100, 64), FAKE, FAKE, 8, 1.0, FAKE, None, 0, ws, big, None) == -2
    assert f(FAKE, -1, _nf4(64, 64), FAKE, FAKE, 8, 1.0, FAKE, None, 0, ws, big, None) == -2
    # workspace missing / too small / misaligned
    assert f(FAKE, 8, _nf4(64, 64), FAKE, FAKE, 8, 1.0, FAKE, None, 0, None, 0, None) == -3
    assert f(FAKE, 8, _nf4(64, 64), FAKE, FAKE, 8, 1.0, FAKE, None, 0, ws, 16, None) == -3
    assert f(FAKE, 8, _nf4(64, 64), FAKE, FAKE, 8, 1.0, FAKE, None, 0, ctypes.c_void_p(0x100010),
             big, None) == -3
    # m == 0 is a no-op that succeeds without touching memory
    assert f(FAKE, 0, _nf4(64, 64), FAKE, FAKE, 8, 1.0, FAKE, None, 0, ws, big, None) == 0
    b = L.qlora_linear_bwd
    assert b(FAKE, FAKE, None, 8, _nf4(64, 64), FAKE, FAKE, 8, 1.0, None, FAKE, FAKE, 0, ws, big,
             None) == -1
    assert b(FAKE, FAKE, FAKE, 8, _nf4(64, 64), FAKE, FAKE, 8, 1.0, None, FAKE, FAKE, 0, None, 0,
             None) == -3


def test_mlp_validation_errors(L):
    ws = ctypes.c_void_p(0x100000)
    big = 1 << 40
    w = _lib.MlpWeights(_nf4(128, 64), _nf4(128, 64), _nf4(64, 128), *([0x3000] * 6), 64, 128, 8,
                        1.0, 0)
    f = L.qlora_mlp_fwd
    args = lambda ww: (FAKE, 8, ctypes.byref(ww), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, ws, big, None)  # noqa: E731
    bad = _lib.MlpWeights.from_buffer_copy(w)
    bad.act = 5
    assert f(*args(bad)) == -1
    bad = _lib.MlpWeights.from_buffer_copy(w)
    bad.r = 65
    assert f(*args(bad)) == -1
    bad = _lib.MlpWeights.from_buffer_copy(w)
    bad.down = _nf4(64, 64)          # down must be [d][h]
    assert f(*args(bad)) == -2
    bad = _lib.MlpWeights.from_buffer_copy(w)
    bad.b_up = 0
    assert f(*args(bad)) == -1
    assert f(FAKE, 0, ctypes.byref(w), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, ws, big, None) == 0
    assert f(FAKE, 8, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, ws, big, None) == -1
    # misaligned: a bf16 matrix off its 16-byte grid, an fp32 U off 4 bytes,
    # NF4 codes off 16 or absmax off 4 bytes, a LoRA factor off 16 bytes
    odd8, odd2 = ctypes.c_void_p(0x1008), ctypes.c_void_p(0x1002)
    assert f(odd8, 8, ctypes.byref(w), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, ws, big, None) == -2
    assert f(FAKE, 8, ctypes.byref(w), FAKE, odd8, FAKE, FAKE, FAKE, FAKE, 0, ws, big, None) == -2
    assert f(FAKE, 8, ctypes.byref(w), FAKE, FAKE, FAKE, FAKE, odd2, FAKE, 0, ws, big, None) == -2
    for field, val in (("gate", _lib.Nf4(0x1008, 0x2000, 128, 64)), ("down", _lib.Nf4(0x1000, 0x2002, 64, 128)),
                       ("a_up", 0x3008)):
        bad = _lib.MlpWeights.from_buffer_copy(w)
        setattr(bad, field, val)
        assert f(*args(bad)) == -2, field


def test_alignment_errors_linear_and_dequant(L):
    ws = ctypes.c_void_p(0x100000)
    big = 1 << 40
    odd8, odd2 = ctypes.c_void_p(0x1008), ctypes.c_void_p(0x1002)
    f = L.qlora_linear_fwd
    ok = (FAKE, 8, _nf4(64, 64), FAKE, FAKE, 8, 1.0, FAKE, FAKE, 0, ws, big, None)
    for i, bad in ((0, odd8), (3, odd8), (4, odd8), (7, odd8), (8, odd2)):
        a = list(ok)
        a[i] = bad
        assert f(*a) == -2, i
    a = list(ok)
    a[2] = _lib.Nf4(0x1008, 0x2000, 64, 64)
    assert f(*a) == -2
    b = L.qlora_linear_bwd
    okb = (FAKE, FAKE, FAKE, 8, _nf4(64, 64), FAKE, FAKE, 8, 1.0, FAKE, FAKE, FAKE, 0, ws, big, None)
    for i, bad in ((0, odd8), (1, odd8), (2, odd2), (9, odd8), (10, ctypes.c_void_p(0x1001)),
                   (11, ctypes.c_void_p(0x1001))):
        a = list(okb)
        a[i] = bad
        assert b(*a) == -2, i
    assert L.qlora_nf4_dequant(_lib.Nf4(0x1008, 0x2000, 64, 64), FAKE, None) == -2
    assert L.qlora_nf4_dequant(_lib.Nf4(0x1000, 0x2002, 64, 64), FAKE, None) == -2
    assert L.qlora_nf4_dequant(_nf4(64, 64), odd8, None) == -2


def test_probe_validation_errors(L):
    d = ctypes.c_double(0)
    assert L.qlora_probe_mfma_peak(100, None, ctypes.byref(d), None) == -1
    assert L.qlora_probe_mfma_peak(100, ctypes.byref(d), None, None) == -1
    assert L.qlora_probe_mfma_peak(0, ctypes.byref(d), ctypes.byref(d), None) == -1


def test_w16_validation_errors(L):
    FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first
    ws = L.qlora_linear16_workspace_bytes(64, 128, 192, 8)
    assert ws > 0
    assert L.qlora_linear16_workspace_bytes(64, 100, 192, 8) == 0        # k not a multiple of 64
    assert L.qlora_linear16_workspace_bytes(64, 128, 192, 65) == 0       # r > 64
    # null weight
    assert L.qlora_linear16_fwd(FAKE, 64, None, 192, 128, FAKE, FAKE, 8, ctypes.c_float(1.0),
                                FAKE, FAKE, FAKE, ws, None) == -1
    # bad shape
    assert L.qlora_linear16_fwd(FAKE, 64, FAKE, 192, 100, FAKE, FAKE, 8, ctypes.c_float(1.0),
                                FAKE, FAKE, FAKE, ws, None) == -2
    # workspace too small
    assert L.qlora_linear16_fwd(FAKE, 64, FAKE, 192, 128, FAKE, FAKE, 8, ctypes.c_float(1.0),
                                FAKE, FAKE, FAKE, 256, None) == -3
    assert L.qlora_mlp16_workspace_bytes(64, 128, 192, 8) > 0
    assert L.qlora_mlp16_workspace_bytes(64, 128, 192, 64) > 0
    assert L.qlora_mlp16_workspace_bytes(64, 128, 192, 65) == 0          # MLP rank limit
    w = _lib.Mlp16Weights(None, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000,
                          128, 192, 8, 1.0, 0)
    assert L.qlora_mlp16_fwd(FAKE, 64, ctypes.byref(w), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                             FAKE, 1 << 30, None) == -1
    w.gate = 0x1000
    w.act = 7
    assert L.qlora_mlp16_fwd(FAKE, 64, ctypes.byref(w), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                             FAKE, 1 << 30, None) == -1


def test_quantize_validation_errors(L):
    FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first
    assert L.qlora_nf4_quantize(None, 4, 64, FAKE, FAKE, None) == -1      # null weights
    assert L.qlora_nf4_quantize(FAKE, 4, 64, FAKE, None, None) == -1      # null absmax
    assert L.qlora_nf4_quantize(FAKE, 4, 96, FAKE, FAKE, None) == -2      # k % 64 != 0
    assert L.qlora_nf4_quantize(FAKE, -1, 64, FAKE, FAKE, None) == -2     # negative rows
    assert L.qlora_nf4_quantize(None, 0, 64, None, None, None) == 0       # empty: no work
    assert L.qlora_nf4_quantize(ctypes.c_void_p(0x1008), 4, 64, FAKE, FAKE, None) == -2   # misaligned


def test_absmax_dq_validation_errors(L):
    FAKE = ctypes.c_void_p(0x1000)
    odd = ctypes.c_void_p(0x1002)
    q = L.qlora_absmax_dq_quantize
    assert q(None, 0, None, None, None, None) == 0                         # empty: no work
    assert q(FAKE, -1, FAKE, FAKE, FAKE, None) == -2
    assert q(None, 10, FAKE, FAKE, FAKE, None) == -1
    assert q(FAKE, 10, FAKE, None, FAKE, None) == -1
    assert q(odd, 10, FAKE, FAKE, FAKE, None) == -2
    dq = L.qlora_absmax_dq_dequant
    assert dq(None, None, None, 0, None, None) == 0
    assert dq(FAKE, FAKE, FAKE, -5, FAKE, None) == -2
    assert dq(FAKE, FAKE, None, 10, FAKE, None) == -1
    assert dq(FAKE, FAKE, FAKE, 10, odd, None) == -2
    # a weight with neither fp32 absmax nor the double-quantized triple is rejected
    w = _lib.Nf4(0x1000, None, 64, 64, 0x3000, None, 0x3000)
    assert L.qlora_nf4_dequant(w, FAKE, None) == -1
    w = _lib.Nf4(0x1000, None, 64, 64, 0x3001, 0x3000, 0x3002)            # offset off 4 bytes
    assert L.qlora_nf4_dequant(w, FAKE, None) == -2


def test_qkv_validation_errors(L):
    FAKE = 0x1000   # never dereferenced: validation fails first
    F = ctypes.c_void_p(FAKE)
    assert L.qlora_qkv_workspace_bytes(64, 128, 128, 64, 64, 16) > 0
    assert L.qlora_qkv_workspace_bytes(64, 128, 128, 64, 100, 16) == 0   # n_v % 64
    assert L.qlora_qkv_workspace_bytes(64, 128, 128, 64, 64, 65) == 0    # r > 64
    nf = lambda n, k: _lib.Nf4(FAKE, FAKE, n, k)  # noqa: E731
    w = _lib.QkvWeights(nf(128, 128), nf(64, 128), nf(64, 128), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                        8, 1.0)
    ws = L.qlora_qkv_workspace_bytes(64, 128, 128, 64, 64, 8)
    args = lambda ldq=128, ldk=64, ldv=64, q=F, wsb=ws: (  # noqa: E731
        F, 64, ctypes.byref(w), q, ldq, F, ldk, F, ldv, F, F, wsb, None)
    assert L.qlora_qkv_fwd(*args(ldq=120)) == -2                # pitch below the width
    assert L.qlora_qkv_fwd(*args(ldq=132)) == -2                # pitch not a multiple of 8
    assert L.qlora_qkv_fwd(*args(q=ctypes.c_void_p(FAKE + 8))) == -2   # misaligned rows
    assert L.qlora_qkv_fwd(*args(wsb=256)) == -3                # workspace too small
    w.v = nf(64, 192)                                           # d mismatch
    assert L.qlora_qkv_fwd(*args()) == -2
    w.v = nf(64, 128)
    w.r = 0
    assert L.qlora_qkv_fwd(*args()) == -1
    w.r = 8
    w.b_k = None
    assert L.qlora_qkv_fwd(*args()) == -1
    w.b_k = FAKE
    g = _lib.QkvGrads(FAKE, FAKE, FAKE, None, FAKE, FAKE)
    assert L.qlora_qkv_bwd(F, 128, F, 64, F, 64, F, F, 64, ctypes.byref(w), F, ctypes.byref(g),
                           F, ws, None) == -1                   # null gradient
    w16 = _lib.Qkv16Weights(FAKE, None, FAKE, 128, 128, 64, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                            8, 1.0)
    assert L.qlora_qkv16_fwd(*(lambda a: (a[0], a[1], ctypes.byref(w16)) + a[3:])(args())) == -1


def test_norm_rope_xent_validation_errors(L):
    F_ = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first
    f = ctypes.c_float
    assert L.qlora_rmsnorm_fwd(F_, 4, 100, F_, f(1e-6), 0, F_, F_, None) == -2      # d % 8
    assert L.qlora_rmsnorm_fwd(F_, 4, 64, None, f(1e-6), 0, F_, F_, None) == -1     # no weight
    assert L.qlora_rmsnorm_fwd(F_, 4, 64, F_, f(-1.0), 0, F_, F_, None) == -1       # eps < 0
    assert L.qlora_rmsnorm_fwd(F_, 4, 64, F_, f(1e-6), 2, F_, F_, None) == -1       # flag
    assert L.qlora_rmsnorm_fwd(None, 0, 64, F_, f(1e-6), 0, None, None, None) == 0  # empty
    assert L.qlora_rmsnorm_bwd(F_, F_, None, 4, 64, F_, 0, F_, None) == -1          # no rstd
    assert L.qlora_rope_fwd(F_, 256, 4, 2, 24, F_, f(1e4), F_, 256, None) == -2     # hd % 16
    assert L.qlora_rope_fwd(F_, 256, 4, 2, 512, F_, f(1e4), F_, 1024, None) == -2   # hd > 256
    assert L.qlora_rope_fwd(F_, 200, 4, 2, 128, F_, f(1e4), F_, 256, None) == -2    # pitch < width
    assert L.qlora_rope_fwd(F_, 256, 4, 2, 128, F_, f(0.0), F_, 256, None) == -1    # base
    assert L.qlora_rope_fwd(F_, 256, 4, 2, 128, F_, f(1e4), F_, 264, None) == -1    # in place, pitches differ
    assert L.qlora_rope_bwd(F_, 256, 4, 2, 128, None, f(1e4), F_, 256, None) == -1  # no positions
    assert L.qlora_cross_entropy_fwd(F_, 100, 4, 100, F_, F_, F_, F_, F_, None) == -2   # pitch % 8
    assert L.qlora_cross_entropy_fwd(F_, 96, 4, 100, F_, F_, F_, F_, F_, None) == -2    # pitch < V
    assert L.qlora_cross_entropy_fwd(F_, 104, 4, 100, F_, F_, F_, None, F_, None) == -1  # no loss
    assert L.qlora_cross_entropy_bwd(F_, 104, 4, 100, F_, F_, None, None, F_, 104, None) == -1
    assert L.qlora_cross_entropy_bwd(F_, 104, 4, 100, F_, F_, None, F_, F_, 112, None) == -1  # in place
    assert L.qlora_cross_entropy_fused(F_, 104, 4, 100, F_, f(1.0), F_, F_, None, F_, F_, 104, None) == -1
    assert L.qlora_cross_entropy_fused(F_, 104, 4, 100, F_, f(float("nan")), F_, F_, F_, F_, F_, 104,
                                       None) == -1
    assert L.qlora_cross_entropy_fused(F_, 104, 4, 100, F_, f(1.0), F_, F_, F_, F_, F_, 100, None) == -2


_NODEV_SCRIPT = r"""
import ctypes, sys
hip = ctypes.CDLL("libamdhip64.so")
n = ctypes.c_int(0)
hip.hipGetDeviceCount(ctypes.byref(n))
if n.value > 0:
    print("SKIP device visible")
    sys.exit(0)
from qlora_fine_tuning_amd import _lib
L = _lib.lib()
FAKE = ctypes.c_void_p(0x1000)
ws = ctypes.c_void_p(0x100000)
nf = lambda n, k: _lib.Nf4(0x1000, 0x2000, n, k)
out = []
out.append(L.qlora_nf4_dequant(nf(64, 64), FAKE, None))
out.append(L.qlora_linear_fwd(FAKE, 8, nf(64, 64), FAKE, FAKE, 8, 1.0, FAKE, FAKE, 0, ws, 1 << 40, None))
w = _lib.MlpWeights(nf(128, 64), nf(128, 64), nf(64, 128), *([0x3000] * 6), 64, 128, 8, 1.0, 0)
out.append(L.qlora_mlp_fwd(FAKE, 8, ctypes.byref(w), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, ws, 1 << 40, None))
print("RC", *out)
print("MSG", L.qlora_last_error().decode())
"""


def test_no_device_returns_ehip():
    """With no GPU visible, a compute call fails at its first HIP call and
    returns QLORA_EHIP with the failing step and HIP's message in
    qlora_last_error (nothing is dereferenced: the pointers are never used).
    Runs in a child process with every device hidden; it checks the device
    count itself and skips the calls if one is still visible."""
    import subprocess
    import sys
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", PYTHONPATH=ROOT)
    res = subprocess.run([sys.executable, "-c", _NODEV_SCRIPT], env=env, capture_output=True,
                         text=True, timeout=300)
    assert res.returncode == 0, res.stderr
    if "SKIP" in res.stdout:
        pytest.skip("a device is still visible")
    rc = [ln for ln in res.stdout.splitlines() if ln.startswith("RC")][0].split()[1:]
    assert rc == ["-4", "-4", "-4"]
    msg = [ln for ln in res.stdout.splitlines() if ln.startswith("MSG")][0]
    assert "mlp_fwd" in msg and "device" in msg
