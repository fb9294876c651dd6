"""The C-ABI boundary, without a GPU: the library loads, exports every entry
point its header declares, and rejects bad arguments before launching
anything (status codes, never an abort).  Also checks that the product
package does not reach the oracle."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qvae.h")
PKG = os.path.join(ROOT, "w8a8_int8_quantized_act_amd")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qvae_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    from w8a8_int8_quantized_act_amd import ops
    if not os.path.exists(ops.LIB_PATH):
        from w8a8_int8_quantized_act_amd import build
        build.build()
    return ops.lib()


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ["qvae_quantize_weights", "qvae_act_absmax", "qvae_act_quantize", "qvae_act_absmax_quant",
              "qvae_causalconv3d_w8a8", "qvae_causalconv3d_w8a8_absmax", "qvae_causalconv3d_w8a8_acc32",
              "qvae_select_layer", "qvae_pack_weights_bf16", "qvae_causalconv3d_bf16",
              "qvae_rmsnorm_silu", "qvae_rmsnorm_silu_absmax", "qvae_causalconv3d_w8a8_qin",
              "qvae_strerror", "qvae_version", "qvae_init"]:
        assert n in names
    assert "qvae_probe_mfma" not in names          # measurement tooling is not part of the library


def test_library_exports_every_declared_symbol(L):
    from w8a8_int8_quantized_act_amd import ops
    out = subprocess.run(["nm", "-D", "--defined-only", ops.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    missing = [n for n in _declared() if n not in exported]
    assert not missing, missing
    for n in _declared():
        getattr(L, n)


def test_version_and_strerror(L):
    assert L.qvae_version() >= 1
    for st in [0, -1, -2, -3, -4, 17]:
        assert isinstance(L.qvae_strerror(st), bytes) and L.qvae_strerror(st)


FAKE = ctypes.c_void_p(0x10000)        # aligned, never dereferenced: validation fails first
FAKE_MIS = ctypes.c_void_p(0x10008)    # misaligned


def conv(L, xq=FAKE, xs=FAKE, cache=None, wq=FAKE, ws=FAKE, b=None, dims=(1, 1, 4, 4, 32, 32, 3, 3, 3),
         y=FAKE):
    return L.qvae_causalconv3d_w8a8(xq, xs, cache, wq, ws, b, *dims, y, None)


def test_conv_rejects_null_and_bad_sizes(L):
    assert conv(L, xq=None) == -1
    assert conv(L, y=None) == -1
    assert conv(L, xs=None) == -1
    assert conv(L, ws=None) == -1
    assert conv(L, dims=(0, 1, 4, 4, 32, 32, 3, 3, 3)) == -1
    assert conv(L, dims=(1, 1, -4, 4, 32, 32, 3, 3, 3)) == -1
    assert conv(L, y=FAKE_MIS) == -1
    assert conv(L, xq=FAKE_MIS) == -1


def test_conv_rejects_unsupported(L):
    assert conv(L, dims=(1, 1, 4, 4, 48, 32, 3, 3, 3)) == -2      # Cin % 32
    assert conv(L, dims=(1, 1, 4, 4, 32, 40, 3, 3, 3)) == -2      # Cout % 32
    assert conv(L, dims=(1, 1, 4, 4, 32, 32, 2, 3, 3)) == -2      # kt = 2
    assert conv(L, dims=(1, 1, 4, 4, 32, 32, 3, 3, 1)) == -2      # kh != kw
    assert conv(L, dims=(1, 1, 4, 4, 32, 32, 3, 5, 5)) == -2      # 5x5
    assert conv(L, dims=(1, 1, 4, 4, 4960, 32, 3, 3, 3)) == -2    # 127^2 * K >= 2^31


def test_conv_absmax_rejects(L):
    f = L.qvae_causalconv3d_w8a8_absmax
    dims = (1, 1, 4, 4, 32, 32, 3, 3, 3)
    assert f(FAKE, FAKE, None, FAKE, FAKE, None, *dims, FAKE, None, None) == -1      # no maximum buffer
    assert f(None, FAKE, None, FAKE, FAKE, None, *dims, FAKE, FAKE, None) == -1
    assert f(FAKE, FAKE, None, FAKE, FAKE, None, 1, 1, 4, 4, 32, 40, 3, 3, 3, FAKE, FAKE, None) == -2


def test_acc32_rejects(L):
    f = L.qvae_causalconv3d_w8a8_acc32
    assert f(None, None, FAKE, 1, 1, 4, 4, 32, 32, 3, 3, 3, FAKE, None) == -1
    assert f(FAKE, None, FAKE, 1, 1, 4, 4, 33, 32, 3, 3, 3, FAKE, None) == -2


def test_quant_entry_points_reject(L):
    assert L.qvae_act_absmax(None, 16, FAKE, None) == -1
    assert L.qvae_act_absmax(FAKE, 0, FAKE, None) == -1
    assert L.qvae_act_absmax(FAKE_MIS, 16, FAKE, None) == -1
    assert L.qvae_act_quantize(FAKE, 16, 1.0, None, FAKE, FAKE, None) == -1
    # clip ratio: (0, 1] is accepted; 0, negative and NaN are invalid, above 1 unsupported
    nan = float("nan")
    for clip, rc in [(0.0, -1), (-0.5, -1), (nan, -1), (1.5, -2), (float("inf"), -2)]:
        assert L.qvae_act_quantize(FAKE, 16, clip, FAKE, FAKE, FAKE, None) == rc, clip
        assert L.qvae_act_absmax_quant(FAKE, 16, clip, FAKE, FAKE, FAKE, None) == rc, clip
        assert L.qvae_quantize_weights(FAKE, 32, 32, 3, 3, 3, clip, FAKE, FAKE, None) == rc, clip
    assert L.qvae_act_absmax_quant(FAKE, 16, 1.0, FAKE, FAKE, FAKE_MIS, None) == -1
    assert L.qvae_act_absmax_quant(FAKE, 16, 0.9, FAKE, FAKE, FAKE_MIS, None) == -1
    assert L.qvae_quantize_weights(None, 32, 32, 3, 3, 3, 1.0, FAKE, FAKE, None) == -1
    assert L.qvae_quantize_weights(FAKE, 32, 32, 3, 3, 3, 0.5, FAKE_MIS, FAKE, None) == -1
    assert L.qvae_quantize_weights(FAKE, 32, 32, 2, 3, 3, 1.0, FAKE, FAKE, None) == -2


def test_bf16_entry_points_reject(L):
    f = L.qvae_causalconv3d_bf16
    dims = (1, 1, 4, 4, 32, 32, 3, 3, 3)
    assert f(None, None, FAKE, None, *dims, FAKE, None) == -1
    assert f(FAKE, None, None, None, *dims, FAKE, None) == -1
    assert f(FAKE, None, FAKE, None, *dims, None, None) == -1
    assert f(FAKE_MIS, None, FAKE, None, *dims, FAKE, None) == -1
    assert f(FAKE, FAKE_MIS, FAKE, None, *dims, FAKE, None) == -1
    assert f(FAKE, None, FAKE, None, 1, 1, 4, 4, 24, 32, 3, 3, 3, FAKE, None) == -2    # Cin % 16
    assert f(FAKE, None, FAKE, None, 1, 1, 4, 4, 32, 48, 3, 3, 3, FAKE, None) == -2    # Cout % 32
    assert f(FAKE, None, FAKE, None, 1, 1, 4, 4, 32, 32, 2, 3, 3, FAKE, None) == -2    # kt = 2
    assert f(FAKE, None, FAKE, None, 1, 1, 4, 4, 32, 32, 3, 1, 3, FAKE, None) == -2    # kh != kw
    p = L.qvae_pack_weights_bf16
    assert p(None, 32, 32, 3, 3, 3, FAKE, None) == -1
    assert p(FAKE, 32, 32, 3, 3, 3, FAKE_MIS, None) == -1
    assert p(FAKE, 32, 0, 3, 3, 3, FAKE, None) == -1
    assert p(FAKE, 40, 32, 3, 3, 3, FAKE, None) == -2
    assert p(FAKE, 32, 24, 3, 3, 3, FAKE, None) == -2


def test_conv_qin_rejects(L):
    f = L.qvae_causalconv3d_w8a8_qin
    dims = (1, 1, 4, 4, 32, 32, 3, 3, 3)
    assert f(FAKE, None, None, 1.0, FAKE, FAKE, None, *dims, None, FAKE, None) == -1        # no maximum buffer
    assert f(FAKE, None, FAKE, 0.0, FAKE, FAKE, None, *dims, None, FAKE, None) == -1        # clip 0
    assert f(FAKE, None, FAKE, float("nan"), FAKE, FAKE, None, *dims, None, FAKE, None) == -1
    assert f(FAKE, None, FAKE, 1.5, FAKE, FAKE, None, *dims, None, FAKE, None) == -2        # clip > 1
    assert f(FAKE, None, FAKE, 1.0, FAKE, None, None, *dims, None, FAKE, None) == -1        # no weight scales
    assert f(FAKE_MIS, None, FAKE, 1.0, FAKE, FAKE, None, *dims, None, FAKE, None) == -1
    assert f(FAKE, FAKE_MIS, FAKE, 1.0, FAKE, FAKE, None, *dims, None, FAKE, None) == -1
    assert f(FAKE, None, FAKE, 1.0, FAKE, FAKE, None, 1, 1, 4, 4, 48, 32, 3, 3, 3, None, FAKE, None) == -2
    assert f(FAKE, None, FAKE, 1.0, FAKE, FAKE, None, 1, 1, 4, 4, 32, 40, 3, 3, 3, None, FAKE, None) == -2
    assert f(FAKE, None, FAKE, 1.0, FAKE, FAKE, None, 1, 1, 4, 4, 4960, 32, 3, 3, 3, None, FAKE, None) == -2


def test_rmsnorm_silu_rejects(L):
    f, fa = L.qvae_rmsnorm_silu, L.qvae_rmsnorm_silu_absmax
    assert f(None, 4, 96, FAKE, 1e-6, FAKE, None) == -1
    assert f(FAKE, 0, 96, FAKE, 1e-6, FAKE, None) == -1
    assert f(FAKE, 4, 96, None, 1e-6, FAKE, None) == -1
    assert f(FAKE, 4, 96, FAKE, 0.0, FAKE, None) == -1
    assert f(FAKE, 4, 96, FAKE, float("nan"), FAKE, None) == -1
    assert f(FAKE_MIS, 4, 96, FAKE, 1e-6, FAKE, None) == -1
    assert f(FAKE, 4, 100, FAKE, 1e-6, FAKE, None) == -2       # C % 8
    assert f(FAKE, 4, 512, FAKE, 1e-6, FAKE, None) == -2       # C > 480
    assert fa(FAKE, 4, 96, FAKE, 1e-6, FAKE, None, None) == -1  # no maximum buffer


def test_force_fail_hook():
    # QVAE_FORCE_FAIL=1: every call returns QVAE_EFORCED before any launch
    code = (
        "import ctypes, sys\n"
        "from w8a8_int8_quantized_act_amd import ops\n"
        "L = ops.lib(); F = ctypes.c_void_p(0x10000)\n"
        "r = [L.qvae_act_absmax(F, 16, F, None),\n"
        "     L.qvae_act_quantize(F, 16, 1.0, F, F, F, None),\n"
        "     L.qvae_act_absmax_quant(F, 16, 1.0, F, F, F, None),\n"
        "     L.qvae_quantize_weights(F, 32, 32, 3, 3, 3, 1.0, F, F, None),\n"
        "     L.qvae_causalconv3d_w8a8(F, F, None, F, F, None, 1, 1, 4, 4, 32, 32, 3, 3, 3, F, None),\n"
        "     L.qvae_causalconv3d_w8a8_acc32(F, None, F, 1, 1, 4, 4, 32, 32, 3, 3, 3, F, None)]\n"
        "sys.exit(0 if r == [-4] * 6 else 1)\n")
    env = dict(os.environ, QVAE_FORCE_FAIL="1")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr


def test_force_fail_w8a8_only():
    # QVAE_FORCE_FAIL=w8a8: the W8A8 calls fail, the native-precision calls still
    # validate their arguments (the fake pointers are rejected as usual, not forced)
    code = (
        "import ctypes, sys\n"
        "from w8a8_int8_quantized_act_amd import ops\n"
        "L = ops.lib(); F = ctypes.c_void_p(0x10000); M = ctypes.c_void_p(0x10008)\n"
        "w8 = [L.qvae_act_absmax(F, 16, F, None),\n"
        "      L.qvae_act_quantize(F, 16, 1.0, F, F, F, None),\n"
        "      L.qvae_quantize_weights(F, 32, 32, 3, 3, 3, 1.0, F, F, None),\n"
        "      L.qvae_causalconv3d_w8a8(F, F, None, F, F, None, 1, 1, 4, 4, 32, 32, 3, 3, 3, F, None),\n"
        "      L.qvae_causalconv3d_w8a8_absmax(F, F, None, F, F, None, 1, 1, 4, 4, 32, 32, 3, 3, 3, F, F, None),\n"
        "      L.qvae_causalconv3d_w8a8_qin(F, None, F, 1.0, F, F, None, 1, 1, 4, 4, 32, 32, 3, 3, 3, None, F, None)]\n"
        "nat = [L.qvae_causalconv3d_bf16(M, None, F, None, 1, 1, 4, 4, 32, 32, 3, 3, 3, F, None),\n"
        "       L.qvae_pack_weights_bf16(F, 32, 32, 3, 3, 3, M, None)]\n"
        "sel = L.qvae_select_layer(3, b'decoder.middle.0.residual.2', 384, 384, 3, 3, 3, 384)\n"
        "sys.exit(0 if w8 == [-4] * 6 and nat == [-1, -1] and sel == 1 else 1)\n")
    env = dict(os.environ, QVAE_FORCE_FAIL="w8a8")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr


def test_binding_raises_when_library_missing(monkeypatch):
    from w8a8_int8_quantized_act_amd import ops
    monkeypatch.setattr(ops, "_lib", None)
    monkeypatch.setattr(ops, "LIB_PATH", "/nonexistent/libqvae.so")
    with pytest.raises(ops.QvaeError):
        ops.lib()


def test_product_never_reaches_the_oracle():
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", src, re.M), f
                assert "qvae_oracle" not in src and "libqvae_oracle" not in src, f


def test_absmax_words_match_header():
    from w8a8_int8_quantized_act_amd import ops
    m = re.search(r"#define\s+QVAE_ABSMAX_WORDS\s+(\d+)", open(HEADER).read())
    assert m and int(m.group(1)) == ops.ABSMAX_WORDS


def test_binding_checks_the_maximum_buffer():
    # the binding rejects an activation-maximum buffer in host memory before any
    # call reaches the library (dtype and length are checked after that)
    import torch
    from w8a8_int8_quantized_act_amd import ops
    with pytest.raises(ValueError, match="device"):
        ops._absmax_buf(torch.zeros(513, dtype=torch.int32))
