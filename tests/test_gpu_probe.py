"""GPU check of the matrix-core rate probe (a measurement aid): after one
round, the sum of a wave's checksums equals, for every instruction it issued,
sum over k of (column sum of A at k) x (row sum of B at k) -- a quantity that
does not depend on how the instruction lays rows and columns over lanes, only
on A and B pairing the same k per (lane group, byte); further rounds add the
same amount again."""
import numpy as np
import pytest
import torch

from tests.test_gpu_parity import DEV

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from w8a8_int8_quantized_act_amd import ops as o
    o.lib()
    return o


def _expected_wave_sum(tab, wave, shape):
    """tab int8 [14, 4096, 16]; rows 0-5 A, 6-13 B; lane l of wave w reads entry 64 w + l."""
    lanes = tab[:, 64 * wave:64 * wave + 64, :].astype(np.int64)   # [14, 64, 16]
    if shape == 0:     # 32x32x32: rows/cols = lane % 32, k = (lane // 32, byte)
        red = lanes.reshape(14, 2, 32, 16).sum(axis=2)             # [14, khalf, byte]
        pairs = [(m + 3 * p, 6 + n + 4 * p) for p in range(2) for m in range(3) for n in range(4)]
    else:              # 16x16x64: rows/cols = lane % 16, k = (lane // 16, byte)
        red = lanes.reshape(14, 4, 16, 16).sum(axis=2)             # [14, kgroup, byte]
        pairs = [(m, 6 + n) for m in range(4) for n in range(8)]
    return sum(int((red[a] * red[b]).sum()) for a, b in pairs)


@pytest.mark.parametrize("shape", [0, 1], ids=["i8_32x32x32", "i8_16x16x64"])
def test_probe_accumulates_the_products(ops, shape):
    g = torch.Generator().manual_seed(40 + shape)
    tab = torch.randint(-9, 10, (14, 4096, 16), generator=g, dtype=torch.int8)
    t_dev = tab.view(torch.int32).reshape(14, 4096, 4).to(DEV)
    out1 = ops.probe_mfma(shape, t_dev, 1, 1).cpu().numpy().astype(np.int64)
    out3 = ops.probe_mfma(shape, t_dev, 3, 1).cpu().numpy().astype(np.int64)
    torch.cuda.synchronize()
    for w in range(4):
        want = _expected_wave_sum(tab.numpy(), w, shape)
        got1 = int(out1[64 * w:64 * w + 64].sum())
        got3 = int(out3[64 * w:64 * w + 64].sum())
        assert got1 == want, f"wave {w}"
        assert got3 == 3 * want, f"wave {w}"


@pytest.mark.parametrize("shape", [2, 3], ids=["bf16_32x32x16", "bf16_16x16x32"])
def test_probe_bf16_runs_and_zero_stays_zero(ops, shape):
    z = torch.zeros((14, 4096, 4), dtype=torch.int32, device=DEV)
    out = ops.probe_mfma(shape, z, 2, 3)
    torch.cuda.synchronize()
    assert out.numel() == 3 * 256 and int(out.abs().max()) == 0


def test_init_loads_the_code_and_changes_nothing(ops):
    """qvae_init (optional set-up) succeeds, may be repeated, and the calls
    after it behave as before."""
    ops.init()
    ops.init()
    z = torch.zeros((14, 4096, 4), dtype=torch.int32, device=DEV)
    out = ops.probe_mfma(0, z, 1, 1)
    torch.cuda.synchronize()
    assert int(out.abs().max()) == 0
