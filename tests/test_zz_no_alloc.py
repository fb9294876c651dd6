"""The allocation-free activation quantizer (qvae_act_absmax_quant_noalloc,
whose activation-maximum words live in the library's static scratch array)
against qvae_act_absmax_quant with a caller workspace, through the C ABI:
calls in a row, each later one on a smaller input whose maximum is smaller,
so a stale maximum left in the scratch by an earlier call would change the
scale.  Scale bits and codes must be equal."""
import ctypes

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def test_noalloc_matches_the_workspace_entry_point():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from w8a8_int8_quantized_act_amd import ops
    L = ops.lib()
    P = ctypes.c_void_p
    stream = P(torch.cuda.current_stream().cuda_stream)
    g = torch.Generator().manual_seed(990)
    # (elements, magnitude, clip): sizes spanning all 512 partial slots down to
    # a few, a ragged tail (numel % 8), and a clip ratio below 1
    for n, mag, clip in [(5_000_003, 9.0, 1.0), (1_234_567, 3.0, 1.0), (4_099, 0.25, 0.5), (13, 0.01, 1.0)]:
        x = (torch.randn(n, generator=g) * mag).to(torch.bfloat16).to(DEV)
        am = torch.empty((ops.ABSMAX_WORDS,), dtype=torch.int32, device=DEV)
        xs_ref = torch.empty((1,), dtype=torch.float32, device=DEV)
        xq_ref = torch.empty((n,), dtype=torch.int8, device=DEV)
        assert L.qvae_act_absmax_quant(P(x.data_ptr()), n, ctypes.c_float(clip), P(am.data_ptr()),
                                       P(xs_ref.data_ptr()), P(xq_ref.data_ptr()), stream) == 0
        xs = torch.full((1,), -1.0, dtype=torch.float32, device=DEV)
        xq = torch.full((n,), 99, dtype=torch.int8, device=DEV)
        assert L.qvae_act_absmax_quant_noalloc(P(x.data_ptr()), n, ctypes.c_float(clip), P(xs.data_ptr()),
                                               P(xq.data_ptr()), stream) == 0
        torch.cuda.synchronize()
        assert xs.cpu().numpy().view(np.uint32)[0] == xs_ref.cpu().numpy().view(np.uint32)[0], n
        assert torch.equal(xq, xq_ref), n
    # arguments are checked before anything runs
    x = torch.zeros((64,), dtype=torch.bfloat16, device=DEV)
    xs = torch.empty((1,), dtype=torch.float32, device=DEV)
    xq = torch.empty((64,), dtype=torch.int8, device=DEV)
    assert L.qvae_act_absmax_quant_noalloc(P(x.data_ptr()), 0, ctypes.c_float(1.0), P(xs.data_ptr()),
                                           P(xq.data_ptr()), stream) == ops.EINVAL
    assert L.qvae_act_absmax_quant_noalloc(P(x.data_ptr()), 64, ctypes.c_float(1.5), P(xs.data_ptr()),
                                           P(xq.data_ptr()), stream) == ops.EUNSUPPORTED
    assert L.qvae_act_absmax_quant_noalloc(None, 64, ctypes.c_float(1.0), P(xs.data_ptr()),
                                           P(xq.data_ptr()), stream) == ops.EINVAL
