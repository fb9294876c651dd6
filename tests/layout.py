"""Test-side layout helper: the packed INT8 weight order that qvae.h documents.

The oracle returns weight codes as [Cout][kt][kh][kw][Cin]; the library's
qvae_quantize_weights writes the same codes as MFMA operand fragments,
  packed[cb][i][s][j][l][L][b] = plain[32*cb + L%32][i][j][l][32*s + 16*(L//32) + b].
This is a permutation only (no arithmetic), written here independently of the
library so that a wrong packing in either place shows up as a mismatch.
"""
import numpy as np


def pack_weight_codes(plain: np.ndarray) -> np.ndarray:
    Co, kt, kh, kw, Ci = plain.shape
    x = plain.reshape(Co // 32, 32, kt, kh, kw, Ci // 32, 2, 16)      # cb r i j l s half b
    x = x.transpose(0, 2, 5, 3, 4, 6, 1, 7)                           # cb i s j l half r b
    return np.ascontiguousarray(x.reshape(Co // 32, kt, Ci // 32, kh, kw, 64, 16))


def pack_weights_bf16(w: np.ndarray) -> np.ndarray:
    """bf16 weights (any 2-byte dtype) [Cout][Cin][kt][kh][kw] -> the packed order
    of qvae_pack_weights_bf16:
      packed[cb][i][s][j][l][L][e] = w[32*cb + L%32][16*s + 8*(L//32) + e][i][j][l]."""
    Co, Ci, kt, kh, kw = w.shape
    x = w.reshape(Co // 32, 32, Ci // 16, 2, 8, kt, kh, kw)            # cb r s half e i j l
    x = x.transpose(0, 5, 2, 6, 7, 3, 1, 4)                           # cb i s j l half r e
    return np.ascontiguousarray(x.reshape(Co // 32, kt, Ci // 16, kh, kw, 64, 8))
