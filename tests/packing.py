"""Test-side packer: codes -> MLX-layout uint32 words, built on numpy's
``packbits(bitorder="little")`` so that it shares nothing with the oracle's
bit-at-a-time unpack. Value k of a row occupies stream bits [k*bits, (k+1)*bits),
least significant bit first; bytes are assembled little-endian into words.
"""
import numpy as np


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    N, K = codes.shape
    assert (K * bits) % 32 == 0
    # bit matrix [N, K, bits], bit i of each code (LSB first)
    bitmat = (codes[:, :, None] >> np.arange(bits, dtype=np.uint8)[None, None, :]) & 1
    stream = bitmat.reshape(N, K * bits)
    packed = np.packbits(stream, axis=1, bitorder="little")  # [N, K*bits/8] bytes
    return np.ascontiguousarray(packed).view("<u4").astype(np.uint32).reshape(N, K * bits // 32)
