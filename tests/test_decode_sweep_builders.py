"""CPU check of the one-hot and +-1 operand builders of the GPU code-sweep tests: each
vector decodes, through the oracle's own decoders, to what the sweep says it holds."""
import numpy as np

from oracle import oracle as orc
from sparse_attention_fp4_amd import workloads as wl

from .test_gpu_decode_codes import _codes, _one_hot, _signed_ones


def test_sweep_vectors_decode_to_what_they_claim():
    for fmt in (wl.MXFP4, wl.NVFP4):
        codes = _codes(fmt)
        nib = np.repeat(np.arange(16, dtype=np.uint8), 3)
        cod = np.tile(codes[[0, codes.size // 2, -1]], 16)
        p, s = _one_hot(nib.size, fmt, cod, nib, seed=1)
        v = orc.dequant(fmt, p, s)
        dec = orc.e8m0 if fmt == wl.MXFP4 else orc.e4m3
        for i in range(nib.size):
            d = (7 * i + 3) % 128
            want = orc.e2m1(int(nib[i])) * dec(int(cod[i]))
            assert v[i, d] == want
            assert np.all(np.delete(v[i], d) == 0)
        p, s = _signed_ones(4, fmt, codes[:2])
        v = orc.dequant(fmt, p, s)
        assert np.all(v[0] == dec(int(codes[0]))) and np.all(v[1] == -dec(int(codes[0])))
        assert np.all(v[2] == dec(int(codes[1]))) and np.all(v[3] == -dec(int(codes[1])))
    # the swept code lists: E8M0 1..254, every E4M3 code but the two NaNs
    assert _codes(wl.MXFP4).tolist() == list(range(1, 255))
    e4 = _codes(wl.NVFP4)
    assert e4.size == 254 and 0x7F not in e4 and 0xFF not in e4 and 0x7E in e4 and 0xFE in e4
    assert orc.e4m3(0x7E) == 448.0 and orc.e4m3(0xFE) == -448.0 and orc.e4m3(0x01) == 2.0 ** -9
