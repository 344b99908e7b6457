"""Pins of the oracle's 3- and 4-bit base quantizer variants (CPU only).

The base quantizer B_b of the summary's §3 step 2 at b = 3 and 4 bits (7 and 15 levels), stored one
code per nibble. Pins: the nibble layout on a hand-worked word; keys lying on a 3- or 4-bit grid
are reproduced exactly, so a rank-0 cache decodes to exact attention (torch fp64); the storage
error falls as bits grow on the same keys.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import oracle as orc
from workloads import synth

from .helpers import value_payload


def test_nibble_layout_worked_word():
    # channels 0..7 carry codes 0..7: channel 2i at nibble i, channel 2i+1 at nibble i + 4
    codes = np.arange(16, dtype=np.uint8)[None, :]      # one token, d = 16: words 0x75316420, 0xfdb9eca8
    kc = np.zeros((1, 8), np.uint8)
    assert orc.lib().orc_pack_kcode4(16, 1, orc._p(codes), orc._p(kc)) == 0
    assert kc[0].tolist() == [0x20, 0x64, 0x31, 0x75, 0xa8, 0xec, 0xb9, 0xfd]


def _grid_keys(rng, T, d, levels):
    K = np.empty((T, d), np.float32)
    for g0 in range(0, T, 32):
        z = rng.integers(-64, 64, size=d) / 16.0
        s = rng.integers(1, 8, size=d) / 16.0
        c = rng.integers(0, levels + 1, size=(32, d))
        c[0, :], c[1, :] = 0, levels
        K[g0:g0 + 32] = (c * s + z).astype(np.float32)
    return K


@pytest.mark.parametrize("bits", [3, 4])
def test_grid_keys_decode_to_exact_attention(bits):
    w = synth.scaled(synth.WORKLOADS["qwen7b_decode"], n_q_heads=4, n_kv_heads=2, batch=1, rank=0, base_bits=bits)
    rng = np.random.default_rng(40 + bits)
    K = np.stack([_grid_keys(rng, 96, 128, (1 << bits) - 1) for _ in range(2)])
    assert np.array_equal(synth.round_to(K, "bf16"), K)  # dyadic grid values survive bf16
    V = synth.stack_streams(w, "values", 1, 96)[0]
    c = orc.empty_cache(1, 2, 96, 128, 0, 0, 1, base_bits=bits)
    for h in range(2):
        orc.write_stream(c, 0, h, 0, K[h], value_payload(V[h], w), None, 0, 1, bits=bits)
    q = synth.decode_queries(w, batch=1)
    _, out = orc.decode(c, q, None, 96, 1.0, 0, 1)
    qt = torch.from_numpy(q.astype(np.float64))[:, :, None, :]
    Kt = torch.from_numpy(K.astype(np.float64)).repeat_interleave(2, dim=0)[None]
    Vt = torch.from_numpy(V.astype(np.float64)).repeat_interleave(2, dim=0)[None]
    ref = F.scaled_dot_product_attention(qt, Kt, Vt)[:, :, 0, :].numpy()
    assert np.allclose(out, ref, rtol=0, atol=1e-12)


def test_storage_error_falls_with_bits():
    w = synth.WORKLOADS["qwen7b_decode"]
    k = synth.keys(w, 0, 0, 256)
    err = {}
    for bits in (2, 3, 4):
        e = orc.encode_keys(k, None, bits=bits)
        gi = np.arange(256) // 32
        k_hat = e["codes"] * orc.f16_bits_to_f32(e["scale"])[gi] + orc.f16_bits_to_f32(e["zero"])[gi]
        err[bits] = float(np.mean((k_hat - k) ** 2))
    assert err[4] < err[3] < err[2]
    assert err[2] / err[4] > 20  # about (15/3)^2 = 25 for errors uniform in a step
