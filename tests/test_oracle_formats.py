"""Pins of the oracle's number formats and byte packing (CPU only).

The binary16 / bfloat16 converters are pinned to library routines (numpy's float16 cast, torch's
bfloat16 cast); the packers to the bit layout by brute force over every code value, and to a
hand-worked fixture under tests/golden/.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as orc

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _f16_boundary_cases():
    # every finite binary16 value, the midpoints between neighbours (ties) and one f32 ulp on
    # either side of each midpoint
    h = np.arange(0, 0x7C00, dtype=np.uint16)
    vals = h.view(np.float16).astype(np.float32)
    nxt = np.append(vals[1:], np.float32(65536.0))
    mid = ((vals.astype(np.float64) + nxt.astype(np.float64)) / 2).astype(np.float32)
    up = np.nextafter(mid, np.float32(np.inf))
    dn = np.nextafter(mid, np.float32(-np.inf))
    x = np.concatenate([vals, mid, up, dn, np.array([65519.0, 65520.0, 65536.0, 1e30, 1e-30, 2.0 ** -25,
                                                      2.0 ** -25 * 1.0000001, 2.0 ** -26, 5.96e-8], np.float32)])
    return np.concatenate([x, -x])


def test_f32_to_f16_matches_numpy_on_all_boundaries():
    x = _f16_boundary_cases()
    ours = orc.f32_to_f16_bits(x)
    ref = x.astype(np.float16).view(np.uint16)
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first x={x[bad[:5]]} ours={ours[bad[:5]]} ref={ref[bad[:5]]}"


def test_f32_to_f16_random_bits_match_numpy():
    rng = np.random.default_rng(5)
    u = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    x = x[np.isfinite(x)]
    assert np.array_equal(orc.f32_to_f16_bits(x), x.astype(np.float16).view(np.uint16))


def test_f16_to_f32_all_patterns():
    h = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    ours = orc.f16_bits_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f32_to_bf16_matches_torch():
    rng = np.random.default_rng(6)
    u = rng.integers(0, 2 ** 32, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    # force many exact ties and near-ties
    u[::3] = (u[::3] & 0xFFFF0000) | 0x8000
    u[1::3] = (u[1::3] & 0xFFFF0000) | 0x7FFF
    x = u.view(np.float32)
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.f32_to_bf16_bits(x), ref)


def test_kcode_pack_every_byte_value_in_every_byte():
    """Key-code word layout: byte k of a 16-channel word holds channels 2k (bits 0-1), 8+2k (2-3),
    2k+1 (4-5) and 9+2k (6-7). Every byte value is produced in every byte position."""
    d, T = 16, 256 * 4
    codes = np.zeros((T, d), np.uint8)
    for k in range(4):
        v = np.arange(256)
        rows = slice(256 * k, 256 * (k + 1))
        codes[rows, 2 * k] = v & 3
        codes[rows, 8 + 2 * k] = (v >> 2) & 3
        codes[rows, 2 * k + 1] = (v >> 4) & 3
        codes[rows, 9 + 2 * k] = (v >> 6) & 3
    out = np.zeros((T, d // 4), np.uint8)
    assert orc.lib().orc_pack_kcode(d, T, orc._p(codes), orc._p(out)) == 0
    for k in range(4):
        blk = out[256 * k:256 * (k + 1)]
        assert np.array_equal(blk[:, k], np.arange(256, dtype=np.uint8))
        assert not np.any(np.delete(blk, k, axis=1))
    # two words per token at d = 32: the second word holds channels 16..31 the same way
    codes2 = np.zeros((1, 32), np.uint8)
    codes2[0, 16 + 9] = 3
    out2 = np.zeros((1, 8), np.uint8)
    assert orc.lib().orc_pack_kcode(32, 1, orc._p(codes2), orc._p(out2)) == 0
    assert list(out2[0]) == [0, 0, 0, 0, 0xC0, 0, 0, 0]
    assert orc.lib().orc_pack_kcode(4, 1, orc._p(codes2), orc._p(out2)) == -1  # d % 16 != 0


def test_scode_pack_roundtrip_all_pairs():
    pairs = np.array([(a, b) for a in range(-7, 8) for b in range(-7, 8)], np.int8)  # r = 2
    T = len(pairs)
    out = np.zeros((T, 1), np.uint8)
    assert orc.lib().orc_pack_scode(2, T, orc._p(pairs), orc._p(out)) == 0
    lo = (out[:, 0] & 0xF).astype(int) - 8
    hi = (out[:, 0] >> 4).astype(int) - 8
    assert np.array_equal(lo, pairs[:, 0]) and np.array_equal(hi, pairs[:, 1])


def test_vcode_and_vdense_layouts_roundtrip():
    """Value-code group block: lane l = 16*(t/8) + c%16 owns d/8 bytes, two per 16-channel tile;
    token item i = t%8 = 4q + 2b + e sits in byte b of the tile's pair at bits 4e + 2q."""
    rng = np.random.default_rng(7)
    T = 64
    for d in (64, 128):
        codes = rng.integers(0, 4, size=(T, d), dtype=np.uint8)
        vc = np.zeros((T // 32, d * 8), np.uint8)
        assert orc.lib().orc_pack_vcode(d, T, orc._p(codes), orc._p(vc)) == 0
        for t in range(T):
            g, tt = divmod(t, 32)
            i = tt % 8
            q, b, e = i // 4, (i % 4) // 2, i % 2
            for c in range(d):
                lane = 16 * (tt // 8) + c % 16
                byte = (lane * (d // 16) + c // 16) * 2 + b
                assert (vc[g, byte] >> (4 * e + 2 * q)) & 3 == codes[t, c]
        # every code bit is used exactly once
        assert vc.size * 4 == codes.size
    d = 64
    v = rng.standard_normal((T, d)).astype(np.float32)
    vd = np.zeros((T // 32, d, 32), np.float32)
    assert orc.lib().orc_pack_vdense(d, T, 4, orc._p(v), orc._p(vd)) == 0
    assert np.array_equal(vd.transpose(0, 2, 1).reshape(T, d), v)


def _read_golden(path):
    sections = {}
    cur = None
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        if line.startswith("[") and line.endswith("]"):
            cur = line[1:-1]
            sections[cur] = []
        else:
            sections[cur].append(line.split())
    return sections


def test_golden_worked_example_base_quantizer():
    """Hand-worked example (tests/golden/base_quant_worked.txt): one 32-token group, 4 channels."""
    import os
    g = _read_golden(os.path.join(os.path.dirname(__file__), "golden", "base_quant_worked.txt"))
    keys = np.array([[float(v) for v in row] for row in g["keys"]], np.float32)
    exp_scale = np.array([float(v) for v in g["scale"][0]], np.float32)
    exp_zero = np.array([float(v) for v in g["zero"][0]], np.float32)
    exp_codes = np.array([[int(v) for v in row] for row in g["codes"]], np.uint8)
    exp_words = np.array([int(v, 16) for v in g["kcode_words"][0]], np.uint32)
    enc = orc.encode_keys(keys, None)
    assert np.array_equal(orc.f16_bits_to_f32(enc["scale"][0]), exp_scale)
    assert np.array_equal(orc.f16_bits_to_f32(enc["zero"][0]), exp_zero)
    assert np.array_equal(enc["codes"], exp_codes)
    # packed in a 16-channel word whose channels 4..15 hold code 0
    codes16 = np.zeros((32, 16), np.uint8)
    codes16[:, :4] = enc["codes"]
    kc = np.zeros((32, 4), np.uint8)
    assert orc.lib().orc_pack_kcode(16, 32, orc._p(codes16), orc._p(kc)) == 0
    assert np.array_equal(kc.view("<u4")[:, 0], exp_words)
    # residuals of the worked example are exact (dyadic keys)
    exp_resid = np.array([[float(v) for v in row] for row in g["residual"]], np.float32)
    assert np.array_equal(enc["resid"], exp_resid)
