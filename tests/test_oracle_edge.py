"""Pins of the oracle on the method's degenerate cases (CPU only).

The base quantizer of "Technische Samenvatting: HeadQ ..." §3 step 2 is a min/max grid per
(32-token group, channel); when a channel is constant over its group the grid collapses: the step
is 0, every code 0 and the reconstruction the binary16 zero alone, so the residual is exactly the
rounding of that zero (reading R4: the reciprocal of a zero step is taken as 0). A group of zero
keys leaves nothing for the side code (reading R6: all side codes 0 when the side step is 0).
Values quantized per (token, 32-channel group) collapse the same way. A zero query scores every
token 0, so the decode's output is the plain mean of the stored values. Each expectation here is
fixed by those definitions and computed with numpy alone (numpy's own binary16 cast).
"""
import numpy as np

from oracle import oracle as orc

G = 32


def _f16_bits(x):
    return np.asarray(x, np.float32).astype(np.float16).view(np.uint16)


def _f16(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float32)


def _degenerate_keys(rng, T=96, d=128):
    K = rng.standard_normal((T, d)).astype(np.float32)
    K[:G, 3] = 1.2345678                 # constant over group 0 only
    K[:G, 40] = -7.3
    K[:, 77] = 0.1                       # constant in every group
    K[:, 100] = 0.0
    K[G:2 * G] = 0.0                     # a whole group of zero keys
    return K


def _basis(rng, d, r):
    return np.linalg.qr(rng.standard_normal((d, r)))[0].astype(np.float32)


def test_constant_channels_collapse_to_the_binary16_zero():
    rng = np.random.default_rng(11)
    K = _degenerate_keys(rng)
    e = orc.encode_keys(K, _basis(rng, 128, 16))
    for gi, c in [(0, 3), (0, 40), (0, 77), (2, 77), (0, 100), (2, 100)]:
        rows = slice(G * gi, G * gi + G)
        assert e["scale"][gi, c] == 0
        assert e["zero"][gi, c] == _f16_bits(K[G * gi, c])
        assert np.all(e["codes"][rows, c] == 0)
        # k - z exactly (Sterbenz: the two are within a factor 2 of each other, or both 0)
        assert np.array_equal(e["resid"][rows, c], K[rows, c] - _f16(e["zero"][gi, c]))
    assert np.all(e["scale"][0, :3] != 0) and np.all(e["scale"][2, :3] != 0)


def test_a_group_of_zero_keys_has_no_error_and_no_side_code():
    rng = np.random.default_rng(12)
    K = _degenerate_keys(rng)
    e = orc.encode_keys(K, _basis(rng, 128, 16))
    rows = slice(G, 2 * G)
    assert np.all(e["scale"][1] == 0) and np.all(e["zero"][1] == 0)
    assert np.all(e["codes"][rows] == 0) and np.all(e["resid"][rows] == 0)
    assert np.all(e["proj"][rows] == 0) and np.all(e["sigma"][rows] == 0) and np.all(e["zc"][rows] == 0)
    assert np.all(e["sigma"][:G] != 0) and np.all(e["sigma"][2 * G:] != 0)


def test_constant_value_groups_are_stored_exactly():
    rng = np.random.default_rng(13)
    V = rng.standard_normal((64, 128)).astype(np.float32)
    V[5, 0:32] = 0.75
    V[9, 64:96] = -3.0
    V[20, :] = 0.0
    q = orc.quantize_values(V)
    for t, cg in [(5, 0), (9, 2), (20, 0), (20, 1), (20, 2), (20, 3)]:
        assert q["scale"][t, cg] == 0
        assert q["zero"][t, cg] == _f16_bits(V[t, 32 * cg])
        assert np.all(q["codes"][t, 32 * cg:32 * cg + 32] == 0)
    assert np.count_nonzero(q["scale"] == 0) == 6


def test_zero_query_attends_uniformly():
    rng = np.random.default_rng(14)
    T, d, r = 96 + 7, 128, 16
    K = _degenerate_keys(rng, T=T)
    V = rng.standard_normal((T, d)).astype(np.float32)
    U = _basis(rng, d, r)
    for vmode in (0, 1):
        c = orc.empty_cache(1, 1, 128, d, r, vmode, 0, key_dtype=0)
        orc.write_stream(c, 0, 0, 0, K[:96], V[:96], U, vmode, 0)
        orc.write_stream(c, 0, 0, 96, K[96:], V[96:], U, vmode, 0)
        q = np.zeros((1, 2, d), np.float32)
        lg, out = orc.decode(c, q, U[None], T, 1.0, vmode, 0)
        assert np.all(lg == 0.0)
        mean = orc.value_rows(c, 0, 0, T, vmode, 0).mean(axis=0)
        assert np.allclose(out[0], mean[None], rtol=0, atol=1e-13)
        if vmode == 0:
            assert np.allclose(mean, V.astype(np.float64).mean(axis=0), rtol=0, atol=1e-13)
