"""Pins of the oracle's A^2 value policy (CPU only).

The pages define the A^2 surrogate sum_j p_j^2 |v_hat_j - v_j|^2 of the value readout error
("Technische Samenvatting: HeadQ ...", §2.2) and pair HeadQ keys with an A^2-weighted value policy
for the full-KV composition (§5), without defining the policy. The oracle's reading: per 32-token
group the P tokens of largest w_j * e_j keep a bfloat16 correction, e_j their 2-bit value error and
w_j = 2^round(2 log2(e) a.k_j / sqrt(d)) with a the mean calibration query. These tests check it
against an independent fp64 recomputation and brute force over subsets, planted cases that fix the
direction of the weighting and its use of the value error, the reconstruction bound of the stored
corrections, and that the policy lowers the surrogate under attention drawn from queries around
the mean direction, by more than protecting random tokens does.
"""
import itertools

import numpy as np
import pytest

from oracle import oracle as orc

D = 64
G = 32


def _independent_prio(k, v, a):
    """w_j * e_j per token from the definitions, in fp64 (numpy's float16 for the metadata)."""
    vq = orc.quantize_values(v, 2)
    T, d = v.shape
    s = vq["scale"].view(np.float16).astype(np.float64)[:, np.arange(d) // G]
    z = vq["zero"].view(np.float16).astype(np.float64)[:, np.arange(d) // G]
    e = np.sum((v.astype(np.float64) - (vq["codes"] * s + z)) ** 2, axis=1)
    n = np.clip(np.rint(k.astype(np.float64) @ a.astype(np.float64) * 2.0 * np.log2(np.e) / np.sqrt(d)), -64, 64)
    return e * np.exp2(n), k.astype(np.float64) @ a.astype(np.float64) * 2.0 * np.log2(np.e) / np.sqrt(d)


def _data(seed, T=4 * G, d=D):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((T, d)).astype(np.float32)
    v = (rng.standard_normal((T, d)) * np.exp(rng.standard_normal((T, 1)) * 0.5)).astype(np.float32)
    a = (rng.standard_normal(d) * 0.4).astype(np.float32)
    return k, v, a


@pytest.mark.parametrize("P", [1, 2, 4])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_choice_is_the_best_subset(P, seed):
    k, v, a = _data(seed)
    pol = orc.value_policy(k, v, a, P)
    prio, x = _independent_prio(k, v, a)
    for g in range(k.shape[0] // G):
        idx = pol["idx"][g]
        chosen = [int(t) for t in idx[:P]]
        assert chosen == sorted(chosen) and len(set(chosen)) == P      # ascending, distinct
        assert np.all(idx[P:] == 0)
        pg = prio[g * G:(g + 1) * G]
        best = max(itertools.combinations(range(G), P), key=lambda S: sum(pg[list(S)]))
        if set(best) != set(chosen):
            # only a rounding boundary of the power-of-two weight may separate f32 and fp64
            xg = x[g * G:(g + 1) * G]
            diff = set(best) ^ set(chosen)
            assert all(abs(abs(xg[t] - np.floor(xg[t])) - 0.5) < 1e-4 for t in diff), (best, chosen)
        np.testing.assert_allclose(pol["prio"][g * G:(g + 1) * G], pg, rtol=1e-5)


def test_weight_direction_and_error_term():
    rng = np.random.default_rng(7)
    s = np.float32(0.25)
    # values on the 2-bit grid of their own 32-channel groups (zero error), except tokens 5, 9, 20
    codes = rng.integers(0, 4, (G, D)).astype(np.float32)
    codes[:, 0], codes[:, 1] = 0, 3                                  # min and max in every channel group
    codes[:, 32], codes[:, 33] = 0, 3
    v = (codes * s - 0.5).astype(np.float32)
    bump = rng.uniform(0.03, 0.09, D).astype(np.float32) * np.where(codes[0] % 3 == 0, 0, 1)
    for t in (5, 9):
        v[t] = v[0] + bump                                          # same rows: the same error e
    v[20] = v[0] + 0.4 * bump                                        # smaller error
    k = np.zeros((G, D), np.float32)
    a = np.zeros(D, np.float32)
    a[3] = 1.0
    k[9, 3], k[5, 3], k[20, 3] = 4.0, 0.0, 6.0                       # weights 2^round(k3 * 2 log2e / 8)
    pol = orc.value_policy(k, v, a, 1)
    e = _independent_prio(k, v, np.zeros_like(a))[0]
    assert e[5] == e[9] > 0 and e[20] > 0 and np.count_nonzero(e) == 3
    # equal errors: the larger a.k wins; reversing the direction reverses the choice
    assert pol["idx"][0, 0] == 20 or pol["idx"][0, 0] == 9
    w = np.exp2(np.rint(k[:, 3] * 2 * np.log2(np.e) / 8))
    assert pol["idx"][0, 0] == int(np.argmax(w * e))
    assert orc.value_policy(k, v, -a, 1)["idx"][0, 0] == 5
    # with the weights equal, the error decides: tokens without error are never chosen
    pol0 = orc.value_policy(k, v, np.zeros_like(a), 2)
    assert list(pol0["idx"][0, :2]) == [5, 9]


@pytest.mark.parametrize("P", [1, 2])
def test_stored_corrections_and_decoded_values(P):
    k, v, a = _data(3, T=3 * G, d=128)
    caches = {}
    for p in (0, P):
        c = orc.empty_cache(1, 1, 3 * G, 128, 0, 1, 1, key_dtype=1, value_protect=p)
        orc.write_stream(c, 0, 0, 0, k, v, None, 1, 1, a_h=a)
        caches[p] = c
    plain = orc.value_rows(caches[0], 0, 0, 3 * G, 1, 1)
    rows = orc.value_rows(caches[P], 0, 0, 3 * G, 1, 1)
    prot = {g * G + int(t) for g in range(3) for t in caches[P]["vpidx"][0, 0, g, :P]}
    for j in range(3 * G):
        if j in prot:
            delta = v[j].astype(np.float64) - plain[j]
            err = np.abs(rows[j] - v[j])
            assert np.all(err <= 2.0 ** -8 * np.abs(delta) + 1e-6 * np.abs(v[j]) + 1e-30)
            assert np.sum(err ** 2) < 1e-3 * np.sum(delta ** 2)
        else:
            assert np.array_equal(rows[j], plain[j])


def test_mean_query_is_the_mean():
    rng = np.random.default_rng(11)
    q = rng.standard_normal((6, 50, 64)).astype(np.float32) + 0.3
    a = orc.mean_query(q, 2)
    ref = q.astype(np.float64).reshape(2, 3 * 50, 64).mean(axis=1)
    np.testing.assert_allclose(a, ref, rtol=1e-6, atol=1e-7)


def test_policy_lowers_the_a2_surrogate_more_than_random_protection():
    """Queries around a mean direction mu; the policy's direction is their sample mean. The A^2
    surrogate of the attention the exact keys give falls with P, and below what protecting the same
    number of random tokens per group gives."""
    rng = np.random.default_rng(5)
    d, T = 64, 16 * G
    k = rng.standard_normal((T, d)).astype(np.float32)
    v = rng.standard_normal((T, d)).astype(np.float32)
    mu = rng.standard_normal(d)
    mu *= 10.0 / np.linalg.norm(mu)                                  # peaked attention
    calib = (mu + 0.3 * rng.standard_normal((1, 256, d))).astype(np.float32)
    a = orc.mean_query(calib, 1)[0]
    queries = mu + 0.3 * rng.standard_normal((64, d))
    s = queries @ k.T.astype(np.float64) / np.sqrt(d)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)

    def a2(rows):
        return float(np.mean((p ** 2) @ np.sum((rows - v) ** 2, axis=1)))

    def rows_of(P):
        c = orc.empty_cache(1, 1, T, d, 0, 1, 1, key_dtype=1, value_protect=P)
        orc.write_stream(c, 0, 0, 0, k, v, None, 1, 1, a_h=a)
        return orc.value_rows(c, 0, 0, T, 1, 1)

    plain = rows_of(0)
    d0, d1, d2 = a2(plain), a2(rows_of(1)), a2(rows_of(2))
    assert d2 < d1 < d0
    for P, dp in ((1, d1), (2, d2)):
        rand = []
        for trial in range(20):
            rows = plain.copy()
            for g in range(T // G):
                for t in rng.choice(G, P, replace=False):
                    rows[g * G + t] = v[g * G + t]          # an exact value: better than any correction
            rand.append(a2(rows))
        assert dp < 0.5 * np.mean(rand), (dp, np.mean(rand))
