"""The equal-key closed forms against the oracle on the CPU, so that the
full-size GPU checks built on them rest on more than their own derivation."""
import numpy as np
import pytest

import equal_keys
import oracle


@pytest.mark.parametrize("S,d,chunk", [(1, 4, 8), (7, 3, 2), (300, 8, 64), (129, 16, 128)])
def test_stream_matches_oracle(S, d, chunk):
    rng = np.random.default_rng([S, d, chunk])
    key = rng.standard_normal(d)
    K = np.repeat(key[None, :], S, axis=0)
    V = rng.standard_normal((S, d))
    q = rng.standard_normal((S, d))
    dO = rng.standard_normal((S, d))
    pos = np.arange(S)
    lse, o, dK, dV = equal_keys.stream(q, dO, V, key, chunk=chunk)
    dq_ref, dK_ref, dV_ref = oracle.attend_rows_bwd(q, pos, K, V, dO)
    np.testing.assert_allclose(lse, oracle.lse_rows(q, pos, K), rtol=0, atol=1e-12)
    np.testing.assert_allclose(o, oracle.attend_rows(q, pos, K, V), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dV, dV_ref, rtol=0, atol=1e-11)
    np.testing.assert_allclose(dK, dK_ref, rtol=0, atol=1e-10)
    np.testing.assert_allclose(dq_ref, 0.0, rtol=0, atol=1e-12)


def test_stream_detects_a_wrong_key():
    """Keys that are not all equal break the closed form (the check is not
    vacuous)."""
    rng = np.random.default_rng(5)
    S, d = 50, 4
    key = rng.standard_normal(d)
    K = np.repeat(key[None, :], S, axis=0)
    K[20] += 1.0
    V, q, dO = (rng.standard_normal((S, d)) for _ in range(3))
    _, _, dK, dV = equal_keys.stream(q, dO, V, key, chunk=16)
    _, dK_ref, dV_ref = oracle.attend_rows_bwd(q, np.arange(S), K, V, dO)
    assert np.max(np.abs(dV - dV_ref)) > 1e-3 and np.max(np.abs(dK - dK_ref)) > 1e-3
