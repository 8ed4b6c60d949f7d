"""CPU tests: the fp64 oracle against the facts that pin it (no GPU)."""
import numpy as np
import pytest

import oracle
from oracle import forms

from oracle_pins import ALL_CHECKS


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(oracle.kda_forward)


def test_oracle_threads_and_pairs_agree():
    rng = np.random.default_rng(3)
    T, H, d = 50, 3, 16
    q = rng.standard_normal((T, H, d))
    k = rng.standard_normal((T, H, d))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, d))
    g = -rng.uniform(0, 2, (T, H, d))
    b = rng.uniform(0, 1, (T, H))
    cu = np.array([0, 20, 50])
    o1, f1 = oracle.kda_forward(q, k, v, g, b, 0.2, cu, None, threads=1)
    o4, f4 = oracle.kda_forward(q, k, v, g, b, 0.2, cu, None, threads=4)
    np.testing.assert_array_equal(o1, o4)
    np.testing.assert_array_equal(f1, f4)
    op, fp = oracle.kda_forward(q, k, v, g, b, 0.2, cu, None, pairs=[(1, 2), (0, 0)])
    np.testing.assert_array_equal(op[20:, 2], o1[20:, 2])
    np.testing.assert_array_equal(op[:20, 0], o1[:20, 0])
    np.testing.assert_array_equal(fp[1, 2], f1[1, 2])
    assert not op[:20, 2].any()


def test_oracle_rejects_bad_arguments():
    z = np.zeros((2, 1, 2))
    with pytest.raises(ValueError):
        oracle.kda_forward(z, z, z, z, np.zeros((2, 1)), 1.0, np.array([0, 3, 2]))


def test_neumann_product_is_exact_for_nilpotent_A():
    """A 16x16 strictly lower-triangular matrix has A^16 = 0, so (I + A)^{-1} = sum_{j<16} (-A)^j
    = (I - A)(I + A^2)(I + A^4)(I + A^8) (smzdm "KDA 内核到底难在哪": 15 terms folded into
    3 doubling stages)."""
    rng = np.random.default_rng(4)
    A = np.tril(rng.standard_normal((16, 16)) * 0.3, -1)
    assert np.array_equal(np.linalg.matrix_power(A, 16), np.zeros((16, 16)))
    assert np.abs(np.linalg.matrix_power(A, 15)).max() > 0
    X = forms._unit_lower_inverse_neumann(A)
    np.testing.assert_allclose(X @ (np.eye(16) + A), np.eye(16), atol=1e-12)
    np.testing.assert_allclose(X, forms._unit_lower_inverse_subst(A), atol=1e-13)


def test_exponent_range_of_16_token_chunks():
    """With g >= -5 a 16-token chunk keeps every e^{+-Gamma} normal in fp32 (|Gamma| <= 80 <
    ln FLT_MAX = 88.7); a 32-token chunk without an anchor overflows (smzdm "反转二": bigger
    chunks need an exponent-centring anchor)."""
    f32 = np.finfo(np.float32)
    G16 = np.float32(-5.0 * 16)
    with np.errstate(over="ignore"):
        assert np.isfinite(np.exp(-G16)) and np.exp(G16) >= f32.tiny
        G32 = np.float32(-5.0 * 32)
        assert not np.isfinite(np.exp(-G32))
        # anchored at the chunk midpoint, the factors stay within e^{+-80}
        assert np.isfinite(np.exp(-(G32 - G32 / 2)))


def test_state_is_32kib_in_bf16():
    """The 128x128 state is exactly 32 KB in bf16 (smzdm "KDA 内核到底难在哪")."""
    assert 128 * 128 * 2 == 32 * 1024
