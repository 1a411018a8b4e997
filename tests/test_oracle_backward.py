"""Pins of the fp64 backward oracle (``oracle/backward.py``) to facts outside itself (no GPU).

The backward is not on the pages; the function it differentiates is the
forward of the aiml.sh page (lab.py, standard_attention).  The pins:

- central finite differences of the C forward oracle (``oracle.attention_dense``
  in fp64), which shares none of the gradient formulas: a wrong sign, a dropped
  softmax-Jacobian term, a missing scale or a transposed product fails them;
- invariants: keys shifted together leave the softmax unchanged, so the
  key gradients sum to zero; the value gradients sum to the sum of dO; the
  causal row 0 sees one key, so its query gradient is zero;
- closed forms: constant value rows (every gradient but dV vanishes) and
  Q = 0 (uniform causal weights 1/(i+1));
- a negative control: the oracle with the delta term dropped fails the
  finite-difference pin.
"""
import numpy as np
import pytest

from oracle import attention_dense
from oracle.backward import attention_backward, row_deltas


def _loss(q, k, v, g, causal, scale):
    o, _ = attention_dense(q, k, v, causal=causal, scale=scale)
    return float((o.reshape(g.shape) * g).sum())


def _finite_difference(q, k, v, g, causal, scale, h=1e-5):
    """d(sum O*g)/d(q, k, v) by central differences of the C forward oracle."""
    grads = []
    for which in range(3):
        base = [q.copy(), k.copy(), v.copy()]
        out = np.zeros_like(base[which])
        it = np.nditer(base[which], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            plus = [t.copy() for t in base]; minus = [t.copy() for t in base]
            plus[which][idx] += h; minus[which][idx] -= h
            out[idx] = (_loss(*plus, g, causal, scale) - _loss(*minus, g, causal, scale)) / (2 * h)
        grads.append(out)
    return grads


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("scale", [0.7, -0.4])
def test_finite_differences_of_the_forward(causal, scale):
    rng = np.random.default_rng(3)
    q, k, v, g = (rng.uniform(-1, 1, (1, 2, 6, 4)) for _ in range(4))
    dq, dk, dv = attention_backward(q, k, v, g, causal=causal, scale=scale)
    fq, fk, fv = _finite_difference(q, k, v, g, causal, scale)
    for name, a, f in (("dq", dq, fq), ("dk", dk, fk), ("dv", dv, fv)):
        assert np.abs(a - f.reshape(a.shape)).max() <= 1e-8, name


def test_negative_control_without_delta_fails():
    """dS = P * dP (delta dropped) must be caught by the finite-difference pin."""
    rng = np.random.default_rng(4)
    q, k, v, g = (rng.uniform(-1, 1, (1, 1, 5, 3)) for _ in range(4))
    scale = 0.9
    qh, kh, vh, gh = q[0, 0], k[0, 0], v[0, 0], g[0, 0]
    s = scale * qh @ kh.T
    s = np.where(np.tril(np.ones((5, 5), dtype=bool)), s, -np.inf)
    p = np.exp(s - s.max(1, keepdims=True)); p /= p.sum(1, keepdims=True)
    wrong_dq = scale * (p * (gh @ vh.T)) @ kh
    fq, _, _ = _finite_difference(q, k, v, g, True, scale)
    assert np.abs(wrong_dq - fq[0, 0]).max() > 1e-3


def test_key_shift_invariance_and_value_sums():
    """Adding one vector to every key leaves each softmax row unchanged, so the key
    gradients sum to zero over keys; each row's weights sum to one, so the value
    gradients sum to the sum of dO rows.  Causal row 0 has one key: dQ_0 = 0."""
    rng = np.random.default_rng(5)
    q, k, v, g = (rng.uniform(-1, 1, (2, 3, 33, 8)) for _ in range(4))
    for causal in (True, False):
        dq, dk, dv = attention_backward(q, k, v, g, causal=causal, scale=0.8)
        assert np.abs(dk.sum(axis=1)).max() <= 1e-12
        assert np.abs(dv.sum(axis=1) - g.reshape(6, 33, 8).sum(axis=1)).max() <= 1e-12
        if causal:
            assert np.abs(dq[:, 0]).max() == 0.0


def test_constant_values_closed_form():
    """v_j = w for all j: O_i = w whatever the weights, so dQ = dK = 0 and
    dV_j = sum_i P_ij dO_i (checked through its column sums with P from scipy-free
    softmax of the scores)."""
    rng = np.random.default_rng(6)
    q, k, g = (rng.uniform(-1, 1, (1, 1, 17, 5)) for _ in range(3))
    w = rng.uniform(-1, 1, 5)
    v = np.broadcast_to(w, (1, 1, 17, 5)).copy()
    dq, dk, dv = attention_backward(q, k, v, g, causal=True, scale=0.6)
    assert np.abs(dq).max() <= 1e-14 and np.abs(dk).max() <= 1e-14
    s = 0.6 * q[0, 0] @ k[0, 0].T
    s = np.where(np.tril(np.ones((17, 17), dtype=bool)), s, -np.inf)
    p = np.exp(s - s.max(1, keepdims=True)); p /= p.sum(1, keepdims=True)
    assert np.abs(dv[0] - p.T @ g[0, 0]).max() <= 1e-14


def test_zero_query_closed_form():
    """Q = 0: causal weights are 1/(i+1), so dV_j = sum_{i>=j} dO_i / (i+1), and
    dQ_i = scale * sum_{j<=i} (dO_i.(v_j - mean_{l<=i} v_l)) / (i+1) * k_j."""
    rng = np.random.default_rng(7)
    S, D, scale = 12, 4, 0.5
    k, v, g = (rng.uniform(-1, 1, (1, 1, S, D)) for _ in range(3))
    q = np.zeros((1, 1, S, D))
    dq, dk, dv = attention_backward(q, k, v, g, causal=True, scale=scale)
    kh, vh, gh = k[0, 0], v[0, 0], g[0, 0]
    want_dv = np.array([sum(gh[i] / (i + 1) for i in range(j, S)) for j in range(S)])
    assert np.abs(dv[0] - want_dv).max() <= 1e-14
    want_dq = np.zeros((S, D))
    for i in range(S):
        mean_v = vh[: i + 1].mean(axis=0)
        for j in range(i + 1):
            want_dq[i] += scale * (gh[i] @ (vh[j] - mean_v)) / (i + 1) * kh[j]
    assert np.abs(dq[0] - want_dq).max() <= 1e-14


def test_row_deltas_equal_the_softmax_weighted_dp():
    """delta_i = dO_i . O_i equals sum_j P_ij (dO V^T)_ij, the form the gradients use."""
    rng = np.random.default_rng(8)
    q, k, v, g = (rng.uniform(-1, 1, (1, 2, 9, 6)) for _ in range(4))
    o, _ = attention_dense(q, k, v, causal=True, scale=0.7)
    delta = row_deltas(o.reshape(q.shape), g)
    for h in range(2):
        s = 0.7 * q[0, h] @ k[0, h].T
        s = np.where(np.tril(np.ones((9, 9), dtype=bool)), s, -np.inf)
        p = np.exp(s - s.max(1, keepdims=True)); p /= p.sum(1, keepdims=True)
        assert np.abs(delta[h] - (p * (g[0, h] @ v[0, h].T)).sum(1)).max() <= 1e-14


def test_bf16_storage_and_head_selection():
    """bf16 bit patterns decode exactly; selected heads equal the full computation."""
    rng = np.random.default_rng(9)
    x = rng.uniform(-1, 1, (4, 2, 10, 8)).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    dec = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    full = attention_backward(dec[0:1], dec[1:2], dec[2:3], dec[3:4], causal=True)
    part = attention_backward(bits[0:1], bits[1:2], bits[2:3], bits[3:4], causal=True, dtype="bf16",
                              bh_idx=[1])
    for a, b in zip(full, part):
        assert np.array_equal(a[1:2], b)
