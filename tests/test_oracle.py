"""Pins of the CPU oracle to facts outside itself (no GPU).

Each test names what it pins and which plausible oracle mistake it would catch:
the page's printed worked example, 40-digit brute force, closed forms,
library routines (scipy's logsumexp/softmax) and invariants of attention.
"""
import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest
import scipy.special

from oracle import attention_dense, tiled_attention
from workloads import bf16_bits_to_float, page_qkv, round_to_bf16


def _golden(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- the page's worked example

def test_page_worked_example_outputs(golden_dir):
    """aiml.sh 'Speed up long contexts with FlashAttention', run-output.txt, equivalence_check.

    The printed first four outputs of rows 0 and 63 (6 decimals) pin the score
    scale, the causal limit, operand order and the normalisation at once.
    """
    g = _golden(golden_dir, "page_equivalence_check.json")
    q, k, v = page_qkv(g["seq_len"], g["head_dim"], seed=42)
    o, _, count = attention_dense(q, k, v, causal=True, with_count=True)
    assert [round(x, 6) for x in o[0, :4]] == g["sample_row0_first4"]
    assert [round(x, 6) for x in o[-1, :4]] == g["sample_last_row_first4"]
    assert count == g["standard_materialized_elements"]


def test_page_worked_example_tiled(golden_dir):
    """The same example through the tiled loop: counters and dense agreement.

    The page prints 1.388e-16 for max |dense - tiled|; the exact digit depends
    on summation order, so the bound is 1e-15 (a few ulps of values below 1).
    """
    g = _golden(golden_dir, "page_equivalence_check.json")
    q, k, v = page_qkv(g["seq_len"], g["head_dim"], seed=42)
    dense, _ = attention_dense(q, k, v, causal=True)
    tiled, _, meta = tiled_attention(q, k, v, g["block_q"], g["block_kv"], causal=True)
    assert np.abs(dense - tiled).max() <= 1e-15
    assert meta["tiles_visited"] == g["flash_tiles_visited"]
    assert meta["max_sram_score_tile_elements"] == g["flash_sram_tile_elements"]
    assert meta["materialized_nxn_elements"] == g["flash_materialized_hbm_elements"]
    assert [round(x, 6) for x in tiled[0, :4]] == g["sample_row0_first4"]
    assert [round(x, 6) for x in tiled[-1, :4]] == g["sample_last_row_first4"]


# ---------------------------------------------------------------- brute force at 40 digits

def _brute(q, k, v, causal, scale):
    getcontext().prec = 40
    S, D = q.shape
    sc = Decimal(scale)
    o = np.zeros((S, D))
    lse = np.zeros(S)
    for i in range(S):
        keys = range(i + 1) if causal else range(S)
        s = [sum(Decimal(q[i, c]) * Decimal(k[j, c]) for c in range(D)) * sc for j in keys]
        m = max(s)
        e = [(x - m).exp() for x in s]
        den = sum(e)
        for c in range(D):
            o[i, c] = float(sum(e[t] * Decimal(v[j, c]) for t, j in enumerate(keys)) / den)
        lse[i] = float(m + den.ln())
    return o, lse


@pytest.mark.parametrize("S,D", [(1, 1), (2, 3), (5, 4), (8, 2), (8, 4)])
@pytest.mark.parametrize("causal", [True, False])
def test_bruteforce_decimal(S, D, causal):
    rng = np.random.default_rng(S * 10 + D)
    q, k, v = (rng.uniform(-1.5, 1.5, size=(S, D)) for _ in range(3))
    scale = 1.0 / math.sqrt(D)
    o, lse = attention_dense(q, k, v, causal=causal, scale=scale)
    ob, lb = _brute(q, k, v, causal, scale)
    assert np.abs(o - ob).max() <= 1e-14
    assert np.abs(lse - lb).max() <= 1e-14


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("causal", [True, False])
def test_zero_query_closed_form(causal):
    """Q = 0 makes every score 0: O_i is the mean of the visible V rows and lse_i = ln(count)."""
    rng = np.random.default_rng(7)
    S, D = 97, 8
    q = np.zeros((S, D))
    k, v = rng.uniform(-0.8, 0.8, size=(2, S, D))
    o, lse = attention_dense(q, k, v, causal=causal)
    n = np.arange(1, S + 1) if causal else np.full(S, S)
    want = np.cumsum(v, axis=0) / n[:, None] if causal else np.broadcast_to(v.mean(0), (S, D))
    assert np.abs(o - want).max() <= 1e-14
    assert np.abs(lse - np.log(n)).max() <= 1e-14


def test_needle_and_no_overflow():
    """A huge scale makes softmax one-hot: O_i = V[argmax], lse_i = max score.

    Scores near 1e4 overflow exp() unless the row max is subtracted first, so
    this also pins the max subtraction.
    """
    rng = np.random.default_rng(3)
    S, D = 40, 4
    q, k, v = rng.uniform(-0.8, 0.8, size=(3, S, D))
    scale = 1e4
    o, lse = attention_dense(q, k, v, causal=True, scale=scale)
    s = (q @ k.T) * scale
    for i in range(S):
        row = s[i, : i + 1]
        j = int(np.argmax(row))
        gap = row[j] - np.partition(row, -2)[-2] if i else np.inf
        assert np.isfinite(o[i]).all()
        # always: max <= lse <= max + ln(number of visible keys)
        assert row[j] - 1e-9 <= lse[i] <= row[j] + math.log(i + 1) + 1e-9
        if gap > 50:
            assert np.abs(o[i] - v[j]).max() <= 1e-12
            assert abs(lse[i] - row[j]) <= 1e-12 * abs(row[j])


@pytest.mark.parametrize("causal", [True, False])
def test_library_softmax(causal):
    """scipy.special.logsumexp / softmax over numpy scores give the same O and lse."""
    rng = np.random.default_rng(11)
    S, D = 33, 16
    q, k, v = rng.uniform(-0.8, 0.8, size=(3, S, D))
    scale = 1.0 / math.sqrt(D)
    o, lse = attention_dense(q, k, v, causal=causal, scale=scale)
    s = (q @ k.T) * scale
    if causal:
        s = np.where(np.tril(np.ones((S, S), bool)), s, -np.inf)
    assert np.abs(lse - scipy.special.logsumexp(s, axis=1)).max() <= 1e-13
    assert np.abs(o - scipy.special.softmax(s, axis=1) @ v).max() <= 1e-14


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("dtype", ["f32", "bf16", "f64"])
def test_causal_row0_is_v0(dtype):
    """Causal row 0 sees only key 0: p_00 = 1, so O[0] = V[0] exactly and lse_0 = scale*q0.k0."""
    rng = np.random.default_rng(5)
    x = rng.uniform(-0.8, 0.8, size=(3, 2, 3, 20, 16)).astype(np.float32)
    if dtype == "bf16":
        q, k, v = (round_to_bf16(t) for t in x)
        vf = bf16_bits_to_float(v).astype(np.float64)
        qf, kf = (bf16_bits_to_float(t).astype(np.float64) for t in (q, k))
    elif dtype == "f32":
        q, k, v = x
        qf, kf, vf = (t.astype(np.float64) for t in x)
    else:
        q, k, v = (t.astype(np.float64) for t in x)
        qf, kf, vf = q, k, v
    o, lse = attention_dense(q, k, v, causal=True, dtype=dtype, scale=0.25)
    o = o.reshape(2, 3, 20, 16)
    lse = lse.reshape(2, 3, 20)
    assert np.array_equal(o[:, :, 0], vf[:, :, 0])
    want = (qf[:, :, 0] * kf[:, :, 0]).sum(-1) * 0.25
    assert np.abs(lse[:, :, 0] - want).max() <= 1e-15


def test_noncausal_single_key_returns_v():
    rng = np.random.default_rng(2)
    q, k, v = rng.uniform(-0.8, 0.8, size=(3, 1, 8))
    o, lse = attention_dense(q, k, v, causal=False)
    assert np.array_equal(o, v)


def test_causality():
    """Changing keys/values after row i leaves rows 0..i unchanged (bitwise)."""
    rng = np.random.default_rng(9)
    S, D, i = 30, 8, 17
    q, k, v = rng.uniform(-0.8, 0.8, size=(3, S, D))
    o1, l1 = attention_dense(q, k, v)
    k2, v2 = k.copy(), v.copy()
    k2[i + 1:] = rng.uniform(-3, 3, size=k2[i + 1:].shape)
    v2[i + 1:] = rng.uniform(-3, 3, size=v2[i + 1:].shape)
    o2, l2 = attention_dense(q, k2, v2)
    assert np.array_equal(o1[: i + 1], o2[: i + 1])
    assert np.array_equal(l1[: i + 1], l2[: i + 1])
    assert not np.array_equal(o1[i + 1:], o2[i + 1:])


def test_noncausal_key_permutation():
    """Non-causal attention is a set function of the (key, value) pairs."""
    rng = np.random.default_rng(4)
    S, D = 45, 8
    q, k, v = rng.uniform(-0.8, 0.8, size=(3, S, D))
    perm = rng.permutation(S)
    o1, l1 = attention_dense(q, k, v, causal=False)
    o2, l2 = attention_dense(q, k[perm], v[perm], causal=False)
    assert np.abs(o1 - o2).max() <= 1e-15
    assert np.abs(l1 - l2).max() <= 1e-14


def test_sampling_matches_full_and_heads_are_independent():
    """Row/head sampling returns the same rows as the full call; heads do not mix."""
    rng = np.random.default_rng(8)
    B, H, S, D = 2, 3, 21, 8
    q, k, v = rng.uniform(-0.8, 0.8, size=(3, B, H, S, D))
    o, lse = attention_dense(q, k, v, n_threads=3)
    bh = np.array([5, 0, 3])
    rows = np.array([20, 0, 7])
    os_, ls_ = attention_dense(q, k, v, bh_idx=bh, row_idx=rows, n_threads=2)
    assert np.array_equal(os_, o[bh][:, rows])
    assert np.array_equal(ls_, lse[bh][:, rows])
    # swapping two heads swaps their outputs
    q2, k2, v2 = (t.reshape(B * H, S, D)[[1, 0, 2, 3, 4, 5]].reshape(B, H, S, D) for t in (q, k, v))
    o2, _ = attention_dense(q2, k2, v2)
    assert np.array_equal(o2[0], o[1]) and np.array_equal(o2[1], o[0])


def test_storage_decoding_is_exact():
    """bf16 bit patterns and fp32 values decode to the same doubles as fp64 input."""
    rng = np.random.default_rng(6)
    x = rng.uniform(-0.8, 0.8, size=(3, 1, 2, 19, 8)).astype(np.float32)
    bits = [round_to_bf16(t) for t in x]
    wide = [bf16_bits_to_float(b).astype(np.float64) for b in bits]
    ob, lb = attention_dense(*bits, dtype="bf16")
    od, ld = attention_dense(*wide)
    assert np.array_equal(ob, od) and np.array_equal(lb, ld)
    of, lf = attention_dense(*x)
    od2, ld2 = attention_dense(*(t.astype(np.float64) for t in x))
    assert np.array_equal(of, od2) and np.array_equal(lf, ld2)


def test_round_to_bf16_ties_to_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e38], dtype=np.float32)
    bits = round_to_bf16(vals)
    back = bf16_bits_to_float(bits)
    assert back[0] == 1.0
    assert back[1] == 1.0                    # halfway, rounds to even
    assert back[2] == 1.0 + 2 ** -6          # halfway, rounds up to even
    assert back[3] == -2.5


def test_invalid_arguments_raise():
    q = np.zeros((4, 2))
    with pytest.raises(RuntimeError):
        attention_dense(q, q, q, row_idx=[4])
    with pytest.raises(RuntimeError):
        attention_dense(q, q, q, row_idx=[-1])


# ---------------------------------------------------------------- the tiled loop

@pytest.mark.parametrize("bq,bk", [(16, 16), (8, 32), (32, 8), (7, 5), (1, 1), (64, 64), (13, 64)])
@pytest.mark.parametrize("causal", [True, False])
def test_tiled_equals_dense(bq, bk, causal):
    """Block-size invariance of the method (page: dense and tiled agree to ~1e-16)."""
    q, k, v = page_qkv(64, 16, seed=42)
    od, ld = attention_dense(q, k, v, causal=causal)
    ot, lt, _ = tiled_attention(q, k, v, bq, bk, causal=causal)
    assert np.abs(od - ot).max() <= 1e-15
    assert np.abs(ld - lt).max() <= 1e-14


def test_tiled_ragged_multihead():
    rng = np.random.default_rng(12)
    q, k, v = rng.uniform(-0.8, 0.8, size=(3, 2, 2, 50, 8))
    od, ld = attention_dense(q, k, v)
    ot, lt, meta = tiled_attention(q, k, v, 16, 12)
    assert np.abs(od.reshape(ot.shape) - ot).max() <= 1e-15
    assert np.abs(ld.reshape(lt.shape) - lt).max() <= 1e-14
    from tiled_online_softmax_causal_amd.costmodel import causal_kv_tiles
    assert meta["tiles_visited"] == 4 * causal_kv_tiles(50, 16, 12)


def test_tiled_stress_rescaling():
    """Wide score range (uniform(-4,4) Q and K): the running max jumps often."""
    rng = np.random.default_rng(13)
    S, D = 96, 16
    q, k = rng.uniform(-4, 4, size=(2, S, D))
    v = rng.uniform(-0.8, 0.8, size=(S, D))
    od, ld = attention_dense(q, k, v)
    ot, lt, _ = tiled_attention(q, k, v, 16, 16)
    assert np.abs(od - ot).max() <= 1e-14
    assert np.abs(ld - lt).max() <= 1e-13


def test_negative_control_missing_rescale_is_caught():
    """The page's switch that skips the accumulator rescale must fail any parity bound used here."""
    q, k, v = page_qkv(64, 16, seed=42)
    od, _ = attention_dense(q, k, v)
    bad, _, _ = tiled_attention(q, k, v, 16, 16, rescale_previous_acc=False)
    assert np.abs(od - bad).max() > 1e-2
