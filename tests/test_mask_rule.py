"""The ping-pong kernel's per-tile mask decisions, restated on the host and
checked against the plain visibility rule of the aiml.sh page "Speed up long
contexts with FlashAttention" (lab.py, tiled_flash_attention: row i sees keys
0..i under the causal rule, 0..S-1 otherwise).

The kernel (csrc/fa_fwd_pingpong.h) copies whole BK-key tiles; a last tile cut
short by S is copied as keys S-BK..S-1, so its first rows repeat keys of the
tile before.  Per item (256 query rows) and wave (32 rows) it bounds the tiles
it multiplies (t < n_w) and the first tile it masks (t_mask), and on a masked
tile it hides element (kb, r) of lane half h, LDS row j = 32 kb + 8 (r // 4) +
4 h + r % 4 (key kv_row0 + j), when the unsigned value c + b exceeds hi, with
c = 32 kb + 8 (r // 4) + r % 4, b = 4 h - (kv0 - kv_row0) and hi = qi - kv0
(causal) or BK.  This test enumerates those decisions for every element of
every tile of every wave over many lengths and checks that each row's visible
keys are exactly the rule's, each counted once, and that an unmasked tile
hides nothing the rule shows and shows nothing it hides.
"""
from __future__ import annotations

import numpy as np
import pytest

BQ, QW, WAVES = 256, 32, 8


def item_tiles(qb: int, S: int, BK: int, causal: bool) -> int:
    kv_end = min(qb * BQ + BQ, S) if causal else S
    return (kv_end + BK - 1) // BK


def span(qb: int, wave: int, S: int, BK: int, causal: bool):
    q0w = qb * BQ + wave * QW
    n_tiles = item_tiles(qb, S, BK, causal)
    if q0w >= S:
        n_w = 0
    else:
        n_w = min(n_tiles, (min(q0w + QW, S) - 1) // BK + 1) if causal else n_tiles
    t_mask = min((q0w + 1) // BK, S // BK) if causal else S // BK
    return q0w, n_w, t_mask


def tile_elements(BK: int):
    """(key offset j within the tile's LDS rows, c, lane half) of every element a lane holds."""
    kb, r, h = np.meshgrid(np.arange(BK // 32), np.arange(16), np.arange(2), indexing="ij")
    c = 32 * kb + 8 * (r // 4) + r % 4
    j = c + 4 * h
    return j.ravel(), c.ravel(), h.ravel()


def check_length(S: int, BK: int, causal: bool):
    j, c, h = tile_elements(BK)
    n_qb = (S + BQ - 1) // BQ
    for qb in range(n_qb):
        for wave in range(WAVES):
            q0w, n_w, t_mask = span(qb, wave, S, BK, causal)
            for col in range(QW):
                qi = q0w + col
                if qi >= S:  # rows past S are computed but never stored
                    continue
                seen = np.zeros(S, dtype=np.int64)
                for t in range(n_w):
                    kv0 = t * BK
                    kv_row0 = min(kv0, S - BK)
                    key = kv_row0 + j
                    assert key.min() >= 0 and key.max() <= S - 1  # whole-tile copies stay inside the sequence
                    rule = (key >= kv0) & ((key <= qi) if causal else np.ones_like(key, dtype=bool))
                    if t < t_mask:
                        # an unmasked tile: every element is one the rule shows
                        assert rule.all(), (S, BK, causal, qb, wave, qi, t)
                        shown = np.ones_like(rule)
                    else:
                        assert not causal or qi >= kv0, (S, BK, qb, wave, qi, t)
                        b = 4 * h - (kv0 - kv_row0)
                        hi = (qi - kv0) if causal else BK
                        hidden = ((c + b) & 0xFFFFFFFF) > hi  # the kernel's unsigned compare
                        shown = ~hidden
                        assert np.array_equal(shown, rule), (S, BK, causal, qb, wave, qi, t)
                    np.add.at(seen, key[shown], 1)
                # tiles past n_w hold no key the row sees
                for t in range(n_w, item_tiles(qb, S, BK, causal)):
                    assert not causal or t * BK > qi, (S, BK, qb, wave, qi, t)
                want = np.zeros(S, dtype=np.int64)
                want[: (qi + 1 if causal else S)] = 1
                assert np.array_equal(seen, want), (S, BK, causal, qb, wave, qi)


LENGTHS = [64, 65, 100, 127, 128, 129, 191, 192, 255, 256, 257, 300, 383, 384, 511, 512, 513, 640, 777, 1000]


@pytest.mark.parametrize("BK", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_mask_decisions_match_visibility_rule(BK, causal):
    for S in LENGTHS:
        if S >= BK:  # the ping-pong variants take S >= BK
            check_length(S, BK, causal)


def test_mask_rule_catches_a_wrong_offset():
    """Negative control: dropping the repeated-rows offset b's shift breaks a cut-short tile."""
    S, BK = 200, 128
    j, c, h = tile_elements(BK)
    t, qi = 1, 199
    kv0, kv_row0 = t * BK, min(t * BK, S - BK)
    key = kv_row0 + j
    rule = (key >= kv0) & (key <= qi)
    wrong = ~((((c + 4 * h) & 0xFFFFFFFF) > qi - kv0))  # b without the - (kv0 - kv_row0) term
    assert not np.array_equal(wrong, rule)
