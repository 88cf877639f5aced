"""Pins for the LVSA mask oracle: hand-worked examples, invariants the page
states, and a brute-force restatement by rank counting."""
import itertools
import json
import os

import numpy as np
import pytest

import oracle


def test_worked_examples(golden_dir):
    with open(os.path.join(golden_dir, "lvsa_worked_examples.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        for t, want in c["sets"].items():
            got = oracle.attend_set(int(t), c["T"], c["C"], c["W"], c["T_per"], c["s"])
            assert got == want, (c, t)


def _rank_window(t, T, k):
    """N_k(t) by rank counting: f is in iff fewer than k frames g have (|g-t|, g) < (|f-t|, f)."""
    out = set()
    for f in range(T):
        r = sum(1 for g in range(T) if (abs(g - t), g) < (abs(f - t), f))
        if r < k:
            out.add(f)
    return out


def _brute(t, T, C, W, T_per, s):
    G = {f for f in range(T) if (f - s) % T_per == 0}
    target = min(C, T)
    for k in range(min(W, T), T + 1):
        A = G | _rank_window(t, T, k)
        if len(A) >= target:
            return sorted(A)
    return sorted(G | set(range(T)))


SWEEP = [
    (T, C, W, T_per, s)
    for T in (1, 2, 3, 5, 8, 11)
    for C in (1, 2, 3, 5, 9, 13)
    for W in (1, 2, 3, 6)
    for T_per in (1, 2, 3, 4)
    for s in (0, 1, 5)
]


@pytest.mark.parametrize("T,C,W,T_per,s", SWEEP[::3])
def test_brute_force(T, C, W, T_per, s):
    for t in range(T):
        assert oracle.attend_set(t, T, C, W, T_per, s) == _brute(t, T, C, W, T_per, s)


@pytest.mark.parametrize("T,C,W,T_per,s", SWEEP)
def test_invariants(T, C, W, T_per, s):
    G = set(oracle.anchors(T, T_per, s))
    for t in range(T):
        A = oracle.attend_set(t, T, C, W, T_per, s)
        As = set(A)
        assert A == sorted(As)
        assert t in As
        assert G <= As
        base = set(sorted(range(T), key=lambda f: (abs(f - t), f))[: min(W, T)])
        assert base <= As
        # window part is one contiguous run of frames containing t
        win = sorted(As - (G - base))
        lo, hi = min(win), max(win)
        assert set(range(lo, hi + 1)) - G <= As
        if len(G | base) <= min(C, T):
            assert len(A) == min(C, T)  # budget met exactly
        else:
            assert As == G | base  # over budget: kept whole, nothing added
        if T <= C:
            assert A == list(range(T))


@pytest.mark.parametrize("T,T_per", [(4, 2), (126, 8), (21, 8), (13, 5), (7, 1)])
def test_rotation_exactly_once(T, T_per):
    for s0 in range(3):
        counts = np.zeros(T, dtype=int)
        for s in range(s0, s0 + T_per):
            for f in oracle.anchors(T, T_per, s):
                counts[f] += 1
        assert np.all(counts == 1)


def test_budget_met_on_long_video():
    # 6x-length Wan-1.3B mask: every query frame sees exactly C = 21 frames for every step
    for s in range(8):
        idx, cnt = oracle.lvsa_mask(126, 21, 5, 8, s)
        assert np.all(cnt == 21)
        assert idx.shape == (126, 21)
        assert np.all(np.diff(idx, axis=1) > 0)
        assert oracle.lvsa_capacity(126, 21, 5, 8, s) == 21


def test_full_mask_when_T_le_C():
    idx, cnt = oracle.lvsa_mask(21, 21, 5, 8, 0)
    assert np.all(cnt == 21)
    assert np.all(idx == np.arange(21)[None, :])


def test_over_budget_capacity():
    # anchors every frame (T_per = 1) plus window 3 with C = 2: A(t) is everything
    idx, cnt = oracle.lvsa_mask(6, 2, 3, 1, 0)
    assert np.all(cnt == 6)
    # G = {0, 3} (T_per=3), W=4 > C=3 -> kept whole: |A(t)| = |G ∪ N_4(t)|
    for t in range(8):
        A = oracle.attend_set(t, 8, 3, 4, 3, 0)
        assert len(A) >= 4
    assert oracle.lvsa_capacity(8, 3, 4, 3, 0) == max(len(oracle.attend_set(t, 8, 3, 4, 3, 0)) for t in range(8))


def test_planted_tie_mistake_is_caught(golden_dir, monkeypatch):
    """A nearest order that breaks ties towards the later frame must fail the worked examples."""
    import oracle.lvsa as L

    monkeypatch.setattr(L, "nearest_order", lambda t, T: sorted(range(T), key=lambda f: (abs(f - t), -f)))
    with open(os.path.join(golden_dir, "lvsa_worked_examples.json")) as f:
        g = json.load(f)
    bad = 0
    for c in g["cases"]:
        for t, want in c["sets"].items():
            bad += L.attend_set(int(t), c["T"], c["C"], c["W"], c["T_per"], c["s"]) != want
    assert bad > 0


def test_rejects_bad_params():
    for args in [(0, 4, 0, 2, 2, 0), (0, 4, 3, 0, 2, 0), (0, 4, 3, 2, 0, 0), (4, 4, 3, 2, 2, 0)]:
        with pytest.raises(ValueError):
            oracle.attend_set(*args)
