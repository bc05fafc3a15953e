"""Pins of the decode-side oracle (oracle/decode.py) against closed forms,
hand-worked cases and brute force.

[FD] = Flash-dLLM paper summary page, 方法步骤详情 steps 2 and 3;
[FST] = Fast-dLLM article, 并行解碼新策略.
"""
import itertools
import math

import numpy as np
import pytest

from oracle import decode as D


# ---------------------------------------------------------------- confidence

@pytest.mark.parametrize("V,c", [(1, 0.0), (7, -3.5), (1000, 12.0), (65536, 0.25)])
def test_uniform_row_has_confidence_one_over_v_and_token_zero(V, c):
    tok, conf = D.confidence_argmax(np.full((2, V), c))
    assert list(tok) == [0, 0]
    assert np.all(conf == 1.0 / V)


@pytest.mark.parametrize("V,p,a", [(2, 1, 1.0), (10, 3, 2.5), (4099, 4098, 9.0), (131072, 77, 14.0)])
def test_single_peak_closed_form(V, p, a):
    z = np.zeros((1, V))
    z[0, p] = a
    tok, conf = D.confidence_argmax(z)
    assert tok[0] == p
    # softmax of one logit a among V-1 zeros
    assert conf[0] == pytest.approx(1.0 / (1.0 + (V - 1) * math.exp(-a)), rel=1e-13)


def test_two_token_row_is_a_sigmoid_of_the_gap():
    for a, b in [(0.0, 1.0), (3.0, -2.0), (-7.25, -7.0)]:
        tok, conf = D.confidence_argmax(np.array([[a, b]]))
        assert tok[0] == (0 if a >= b else 1)
        assert conf[0] == pytest.approx(1.0 / (1.0 + math.exp(-abs(a - b))), rel=1e-14)


def test_tied_peaks_take_the_lowest_token():
    V = 5000
    z = np.zeros((3, V))
    for r, (p1, p2) in enumerate([(10, 4000), (0, 4999), (2047, 2048)]):
        z[r, p1] = z[r, p2] = 6.0
    tok, conf = D.confidence_argmax(z)
    assert list(tok) == [10, 0, 2047]
    assert np.allclose(conf, 1.0 / (2.0 + (V - 2) * math.exp(-6.0)), rtol=1e-13)


def test_confidence_against_the_unshifted_softmax_and_shift_invariance():
    rng = np.random.default_rng(5)
    z = rng.normal(0, 3, size=(6, 37))
    tok, conf = D.confidence_argmax(z)
    for r in range(6):
        e = [math.exp(v) for v in z[r]]            # small logits: no overflow
        p = [v / sum(e) for v in e]
        assert tok[r] == max(range(37), key=lambda i: (p[i], -i))
        assert conf[r] == pytest.approx(max(p), rel=1e-13)
    tok2, conf2 = D.confidence_argmax(z + 1000.0)  # shifted: overflows unless max is subtracted
    assert np.array_equal(tok, tok2)
    assert np.allclose(conf, conf2, rtol=1e-12)


# ---------------------------------------------------------------- commit rule

def test_commit_hand_example():
    conf = np.array([0.95, 0.5, 0.9, 0.2,      # seq 0: two at or above 0.9
                     0.3, 0.6, 0.6,            # seq 1: none; tie -> lowest row
                     0.91])                    # seq 3 (seq 2 is empty)
    cu = [0, 4, 7, 7, 8]
    commit, n = D.confidence_commit(conf, cu, 0.9)
    assert commit.tolist() == [True, False, True, False, False, True, False, True]
    assert n.tolist() == [2, 1, 0, 1]


def test_commit_brute_force_properties():
    rng = np.random.default_rng(11)
    for trial in range(300):
        lens = rng.integers(0, 6, size=rng.integers(1, 5))
        cu = np.concatenate([[0], np.cumsum(lens)])
        conf = rng.choice([0.1, 0.5, 0.8, 0.9, 0.95], size=int(cu[-1]))
        eps = float(rng.choice([0.8, 0.9]))
        commit, n = D.confidence_commit(conf, cu, eps)
        for b in range(len(lens)):
            s = slice(cu[b], cu[b + 1])
            c, m = conf[s], commit[s]
            assert n[b] == m.sum()
            if len(c) == 0:
                assert n[b] == 0
            elif (c >= eps).any():
                assert np.array_equal(m, c >= eps)
            else:
                # exactly one: the first row holding the sequence's largest confidence
                want = [i == min(j for j in range(len(c)) if c[j] == c.max()) for i in range(len(c))]
                assert m.tolist() == want


# ---------------------------------------------------------------- verify scan

def test_verify_hand_example():
    draft = [5, 6, 7, 8, 9,   1, 2,   3]
    pred = [5, 6, 0, 8, 9,    1, 2,   4]
    conf = [0.9, 0.8, 0.99, 0.99, 0.99,   0.85, 0.79,   0.99]
    cu = [0, 5, 7, 7, 8]
    acc, n = D.verify_accept(draft, pred, conf, cu, 0.8)
    # seq 0: row 1 sits exactly at gamma (accepted), row 2 mismatches, rows 3-4
    # match but come after the first failure
    assert acc.tolist() == [True, True, False, False, False, True, False, False]
    assert n.tolist() == [2, 1, 0, 0]


@pytest.mark.parametrize("L", range(0, 7))
def test_verify_exhaustive_prefix_length(L):
    for bits in itertools.product([0, 1, 2], repeat=L):
        # 0: accepted, 1: token mismatch, 2: confidence below gamma
        draft = [3] * L
        pred = [4 if b == 1 else 3 for b in bits]
        conf = [0.5 if b == 2 else 0.9 for b in bits]
        acc, n = D.verify_accept(draft, pred, conf, [0, L], 0.8)
        s = "".join("a" if b == 0 else "x" for b in bits)
        lead = len(s) - len(s.lstrip("a"))
        assert n[0] == lead
        assert acc.tolist() == [i < lead for i in range(L)]
