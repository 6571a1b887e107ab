"""Pins of the oracle's LM head + confidence + candidate (no GPU).

Each test fixes the oracle against something other than itself: a closed
form, a hand-built case, brute-force loops, or a property of the softmax.
"""
import math

import numpy as np
import pytest

from oracle import token_stats, lm_head_logits
from decoding_step_amd.synth import bf16_bits, bf16_to_f32, make_weights, stream


def f32(x):
    return np.float32(x)


def test_zero_hidden_gives_uniform_confidence():
    # h = 0 => every logit is 0 => softmax is uniform: conf = 1/V, tie => token 0, gap 0.
    V, H = 1024, 64
    W = make_weights(V, H, "f32")
    st = token_stats(np.zeros((3, H), np.float32), W)
    assert np.all(st["conf"] == f32(1.0 / 1024))            # 0.0009765625 exactly
    assert np.all(st["tok"] == 0)
    assert np.all(st["gap"] == 0)


def test_two_token_vocabulary_is_a_sigmoid():
    # V = 2, H = 1: z = (x w0, x w1); conf = 1 / (1 + exp(-|z1 - z0|)).
    cases = [(1.5, 0.25, -0.75), (-2.0, 0.5, 0.125), (0.375, 3.0, 3.0), (4.0, -1.0, 0.5)]
    for x, w0, w1 in cases:
        st = token_stats(np.array([[x]], np.float32), np.array([[w0], [w1]], np.float32))
        d = abs(x * w1 - x * w0)
        assert st["conf"][0] == f32(1.0 / (1.0 + math.exp(-d)))
        want = 0 if x * w0 >= x * w1 else 1
        assert st["tok"][0] == want
        assert st["gap"][0] == f32(d)


def test_hand_built_softmax(golden):
    g = golden("softmax_handbuilt.json")
    h = np.array([g["hidden"]], np.float32)
    W = np.array(g["W"], np.float32)
    st = token_stats(h, W)
    assert st["tok"][0] == g["tok"]
    assert abs(float(st["conf"][0]) - g["conf"]) < 1e-6
    assert abs(float(st["gap"][0]) - g["gap"]) < 1e-6


def _brute(hf, Wf):
    """Loops over rows, tokens and the hidden dimension with exactly rounded sums."""
    out = []
    for r in range(hf.shape[0]):
        z = [math.fsum(float(hf[r, k]) * float(Wf[v, k]) for k in range(hf.shape[1])) for v in range(Wf.shape[0])]
        z32 = [float(np.float32(x)) for x in z]
        best = 0
        for v in range(1, len(z32)):
            if z32[v] > z32[best]:
                best = v
        second = max([z32[v] for v in range(len(z32)) if v != best], default=-math.inf)
        zmax = max(z)
        S = math.fsum(math.exp(x - zmax) for x in z)
        out.append((best, 1.0 / S, z32[best] - second))
    return out


@pytest.mark.parametrize("V,H,M,dt", [(37, 12, 5, "bf16"), (53, 7, 3, "f32"), (16, 33, 4, "bf16")])
def test_brute_force_tiny(V, H, M, dt):
    g = stream(123, V, H)
    Wf = (g.standard_normal((V, H)) * 0.7).astype(np.float32)
    hf = (g.standard_normal((M, H)) * 2.0).astype(np.float32)
    if dt == "bf16":
        W, h = bf16_bits(Wf), bf16_bits(hf)
        Wf, hf = bf16_to_f32(W), bf16_to_f32(h)
    else:
        W, h = Wf, hf
    st = token_stats(h, W)
    for r, (tok, conf, gap) in enumerate(_brute(hf, Wf)):
        assert st["tok"][r] == tok
        assert st["conf"][r] == f32(conf)
        assert abs(float(st["gap"][r]) - gap) <= 1e-6 * max(1.0, abs(gap))


def test_logit_orientation_non_square():
    # z[r, v] = sum_k h[r, k] W[v, k]: a transposed operand or swapped axis fails on these shapes.
    h = np.array([[1, 2, 3]], np.float32)
    W = np.array([[1, 0, 0], [0, 1, 0], [0, 0, 1], [1, 1, 1], [0, 0, -1]], np.float32)
    z = lm_head_logits(h, W)
    assert z.shape == (1, 5)
    assert np.array_equal(z[0], [1, 2, 3, 6, -3])
    st = token_stats(h, W)
    assert st["tok"][0] == 3 and st["gap"][0] == 3


def test_exact_tie_goes_to_lowest_token():
    V, H = 64, 16
    g = stream(7)
    W = (g.standard_normal((V, H))).astype(np.float32)
    W[41] = W[13] = W[13] * 0 + 3 * np.abs(W[13])     # two identical, dominant rows
    h = np.abs(g.standard_normal((2, H))).astype(np.float32)
    st = token_stats(h, W)
    assert np.all(st["tok"] == 13)
    assert np.all(st["gap"] == 0)


def test_permuting_the_vocabulary_permutes_the_candidate():
    V, H = 211, 24
    g = stream(11)
    W = bf16_bits(g.standard_normal((V, H)).astype(np.float32))
    h = bf16_bits((g.standard_normal((6, H)) * 3).astype(np.float32))
    perm = g.permutation(V)
    a = token_stats(h, W)
    b = token_stats(h, W[perm])
    assert np.array_equal(perm[b["tok"]], a["tok"])
    np.testing.assert_allclose(b["conf"], a["conf"], rtol=1e-6)
    np.testing.assert_allclose(b["gap"], a["gap"], rtol=1e-6)


def test_common_logit_shift_changes_nothing():
    # Append a constant input 1 and a constant weight c: every logit moves by c.  With c = 1000 a
    # softmax that forgot to subtract the maximum overflows.
    V, H = 97, 16
    g = stream(5)
    W = g.standard_normal((V, H)).astype(np.float32)
    h = (g.standard_normal((4, H)) * 2).astype(np.float32)
    W2 = np.concatenate([W, np.full((V, 1), 1000.0, np.float32)], axis=1)
    h2 = np.concatenate([h, np.ones((4, 1), np.float32)], axis=1)
    a, b = token_stats(h, W), token_stats(h2, W2)
    assert np.array_equal(a["tok"], b["tok"])
    np.testing.assert_allclose(b["conf"], a["conf"], rtol=1e-5)
    assert np.all(np.isfinite(b["conf"]))


def test_one_token_vocabulary():
    st = token_stats(np.ones((2, 4), np.float32), np.ones((1, 4), np.float32))
    assert np.all(st["conf"] == 1) and np.all(st["tok"] == 0) and np.all(np.isinf(st["gap"]))


@pytest.mark.slow
def test_planted_peak_at_full_vocabulary():
    # 8B-class shape: a hidden state 45 x W[t]/||W[t]|| + N(0,1) puts logit ~40.7 on t and at most ~7
    # elsewhere, so the softmax mass outside t is ~1e-12: candidate t, confidence 1.0 in float32.
    V, H = 126464, 2048
    W = make_weights(V, H, "bf16")
    g = stream(99)
    t = np.array([5, 126463])
    w = bf16_to_f32(W[t]).astype(np.float64)
    h = 45.0 * w / np.linalg.norm(w, axis=1, keepdims=True) + g.standard_normal((2, H))
    st = token_stats(bf16_bits(h.astype(np.float32)), W)
    assert np.array_equal(st["tok"], t)
    assert np.all(st["conf"] == f32(1.0))
    assert np.all(st["gap"] > 20)
