"""Pins of the oracle's top-k candidate export (no GPU).

Readings T1-T4: the k tokens with the largest float32-rounded logits, ties to the lower id, with
their softmax probabilities over the whole vocabulary; token -1 / probability 0 past V; every
row.  Pinned by a hand-built case with rational probabilities, brute-force loops that rank by
repeated selection instead of sorting, the k = 1 case against the separately pinned statistics,
the k = V case (a permutation whose probabilities sum to one), and exact ties.
"""
import math

import numpy as np
import pytest

from oracle import token_stats, topk_candidates
from decoding_step_amd.synth import BlockStream, make_weights, stream


def test_topk_hand_built(golden):
    g = golden("topk_handbuilt.json")
    h = np.array([g["hidden"]], np.float32)
    W = np.array(g["W"], np.float32)
    out = topk_candidates(h, W, g["k"])
    assert out["tok"][0].tolist() == g["tok"]
    np.testing.assert_allclose(out["prob"][0], g["prob"], rtol=1e-6, atol=0)


def _brute(hf, Wf, k):
    """Loops: exactly rounded logits, ranking by repeated selection of the best remaining token."""
    out = []
    V = Wf.shape[0]
    for r in range(hf.shape[0]):
        z = [math.fsum(float(hf[r, j]) * float(Wf[v, j]) for j in range(hf.shape[1])) for v in range(V)]
        z32 = [float(np.float32(x)) for x in z]
        zmax = max(z)
        S = math.fsum(math.exp(x - zmax) for x in z)
        left = list(range(V))
        toks, probs = [], []
        for _ in range(k):
            if not left:
                toks.append(-1)
                probs.append(0.0)
                continue
            best = left[0]
            for v in left[1:]:
                if z32[v] > z32[best]:       # strict: an equal logit keeps the lower id
                    best = v
            left.remove(best)
            toks.append(best)
            probs.append(math.exp(z[best] - zmax) / S)
        out.append((toks, probs))
    return out


@pytest.mark.parametrize("V,H,k,dtype", [(37, 8, 5, "f32"), (64, 16, 8, "bf16"), (5, 4, 8, "f32"), (1, 8, 3, "bf16")])
def test_topk_brute_force(V, H, k, dtype):
    W = make_weights(V, H, dtype, seed=3)
    g = stream(41, V, H)
    h = (g.standard_normal((6, H)) * 2.0).astype(np.float32)
    if dtype == "bf16":
        from decoding_step_amd.synth import bf16_bits, bf16_to_f32
        h = bf16_bits(h)
        hf, Wf = bf16_to_f32(h), bf16_to_f32(W)
    else:
        hf, Wf = h, W
    got = topk_candidates(h, W, k)
    for r, (toks, probs) in enumerate(_brute(hf, Wf, k)):
        assert got["tok"][r].tolist() == toks
        np.testing.assert_allclose(got["prob"][r], np.array(probs, np.float32), rtol=1e-6, atol=1e-30)


def test_k1_is_the_candidate_and_its_confidence():
    W = make_weights(3001, 64, "bf16")
    h = BlockStream(W, 24, 5, 40.0).hidden(0, 0)
    st = token_stats(h, W)
    tk = topk_candidates(h, W, 1)
    assert np.array_equal(tk["tok"][:, 0], st["tok"])
    np.testing.assert_allclose(tk["prob"][:, 0], st["conf"], rtol=1e-7)


def test_k_equal_v_is_a_permutation_that_sums_to_one():
    V, H = 97, 32
    W = make_weights(V, H, "f32", seed=5)
    h = (stream(42, V).standard_normal((5, H)) * 3.0).astype(np.float32)
    tk = topk_candidates(h, W, V)
    for r in range(5):
        assert sorted(tk["tok"][r].tolist()) == list(range(V))
        assert abs(math.fsum(tk["prob"][r].astype(np.float64)) - 1.0) < 1e-5
        assert np.all(np.diff(tk["prob"][r]) <= 0)              # best first


def test_exact_ties_rank_by_id():
    # zero hidden state: every logit 0, so the ranking is 0, 1, 2, ... with probability 1/V each
    V, H = 50, 16
    W = make_weights(V, H, "f32")
    tk = topk_candidates(np.zeros((2, H), np.float32), W, 6)
    assert tk["tok"].tolist() == [[0, 1, 2, 3, 4, 5]] * 2
    assert np.all(tk["prob"] == np.float32(1.0 / V))
    # duplicated vocabulary rows give equal logits: the copies rank in id order, adjacent
    W2 = make_weights(40, H, "f32", seed=9)
    W2[[7, 21, 33]] = W2[12]
    h = (W2[12] * 4.0)[None, :]
    tk = topk_candidates(h, W2, 4)
    assert tk["tok"][0].tolist() == [7, 12, 21, 33]
    assert len(set(tk["prob"][0].tolist())) == 1


def test_planted_token_ranks_first_and_shapes_follow_hidden():
    W = make_weights(2003, 64, "bf16")
    bs = BlockStream(W, 6, 77, 200.0)
    h = bs.hidden(0, 0)
    tk = topk_candidates(h.reshape(2, 3, 64), W, 3)
    assert tk["tok"].shape == (2, 3, 3) and tk["prob"].shape == (2, 3, 3)
    assert np.array_equal(tk["tok"].reshape(6, 3)[:, 0], bs.planted(0, 0))


def test_ranking_uses_float32_rounded_logits():
    # z0 = 1 and z1 = 1 + 2^-30 differ in float64 but round to the same float32: a tie, so the
    # lower id ranks first (the arg-max takes the same decision in the same precision)
    W = np.array([[1.0, 0.0], [1.0, 2.0 ** -30], [0.5, 0.0]], np.float32)
    h = np.array([[1.0, 1.0]], np.float32)
    tk = topk_candidates(h, W, 3)
    assert tk["tok"][0].tolist() == [0, 1, 2]
    assert token_stats(h, W)["tok"][0] == 0
