"""The validity checks the GPU parity tests apply where several answers are correct
(tests/parity_util.py), run on the CPU: they accept the oracle's own answers and reject planted
mistakes (a wrong commit, a commit outside the mask, a missing forced commit, a wrong credit
update, a token that is not near-maximal)."""
import numpy as np
import pytest

import oracle
from parity_util import check_near_max_tokens, check_policy_replay

L = 8


def _step(rule, conf, tok, mask, ctok=None, cval=None):
    """The oracle's step on given confidences / candidates, packaged like the GPU's outputs."""
    ctok = np.full((L, 4), -1, np.int32) if ctok is None else ctok
    cval = np.zeros((L, 4), np.float32) if cval is None else cval
    out = oracle.decode_step(np.zeros((1, L, 1), np.float32), np.zeros((1, 1), np.float32), mask[None], [rule],
                             ctok[None], cval[None], auto_advance=True,
                             stats={"conf": conf[None], "tok": tok[None], "gap": np.ones((1, L), np.float32)})
    g = {"conf": conf[None].copy(), "tokens": out["tokens"].copy(), "commit": out["commit"].copy(),
         "mask": out["mask"].copy(), "ctok": out["credit_tok"].copy(), "cval": out["credit_val"].copy()}
    return g, ctok, cval


CONF = np.array([0.95, 0.2, 0.91, 0.5, 0.89, 0.99, 0.1, 0.3], np.float32)
TOK = np.arange(L, dtype=np.int64) + 10


@pytest.mark.parametrize("rule", [(oracle.THRESHOLD, 0.9, 0.0, 0), (oracle.HIERARCHICAL, 0.7, 0.0, 0),
                                  (oracle.CREDIT, 1.2, 0.7, 0)])
def test_replay_accepts_the_rule_and_rejects_planted_mistakes(rule):
    mask = np.ones(L, np.uint8)
    g, ctok, cval = _step(rule, CONF, TOK, mask)
    check_policy_replay(rule, mask, ctok, cval, g, 0, True, "as computed")
    committed = np.nonzero(g["commit"][0])[0]
    assert len(committed) >= 1

    bad = {k: v.copy() for k, v in g.items()}          # one commit dropped (mask left consistent)
    bad["commit"][0, committed[0]] = 0
    bad["mask"][0, committed[0]] = 1
    with pytest.raises(AssertionError):
        check_policy_replay(rule, mask, ctok, cval, bad, 0, True, "dropped commit")

    free = [l for l in range(L) if not g["commit"][0, l]]
    bad = {k: v.copy() for k, v in g.items()}          # one extra commit
    bad["commit"][0, free[0]] = 1
    bad["mask"][0, free[0]] = 0
    with pytest.raises(AssertionError):
        check_policy_replay(rule, mask, ctok, cval, bad, 0, True, "extra commit")

    if rule[0] == oracle.CREDIT:
        bad = {k: v.copy() for k, v in g.items()}      # a credit update off by one ulp
        bad["cval"][0, 0, 0] = np.nextafter(bad["cval"][0, 0, 0], np.float32(2))
        with pytest.raises(AssertionError):
            check_policy_replay(rule, mask, ctok, cval, bad, 0, True, "credit")


def test_replay_rejects_a_commit_outside_the_mask_and_a_missing_forced_commit():
    rule = (oracle.THRESHOLD, 0.9, 0.0, 0)
    mask = np.array([0, 1, 1, 0, 1, 1, 1, 0], np.uint8)
    low = np.full(L, 0.3, np.float32)
    low[4] = 0.5                                        # nothing passes: position 4 is forced
    g, ctok, cval = _step(rule, low, TOK, mask)
    assert g["commit"][0].tolist() == [0, 0, 0, 0, 1, 0, 0, 0]
    check_policy_replay(rule, mask, ctok, cval, g, 0, True, "forced")
    bad = {k: v.copy() for k, v in g.items()}
    bad["commit"][0, 4] = 0                             # no commit while positions are masked
    bad["mask"][0, 4] = 1
    with pytest.raises(AssertionError):
        check_policy_replay(rule, mask, ctok, cval, bad, 0, True, "no commit")
    bad = {k: v.copy() for k, v in g.items()}
    bad["commit"][0, 0] = 1                             # position 0 was not masked
    with pytest.raises(AssertionError):
        check_policy_replay(rule, mask, ctok, cval, bad, 0, True, "outside the mask")


def test_near_max_tokens():
    H = 16
    rng = np.random.default_rng(0)
    W = rng.standard_normal((40, H)).astype(np.float32)
    W[5] = W[3] * np.float32(1.0 + 1e-5)                # rows 3 and 5: a near-tie for h along W[3]
    h = np.stack([W[3] * 4, W[9] * 4]).astype(np.float32)
    W64 = oracle.as_f64(W)
    ref = oracle.token_stats(h, W64)
    assert ref["gap"][0] < 1e-2 <= ref["gap"][1]
    assert check_near_max_tokens(h, W64, ref["tok"], ref["tok"], ref["gap"], "oracle") == 1
    other = 5 if ref["tok"][0] == 3 else 3              # the other member of the near-tie: valid
    assert check_near_max_tokens(h, W64, np.array([other, 0]), ref["tok"], ref["gap"], "other") == 1
    with pytest.raises(AssertionError):                 # a token far below the top: invalid
        check_near_max_tokens(h, W64, np.array([9, 0]), ref["tok"], ref["gap"], "far")
    with pytest.raises(AssertionError):                 # outside the vocabulary
        check_near_max_tokens(h, W64, np.array([40, 0]), ref["tok"], ref["gap"], "oob")
