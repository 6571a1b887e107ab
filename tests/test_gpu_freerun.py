"""Free-running parity: the HIP path and the oracle each run on their OWN state, step after step.

Unlike the lockstep tests, nothing is re-synchronised: the GPU's mask and credit after a step are
its input to the next one, and the oracle's likewise.  While the two states agree both sides
see the same hidden states (inputs depend only on the block and iteration a sequence is at).
Every step where a followed sequence's commits, mask or credit slots differ must be a step the
oracle flags for that sequence (F2 / F3, or F1 under credit decoding); the sequence is then no
longer followed, and the divergences are reported with the step and flag that explain them.
"""
import numpy as np
import pytest

import oracle
from parity_util import GAP_FLAG, check_near_max_tokens, check_policy_replay, sequence_flags, say

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decoding_step_amd import _native
    _native.load()


@pytest.mark.parametrize("name,steps,sample", [   # each workload's whole run (a margin past it at B=1)
    ("tiny_threshold_f32", 24, [0]),             # three blocks
    ("threshold_b1_l32", 120, [0]),              # 32 blocks take ~108 steps
    ("credit_b1_l32", 120, [0]),                 # ~107
    ("hierarchical_b1_l64", 190, [0]),           # ~180
    ("mixed_b16_l32", 64, [0, 7, 8, 15]),        # the workload's 64 steps; threshold 0, 7, credit 8, 15
])
def test_free_running(name, steps, sample):
    from decoding_step_amd import _native as nat
    from decoding_step_amd.device import Decoder, credit_tokens, credit_values, new_credit, to_device
    from decoding_step_amd.synth import BlockStream, make_weights
    from decoding_step_amd.workloads import WORKLOADS
    wl = WORKLOADS[name]
    B, L = wl.B, wl.L
    say(f"gpu: free-running {name}, {steps} steps")
    W = make_weights(wl.V, wl.H, wl.dtype)
    W64 = oracle.as_f64(W)
    seq = [(p.kind, p.threshold, p.decay, p.max_depth) for p in wl.policies]
    dec = Decoder(to_device(W), B, L, seq, flags=nat.DLM_AUTO_ADVANCE)
    streams = [BlockStream(W, L, s, wl.a_max, rp) for s, rp in zip(wl.seeds, wl.redraw_p)]
    pos = [[0, 0] for _ in range(B)]
    mask = torch.ones((B, L), dtype=torch.uint8, device="cuda")
    credit = new_credit(B, L)
    o_mask = {b: np.ones(L, np.uint8) for b in sample}
    o_ctok = {b: np.full((L, 4), -1, np.int32) for b in sample}
    o_cval = {b: np.zeros((L, 4), np.float32) for b in sample}
    following, diverged = set(sample), []
    compared = commits = near_ties = 0
    # the GPU's own state before each step (the rule replay starts from it: in free running the GPU's
    # credit values may differ from the oracle's in the last bits while everything else agrees)
    p_mask = np.ones((B, L), np.uint8)
    p_ctok = np.full((B, L, 4), -1, np.int32)
    p_cval = np.zeros((B, L, 4), np.float32)
    for n in range(steps):
        h = np.stack([streams[b].hidden(*pos[b]) for b in range(B)])
        dec.step(to_device(h), mask, credit)
        torch.cuda.synchronize()
        g_mask, g_com, g_tok = mask.cpu().numpy(), dec.out_commit.cpu().numpy(), dec.out_tokens.cpu().numpy()
        g_ctok, g_cval = credit_tokens(credit).cpu().numpy(), credit_values(credit).cpu().numpy()
        g = {"conf": dec.conf.cpu().numpy(), "tokens": g_tok, "commit": g_com, "mask": g_mask, "ctok": g_ctok,
             "cval": g_cval}
        sel = sorted(following)
        if sel:
            # the followed sequences' states agree with the oracle's, so they sit at the same
            # (block, iteration) and h[b] is the oracle's input too
            ref = oracle.decode_step(h[sel], W64, np.stack([o_mask[b] for b in sel]), [seq[b] for b in sel],
                                     np.stack([o_ctok[b] for b in sel]), np.stack([o_cval[b] for b in sel]),
                                     auto_advance=True)
            for i, b in enumerate(sel):
                ref_b = {k: ref[k][i] for k in ("conf", "score", "gap", "commit")}
                fl = sequence_flags(seq[b][0], seq[b][1], o_mask[b], ref_b, True)
                flagged = bool(fl & {"F2", "F3"}) or (seq[b][0] == oracle.CREDIT and "F1" in fl)
                sure = ref["gap"][i] >= GAP_FLAG
                assert np.array_equal(g_tok[b][sure], ref["tokens"][i][sure]), f"token, seq {b} step {n}"
                # flagged or not, the GPU's decision is a valid one: near-maximal tokens on near-ties,
                # and its commits / mask / credit are its rule applied to its own values
                near_ties += check_near_max_tokens(h[b], W64, g_tok[b], ref["tokens"][i], ref["gap"][i],
                                                   f"seq {b} step {n}")
                check_policy_replay(seq[b], p_mask[b], p_ctok[b], p_cval[b], g, b, True, f"seq {b} step {n}")
                same = (np.array_equal(g_com[b], ref["commit"][i]) and np.array_equal(g_mask[b], ref["mask"][i])
                        and np.array_equal(g_ctok[b], ref["credit_tok"][i]))
                if same and seq[b][0] == oracle.CREDIT:
                    np.testing.assert_allclose(g_cval[b], ref["credit_val"][i], rtol=1e-3, atol=1e-6)
                if same:
                    compared += 1
                    commits += int(g_com[b].sum())
                    o_mask[b], o_ctok[b], o_cval[b] = ref["mask"][i], ref["credit_tok"][i], ref["credit_val"][i]
                else:
                    assert flagged, f"sequence {b} diverged at step {n} with no near-tie flag ({sorted(fl)})"
                    diverged.append((b, n, sorted(fl)))
                    following.discard(b)
        p_mask, p_ctok, p_cval = g_mask.copy(), g_ctok.copy(), g_cval.copy()
        for b in range(B):
            pos[b] = [pos[b][0] + 1, 0] if not g_mask[b].any() else [pos[b][0], pos[b][1] + 1]
    say(f"[{name}] free-running: {compared} sequence-steps equal, {commits} commits, "
        f"{near_ties} near-tie rows with a near-maximal token, divergences {diverged if diverged else 'none'}")
    assert compared >= min(steps, 4) * len(sample) // 2
