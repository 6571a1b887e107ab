"""GPU parity of early stop on the end token (readings E1-E4), through the C ABI.

The commit path is compared bit for bit with the oracle on the hand-worked block and on random
states; whole steps run in lockstep with the oracle on the streaming and the GEMM path, with an
end token chosen among the planted tokens so that sequences do finish.
"""
import numpy as np
import pytest

import oracle
from parity_util import GAP_FLAG, sequence_flags, say

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decoding_step_amd import _native
    _native.load()


def _commit_gpu(conf, tok, mask, ctok, cval, done, seq, flags=0):
    from decoding_step_amd import _native as nat
    from decoding_step_amd.device import credit_from_numpy, credit_tokens, credit_values
    B, L = conf.shape
    d_conf = torch.from_numpy(np.ascontiguousarray(conf, np.float32)).cuda()
    d_tok = torch.from_numpy(np.ascontiguousarray(tok, np.int32)).cuda()
    d_mask = torch.from_numpy(np.ascontiguousarray(mask, np.uint8)).cuda()
    d_done = torch.from_numpy(np.ascontiguousarray(done, np.uint8)).cuda()
    credit = credit_from_numpy(ctok, cval)
    out = torch.empty((B, L), dtype=torch.uint8, device="cuda")
    pol = nat.StepPolicy(B, L, 32, 1, nat.DLM_BF16, seq, flags=flags, seq_done=d_done)
    nat.dlm_commit(d_conf, d_tok, d_mask, credit, pol, out)
    torch.cuda.synchronize()
    return (out.cpu().numpy(), d_mask.cpu().numpy(), credit_tokens(credit).cpu().numpy(),
            credit_values(credit).cpu().numpy(), d_done.cpu().numpy())


def test_eos_hand_worked_on_gpu(golden):
    say("gpu: hand-worked early stop")
    g = golden("eos_threshold_L8.json")
    L = g["L"]
    seq = [(oracle.THRESHOLD, g["tau"], 0.0, 0, g["eos"])]
    mask = np.ones((1, L), np.uint8)
    ctok = np.full((1, L, 4), -1, np.int32)
    cval = np.zeros((1, L, 4), np.float32)
    done = np.zeros(1, np.uint8)
    for it in g["iterations"]:
        conf = np.array([it["conf"]], np.float32)
        tok = np.array([it["tok"]], np.int32)
        commit, mask, ctok, cval, done = _commit_gpu(conf, tok, mask, ctok, cval, done, seq,
                                                     flags=1 if it.get("advance") else 0)
        assert sorted(np.nonzero(commit[0])[0].tolist()) == it["commit"]
        assert int(done[0]) == it["state"]
    assert not mask.any()


@pytest.mark.parametrize("L", [1, 6, 32, 64])
@pytest.mark.parametrize("advance", [0, 1])
def test_eos_random_states_bit_exact(L, advance):
    say(f"gpu: early stop, random states L={L} advance={advance}")
    from decoding_step_amd.synth import stream
    g = stream(91, L, advance)
    rules = [(0, 0.9, 0.0, 0, 2), (0, 1.1, 0.0, 0, 3), (1, 0.7, 0.0, 0, 2), (1, 0.5, 0.0, 1, 1),
             (2, 1.2, 0.7, 0, 2), (2, 0.9, 0.0, 0, 4), (0, 0.9, 0.0, 0, -1), (2, 1.0, 0.5, 0, -1)]
    B = 48
    seq = [rules[b % len(rules)] for b in range(B)]
    mask = (g.random((B, L)) < 0.75).astype(np.uint8)
    mask[::9] = 0
    done = g.integers(0, 3, B).astype(np.uint8)                 # all three states on entry
    ctok = np.full((B, L, 4), -1, np.int32)
    cval = np.zeros((B, L, 4), np.float32)
    levels = np.array([0.05, 0.3, 0.5, 0.62, 0.7, 0.75, 0.9, 0.95, 1.0], np.float32)
    for it in range(8):
        conf = levels[g.integers(0, len(levels), (B, L))]
        tok = g.integers(0, 6, (B, L)).astype(np.int32)
        got = _commit_gpu(conf, tok, mask, ctok, cval, done, seq, flags=advance)
        ref = oracle.decode_step(np.zeros((B, L, 1), np.float32), np.zeros((1, 1), np.float32), mask, seq,
                                 ctok, cval, auto_advance=bool(advance), seq_done=done,
                                 stats={"conf": conf, "tok": tok, "gap": np.ones((B, L), np.float32)})
        np.testing.assert_array_equal(got[0], ref["commit"], err_msg=f"commit it {it}")
        np.testing.assert_array_equal(got[1], ref["mask"], err_msg=f"mask it {it}")
        np.testing.assert_array_equal(got[4], ref["seq_done"], err_msg=f"state it {it}")
        credit_rows = [b for b in range(B) if seq[b][0] == oracle.CREDIT]
        np.testing.assert_array_equal(got[2][credit_rows], ref["credit_tok"][credit_rows])
        np.testing.assert_array_equal(got[3][credit_rows], ref["credit_val"][credit_rows])
        mask, ctok, cval, done = ref["mask"], ref["credit_tok"], ref["credit_val"], ref["seq_done"]


@pytest.mark.parametrize("name,sample,steps", [
    ("tiny_threshold_f32", [0], 14),           # streaming kernel
    ("mixed_b16_l32", [0, 9], 6),              # GEMM path, threshold and credit sequences
])
def test_eos_whole_steps_lockstep(name, sample, steps):
    """Whole steps with early stop, both sides fed the oracle's state each step."""
    from decoding_step_amd import _native as nat
    from decoding_step_amd.device import (Decoder, credit_from_numpy, credit_tokens, credit_values,
                                          to_device)
    from decoding_step_amd.synth import BlockStream, make_weights, stream
    from decoding_step_amd.workloads import WORKLOADS
    wl = WORKLOADS[name]
    B, L = wl.B, wl.L
    W = make_weights(wl.V, wl.H, wl.dtype)
    W64 = oracle.as_f64(W)
    # the end token: the token planted at position L*5/8 of sequence 0's first block
    eos = int(stream(wl.seeds[0], 1, 0).integers(0, wl.V, L)[(5 * L) // 8])
    seq = [(p.kind, p.threshold, p.decay, p.max_depth, eos) for p in wl.policies]
    say(f"gpu: early stop lockstep {name}, end token {eos}")
    dec = Decoder(to_device(W), B, L, seq, flags=nat.DLM_AUTO_ADVANCE)
    d_done = torch.zeros(B, dtype=torch.uint8, device="cuda")
    dec.policy.set_seq_done(d_done)
    streams = [BlockStream(W, L, s, wl.a_max, rp) for s, rp in zip(wl.seeds, wl.redraw_p)]
    pos = [[0, 0] for _ in range(B)]
    mask = np.ones((B, L), np.uint8)
    ctok = np.full((B, L, 4), -1, np.int32)
    cval = np.zeros((B, L, 4), np.float32)
    done = np.zeros(B, np.uint8)
    compared, padded = 0, 0
    for n in range(steps):
        h = np.stack([streams[b].hidden(*pos[b]) for b in range(B)])
        d_mask = torch.from_numpy(mask.copy()).cuda()
        d_credit = credit_from_numpy(ctok, cval)
        d_done.copy_(torch.from_numpy(done.copy()))
        dec.step(to_device(h), d_mask, d_credit)
        torch.cuda.synchronize()
        g_tok, g_com = dec.out_tokens.cpu().numpy(), dec.out_commit.cpu().numpy()
        g_mask, g_done = d_mask.cpu().numpy(), d_done.cpu().numpy()
        ref = oracle.decode_step(h[sample], W64, mask[sample], [seq[b] for b in sample], ctok[sample],
                                 cval[sample], auto_advance=True, seq_done=done[sample])
        for i, b in enumerate(sample):
            ref_b = {k: ref[k][i] for k in ("conf", "score", "gap", "commit")}
            fl = sequence_flags(seq[b][0], seq[b][1], mask[b], ref_b, True)
            sure = ref["gap"][i] >= GAP_FLAG
            np.testing.assert_array_equal(g_tok[b][sure], ref["tokens"][i][sure], err_msg=f"tokens seq {b} step {n}")
            if fl & {"F2", "F3"} or (seq[b][0] == oracle.CREDIT and "F1" in fl):
                continue
            compared += 1
            padded += int(((ref["tokens"][i] == eos) & (ref["commit"][i] == 1)).sum())
            np.testing.assert_array_equal(g_com[b], ref["commit"][i], err_msg=f"commit seq {b} step {n}")
            np.testing.assert_array_equal(g_mask[b], ref["mask"][i], err_msg=f"mask seq {b} step {n}")
            assert g_done[b] == ref["seq_done"][i], f"state seq {b} step {n}"
            if seq[b][0] == oracle.CREDIT:
                np.testing.assert_array_equal(credit_tokens(d_credit).cpu().numpy()[b], ref["credit_tok"][i])
        # continue from the oracle's state on the sampled sequences, from the GPU's elsewhere
        new_mask, new_done = g_mask.copy(), g_done.copy()
        new_ctok, new_cval = credit_tokens(d_credit).cpu().numpy(), credit_values(d_credit).cpu().numpy()
        for i, b in enumerate(sample):
            new_mask[b], new_done[b] = ref["mask"][i], ref["seq_done"][i]
            new_ctok[b], new_cval[b] = ref["credit_tok"][i], ref["credit_val"][i]
        mask, done, ctok, cval = new_mask, new_done, new_ctok, new_cval
        for b in range(B):
            if done[b] == oracle.FINISHED:
                continue
            pos[b] = [pos[b][0] + 1, 0] if not mask[b].any() else [pos[b][0], pos[b][1] + 1]
    say(f"[{name}] {compared} sequence-steps compared, end-token commits {padded}, states {done[sample].tolist()}")
    assert done[sample[0]] == oracle.FINISHED           # sequence 0 met its end token and finished
    assert compared >= len(sample) * 2
