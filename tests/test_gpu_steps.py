"""GPU: several decode steps in one call (dlm_decode_steps), and that call inside a HIP graph.

The multi-step call must equal the same steps made one call at a time, bit for bit (the
kernels are deterministic), and the oracle run over the same staged inputs wherever no
near-tie flag is raised.  A captured graph of the call is replayed several times, with eager
work between the replays, and every replay must equal the eager result.
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


def _setup(name):
    from decoding_step_amd import _native as nat
    from decoding_step_amd.device import Decoder, to_device
    from decoding_step_amd.synth import make_weights
    from decoding_step_amd.workloads import WORKLOADS
    wl = WORKLOADS[name]
    W = make_weights(wl.V, wl.H, wl.dtype)
    Wd = to_device(W)
    seq = [(p.kind, p.threshold, p.decay, p.max_depth) for p in wl.policies]
    dec = Decoder(Wd, wl.B, wl.L, seq, flags=nat.DLM_AUTO_ADVANCE)
    return wl, W, Wd, seq, dec


def _stage_one_by_one(wl, W, dec, n):
    """n single steps from a fresh state; returns the staged inputs and every step's outputs."""
    from decoding_step_amd.device import credit_tokens, credit_values, new_credit, to_device
    from decoding_step_amd.synth import BlockStream
    streams = [BlockStream(W, wl.L, s, wl.a_max, rp) for s, rp in zip(wl.seeds, wl.redraw_p)]
    pos = [[0, 0] for _ in range(wl.B)]
    mask = torch.ones((wl.B, wl.L), dtype=torch.uint8, device="cuda")
    credit = new_credit(wl.B, wl.L)
    h_np, toks, coms = [], [], []
    for _ in range(n):
        h = np.stack([streams[b].hidden(*pos[b]) for b in range(wl.B)])
        h_np.append(h)
        dec.step(to_device(h), mask, credit)
        toks.append(dec.out_tokens.cpu().numpy())
        coms.append(dec.out_commit.cpu().numpy())
        m = mask.cpu().numpy()
        for b in range(wl.B):
            pos[b] = [pos[b][0] + 1, 0] if not m[b].any() else [pos[b][0], pos[b][1] + 1]
    final = (mask.cpu().numpy(), credit_tokens(credit).cpu().numpy(), credit_values(credit).cpu().numpy())
    return np.stack(h_np), np.stack(toks), np.stack(coms), final


def _run_steps(wl, dec, hidden_steps):
    from decoding_step_amd.device import credit_tokens, credit_values, new_credit
    n = hidden_steps.shape[0]
    mask = torch.ones((wl.B, wl.L), dtype=torch.uint8, device="cuda")
    credit = new_credit(wl.B, wl.L)
    tok = torch.full((n, wl.B, wl.L), -1, dtype=torch.int32, device="cuda")
    com = torch.full((n, wl.B, wl.L), 7, dtype=torch.uint8, device="cuda")
    dec.steps(hidden_steps, mask, credit, tok, com)
    torch.cuda.synchronize()
    return (tok.cpu().numpy(), com.cpu().numpy(),
            (mask.cpu().numpy(), credit_tokens(credit).cpu().numpy(), credit_values(credit).cpu().numpy()))


def _oracle_compare(wl, W, seq, h_np, toks, coms, sample):
    """Oracle over the staged inputs, per sampled sequence, while its state matches the GPU's."""
    W64 = oracle.as_f64(W)
    B, L = wl.B, wl.L
    mask = np.ones((B, L), np.uint8)
    ctok = np.full((B, L, 4), -1, np.int32)
    cval = np.zeros((B, L, 4), np.float32)
    compared, flagged = 0, 0
    live = set(sample)
    for n in range(h_np.shape[0]):
        sel = sorted(live)
        if not sel:
            break
        ref = oracle.decode_step(h_np[n][sel], W64, mask[sel], [seq[b] for b in sel], ctok[sel], cval[sel],
                                 auto_advance=True)
        for i, b in enumerate(sel):
            ref_b = {k: ref[k][i] for k in ("conf", "score", "gap", "commit")}
            fl = sequence_flags(seq[b][0], seq[b][1], mask[b], ref_b, True)
            sure = ref["gap"][i] >= GAP_FLAG
            np.testing.assert_array_equal(toks[n][b][sure], ref["tokens"][i][sure], err_msg=f"tokens seq {b} step {n}")
            if fl & {"F2", "F3"} or (seq[b][0] == oracle.CREDIT and "F1" in fl):
                flagged += 1
                live.discard(b)       # the two sides may part ways here; stop following this sequence
                continue
            np.testing.assert_array_equal(coms[n][b], ref["commit"][i], err_msg=f"commit seq {b} step {n}")
            compared += 1
            mask[b], ctok[b], cval[b] = ref["mask"][i], ref["credit_tok"][i], ref["credit_val"][i]
    return compared, flagged


@pytest.mark.parametrize("name,n,sample", [
    ("credit_b1_l32", 8, [0]),                 # streaming kernel, credit state carried across steps
    ("mixed_b16_l32", 4, [0, 9]),              # GEMM path, threshold and credit sequences
])
def test_decode_steps_equals_single_steps_and_oracle(name, n, sample):
    say(f"gpu: dlm_decode_steps {name} n={n}")
    from decoding_step_amd.device import to_device
    wl, W, Wd, seq, dec = _setup(name)
    h_np, toks, coms, final = _stage_one_by_one(wl, W, dec, n)
    hidden_steps = to_device(h_np.reshape(n, wl.B, wl.L, wl.H))
    tok2, com2, final2 = _run_steps(wl, dec, hidden_steps)
    np.testing.assert_array_equal(tok2, toks)
    np.testing.assert_array_equal(com2, coms)
    for a, b in zip(final, final2):
        np.testing.assert_array_equal(a, b)
    compared, flagged = _oracle_compare(wl, W, seq, h_np, tok2, com2, sample)
    say(f"[{name}] oracle: {compared} sequence-steps compared bit for bit, {flagged} flagged")
    assert compared >= 2


@pytest.mark.parametrize("name", [
    "credit_b1_l32",        # streaming kernel: one launch per step
    "mixed_b16_l32",        # GEMM path: pack, head and finalize kernels per step
])
def test_decode_steps_inside_a_graph(name):
    say(f"gpu: dlm_decode_steps {name} captured in a HIP graph, replayed 3 times")
    from decoding_step_amd.device import credit_tokens, credit_values, new_credit, to_device
    n = 4
    wl, W, Wd, seq, dec = _setup(name)
    h_np, _, _, _ = _stage_one_by_one(wl, W, dec, n)
    hidden_steps = to_device(h_np.reshape(n, wl.B, wl.L, wl.H))
    ref_tok, ref_com, ref_final = _run_steps(wl, dec, hidden_steps)
    mask = torch.ones((wl.B, wl.L), dtype=torch.uint8, device="cuda")
    credit = new_credit(wl.B, wl.L)
    credit0 = credit.clone()
    tok = torch.empty((n, wl.B, wl.L), dtype=torch.int32, device="cuda")
    com = torch.empty((n, wl.B, wl.L), dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                     # warm-up on the capture stream
        dec.policy.set_stream(side)
        dec.steps(hidden_steps, mask, credit, tok, com)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    mask.fill_(1)
    credit.copy_(credit0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        dec.policy.set_stream(torch.cuda.current_stream())
        dec.steps(hidden_steps, mask, credit, tok, com)
    dec.policy.set_stream(None)
    for rep in range(3):
        mask.fill_(1)                                  # eager work between replays
        credit.copy_(credit0)
        tok.fill_(-5)
        com.fill_(3)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(tok.cpu().numpy(), ref_tok, err_msg=f"replay {rep}")
        np.testing.assert_array_equal(com.cpu().numpy(), ref_com, err_msg=f"replay {rep}")
        np.testing.assert_array_equal(mask.cpu().numpy(), ref_final[0], err_msg=f"replay {rep}")
        np.testing.assert_array_equal(credit_tokens(credit).cpu().numpy(), ref_final[1], err_msg=f"replay {rep}")
        np.testing.assert_array_equal(credit_values(credit).cpu().numpy(), ref_final[2], err_msg=f"replay {rep}")
    say("[graph] 3 replays equal the eager call")
