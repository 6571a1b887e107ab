"""GPU parity of the top-k candidate export (readings T1-T4), through the C ABI.

The HIP path is compared with the oracle's topk_candidates row by row: a rank's token must
match wherever the oracle's float32 logits separate it from both neighbours by at least 1e-2
(the near-tie rule of the candidate), a rank's probability must match to 1e-3 relative
everywhere (the i-th largest probability does not depend on which of two tied tokens holds it).
Entry 0 must equal the call's own candidate and confidence exactly, and turning the export on
must not change the step's statistics or commits.
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


def _stats_topk(h, W, B, L, k, dtype_code):
    """dlm_token_stats with the export on; returns conf, tok, gap, topk tokens, topk prob."""
    from decoding_step_amd import _native as nat
    from decoding_step_amd.device import to_device
    V, H = W.shape
    M = B * L
    ws = torch.zeros(nat.dlm_workspace_bytes_topk(B, L, H, V, dtype_code, k), dtype=torch.uint8, device="cuda")
    assert ws.numel() > 0
    tt = torch.full((M, k), -7, dtype=torch.int32, device="cuda")
    tp = torch.full((M, k), -7.0, dtype=torch.float32, device="cuda")
    pol = nat.StepPolicy(B, L, H, V, dtype_code, [(0, 0.9, 0, 0)] * B, ws, topk=k, out_topk_tokens=tt,
                         out_topk_prob=tp)
    conf = torch.empty(M, dtype=torch.float32, device="cuda")
    tok = torch.empty(M, dtype=torch.int32, device="cuda")
    gap = torch.empty(M, dtype=torch.float32, device="cuda")
    nat.dlm_token_stats(to_device(h), to_device(W), pol, conf, tok, gap)
    torch.cuda.synchronize()
    return (conf.cpu().numpy(), tok.cpu().numpy(), gap.cpu().numpy(), tt.cpu().numpy(), tp.cpu().numpy())


def _check_against_oracle(h, W, rows, k, got_tok, got_prob):
    """Compare sampled rows with the oracle; returns (ranks compared, ranks exempt)."""
    V = W.shape[0]
    ref = oracle.topk_candidates(h[rows], W, min(k + 1, V))
    z32 = oracle.lm_head_logits(h[rows], W).astype(np.float32)
    compared = exempt = 0
    for i in range(len(rows)):
        order = ref["tok"][i]
        zs = [float(z32[i, t]) for t in order]
        for r in range(k):
            if r >= V:
                assert got_tok[i, r] == -1 and got_prob[i, r] == 0.0, (rows[i], r)
                continue
            lo = zs[r] - zs[r + 1] if r + 1 < len(zs) else np.inf
            hi = zs[r - 1] - zs[r] if r > 0 else np.inf
            if min(lo, hi) >= GAP_FLAG:
                assert got_tok[i, r] == order[r], (rows[i], r, got_tok[i], order)
                compared += 1
            else:
                exempt += 1
        np.testing.assert_allclose(got_prob[i, :min(k, V)], ref["prob"][i, :min(k, V)], rtol=1e-3, atol=1e-30,
                                   err_msg=f"row {rows[i]}")
    return compared, exempt


def _valid(tok, prob, V, k):
    for i in range(tok.shape[0]):
        real = tok[i][tok[i] >= 0]
        assert len(real) == min(k, V) and len(set(real.tolist())) == len(real)
        assert np.all(real < V)
        assert np.all(np.diff(prob[i]) <= 0)                   # best first
        assert np.all((prob[i] >= 0) & (prob[i] <= 1))


@pytest.mark.parametrize("B,L,H,V,dtype,k", [
    (1, 8, 64, 1024, "f32", 8),            # tiny float32
    (1, 32, 2048, 126464, "bf16", 8),      # the batch-1 block shape, all rows
    (2, 13, 256, 3001, "bf16", 5),         # ragged rows and tiles
    (1, 5, 64, 5, "f32", 8),               # fewer tokens than k: padding
    (1, 3, 64, 1, "bf16", 3),              # one-token vocabulary
    (3, 40, 4096, 5003, "bf16", 4),        # 16 K fragments per wavefront, two 16-row blocks per group
    (5, 20, 128, 20011, "f32", 8),         # four 16-row blocks per group
    (16, 32, 2048, 30011, "bf16", 8),      # 512 rows: the GEMM-shaped head's chunk lists, ragged tile
    (16, 32, 2048, 157184, "bf16", 8),     # the batched workload's shape: GEMM-shaped head, no partial tile
    (5, 13, 256, 3001, "bf16", 8),         # 65 rows on the GEMM-shaped head (512-row group, mostly padding)
    (3, 32, 256, 5, "bf16", 8),            # fewer tokens than k on the GEMM-shaped head
    (8, 32, 256, 20011, "f32", 6),         # 256 float32 rows: the streaming head with the fold
    (1, 32, 2048, 126464, "bf16", 1),      # k = 1 on the streaming head: the export is the candidate
    (16, 32, 256, 5003, "bf16", 1),        # k = 1 on the GEMM-shaped head
])
def test_topk_token_stats(B, L, H, V, dtype, k):
    from decoding_step_amd import _native as nat
    from decoding_step_amd.synth import BlockStream, make_weights
    M = B * L
    say(f"gpu: top-k stats B={B} L={L} H={H} V={V} {dtype} k={k}")
    W = make_weights(V, H, dtype)
    h = BlockStream(W, M, 3 * M + V, 30.0).hidden(0, 0)
    code = nat.DLM_BF16 if dtype == "bf16" else nat.DLM_F32
    conf, tok, gap, tt, tp = _stats_topk(h, W, B, L, k, code)
    _valid(tt, tp, V, k)
    assert np.array_equal(tt[:, 0], tok)                       # entry 0 is the candidate ...
    assert np.array_equal(tp[:, 0], conf)                      # ... with its confidence, bit for bit
    rows = np.arange(M)
    if M > 64:
        rows = np.unique(np.r_[0, M - 1, np.arange(0, M, 37), 63, 64, 65, 255, 256])
        rows = rows[rows < M]
    compared, exempt = _check_against_oracle(h, W, rows, k, tt[rows], tp[rows])
    ref = oracle.token_stats(h[rows], W)
    np.testing.assert_allclose(conf[rows], ref["conf"], rtol=1e-3)
    say(f"[top-k] {len(rows)} rows, {compared} ranks compared exactly, {exempt} within 1e-2 of a neighbour")
    assert compared >= len(rows) // 2


def test_topk_gemm_head_largest_vocabulary():
    """The GEMM head's chunk entries pack the id and the gap code into 32 bits: at V = 2^22 - 1
    the id takes 22 bits and the gap code keeps 6 mantissa bits, the coarsest it gets.  65 rows
    (GEMM path, ragged last tile), sampled rows against the oracle."""
    from decoding_step_amd import _native as nat
    from decoding_step_amd.synth import BlockStream, make_weights
    B, L, H, V, k = 5, 13, 256, (1 << 22) - 1, 8
    say(f"gpu: top-k on the GEMM head at the largest vocabulary, B={B} L={L} H={H} V={V}")
    W = make_weights(V, H, "bf16", seed=7)
    h = BlockStream(W, B * L, 11, 30.0).hidden(0, 0)
    conf, tok, gap, tt, tp = _stats_topk(h, W, B, L, k, nat.DLM_BF16)
    _valid(tt, tp, V, k)
    assert np.array_equal(tt[:, 0], tok)
    assert np.array_equal(tp[:, 0], conf)
    rows = np.array([0, 1, 17, 31, 32, 63, 64])
    compared, exempt = _check_against_oracle(h, W, rows, k, tt[rows], tp[rows])
    say(f"[top-k] {len(rows)} rows, {compared} ranks compared exactly, {exempt} within 1e-2 of a neighbour")
    assert compared >= len(rows) // 2


def test_topk_exact_ties_across_workgroups():
    """Copies of one vocabulary row give bit-equal logits wherever they sit (same K order), so
    they must come out adjacent and in id order: within a thread's stream (ids 16 apart), across
    slots of a tile, and across vocabulary ranges of different workgroups."""
    from decoding_step_amd import _native as nat
    from decoding_step_amd.synth import make_weights
    V, H = 30011, 256
    W = make_weights(V, H, "f32", seed=4)
    copies = [5, 21, 22, 4000, 17333, 30010]
    W[copies] = W[12]
    h = np.stack([W[12] * 6.0, W[12] * 6.0 + 0.01])           # the copies are far ahead of every other token
    conf, tok, gap, tt, tp = _stats_topk(h.astype(np.float32), W, 1, 2, 8, nat.DLM_F32)
    want = sorted(copies + [12])
    for r in range(2):
        assert tt[r, :7].tolist() == want, tt[r]
        assert len(set(tp[r, :7].tolist())) == 1
        assert tok[r] == 5 and gap[r] == 0.0
    ref = oracle.topk_candidates(h.astype(np.float32), W, 8)
    assert ref["tok"][:, :7].tolist() == [want, want]


def test_topk_gemm_head_ties_inside_one_chunk():
    """GEMM-shaped head (96 rows): a row whose best tokens share one chunk (a lane's 16 ids of one
    32-row vocabulary block) must be recomputed exactly, and exact ties (copied rows, in the same
    chunk and in other chunks) must come out adjacent and in id order with equal probabilities."""
    from decoding_step_amd import _native as nat
    from decoding_step_amd.synth import BlockStream, bf16_bits, bf16_to_f32, make_weights
    B, L, H, V, k = 3, 32, 256, 4096, 8
    say(f"gpu: top-k ties inside a chunk, GEMM-shaped head B={B} L={L} V={V}")
    W = make_weights(V, H, "bf16", seed=9)
    a, b, c = 65, 73, 2000                # a and b: ids 64 + {1, 9}, both in half 0 of block 64..95
    W[b] = W[a]
    W[c] = W[a]
    h = BlockStream(W, B * L, 77, 30.0).hidden(0, 0)
    wa = bf16_to_f32(W[a])
    h[0] = bf16_bits(wa * 8.0)            # a, b, c tie far ahead of every other token
    w2 = bf16_to_f32(W[a + 2])            # id 67: same chunk as a and b
    h[1] = bf16_bits(wa * 6.0 + w2 * 6.0)
    conf, tok, gap, tt, tp = _stats_topk(h, W, B, L, k, nat.DLM_BF16)
    _valid(tt, tp, V, k)
    assert np.array_equal(tt[:, 0], tok) and np.array_equal(tp[:, 0], conf)
    assert tt[0, :3].tolist() == [a, b, c], tt[0]
    assert tp[0, 0] == tp[0, 1] == tp[0, 2]
    ref = oracle.topk_candidates(h[:2], W, k)
    assert ref["tok"][0, :3].tolist() == [a, b, c]
    rows = np.arange(B * L)
    compared, exempt = _check_against_oracle(h, W, rows, k, tt, tp)
    say(f"[top-k ties] {compared} ranks compared exactly, {exempt} near-ties")
    assert compared >= len(rows) * 4


def _plain_and_topk_steps(name, k, n_steps):
    from decoding_step_amd import _native as nat
    from decoding_step_amd.device import Decoder, new_credit, to_device
    from decoding_step_amd.synth import BlockStream, make_weights
    from decoding_step_amd.workloads import WORKLOADS
    wl = WORKLOADS[name]
    W = make_weights(wl.V, wl.H, wl.dtype)
    Wd = to_device(W)
    seq = [(p.kind, p.threshold, p.decay, p.max_depth) for p in wl.policies]
    plain = Decoder(Wd, wl.B, wl.L, seq, flags=nat.DLM_AUTO_ADVANCE)
    withk = Decoder(Wd, wl.B, wl.L, seq, flags=nat.DLM_AUTO_ADVANCE, topk=k)
    streams = [BlockStream(W, wl.L, s, wl.a_max, rp) for s, rp in zip(wl.seeds, wl.redraw_p)]
    pos = [[0, 0] for _ in range(wl.B)]
    m1 = torch.ones((wl.B, wl.L), dtype=torch.uint8, device="cuda")
    m2 = m1.clone()
    c1, c2 = new_credit(wl.B, wl.L), new_credit(wl.B, wl.L)
    for _ in range(n_steps):
        h = np.stack([streams[b].hidden(*pos[b]) for b in range(wl.B)])
        hd = to_device(h)
        plain.step(hd, m1, c1)
        withk.step(hd, m2, c2)
        torch.cuda.synchronize()
        m = m1.cpu().numpy()
        for b in range(wl.B):
            pos[b] = [pos[b][0] + 1, 0] if not m[b].any() else [pos[b][0], pos[b][1] + 1]
        yield wl, W, seq, h, plain, withk, m1.cpu().numpy(), m2.cpu().numpy(), c1, c2


@pytest.mark.parametrize("name", ["threshold_b1_l32", "credit_b1_l32", "hierarchical_b1_l64"])
def test_topk_leaves_the_step_unchanged(name):
    """Batch-1 workloads run the same streaming fold either way: statistics, commits, state bit-equal."""
    from decoding_step_amd.device import credit_tokens, credit_values
    say(f"gpu: step with and without top-k, {name}")
    n = 0
    for wl, W, seq, h, plain, withk, m1, m2, c1, c2 in _plain_and_topk_steps(name, 8, 6):
        assert np.array_equal(plain.out_tokens.cpu().numpy(), withk.out_tokens.cpu().numpy())
        assert np.array_equal(plain.out_commit.cpu().numpy(), withk.out_commit.cpu().numpy())
        assert np.array_equal(plain.conf.cpu().numpy(), withk.conf.cpu().numpy())
        assert np.array_equal(plain.gap.cpu().numpy(), withk.gap.cpu().numpy())
        assert np.array_equal(m1, m2)
        assert np.array_equal(credit_tokens(c1).cpu().numpy(), credit_tokens(c2).cpu().numpy())
        assert np.array_equal(credit_values(c1).cpu().numpy(), credit_values(c2).cpu().numpy())
        tt = withk.topk_tokens.cpu().numpy().reshape(-1, 8)
        tp = withk.topk_prob.cpu().numpy().reshape(-1, 8)
        assert np.array_equal(tt[:, 0], withk.out_tokens.cpu().numpy().reshape(-1))
        assert np.array_equal(tp[:, 0], withk.conf.cpu().numpy().reshape(-1))
        if n == 0:
            rows = np.arange(wl.B * wl.L)
            compared, _ = _check_against_oracle(h.reshape(-1, wl.H), W, rows, 8, tt, tp)
            assert compared >= len(rows)
        n += 1
    say(f"[{name}] {n} steps identical with the export on")


def test_topk_step_on_the_batched_workload():
    """512 rows: the step with top-k runs the GEMM-shaped head with its chunk lists; statistics,
    commits and state must equal the plain step's bit for bit, commits are checked against the
    oracle on sampled sequences (near-tie rules as elsewhere), the export on sampled rows."""
    from decoding_step_amd.device import credit_tokens, credit_values
    say("gpu: step with top-k, mixed_b16_l32")
    first_done = False
    for wl, W, seq, h, plain, withk, m1, m2, c1, c2 in _plain_and_topk_steps("mixed_b16_l32", 8, 2):
        assert np.array_equal(plain.out_tokens.cpu().numpy(), withk.out_tokens.cpu().numpy())
        assert np.array_equal(plain.out_commit.cpu().numpy(), withk.out_commit.cpu().numpy())
        assert np.array_equal(plain.conf.cpu().numpy(), withk.conf.cpu().numpy())
        assert np.array_equal(plain.gap.cpu().numpy(), withk.gap.cpu().numpy())
        assert np.array_equal(m1, m2)
        assert np.array_equal(credit_tokens(c1).cpu().numpy(), credit_tokens(c2).cpu().numpy())
        assert np.array_equal(credit_values(c1).cpu().numpy(), credit_values(c2).cpu().numpy())
        if first_done:
            continue                       # the oracle check below starts from fresh blocks: first step only
        first_done = True
        sample = [0, 5, 9, 15]
        ref = oracle.decode_step(h[sample], oracle.as_f64(W), np.ones((len(sample), wl.L), np.uint8),
                                 [seq[b] for b in sample], auto_advance=True)
        g_com, g_tok = withk.out_commit.cpu().numpy(), withk.out_tokens.cpu().numpy()
        compared = 0
        for i, b in enumerate(sample):
            ref_b = {key: ref[key][i] for key in ("conf", "score", "gap", "commit")}
            fl = sequence_flags(seq[b][0], seq[b][1], np.ones(wl.L, np.uint8), ref_b, True)
            sure = ref["gap"][i] >= GAP_FLAG
            assert np.array_equal(g_tok[b][sure], ref["tokens"][i][sure])
            if fl & {"F2", "F3"} or (seq[b][0] == oracle.CREDIT and "F1" in fl):
                continue
            assert np.array_equal(g_com[b], ref["commit"][i]), b
            assert np.array_equal(m2[b], ref["mask"][i]), b
            compared += 1
        tt = withk.topk_tokens.cpu().numpy()
        tp = withk.topk_prob.cpu().numpy()
        rows = np.array([0, 31, 160, 300, 511])
        c, _ = _check_against_oracle(h.reshape(-1, wl.H), W, rows, 8, tt.reshape(-1, 8)[rows], tp.reshape(-1, 8)[rows])
        say(f"[mixed top-k] {compared} sequences' commits and {c} ranks compared")
        assert compared >= 2 and c >= len(rows) * 4


def _topk_steps_setup(name, k, n):
    """A Decoder with the export on, and n steps of the workload one call each (each sequence
    advancing to its next block when its mask empties): the staged hidden blocks and each step's
    export."""
    from decoding_step_amd import _native as nat
    from decoding_step_amd.device import Decoder, new_credit, to_device
    from decoding_step_amd.synth import BlockStream, make_weights
    from decoding_step_amd.workloads import WORKLOADS
    wl = WORKLOADS[name]
    W = make_weights(wl.V, wl.H, wl.dtype)
    Wd = to_device(W)
    seq = [(p.kind, p.threshold, p.decay, p.max_depth) for p in wl.policies]
    dec = Decoder(Wd, wl.B, wl.L, seq, flags=nat.DLM_AUTO_ADVANCE, topk=k)
    streams = [BlockStream(W, wl.L, s, wl.a_max, rp) for s, rp in zip(wl.seeds, wl.redraw_p)]
    mask = torch.ones((wl.B, wl.L), dtype=torch.uint8, device="cuda")
    credit = new_credit(wl.B, wl.L)
    pos = [[0, 0] for _ in range(wl.B)]
    hs, ref = [], {"tok": [], "com": [], "tt": [], "tp": []}
    for _ in range(n):
        h = np.stack([streams[b].hidden(*pos[b]) for b in range(wl.B)])
        hs.append(h)
        dec.step(to_device(h), mask, credit)
        ref["tok"].append(dec.out_tokens.cpu().numpy().copy())
        ref["com"].append(dec.out_commit.cpu().numpy().copy())
        ref["tt"].append(dec.topk_tokens.cpu().numpy().copy())
        ref["tp"].append(dec.topk_prob.cpu().numpy().copy())
        m = mask.cpu().numpy()
        for b in range(wl.B):
            pos[b] = [pos[b][0] + 1, 0] if not m[b].any() else [pos[b][0], pos[b][1] + 1]
    ref = {key: np.stack(v) for key, v in ref.items()}
    ref["mask"] = mask.cpu().numpy()
    return wl, dec, to_device(np.stack(hs)), ref


def _topk_steps_buffers(wl, k, n):
    tok = torch.full((n, wl.B, wl.L), -5, dtype=torch.int32, device="cuda")
    com = torch.full((n, wl.B, wl.L), 3, dtype=torch.uint8, device="cuda")
    tt = torch.full((n, wl.B, wl.L, k), -9, dtype=torch.int32, device="cuda")
    tp = torch.full((n, wl.B, wl.L, k), -9.0, dtype=torch.float32, device="cuda")
    return tok, com, tt, tp


def _topk_steps_check(ref, mask, tok, com, tt, tp, label):
    np.testing.assert_array_equal(tok.cpu().numpy(), ref["tok"], err_msg=f"{label}: tokens")
    np.testing.assert_array_equal(com.cpu().numpy(), ref["com"], err_msg=f"{label}: commits")
    np.testing.assert_array_equal(mask.cpu().numpy(), ref["mask"], err_msg=f"{label}: mask")
    np.testing.assert_array_equal(tt.cpu().numpy(), ref["tt"], err_msg=f"{label}: export tokens")
    np.testing.assert_array_equal(tp.cpu().numpy(), ref["tp"], err_msg=f"{label}: export probabilities")


@pytest.mark.parametrize("name,k,n", [
    ("credit_b1_l32", 5, 4),      # streaming head: one launch per step
    ("mixed_b16_l32", 8, 3),      # GEMM-shaped head: pack, head with chunk lists, finalize per step
])
def test_topk_in_decode_steps(name, k, n):
    """dlm_decode_steps writes one export per step; each equals the single-step call's, and the
    Decoder's own export buffers are back in the policy afterwards."""
    from decoding_step_amd.device import new_credit
    say(f"gpu: dlm_decode_steps with top-{k}, {name}, {n} steps")
    wl, dec, hidden_steps, ref = _topk_steps_setup(name, k, n)
    mask = torch.ones((wl.B, wl.L), dtype=torch.uint8, device="cuda")
    credit = new_credit(wl.B, wl.L)
    tok, com, tt, tp = _topk_steps_buffers(wl, k, n)
    dec.steps(hidden_steps, mask, credit, tok, com, tt, tp)
    torch.cuda.synchronize()
    _topk_steps_check(ref, mask, tok, com, tt, tp, name)
    dec.step(hidden_steps[0], torch.ones_like(mask), new_credit(wl.B, wl.L))
    torch.cuda.synchronize()
    assert np.array_equal(dec.topk_tokens.cpu().numpy(), ref["tt"][0])
    say(f"[{name}] {n} steps' exports equal the single-step calls'")


@pytest.mark.parametrize("name,k,n", [
    ("threshold_b1_l32", 8, 3),   # streaming head
    ("mixed_b16_l32", 8, 3),      # GEMM-shaped head
])
def test_topk_decode_steps_inside_a_graph(name, k, n):
    """dlm_decode_steps with the export on, captured in a HIP graph and replayed three times with
    eager work between the replays: every replay equals the single-step calls."""
    from decoding_step_amd.device import new_credit
    say(f"gpu: dlm_decode_steps with top-{k}, {name}, captured in a HIP graph, replayed 3 times")
    wl, dec, hidden_steps, ref = _topk_steps_setup(name, k, n)
    mask = torch.ones((wl.B, wl.L), dtype=torch.uint8, device="cuda")
    credit = new_credit(wl.B, wl.L)
    credit0 = credit.clone()
    tok, com, tt, tp = _topk_steps_buffers(wl, k, n)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                     # warm-up on the capture stream
        dec.policy.set_stream(side)
        dec.steps(hidden_steps, mask, credit, tok, com, tt, tp)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    _topk_steps_check(ref, mask, tok, com, tt, tp, f"{name} eager")
    g = torch.cuda.CUDAGraph()
    mask.fill_(1)
    credit.copy_(credit0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        dec.policy.set_stream(torch.cuda.current_stream())
        dec.steps(hidden_steps, mask, credit, tok, com, tt, tp)
    dec.policy.set_stream(None)
    for rep in range(3):
        mask.fill_(1)                                  # eager work between replays
        credit.copy_(credit0)
        tok.fill_(-5)
        com.fill_(3)
        tt.fill_(-9)
        tp.fill_(-9.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _topk_steps_check(ref, mask, tok, com, tt, tp, f"{name} replay {rep}")
    say(f"[{name}] 3 replays with the export equal the single-step calls")
