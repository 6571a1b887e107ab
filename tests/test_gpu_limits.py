"""GPU parity at the limits of the supported shapes, through the C ABI.

Every row goes through the head on the GPU; the oracle recomputes a sample of rows (first and
last of every row group among them), which it can afford at these sizes.  Shapes: the largest
B and L (16384 rows, the GEMM path with 32 row groups of 512), the largest B with L = 1, the largest
hidden size on the streaming and on the GEMM path, and a one-token vocabulary on the GEMM path.
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


def _sample_rows(M, n=40, group=256, seed=3):
    rows = {0, M - 1}
    for g0 in range(0, M, group):                 # first and last row of every group
        rows |= {g0, min(M, g0 + group) - 1}
    rng = np.random.default_rng(seed)
    rows |= set(rng.integers(0, M, n).tolist())
    return np.array(sorted(rows))


@pytest.mark.parametrize("B,L,H,V", [
    (256, 64, 2048, 30011),    # the largest block batch: 16384 rows, GEMM path, 32 row groups
    (256, 1, 1024, 20011),     # the largest B with L = 1 (256 rows)
    (1, 8, 4096, 5003),        # the largest hidden size of the streaming kernel (bf16)
    (9, 32, 4096, 5003),       # the GEMM path at H = 4096
    (3, 32, 256, 1),           # the GEMM path with a one-token vocabulary
])
def test_token_stats_at_the_limits(B, L, H, V):
    M = B * L
    say(f"gpu: limits B={B} L={L} H={H} V={V} ({M} rows)")
    from decoding_step_amd import _native as nat
    from decoding_step_amd.device import to_device
    from decoding_step_amd.synth import BlockStream, make_weights
    W = make_weights(V, H, "bf16")
    h = BlockStream(W, M, M + V, 60.0).hidden(0, 0)
    ws = torch.zeros(nat.dlm_workspace_bytes(B, L, H, V, nat.DLM_BF16), dtype=torch.uint8, device="cuda")
    assert ws.numel() > 0
    pol = nat.StepPolicy(B, L, H, V, nat.DLM_BF16, [(0, 0.9, 0, 0)] * B, ws)
    conf = torch.empty(M, dtype=torch.float32, device="cuda")
    tok = torch.empty(M, dtype=torch.int32, device="cuda")
    gap = torch.empty(M, dtype=torch.float32, device="cuda")
    nat.dlm_token_stats(to_device(h), to_device(W), pol, conf, tok, gap)
    torch.cuda.synchronize()
    rows = _sample_rows(M)
    ref = oracle.token_stats(h[rows], W)
    conf, tok, gap = conf.cpu().numpy()[rows], tok.cpu().numpy()[rows], gap.cpu().numpy()[rows]
    sure = ref["gap"] >= 1e-2
    np.testing.assert_array_equal(tok[sure], ref["tok"][sure])
    check_near_max_tokens(h[rows], oracle.as_f64(W), tok, ref["tok"], ref["gap"], f"B={B} L={L} H={H} V={V}")
    np.testing.assert_allclose(conf, ref["conf"], rtol=1e-3)
    fin = np.isfinite(ref["gap"])
    np.testing.assert_allclose(gap[fin], ref["gap"][fin], rtol=1e-3, atol=2e-3)
    assert np.all(np.isinf(gap[~fin]))
    assert np.all(conf <= 1.0) and np.all(conf > 0.0)      # the largest probability lies in (0, 1]
    if V == 1:
        assert np.all(tok == 0)
    say(f"[limits] {len(rows)} rows compared, {int((~sure).sum())} near-ties")


def test_largest_block_batch_whole_step():
    """One full step at B=256, L=64 (threshold and credit rules), commits checked on sampled
    sequences against the oracle from the same state."""
    from decoding_step_amd import _native as nat
    from decoding_step_amd.device import Decoder, credit_tokens, credit_values, new_credit, to_device
    from decoding_step_amd.synth import BlockStream, make_weights
    B, L, H, V = 256, 64, 1024, 12007
    say(f"gpu: whole step at B={B} L={L}")
    W = make_weights(V, H, "bf16")
    seq = [(oracle.THRESHOLD, 0.9, 0.0, 0) if b % 2 == 0 else (oracle.CREDIT, 1.2, 0.7, 0) for b in range(B)]
    h = np.stack([BlockStream(W, L, 1000 + b, 60.0).hidden(0, 0) for b in range(B)])
    dec = Decoder(to_device(W), B, L, seq, flags=nat.DLM_AUTO_ADVANCE)
    mask = torch.ones((B, L), dtype=torch.uint8, device="cuda")
    credit = new_credit(B, L)
    dec.step(to_device(h), mask, credit)
    torch.cuda.synchronize()
    sample = [0, 1, 127, 128, 254, 255]
    W64 = oracle.as_f64(W)
    ref = oracle.decode_step(h[sample], W64, np.ones((len(sample), L), np.uint8),
                             [seq[b] for b in sample], auto_advance=True)
    g_com, g_mask = dec.out_commit.cpu().numpy(), mask.cpu().numpy()
    g_tok, g_ctok = dec.out_tokens.cpu().numpy(), credit_tokens(credit).cpu().numpy()
    g = {"conf": dec.conf.cpu().numpy(), "tokens": g_tok, "commit": g_com, "mask": g_mask, "ctok": g_ctok,
         "cval": credit_values(credit).cpu().numpy()}
    compared = 0
    for i, b in enumerate(sample):
        ref_b = {k: ref[k][i] for k in ("conf", "score", "gap", "commit")}
        fl = sequence_flags(seq[b][0], seq[b][1], np.ones(L, np.uint8), ref_b, True)
        sure = ref["gap"][i] >= GAP_FLAG
        np.testing.assert_array_equal(g_tok[b][sure], ref["tokens"][i][sure], err_msg=f"tokens seq {b}")
        check_near_max_tokens(h[b], W64, g_tok[b], ref["tokens"][i], ref["gap"][i], f"seq {b}")
        check_policy_replay(seq[b], np.ones(L, np.uint8), np.full((L, 4), -1, np.int32), np.zeros((L, 4), np.float32),
                            g, b, True, f"seq {b}")
        if fl & {"F2", "F3"} or (seq[b][0] == oracle.CREDIT and "F1" in fl):
            continue
        compared += 1
        np.testing.assert_array_equal(g_com[b], ref["commit"][i], err_msg=f"commit seq {b}")
        np.testing.assert_array_equal(g_mask[b], ref["mask"][i], err_msg=f"mask seq {b}")
        if seq[b][0] == oracle.CREDIT:
            np.testing.assert_array_equal(g_ctok[b], ref["credit_tok"][i], err_msg=f"credit seq {b}")
    say(f"[B=256 L=64] {compared} of {len(sample)} sampled sequences compared bit for bit")
    assert compared >= 3
    assert g_com.sum(axis=1).min() >= 1                # at least one commit per sequence
