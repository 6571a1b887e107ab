"""GPU parity of the vocabulary-sharded head (readings V1-V3), through the C ABI.

One GPU runs every shard's dlm_shard_stats at the real shard shape, the records land in one
[G][B*L] buffer as an all-gather would leave them, and dlm_merge_commit merges and commits.  The
shard records are compared with the oracle's shard_stats; the merged step with the oracle's
decode_step in lockstep (same flags as the unsharded parity tests) and with the unsharded
dlm_decode_step on the same inputs.
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


def _cuts(V, G, uneven=False):
    if uneven:
        return [0, V // 25, V // 25 + V // 2 + 1, V]
    return [V * g // G for g in range(G + 1)]


class Sharded:
    """Per-shard workspaces, policies and W slices on the device, plus the gathered records."""

    def __init__(self, W, B, L, cuts, seq, flags=0):
        from decoding_step_amd import _native as nat
        from decoding_step_amd.device import to_device, torch_dtype_code
        V, H = W.shape
        self.B, self.L, self.cuts = B, L, cuts
        self.G = len(cuts) - 1
        self.W_shards = [to_device(np.ascontiguousarray(W[a:b])) for a, b in zip(cuts[:-1], cuts[1:])]
        code = torch_dtype_code(self.W_shards[0])
        self.ws = [torch.zeros(nat.dlm_workspace_bytes(B, L, H, b - a, code), dtype=torch.uint8, device="cuda")
                   for a, b in zip(cuts[:-1], cuts[1:])]
        self.pol = [nat.StepPolicy(B, L, H, b - a, code, [(0, 0.9, 0, 0)] * B, ws)
                    for (a, b), ws in zip(zip(cuts[:-1], cuts[1:]), self.ws)]
        self.records = torch.empty((self.G, B * L, 4), dtype=torch.float32, device="cuda")
        self.conf = torch.empty((B, L), dtype=torch.float32, device="cuda")
        self.gap = torch.empty((B, L), dtype=torch.float32, device="cuda")
        self.merge_pol = nat.StepPolicy(B, L, H, V, code, seq, flags=flags, out_conf=self.conf, out_gap=self.gap)
        self.out_tokens = torch.empty((B, L), dtype=torch.int32, device="cuda")
        self.out_commit = torch.empty((B, L), dtype=torch.uint8, device="cuda")

    def shard_stats(self, hd):
        from decoding_step_amd import _native as nat
        for g in range(self.G):
            nat.dlm_shard_stats(hd, self.W_shards[g], self.cuts[g], self.pol[g], self.records[g])

    def step(self, hd, mask, credit):
        from decoding_step_amd import _native as nat
        self.shard_stats(hd)
        nat.dlm_merge_commit(self.records, self.G, mask, credit, self.merge_pol, self.out_tokens, self.out_commit)


def _records_np(rec):
    r = rec.cpu().numpy()
    return r[..., 0], r[..., 1], r[..., 2].view(np.int32), r[..., 3]


@pytest.mark.parametrize("B,L,H,V,G,dtype,shard", [
    (1, 32, 2048, 126464, 8, "bf16", 3),     # batch-1 block, one eighth of the vocabulary (15808 rows)
    (16, 32, 2048, 157184, 8, "bf16", 7),    # 512 rows: the GEMM-shaped head on 19648 rows
    (2, 5, 64, 1000, 3, "f32", 2),           # tiny float32, ragged shard
])
def test_shard_records_against_the_oracle(B, L, H, V, G, dtype, shard):
    from decoding_step_amd.device import to_device
    from decoding_step_amd.synth import BlockStream, make_weights
    say(f"gpu: shard records B={B} L={L} V={V} shard {shard}/{G}")
    W = make_weights(V, H, dtype)
    M = B * L
    h = BlockStream(W, M, 11 + M, 40.0).hidden(0, 0)
    cuts = _cuts(V, G)
    sh = Sharded(W, B, L, cuts, [(0, 0.9, 0, 0)] * B)
    from decoding_step_amd import _native as nat
    a, b = cuts[shard], cuts[shard + 1]
    nat.dlm_shard_stats(to_device(h), sh.W_shards[shard], a, sh.pol[shard], sh.records[shard])
    torch.cuda.synchronize()
    m, s, tok, sec = (x[shard] for x in _records_np(sh.records))
    rows = np.arange(M) if M <= 64 else np.r_[0:8, 250:262, M - 8:M]
    ref = oracle.shard_stats(h[rows], W[a:b], a)
    sure = (ref["top32"] - ref["second32"]) >= GAP_FLAG
    assert np.array_equal(tok[rows][sure], ref["tok"][sure])
    assert np.all((tok[rows] >= a) & (tok[rows] < b))
    np.testing.assert_allclose(m[rows], ref["m"], rtol=1e-5, atol=1e-4)
    np.testing.assert_allclose(s[rows], ref["s"], rtol=1e-3)
    fin = np.isfinite(ref["second32"])
    np.testing.assert_allclose(sec[rows][fin], ref["second32"][fin], rtol=1e-3, atol=2e-3)
    assert np.all(s[rows] >= 1.0 - 1e-4)                       # the maximum's own term is 1 (to rounding)
    say(f"[shard] {len(rows)} rows, tokens {int(sure.sum())} exact")


@pytest.mark.parametrize("name,G,uneven,steps,sample", [
    ("threshold_b1_l32", 8, False, 3, [0]),
    ("credit_b1_l32", 8, False, 4, [0]),
    ("credit_b1_l32", 3, True, 3, [0]),
    ("mixed_b16_l32", 8, False, 2, [0, 9]),
])
def test_sharded_step_in_lockstep(name, G, uneven, steps, sample):
    """Both sides continue from the oracle's state; the unsharded step runs beside on the same state."""
    from decoding_step_amd import _native as nat
    from decoding_step_amd.device import Decoder, credit_from_numpy, credit_tokens, to_device
    from decoding_step_amd.synth import BlockStream, make_weights
    from decoding_step_amd.workloads import WORKLOADS
    wl = WORKLOADS[name]
    B, L = wl.B, wl.L
    say(f"gpu: sharded step {name} G={G}{' uneven' if uneven else ''}")
    W = make_weights(wl.V, wl.H, wl.dtype)
    W64 = oracle.as_f64(W)
    seq = [(p.kind, p.threshold, p.decay, p.max_depth) for p in wl.policies]
    sh = Sharded(W, B, L, _cuts(wl.V, G, uneven), seq, flags=nat.DLM_AUTO_ADVANCE)
    whole = Decoder(to_device(W), B, L, seq, flags=nat.DLM_AUTO_ADVANCE)
    streams = [BlockStream(W, L, s, wl.a_max, rp) for s, rp in zip(wl.seeds, wl.redraw_p)]
    pos = [[0, 0] for _ in range(B)]
    mask = np.ones((B, L), np.uint8)
    ctok = np.full((B, L, 4), -1, np.int32)
    cval = np.zeros((B, L, 4), np.float32)
    compared = agree = 0
    for n in range(steps):
        h = np.stack([streams[b].hidden(*pos[b]) for b in range(B)])
        hd = to_device(h)
        m1, c1 = torch.from_numpy(mask.copy()).cuda(), credit_from_numpy(ctok, cval)
        m2, c2 = torch.from_numpy(mask.copy()).cuda(), credit_from_numpy(ctok, cval)
        sh.step(hd, m1, c1)
        whole.step(hd, m2, c2)
        torch.cuda.synchronize()
        s_tok, s_com, s_mask = sh.out_tokens.cpu().numpy(), sh.out_commit.cpu().numpy(), m1.cpu().numpy()
        w_tok, w_com, w_conf = whole.out_tokens.cpu().numpy(), whole.out_commit.cpu().numpy(), whole.conf.cpu().numpy()
        s_conf = sh.conf.cpu().numpy()
        # two merge orders of the same sums: each rescaling exp2 carries the rounding of m*log2(e)
        # (about 6e-6 relative at logits near 100), far inside the 1e-3 bar against the oracle
        np.testing.assert_allclose(s_conf, w_conf, rtol=2e-4)
        ref = oracle.decode_step(h[sample], W64, mask[sample], [seq[b] for b in sample], ctok[sample], cval[sample],
                                 auto_advance=True)
        for i, b in enumerate(sample):
            ref_b = {k: ref[k][i] for k in ("conf", "score", "gap", "commit")}
            fl = sequence_flags(seq[b][0], seq[b][1], mask[b], ref_b, True)
            sure = ref["gap"][i] >= GAP_FLAG
            assert np.array_equal(s_tok[b][sure], ref["tokens"][i][sure]), (b, n)
            assert np.array_equal(s_tok[b][sure], w_tok[b][sure]), (b, n)
            np.testing.assert_allclose(s_conf[b], ref["conf"][i], rtol=1e-3)
            if fl & {"F2", "F3"} or (seq[b][0] == oracle.CREDIT and "F1" in fl):
                continue
            compared += 1
            assert np.array_equal(s_com[b], ref["commit"][i]), (b, n)
            assert np.array_equal(s_mask[b], ref["mask"][i]), (b, n)
            if seq[b][0] == oracle.CREDIT:
                assert np.array_equal(credit_tokens(c1).cpu().numpy()[b], ref["credit_tok"][i]), (b, n)
            agree += int(np.array_equal(s_com[b], w_com[b]))
        # continue from the oracle's state on the sampled sequences, from the sharded run's elsewhere
        new_mask = s_mask.copy()
        new_ctok = credit_tokens(c1).cpu().numpy()
        from decoding_step_amd.device import credit_values
        new_cval = credit_values(c1).cpu().numpy()
        for i, b in enumerate(sample):
            new_mask[b], new_ctok[b], new_cval[b] = ref["mask"][i], ref["credit_tok"][i], ref["credit_val"][i]
        mask, ctok, cval = new_mask, new_ctok, new_cval
        for b in range(B):
            pos[b] = [pos[b][0] + 1, 0] if not mask[b].any() else [pos[b][0], pos[b][1] + 1]
    say(f"[{name} G={G}] {compared} sequence-steps bit-exact with the oracle, {agree} equal to the unsharded step")
    assert compared >= steps * len(sample) // 2


def test_merge_commit_is_deterministic():
    from decoding_step_amd import _native as nat
    from decoding_step_amd.device import new_credit, to_device
    from decoding_step_amd.synth import BlockStream, make_weights
    say("gpu: dlm_merge_commit three times on the same records")
    W = make_weights(30011, 256, "bf16")
    h = BlockStream(W, 32, 5, 40.0).hidden(0, 0)[None]
    sh = Sharded(W, 1, 32, _cuts(30011, 5), [(2, 1.1, 0.6, 0)])
    sh.shard_stats(to_device(h))
    outs = []
    for _ in range(3):
        mask = torch.ones((1, 32), dtype=torch.uint8, device="cuda")
        credit = new_credit(1, 32)
        nat.dlm_merge_commit(sh.records, sh.G, mask, credit, sh.merge_pol, sh.out_tokens, sh.out_commit)
        torch.cuda.synchronize()
        outs.append((sh.out_tokens.cpu().numpy(), sh.out_commit.cpu().numpy(), mask.cpu().numpy(),
                     sh.conf.cpu().numpy(), credit.cpu().numpy()))
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert np.array_equal(a, b)
