"""GPU parity: the HIP decode step against the CPU oracle, through the C ABI.

Commit policies are compared bit for bit on identical confidences; the LM
head + statistics on ragged and full shapes; whole steps in lockstep on all
five workloads (the batched one on sampled sequences).  Near-tie decisions
are flagged and counted (tests/parity_util.py).
"""
import numpy as np
import pytest

import oracle
from parity_util import Lockstep, check_near_max_tokens, say

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decoding_step_amd import _native
    _native.load()


_W_CACHE = {}


def weights(V, H, dtype):
    from decoding_step_amd.device import to_device
    from decoding_step_amd.synth import make_weights
    key = (V, H, dtype)
    if key not in _W_CACHE:
        _W_CACHE.clear()
        W = make_weights(V, H, dtype)
        _W_CACHE[key] = (W, to_device(W), oracle.as_f64(W))
    return _W_CACHE[key]


def decoder(Wd, B, L, seq, flags=None):
    from decoding_step_amd import _native as nat
    from decoding_step_amd.device import Decoder
    return Decoder(Wd, B, L, seq, flags=nat.DLM_AUTO_ADVANCE if flags is None else flags)


# ---------------------------------------------------------------------------------- commit only
def _commit_gpu(conf, tok, mask, ctok, cval, seq, flags=0):
    from decoding_step_amd import _native as nat
    from decoding_step_amd.device import credit_from_numpy, credit_tokens, credit_values
    B, L = conf.shape
    dev_conf = torch.from_numpy(np.ascontiguousarray(conf, np.float32)).cuda()
    dev_tok = torch.from_numpy(np.ascontiguousarray(tok, np.int32)).cuda()
    dev_mask = torch.from_numpy(np.ascontiguousarray(mask, np.uint8)).cuda()
    credit = credit_from_numpy(ctok, cval)
    out = torch.empty((B, L), dtype=torch.uint8, device="cuda")
    pol = nat.StepPolicy(B, L, 32, 1, nat.DLM_BF16, seq, flags=flags)
    nat.dlm_commit(dev_conf, dev_tok, dev_mask, credit, pol, out)
    torch.cuda.synchronize()
    return (out.cpu().numpy(), dev_mask.cpu().numpy(), credit_tokens(credit).cpu().numpy(),
            credit_values(credit).cpu().numpy())


@pytest.mark.parametrize("name", ["threshold_L8.json", "hierarchical_L8.json", "credit_L6.json"])
def test_hand_worked_sequences_on_gpu(golden, name):
    say(f"gpu: hand-worked {name}")
    g = golden(name)
    L = g["L"]
    if "tau" in g:
        kind = oracle.THRESHOLD if name.startswith("threshold") else oracle.HIERARCHICAL
        seq = [(kind, g["tau"], 0.0, 0)]
    else:
        seq = [(oracle.CREDIT, g["theta"], g["decay"], 0)]
    mask = np.ones((1, L), np.uint8)
    ctok = np.full((1, L, 4), -1, np.int32)
    cval = np.zeros((1, L, 4), np.float32)
    for it in g["iterations"]:
        conf = np.array([it["conf"]], np.float32)
        tok = np.array([it.get("tok", [0] * L)], np.int32)
        commit, mask, ctok, cval = _commit_gpu(conf, tok, mask, ctok, cval, seq)
        assert sorted(np.nonzero(commit[0])[0].tolist()) == it["commit"]
    assert not mask.any()


@pytest.mark.parametrize("L", [1, 5, 8, 31, 32, 63, 64])
@pytest.mark.parametrize("advance", [0, 1])
def test_commit_random_states_bit_exact(L, advance):
    say(f"gpu: random commit states L={L} advance={advance}")
    from decoding_step_amd.synth import stream
    g = stream(77, L, advance)
    rules = [(0, 0.9, 0.0, 0), (0, 1.1, 0.0, 0), (1, 0.7, 0.0, 0), (1, 0.5, 0.0, 1), (1, 0.6, 0.0, 2),
             (2, 1.2, 0.7, 0), (2, 0.9, 0.0, 0), (2, 1.0, 0.5, 0)]
    B = 40
    seq = [rules[b % len(rules)] for b in range(B)]
    mask = (g.random((B, L)) < 0.7).astype(np.uint8)
    mask[::7] = 0                                              # some empty rows
    ctok = np.full((B, L, 4), -1, np.int32)
    cval = np.zeros((B, L, 4), np.float32)
    levels = np.array([0.05, 0.3, 0.5, 0.62, 0.7, 0.75, 0.9, 0.95, 1.0], np.float32)
    for it in range(6):
        conf = levels[g.integers(0, len(levels), (B, L))]     # ties on purpose
        tok = g.integers(0, 6, (B, L)).astype(np.int32)
        got = _commit_gpu(conf, tok, mask, ctok, cval, seq, flags=advance)
        ref = oracle.decode_step(np.zeros((B, L, 1), np.float32), np.zeros((1, 1), np.float32), mask, seq,
                                 ctok, cval, auto_advance=bool(advance),
                                 stats={"conf": conf, "tok": tok, "gap": np.ones((B, L), np.float32)})
        np.testing.assert_array_equal(got[0], ref["commit"], err_msg=f"commit it {it}")
        np.testing.assert_array_equal(got[1], ref["mask"], err_msg=f"mask it {it}")
        credit_rows = [b for b in range(B) if seq[b][0] == oracle.CREDIT]
        np.testing.assert_array_equal(got[2][credit_rows], ref["credit_tok"][credit_rows])
        np.testing.assert_array_equal(got[3][credit_rows], ref["credit_val"][credit_rows])
        mask, ctok, cval = ref["mask"], ref["credit_tok"], ref["credit_val"]


# ---------------------------------------------------------------------------------- LM head stats
def _stats_inputs(M, H, V, dtype, seed):
    from decoding_step_amd.synth import BlockStream, bf16_bits, bf16_to_f32, make_weights
    W = make_weights(V, H, dtype)
    if V > 40:
        W[V - 3] = W[7]                                        # duplicated row: exact tie with id 7
    h = BlockStream(W, M, seed, 60.0).hidden(0, 0)
    if M > 2:
        h[1] = 0                                               # all-zero row: uniform softmax
        if V > 40:                                             # row aimed at the duplicated pair
            w7 = W[7].astype(np.float32) if dtype == "f32" else bf16_to_f32(W[7])
            h[2] = (w7 * 400).astype(np.float32) if dtype == "f32" else bf16_bits(w7 * 400)
    return W, h


@pytest.mark.parametrize("B,L,H,V,dtype", [
    (1, 8, 64, 1024, "f32"),        # tiny workload shape
    (1, 5, 96, 1000, "bf16"),       # ragged last tile
    (1, 37, 128, 4099, "bf16"),     # two row groups, ragged rows and tile
    (2, 35, 64, 2500, "f32"),       # three row groups, float32
    (1, 3, 32, 17, "bf16"),         # fewer tiles than wavefronts
    (1, 2, 32, 1, "bf16"),          # one-token vocabulary
    (1, 16, 2048, 20011, "bf16"),   # full hidden size, prime vocabulary
    (5, 13, 256, 3001, "bf16"),     # GEMM path, 256-row groups: 65 rows, ragged last tile
    (4, 30, 256, 1000, "bf16"),     # GEMM path, 256-row groups: 120 rows, fewer tiles than workgroups
    (8, 32, 256, 30011, "bf16"),    # GEMM path: a full 256-row group, ragged last tile
    (17, 31, 512, 5003, "bf16"),    # GEMM path, 512-row groups: 527 rows = two groups, 40 workgroups each
    (5, 13, 128, 3001, "bf16"),     # 65 rows with H % 256 != 0: streaming kernel, row groups
    (16, 32, 2048, 30011, "bf16"),  # GEMM path at the batched workload's row count (one 512-row group)
    (9, 32, 512, 40013, "bf16"),    # GEMM path: 288 rows, one 512-row group mostly padding
    (16, 32, 256, 65613, "bf16"),   # GEMM path: a full 512-row group, ragged last tile
    (24, 32, 256, 30011, "bf16"),   # GEMM path: 768 rows = 2 groups paired on one XCD, ragged tile
    (4, 32, 256, 30208, "bf16"),    # GEMM path, 256-row group, V = 118 x 256: no partial tile
    (16, 32, 2048, 157184, "bf16"), # the batched workload's shape: V = 1228 x 128, no partial tile
])
def test_token_stats_against_oracle(B, L, H, V, dtype):
    M = B * L
    say(f"gpu: token stats B={B} L={L} H={H} V={V} {dtype}")
    from decoding_step_amd import _native as nat
    from decoding_step_amd.device import to_device
    W, h = _stats_inputs(M, H, V, dtype, seed=M + V)
    Wd, hd = to_device(W), to_device(h)
    W64 = oracle.as_f64(W)                                     # widened once for all row chunks
    code = nat.DLM_BF16 if dtype == "bf16" else nat.DLM_F32
    ws = torch.zeros(nat.dlm_workspace_bytes(B, L, H, V, code), dtype=torch.uint8, device="cuda")
    pol = nat.StepPolicy(B, L, H, V, code, [(0, 0.9, 0, 0)] * B, ws)
    conf = torch.empty(M, dtype=torch.float32, device="cuda")
    tok = torch.empty(M, dtype=torch.int32, device="cuda")
    gap = torch.empty(M, dtype=torch.float32, device="cuda")
    nat.dlm_token_stats(hd, Wd, pol, conf, tok, gap)
    torch.cuda.synchronize()
    ref = oracle.token_stats(h, W64)
    conf, tok, gap = conf.cpu().numpy(), tok.cpu().numpy(), gap.cpu().numpy()
    sure = ref["gap"] >= 1e-2
    np.testing.assert_array_equal(tok[sure], ref["tok"][sure])
    near = check_near_max_tokens(h, W64, tok, ref["tok"], ref["gap"], f"B={B} L={L} V={V}")
    np.testing.assert_allclose(conf, ref["conf"], rtol=1e-3)
    assert np.all(conf <= 1.0) and np.all(conf > 0.0)       # the largest probability lies in (0, 1]
    fin = np.isfinite(ref["gap"])
    np.testing.assert_allclose(gap[fin], ref["gap"][fin], rtol=1e-3, atol=2e-3)
    assert np.all(np.isinf(gap[~fin]))
    if M > 2:
        assert tok[1] == 0 and conf[1] == np.float32(1.0 / V)   # zero row: exact uniform
        if V > 40:
            assert tok[2] == 7 and gap[2] == 0                    # duplicated row: lower id, zero gap
    say(f"[token stats] all {M} rows compared; {near} near-tie rows, each with a near-maximal token")


def test_repeated_calls_are_bit_identical():
    say("gpu: determinism")
    from decoding_step_amd import _native as nat
    from decoding_step_amd.device import to_device
    W, h = _stats_inputs(32, 2048, 126464 // 4, "bf16", seed=5)
    Wd, hd = to_device(W), to_device(h)
    ws = torch.zeros(nat.dlm_workspace_bytes(1, 32, 2048, W.shape[0], 1), dtype=torch.uint8, device="cuda")
    pol = nat.StepPolicy(1, 32, 2048, W.shape[0], 1, [(0, 0.9, 0, 0)], ws)
    outs = []
    for _ in range(3):
        conf = torch.empty(32, dtype=torch.float32, device="cuda")
        tok = torch.empty(32, dtype=torch.int32, device="cuda")
        gap = torch.empty(32, dtype=torch.float32, device="cuda")
        nat.dlm_token_stats(hd, Wd, pol, conf, tok, gap)
        outs.append((conf.cpu().numpy(), tok.cpu().numpy(), gap.cpu().numpy()))
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert np.array_equal(a, b)


def test_failed_call_writes_nothing():
    say("gpu: error path leaves state untouched")
    from decoding_step_amd import _native as nat
    mask = torch.ones((1, 8), dtype=torch.uint8, device="cuda")
    out_t = torch.full((1, 8), -7, dtype=torch.int32, device="cuda")
    out_c = torch.full((1, 8), 9, dtype=torch.uint8, device="cuda")
    h = torch.zeros((1, 8, 64), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((100, 64), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    pol = nat.StepPolicy(1, 8, 64, 100, nat.DLM_BF16, [(5, 0.9, 0, 0)], ws)
    with pytest.raises(nat.DlmError):
        nat.dlm_decode_step(h, W, mask, None, pol, out_t, out_c)
    torch.cuda.synchronize()
    assert torch.all(mask == 1) and torch.all(out_t == -7) and torch.all(out_c == 9)


# ---------------------------------------------------------------------------------- whole steps
def _lockstep(name, **run):
    from decoding_step_amd.workloads import WORKLOADS
    wl = WORKLOADS[name]
    W, Wd, W64 = weights(wl.V, wl.H, wl.dtype)
    sample = run.pop("sample", None)
    say(f"gpu: lockstep {name} {run}")
    return Lockstep(wl, W, Wd, W64, decoder, sample_seqs=sample).run(label=name, **run)


def test_lockstep_tiny_threshold_f32():
    ls = _lockstep("tiny_threshold_f32", blocks=3)
    assert ls.commits == 3 * 8


def test_lockstep_threshold_b1_l32():
    ls = _lockstep("threshold_b1_l32", blocks=2)
    assert ls.commits == 2 * 32


def test_lockstep_credit_b1_l32():
    ls = _lockstep("credit_b1_l32", blocks=2)
    assert ls.commits == 2 * 32


def test_lockstep_hierarchical_b1_l64():
    ls = _lockstep("hierarchical_b1_l64", blocks=1)
    assert ls.commits == 64


def test_lockstep_mixed_b16_l32_all_sequences():
    # every one of the 16 sequences (all 512 rows, i.e. every wavefront of the GEMM-shaped head's
    # non-tail kernel) against the oracle, three steps
    ls = _lockstep("mixed_b16_l32", steps=3)
    assert ls.checked["rule replays"] == 3 * 16
