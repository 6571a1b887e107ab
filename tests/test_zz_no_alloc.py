"""dlm_decode_step_noalloc (workspace in the library's static per-GPU scratch) against
dlm_decode_step (caller's workspace): the same kernels, so every output and every state array
must be the same bits.  Calls follow one another with different shapes, the second smaller than
the first, then back to the first (the shared scratch keeps the last call's contents; the counter
region must be zero again after every call whatever the shape)."""
import numpy as np
import pytest
import torch

from decoding_step_amd import _native as nat
from decoding_step_amd.device import new_credit, to_device, torch_dtype_code
from decoding_step_amd.synth import BlockStream, make_weights

pytestmark = pytest.mark.gpu

THR = (nat.DLM_THRESHOLD, 0.9, 0.0, 0)
CRED = (nat.DLM_CREDIT, 1.2, 0.7, 0)
HIER = (nat.DLM_HIERARCHICAL, 0.7, 0.0, 0)


def say(msg):
    print(msg, flush=True)


def one_pair(W, Wd, B, L, seq, it, topk=0):
    """One step of each entry point from the same state; returns both sides' outputs (host)."""
    V, H = W.shape
    dev = Wd.device
    code = torch_dtype_code(Wd)
    streams = [BlockStream(W, L, seed=b, a_max=60.0, redraw_p=0.3 if s[0] == nat.DLM_CREDIT else 0.0)
               for b, s in enumerate(seq)]
    h = to_device(np.stack([s.hidden(0, it) for s in streams]), dev)
    rng = np.random.default_rng(100 + it)
    mask0 = torch.from_numpy((rng.random((B, L)) < 0.7).astype(np.uint8)).to(dev)
    credit0 = new_credit(B, L, dev)
    out = []
    for noalloc in (False, True):
        mask, credit = mask0.clone(), credit0.clone()
        tok = torch.full((B, L), -7, dtype=torch.int32, device=dev)
        com = torch.full((B, L), 7, dtype=torch.uint8, device=dev)
        conf = torch.full((B, L), -1.0, dtype=torch.float32, device=dev)
        gap = torch.full((B, L), -1.0, dtype=torch.float32, device=dev)
        tk_tok = torch.full((B, L, topk), -7, dtype=torch.int32, device=dev) if topk else None
        tk_prob = torch.full((B, L, topk), -1.0, dtype=torch.float32, device=dev) if topk else None
        if noalloc:
            pol = nat.StepPolicy(B, L, H, V, code, seq, None, 0, flags=nat.DLM_AUTO_ADVANCE, out_conf=conf,
                                 out_gap=gap, topk=topk, out_topk_tokens=tk_tok, out_topk_prob=tk_prob)
            nat.dlm_decode_step_noalloc(h, Wd, mask, credit, pol, tok, com)
        else:
            ws = torch.zeros(nat.dlm_workspace_bytes_topk(B, L, H, V, code, topk), dtype=torch.uint8, device=dev)
            pol = nat.StepPolicy(B, L, H, V, code, seq, ws, flags=nat.DLM_AUTO_ADVANCE, out_conf=conf, out_gap=gap,
                                 topk=topk, out_topk_tokens=tk_tok, out_topk_prob=tk_prob)
            nat.dlm_decode_step(h, Wd, mask, credit, pol, tok, com)
        torch.cuda.synchronize()
        o = {"tokens": tok, "commit": com, "mask": mask, "credit": credit, "conf": conf, "gap": gap}
        if topk:
            o["topk_tokens"], o["topk_prob"] = tk_tok, tk_prob
        out.append({k: v.cpu().numpy() for k, v in o.items()})
    return out


def check_pair(label, ref, got):
    for k in ref:
        assert np.array_equal(ref[k].view(np.uint8), got[k].view(np.uint8)), f"{label}: {k} differs"
    assert ref["commit"].max() == 1, f"{label}: no commit at all"   # the case exercises the policies


def test_noalloc_matches_workspace_entry_point_across_shapes():
    dev = torch.device("cuda:0")
    V, H = 5003, 256                       # ragged last tile on both heads
    W = make_weights(V, H, "bf16")
    Wd = to_device(W, dev)
    cases = [
        # (label, B, L, per-sequence rules, top-k)
        ("batched 16x32 (GEMM-shaped head)", 16, 32, [THR] * 8 + [CRED] * 8, 0),
        ("single 1x32 (streaming head), smaller", 1, 32, [THR], 0),
        ("batched 16x32 again", 16, 32, [THR] * 8 + [CRED] * 8, 0),
        ("2x64 hierarchical + credit, top-4 export, smaller", 2, 64, [HIER, CRED], 4),
        ("single 1x32 again", 1, 32, [CRED], 0),
    ]
    for it, (label, B, L, seq, k) in enumerate(cases):
        say(f"[noalloc] {label}: B={B} L={L} H={H} V={V} topk={k}")
        ref, got = one_pair(W, Wd, B, L, seq, it, k)
        check_pair(label, ref, got)
        say(f"[noalloc] {label}: bit-identical ({int(ref['commit'].sum())} commits)")


def test_noalloc_batched_workload_shape():
    """The batched workload's full shape (16 x 32 rows, V = 157184, H = 2048), then the headline
    shape (1 x 32, V = 126464): both through the static scratch, equal to the workspace calls."""
    dev = torch.device("cuda:0")
    for B, L, V, seq in [(16, 32, 157184, [THR] * 8 + [CRED] * 8), (1, 32, 126464, [THR])]:
        say(f"[noalloc] full shape B={B} L={L} H=2048 V={V}")
        W = make_weights(V, 2048, "bf16")
        Wd = to_device(W, dev)
        ref, got = one_pair(W, Wd, B, L, seq, 0)
        check_pair(f"B={B} L={L} V={V}", ref, got)
        del Wd
        torch.cuda.empty_cache()
