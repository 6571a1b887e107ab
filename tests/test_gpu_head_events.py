"""GPU: the head-timing events of dlm_policy (head_events).

The library records the pair right before and right after the kernel that streams W_vocab:
on the streaming path that kernel is the whole step, on the GEMM-shaped path it sits between
the hidden-row packing and the merge + commit kernel.  The pair must bracket a positive time no
longer than the whole call, and a step with the events set must produce the same outputs as a
step without them.
"""
import pytest

from parity_util import say

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from decoding_step_amd import _native
    _native.load()


@pytest.mark.parametrize("B,L,H,V", [
    (1, 32, 2048, 20011),     # streaming path: one kernel per step
    (16, 32, 2048, 30011),    # GEMM path, 512-row group: pack, head, finalize
    (4, 32, 256, 5003),       # GEMM path, 256-row group
])
def test_head_events_bracket_the_head_kernel(B, L, H, V):
    say(f"gpu: head events B={B} L={L} H={H} V={V}")
    from decoding_step_amd import _native as nat
    from decoding_step_amd.device import Decoder, new_credit, to_device
    from decoding_step_amd.synth import make_weights
    W = to_device(make_weights(V, H, "bf16"))
    seq = [(nat.DLM_THRESHOLD, 0.9, 0.0, 0)] * B
    g = torch.Generator(device="cuda").manual_seed(3)
    h = (torch.randn((B, L, H), device="cuda", generator=g) * 2).to(torch.bfloat16)
    outs = []
    for timed in (False, True):
        dec = Decoder(W, B, L, seq)
        mask = torch.ones((B, L), dtype=torch.uint8, device="cuda")
        credit = new_credit(B, L)
        call0, head0, head1, call1 = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        if timed:
            dec.policy.set_head_events(head0, head1)
        call0.record()
        dec.step(h, mask, credit)
        call1.record()
        torch.cuda.synchronize()
        outs.append((dec.out_tokens.clone(), dec.out_commit.clone(), mask.clone()))
        if timed:
            t_head, t_call = head0.elapsed_time(head1), call0.elapsed_time(call1)
            say(f"  head {t_head * 1e3:.1f} us of {t_call * 1e3:.1f} us")
            assert 0.0 < t_head <= t_call
    for a, b in zip(*outs):
        assert torch.equal(a, b)
