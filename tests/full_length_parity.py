"""Full-length lockstep parity on the GPU: each workload for its whole run, not a prefix.

tests/test_gpu_full_runs.py runs it for every workload in the GPU suite; it also runs by name on
a GPU machine:

    python tests/full_length_parity.py [workload ...]

The protocol is the lockstep of the GPU parity tests (parity_util.Lockstep): every step both
sides consume the oracle's state for the followed sequences; tokens must match where the
oracle's top-2 gap is at least 1e-2, confidences within 1e-3 relative, and commits, masks and
credit slots bit for bit unless the step is flagged (F1 for credit decoding, F2, F3).  Any
mismatch raises.  Run lengths, from the workload definitions:

    tiny_threshold_f32    one block (until its 8 positions are committed)
    threshold_b1_l32      32 blocks of 32 (generation length 1024)
    credit_b1_l32         32 blocks of 32
    hierarchical_b1_l64   32 blocks of 64 (generation length 2048)
    mixed_b16_l32         64 steps; the oracle follows sequences 0, 7 (threshold) and 8, 15 (credit)
"""
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
for p in (HERE, ROOT):
    if p not in sys.path:
        sys.path.insert(0, p)

import oracle  # noqa: E402
from parity_util import Lockstep, say  # noqa: E402

RUNS = {
    "tiny_threshold_f32": dict(blocks=1),
    "threshold_b1_l32": dict(blocks=32),
    "credit_b1_l32": dict(blocks=32),
    "hierarchical_b1_l64": dict(blocks=32),
    "mixed_b16_l32": dict(steps=64, sample=[0, 7, 8, 15]),
}


def run(name):
    import torch
    from decoding_step_amd import _native as nat
    from decoding_step_amd.device import Decoder, to_device
    from decoding_step_amd.synth import make_weights
    from decoding_step_amd.workloads import WORKLOADS
    wl = WORKLOADS[name]
    spec = dict(RUNS[name])
    sample = spec.pop("sample", None)
    say(f"[{name}] weights V={wl.V} H={wl.H} {wl.dtype}; run {spec}")
    W = make_weights(wl.V, wl.H, wl.dtype)
    Wd, W64 = to_device(W), oracle.as_f64(W)
    ls = Lockstep(wl, W, Wd, W64, lambda w, B, L, seq: Decoder(w, B, L, seq, flags=nat.DLM_AUTO_ADVANCE),
                  sample_seqs=sample)
    t0 = time.time()
    while True:
        if "steps" in spec and ls.steps >= spec["steps"]:
            break
        if "blocks" in spec and min(p[0] for p in ls.pos) >= spec["blocks"]:
            break
        ls.step()
        if ls.steps % 8 == 0:
            say(f"[{name}] step {ls.steps}, blocks done {min(p[0] for p in ls.pos)}, {time.time() - t0:.0f}s")
    say(f"[{name}] PASS: {ls.steps} steps, {ls.commits} commits of followed sequences, flags {dict(ls.flags)}, "
        f"sequence-steps checked bit for bit {dict(ls.checked)}, {time.time() - t0:.0f}s")
    del W, Wd, W64, ls
    torch.cuda.empty_cache()


def main(argv):
    import torch
    if not torch.cuda.is_available():
        sys.exit("full_length_parity.py needs a GPU")
    for name in (argv or list(RUNS)):
        run(name)


if __name__ == "__main__":
    main(sys.argv[1:])
