"""The C ABI without a GPU: exports, sizing, and every host-side validation error.

Validation happens before any HIP call, so these calls pass fake (non-NULL,
never dereferenced) device addresses and expect the documented status.
"""
import ctypes
import math
import os
import re

import pytest

from decoding_step_amd import _native as nat

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dlm.h")
FAKE = 0x10000          # 256-byte aligned, never dereferenced
MISALIGNED = 0x10008


@pytest.fixture(scope="module")
def lib():
    return nat.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(dlm_[a-z_]+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) >= {"dlm_decode_step", "dlm_token_stats", "dlm_commit", "dlm_workspace_bytes",
                          "dlm_workspace_init", "dlm_last_error", "dlm_version"}
    for n in names:
        assert hasattr(lib, n), n


def test_version_matches_header(lib):
    m = re.search(r'#define DLM_VERSION_STRING "([^"]+)"', open(HEADER).read())
    assert nat.dlm_version() == m.group(1)


def test_header_constants_match_binding():
    text = open(HEADER).read()
    for name in ["DLM_MAX_SEQS", "DLM_MAX_L", "DLM_CREDIT_SLOTS", "DLM_MAX_RULES", "DLM_MAX_TOPK", "DLM_MAX_SHARDS"]:
        assert int(re.search(rf"#define {name} (\d+)", text).group(1)) == getattr(nat, name)
    assert int(re.search(r"#define DLM_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text).group(1)) << \
        int(re.search(r"#define DLM_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text).group(2)) == \
        nat.DLM_NOALLOC_SCRATCH_BYTES
    for name in ["DLM_SEQ_RUNNING", "DLM_SEQ_FINISHED", "DLM_SEQ_EOS_IN_BLOCK"]:
        assert int(re.search(rf"{name} = (\d+)", text).group(1)) == getattr(nat, name)
    assert ctypes.sizeof(nat.dlm_credit_slot) == 8
    assert ctypes.sizeof(nat.dlm_shard_record) == 16
    assert ctypes.sizeof(nat.dlm_seq_policy) == 20       # the library asserts the same sizes
    assert ctypes.sizeof(nat.dlm_policy) == 136


def test_workspace_sizes():
    # streaming plan: counters (one global + one per group of 16 vocabulary ranges, padded to
    # 256 B) + one 16-byte record per (padded row, vocabulary range) + one second-level record
    # per (padded row, group); rows are padded to 16, 32 or 64 per row group and there are at most
    # 256 vocabulary ranges (16 groups)
    assert nat.dlm_workspace_bytes(1, 32, 2048, 126464, nat.DLM_BF16) == 256 + 32 * 256 * 16 + 32 * 16 * 16
    assert nat.dlm_workspace_bytes(1, 64, 2048, 126464, nat.DLM_BF16) == 256 + 64 * 256 * 16 + 64 * 16 * 16
    assert nat.dlm_workspace_bytes(1, 8, 64, 1024, nat.DLM_F32) == 256 + 16 * 64 * 16 + 16 * 4 * 16  # 64 tiles
    # GEMM-shaped path (bf16, more than 64 rows): records for every (padded row, workgroup of its
    # row group), then the hidden rows in fragment order (rows padded to 32), then one 16-byte
    # value per row for the commit; a counter per sequence first (padded to 256 B); up to 256 rows
    # one 256-row group against 256-row vocabulary tiles, beyond that 512-row groups against
    # 128-row tiles; workgroups per group a multiple of 8 where there are enough tiles
    assert nat.dlm_workspace_bytes(8, 32, 2048, 157184, nat.DLM_BF16) == \
        256 + 256 * 256 * 16 + 256 * 2048 * 2 + 256 * 16
    assert nat.dlm_workspace_bytes(16, 32, 2048, 157184, nat.DLM_BF16) == \
        256 + 512 * 256 * 16 + 512 * 2048 * 2 + 512 * 16   # 1228 tiles, one group of 256 workgroups
    assert nat.dlm_workspace_bytes(17, 31, 512, 5003, nat.DLM_BF16) == \
        256 + 1024 * 40 * 16 + 544 * 512 * 2 + 527 * 16   # 40 tiles, 2 groups, 527 rows padded to 544
    assert nat.dlm_workspace_bytes(128, 8, 256, 5003, nat.DLM_BF16) == \
        512 + 1024 * 40 * 16 + 1024 * 256 * 2 + 1024 * 16   # 128 counters: 512 B
    for bad in [(0, 8, 64, 64, 0), (1, 65, 64, 64, 0), (1, 8, 48, 64, 0), (1, 8, 64, 0, 0), (1, 8, 64, 64, 5),
                (257, 8, 64, 64, 1), (1, 8, 1 << 20, 64, 1), (1, 8, 4128, 64, 1), (1, 8, 2080, 64, 0)]:
        assert nat.dlm_workspace_bytes(*bad) == 0, bad


def policy(B=1, L=8, H=64, V=1024, dtype=nat.DLM_BF16, seq=None, ws=FAKE, ws_bytes=1 << 20, flags=0, topk=0,
           topk_tokens=FAKE):
    seq = seq if seq is not None else [(nat.DLM_THRESHOLD, 0.9, 0.0, 0)] * B
    return nat.StepPolicy(B, L, H, V, dtype, seq, workspace=ws, workspace_bytes=ws_bytes, flags=flags, topk=topk,
                          out_topk_tokens=topk_tokens if topk else None)


def status_of(fn, *args):
    try:
        fn(*args)
    except nat.DlmError as e:
        assert nat.dlm_last_error() != ""
        return e.status
    return nat.DLM_OK


def step(p, hidden=FAKE, W=FAKE, mask=FAKE, credit=FAKE, out_tok=FAKE, out_commit=FAKE):
    return status_of(nat.dlm_decode_step, hidden, W, mask, credit, p, out_tok, out_commit)


def test_null_pointers():
    p = policy()
    assert step(p, hidden=None) == nat.DLM_ERR_NULL
    assert step(p, W=None) == nat.DLM_ERR_NULL
    assert step(p, mask=None) == nat.DLM_ERR_NULL
    assert step(p, out_tok=None) == nat.DLM_ERR_NULL
    assert step(p, out_commit=None) == nat.DLM_ERR_NULL
    assert nat.load().dlm_decode_step(FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE) == nat.DLM_ERR_NULL
    assert step(policy(ws=None)) == nat.DLM_ERR_NULL
    assert step(policy(seq=[]), credit=None) == nat.DLM_ERR_NULL           # seq == NULL
    credit_pol = policy(seq=[(nat.DLM_CREDIT, 1.2, 0.7, 0)])
    assert step(credit_pol, credit=None) == nat.DLM_ERR_NULL


def test_bad_dtype():
    assert step(policy(dtype=2)) == nat.DLM_ERR_DTYPE
    assert step(policy(dtype=-1)) == nat.DLM_ERR_DTYPE


@pytest.mark.parametrize("kw", [dict(B=0), dict(B=257, seq=[(0, 0.9, 0, 0)] * 257), dict(L=0), dict(L=65),
                                dict(H=0), dict(H=48), dict(H=16), dict(V=0), dict(H=1 << 16)])
def test_bad_shapes(kw):
    assert step(policy(**kw)) == nat.DLM_ERR_SHAPE


@pytest.mark.parametrize("seq", [
    [(7, 0.9, 0.0, 0)],
    [(-1, 0.9, 0.0, 0)],
    [(nat.DLM_THRESHOLD, math.nan, 0.0, 0)],
    [(nat.DLM_THRESHOLD, math.inf, 0.0, 0)],
    [(nat.DLM_CREDIT, 1.2, 1.0, 0)],
    [(nat.DLM_CREDIT, 1.2, -0.1, 0)],
    [(nat.DLM_HIERARCHICAL, 0.7, 0.0, -1)],
])
def test_bad_policies(seq):
    assert step(policy(seq=seq)) == nat.DLM_ERR_POLICY


def test_bad_end_tokens():
    assert step(policy_with_done(V=1024, eos=-2)) == nat.DLM_ERR_POLICY
    assert step(policy_with_done(V=1024, eos=1024)) == nat.DLM_ERR_POLICY
    # dlm_commit knows no vocabulary: any token id >= 0 passes, -2 does not
    p = policy_with_done(V=1024, eos=-2)
    assert status_of(nat.dlm_commit, FAKE, FAKE, FAKE, FAKE, p, FAKE) == nat.DLM_ERR_POLICY


def policy_with_done(V, eos):
    return nat.StepPolicy(1, 8, 64, V, nat.DLM_BF16, [(nat.DLM_THRESHOLD, 0.9, 0.0, 0, eos)], workspace=FAKE,
                          workspace_bytes=1 << 20, seq_done=FAKE)


def test_too_many_distinct_rules():
    seq = [(nat.DLM_THRESHOLD, 0.5 + 0.01 * i, 0.0, 0) for i in range(9)]
    assert step(policy(B=9, seq=seq)) == nat.DLM_ERR_POLICY
    seq = [(nat.DLM_THRESHOLD, 0.5 + 0.01 * (i % 8), 0.0, 0) for i in range(200)]
    # 8 distinct rules over 200 sequences pass validation; a tiny workspace then stops the call
    assert step(policy(B=200, seq=seq, ws_bytes=16)) == nat.DLM_ERR_WORKSPACE


def test_workspace_too_small():
    need = nat.dlm_workspace_bytes(1, 8, 64, 1024, nat.DLM_BF16)
    assert step(policy(ws_bytes=need - 1)) == nat.DLM_ERR_WORKSPACE


def test_misaligned_pointers():
    need = nat.dlm_workspace_bytes(1, 8, 64, 1024, nat.DLM_BF16)
    assert step(policy(ws_bytes=need), hidden=MISALIGNED) == nat.DLM_ERR_SHAPE
    assert step(policy(ws_bytes=need), W=MISALIGNED) == nat.DLM_ERR_SHAPE
    assert step(policy(ws=MISALIGNED, ws_bytes=need)) == nat.DLM_ERR_SHAPE


def test_token_stats_and_commit_validation():
    p = policy()
    assert status_of(nat.dlm_token_stats, None, FAKE, p, FAKE, FAKE) == nat.DLM_ERR_NULL
    assert status_of(nat.dlm_token_stats, FAKE, FAKE, p, None, FAKE) == nat.DLM_ERR_NULL
    assert status_of(nat.dlm_token_stats, FAKE, FAKE, policy(L=100), FAKE, FAKE) == nat.DLM_ERR_SHAPE
    assert status_of(nat.dlm_commit, None, FAKE, FAKE, FAKE, p, FAKE) == nat.DLM_ERR_NULL
    assert status_of(nat.dlm_commit, FAKE, FAKE, FAKE, FAKE, policy(L=65), FAKE) == nat.DLM_ERR_SHAPE
    assert status_of(nat.dlm_commit, FAKE, FAKE, FAKE, FAKE, policy(seq=[(9, 0.9, 0, 0)]), FAKE) == nat.DLM_ERR_POLICY
    assert status_of(nat.dlm_commit, FAKE, FAKE, FAKE, None, policy(seq=[(2, 1.2, 0.7, 0)]), FAKE) == nat.DLM_ERR_NULL
    assert status_of(nat.dlm_workspace_init, None, 16) == nat.DLM_ERR_NULL


def test_decode_steps_validation():
    # every check of dlm_decode_step, plus the step count, before anything is enqueued
    need = nat.dlm_workspace_bytes(1, 8, 64, 1024, nat.DLM_BF16)
    p = policy(ws_bytes=need)
    steps = lambda pol, n=2, hidden=FAKE, tok=FAKE, com=FAKE: status_of(
        nat.dlm_decode_steps, hidden, FAKE, FAKE, FAKE, pol, n, tok, com)
    assert steps(p, n=0) == nat.DLM_ERR_SHAPE
    assert steps(p, n=-3) == nat.DLM_ERR_SHAPE
    assert steps(p, hidden=None) == nat.DLM_ERR_NULL
    assert steps(p, tok=None) == nat.DLM_ERR_NULL
    assert steps(p, com=None) == nat.DLM_ERR_NULL
    assert steps(p, hidden=MISALIGNED) == nat.DLM_ERR_SHAPE
    assert steps(policy(ws_bytes=need - 1)) == nat.DLM_ERR_WORKSPACE
    assert steps(policy(L=65)) == nat.DLM_ERR_SHAPE
    assert steps(policy(seq=[(7, 0.9, 0, 0)])) == nat.DLM_ERR_POLICY
    assert nat.load().dlm_decode_steps(FAKE, FAKE, FAKE, FAKE, None, 2, FAKE, FAKE) == nat.DLM_ERR_NULL


def test_topk_workspace_sizes():
    # top-k on, streaming plan (up to 64 rows, or float32): one list of 8 (logit, id) pairs (64
    # bytes) per (padded row, vocabulary range) after the statistics records, then one merged list
    # per (padded row, group of 16 ranges)
    base = 256 + 32 * 256 * 16 + 32 * 16 * 16
    assert nat.dlm_workspace_bytes_topk(1, 32, 2048, 126464, nat.DLM_BF16, 8) == base + 32 * 256 * 64 + 32 * 16 * 64
    assert nat.dlm_workspace_bytes_topk(1, 32, 2048, 126464, nat.DLM_BF16, 3) == base + 32 * 256 * 64 + 32 * 16 * 64
    assert nat.dlm_workspace_bytes_topk(8, 32, 256, 20011, nat.DLM_F32, 8) == \
        256 + 256 * 64 * 16 + 256 * 4 * 16 + 256 * 64 * 64 + 256 * 4 * 64   # 4 groups of 64 rows, 64 ranges
    # GEMM-shaped plan beyond 64 bf16 rows: always the 512-row group shape; after the plain GEMM
    # workspace, one list of 8 chunk entries (64 bytes) per (padded row, workgroup)
    assert nat.dlm_workspace_bytes_topk(16, 32, 2048, 157184, nat.DLM_BF16, 8) == \
        nat.dlm_workspace_bytes(16, 32, 2048, 157184, nat.DLM_BF16) + 512 * 256 * 64
    assert nat.dlm_workspace_bytes_topk(5, 13, 256, 3001, nat.DLM_BF16, 8) == \
        256 + 512 * 24 * 16 + 96 * 256 * 2 + 65 * 16 + 512 * 24 * 64     # 24 tiles of 128: 24 workgroups
    # the largest vocabulary of the GEMM head with chunk lists: V = 2^22 - 1 (22-bit ids, 128 rows
    # in one 512-row group, 256 workgroups); at V = 2^22 W passes 2 GiB and the streaming plan
    # takes the 128 rows (two 64-row groups, 128 ranges, 8 groups of ranges)
    assert nat.dlm_workspace_bytes_topk(2, 64, 256, (1 << 22) - 1, nat.DLM_BF16, 8) == \
        256 + 512 * 256 * 16 + 128 * 256 * 2 + 128 * 16 + 512 * 256 * 64
    assert nat.dlm_workspace_bytes_topk(2, 64, 256, 1 << 22, nat.DLM_BF16, 8) == \
        256 + 2 * 64 * 128 * 16 + 2 * 64 * 8 * 16 + 2 * 64 * 128 * 64 + 2 * 64 * 8 * 64
    for B, L, H, V, dt in [(1, 32, 2048, 126464, 1), (16, 32, 2048, 157184, 1), (1, 8, 64, 1024, 0)]:
        assert nat.dlm_workspace_bytes_topk(B, L, H, V, dt, 0) == nat.dlm_workspace_bytes(B, L, H, V, dt)
    assert nat.dlm_workspace_bytes_topk(1, 32, 2048, 126464, nat.DLM_BF16, 9) == 0
    assert nat.dlm_workspace_bytes_topk(1, 32, 2048, 126464, nat.DLM_BF16, -1) == 0
    assert nat.dlm_workspace_bytes_topk(0, 32, 2048, 126464, nat.DLM_BF16, 4) == 0


def test_topk_validation():
    need = nat.dlm_workspace_bytes_topk(1, 8, 64, 1024, nat.DLM_BF16, 4)
    assert need > nat.dlm_workspace_bytes(1, 8, 64, 1024, nat.DLM_BF16)
    assert step(policy(ws_bytes=need, topk=9)) == nat.DLM_ERR_POLICY
    assert step(policy(ws_bytes=need, topk=-2)) == nat.DLM_ERR_POLICY
    assert step(policy(ws_bytes=need, topk=4, topk_tokens=None)) == nat.DLM_ERR_NULL
    assert step(policy(ws_bytes=need - 1, topk=4)) == nat.DLM_ERR_WORKSPACE
    small = nat.dlm_workspace_bytes(1, 8, 64, 1024, nat.DLM_BF16)
    assert status_of(nat.dlm_token_stats, FAKE, FAKE, policy(ws_bytes=small, topk=4), FAKE, FAKE) == nat.DLM_ERR_WORKSPACE
    assert status_of(nat.dlm_token_stats, FAKE, FAKE, policy(ws_bytes=need, topk=99), FAKE, FAKE) == nat.DLM_ERR_POLICY
    steps = lambda pol: status_of(nat.dlm_decode_steps, FAKE, FAKE, FAKE, FAKE, pol, 2, FAKE, FAKE)
    assert steps(policy(ws_bytes=need, topk=4, topk_tokens=None)) == nat.DLM_ERR_NULL
    assert steps(policy(ws_bytes=need, topk=12)) == nat.DLM_ERR_POLICY


def test_decoder_steps_needs_per_step_topk_buffers():
    # with the export on, dlm_decode_steps writes one [B][L][k] export per step: the Decoder
    # refuses buffers that cannot hold them instead of passing its single-step ones
    torch = pytest.importorskip("torch")
    from decoding_step_amd.device import Decoder
    W = torch.zeros((1024, 64), dtype=torch.bfloat16)
    dec = Decoder(W, 1, 8, [(nat.DLM_THRESHOLD, 0.9, 0.0, 0)], topk=4)
    assert dec.workspace.numel() == nat.dlm_workspace_bytes_topk(1, 8, 64, 1024, nat.DLM_BF16, 4)
    hs = torch.zeros((3, 1, 8, 64), dtype=torch.bfloat16)
    out_t = torch.zeros((3, 1, 8), dtype=torch.int32)
    out_c = torch.zeros((3, 1, 8), dtype=torch.uint8)
    with pytest.raises(ValueError, match="top-k is on"):
        dec.steps(hs, torch.ones((1, 8), dtype=torch.uint8), None, out_t, out_c)
    with pytest.raises(ValueError, match="top-k is on"):
        dec.steps(hs, torch.ones((1, 8), dtype=torch.uint8), None, out_t, out_c,
                  torch.zeros((2, 1, 8, 4), dtype=torch.int32))


def test_shard_calls_validation():
    need = nat.dlm_workspace_bytes(1, 8, 64, 1024, nat.DLM_BF16)
    p = policy(ws_bytes=need)
    shard = lambda pol, hidden=FAKE, W=FAKE, v0=0, out=FAKE: status_of(nat.dlm_shard_stats, hidden, W, v0, pol, out)
    assert shard(p, hidden=None) == nat.DLM_ERR_NULL
    assert shard(p, W=None) == nat.DLM_ERR_NULL
    assert shard(p, out=None) == nat.DLM_ERR_NULL
    assert shard(p, v0=-1) == nat.DLM_ERR_SHAPE
    assert shard(p, v0=(1 << 31) - 1024) == nat.DLM_ERR_SHAPE       # the shard's last id would overflow
    assert shard(p, out=MISALIGNED) == nat.DLM_ERR_SHAPE
    assert shard(policy(ws_bytes=need, topk=2)) == nat.DLM_ERR_POLICY
    assert shard(policy(ws_bytes=need - 1)) == nat.DLM_ERR_WORKSPACE
    assert shard(policy(L=65)) == nat.DLM_ERR_SHAPE
    assert nat.load().dlm_shard_stats(FAKE, FAKE, 0, None, FAKE) == nat.DLM_ERR_NULL
    merge = lambda pol, rec=FAKE, g=8, mask=FAKE, credit=FAKE, tok=FAKE, com=FAKE: status_of(
        nat.dlm_merge_commit, rec, g, mask, credit, pol, tok, com)
    assert merge(p, rec=None) == nat.DLM_ERR_NULL
    assert merge(p, mask=None) == nat.DLM_ERR_NULL
    assert merge(p, tok=None) == nat.DLM_ERR_NULL
    assert merge(p, com=None) == nat.DLM_ERR_NULL
    assert merge(p, g=0) == nat.DLM_ERR_SHAPE
    assert merge(p, g=257) == nat.DLM_ERR_SHAPE
    assert merge(p, rec=MISALIGNED) == nat.DLM_ERR_SHAPE
    assert merge(policy(L=65)) == nat.DLM_ERR_SHAPE
    assert merge(policy(B=0, seq=[])) == nat.DLM_ERR_SHAPE
    assert merge(policy(seq=[(9, 0.9, 0, 0)])) == nat.DLM_ERR_POLICY
    assert merge(policy(seq=[(2, 1.2, 0.7, 0)]), credit=None) == nat.DLM_ERR_NULL
    assert merge(policy(seq=[(0, 0.9, 0, 0, 1024)])) == nat.DLM_ERR_POLICY      # end token past V
    assert nat.load().dlm_merge_commit(FAKE, 2, FAKE, FAKE, None, FAKE, FAKE) == nat.DLM_ERR_NULL


def test_binding_raises_without_library(tmp_path):
    saved = nat._lib
    try:
        nat._lib = None
        with pytest.raises(RuntimeError, match="not built"):
            nat.load(str(tmp_path / "missing.so"))
    finally:
        nat._lib = saved


def noalloc_step(p, hidden=FAKE, W=FAKE, mask=FAKE, credit=FAKE, out_tok=FAKE, out_commit=FAKE):
    return status_of(nat.dlm_decode_step_noalloc, hidden, W, mask, credit, p, out_tok, out_commit)


def test_noalloc_validation():
    # the same checks as dlm_decode_step, all before any HIP call; the policy's workspace is ignored
    p = policy(ws=None, ws_bytes=0)
    assert noalloc_step(p, hidden=None) == nat.DLM_ERR_NULL
    assert noalloc_step(p, out_commit=None) == nat.DLM_ERR_NULL
    assert nat.load().dlm_decode_step_noalloc(FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE) == nat.DLM_ERR_NULL
    assert noalloc_step(policy(ws=None, dtype=2)) == nat.DLM_ERR_DTYPE
    assert noalloc_step(policy(ws=None, L=65)) == nat.DLM_ERR_SHAPE
    assert noalloc_step(policy(ws=None, seq=[(7, 0.9, 0.0, 0)])) == nat.DLM_ERR_POLICY
    assert noalloc_step(policy(ws=None, seq=[(nat.DLM_CREDIT, 1.2, 0.7, 0)]), credit=None) == nat.DLM_ERR_NULL
    # shapes beyond the static scratch: rejected with a clear message, nothing enqueued
    big = dict(B=256, L=64, H=2048, V=157184)
    assert nat.dlm_workspace_bytes(*big.values(), nat.DLM_BF16) > nat.DLM_NOALLOC_SCRATCH_BYTES
    assert noalloc_step(policy(ws=None, seq=[(nat.DLM_THRESHOLD, 0.9, 0.0, 0)] * 256, **big)) == nat.DLM_ERR_WORKSPACE
    assert "DLM_NOALLOC_SCRATCH_BYTES" in nat.dlm_last_error()
    # the batched workload's shape, with and without the top-k export at one sequence, fits
    # (the workspace plus the 8 KB counter region)
    for B, L, H, V, k in [(16, 32, 2048, 157184, 0), (1, 32, 2048, 126464, 8), (1, 64, 2048, 126464, 8)]:
        need = nat.dlm_workspace_bytes_topk(B, L, H, V, nat.DLM_BF16, k)
        assert 0 < need and need - 256 + 8192 <= nat.DLM_NOALLOC_SCRATCH_BYTES, (B, L, k, need)
    assert noalloc_step(policy(ws=None), hidden=MISALIGNED) == nat.DLM_ERR_SHAPE
