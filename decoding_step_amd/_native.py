"""ctypes binding of ``libdlm.so`` -- argument marshalling only.

Every entry point keeps the C name and argument order of ``include/dlm.h``.
Tensor arguments may be torch tensors (their ``data_ptr()`` is passed) or raw
integer addresses; shapes come from the :class:`StepPolicy`.  All checking
is done by the library, which returns a status; a non-zero status raises
:class:`DlmError` with ``dlm_last_error()``.  There is no fallback: without
the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdlm.so")

DLM_OK, DLM_ERR_NULL, DLM_ERR_DTYPE, DLM_ERR_SHAPE, DLM_ERR_POLICY, DLM_ERR_WORKSPACE, DLM_ERR_HIP = 0, -1, -2, -3, -4, -5, -6
DLM_F32, DLM_BF16 = 0, 1
DLM_THRESHOLD, DLM_HIERARCHICAL, DLM_CREDIT = 0, 1, 2
DLM_AUTO_ADVANCE = 1
DLM_SEQ_RUNNING, DLM_SEQ_FINISHED, DLM_SEQ_EOS_IN_BLOCK = 0, 1, 2
DLM_MAX_SEQS, DLM_MAX_L, DLM_CREDIT_SLOTS, DLM_MAX_RULES, DLM_MAX_TOPK, DLM_MAX_SHARDS = 256, 64, 4, 8, 8, 256
DLM_NOALLOC_SCRATCH_BYTES = 8 << 20

STATUS_NAMES = {0: "DLM_OK", -1: "DLM_ERR_NULL", -2: "DLM_ERR_DTYPE", -3: "DLM_ERR_SHAPE",
                -4: "DLM_ERR_POLICY", -5: "DLM_ERR_WORKSPACE", -6: "DLM_ERR_HIP"}


class dlm_credit_slot(ctypes.Structure):
    _fields_ = [("token", ctypes.c_int32), ("credit", ctypes.c_float)]


class dlm_shard_record(ctypes.Structure):
    _fields_ = [("max_logit", ctypes.c_float), ("sum_exp", ctypes.c_float), ("token", ctypes.c_int32),
                ("second_logit", ctypes.c_float)]


class dlm_seq_policy(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("threshold", ctypes.c_float),
                ("decay", ctypes.c_float), ("max_depth", ctypes.c_int32), ("eos_token", ctypes.c_int32)]


class dlm_policy(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("L", ctypes.c_int64), ("H", ctypes.c_int64), ("V", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("seq", ctypes.POINTER(dlm_seq_policy)),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("stream", ctypes.c_void_p),
                ("out_conf", ctypes.c_void_p), ("out_gap", ctypes.c_void_p),
                ("seq_done", ctypes.c_void_p),
                ("topk", ctypes.c_int32), ("out_topk_tokens", ctypes.c_void_p), ("out_topk_prob", ctypes.c_void_p),
                ("head_events", ctypes.c_void_p * 2)]


class DlmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run __graft_entry__.build() (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    pol = ctypes.POINTER(dlm_policy)
    lib.dlm_decode_step.argtypes = [vp, vp, vp, vp, pol, vp, vp]
    lib.dlm_decode_step.restype = ctypes.c_int
    lib.dlm_decode_step_noalloc.argtypes = [vp, vp, vp, vp, pol, vp, vp]
    lib.dlm_decode_step_noalloc.restype = ctypes.c_int
    lib.dlm_decode_steps.argtypes = [vp, vp, vp, vp, pol, i64, vp, vp]
    lib.dlm_decode_steps.restype = ctypes.c_int
    lib.dlm_token_stats.argtypes = [vp, vp, pol, vp, vp, vp]
    lib.dlm_token_stats.restype = ctypes.c_int
    lib.dlm_commit.argtypes = [vp, vp, vp, vp, pol, vp]
    lib.dlm_commit.restype = ctypes.c_int
    lib.dlm_shard_stats.argtypes = [vp, vp, i64, pol, vp]
    lib.dlm_shard_stats.restype = ctypes.c_int
    lib.dlm_merge_commit.argtypes = [vp, i64, vp, vp, pol, vp, vp]
    lib.dlm_merge_commit.restype = ctypes.c_int
    lib.dlm_workspace_bytes.argtypes = [i64, i64, i64, i64, i32]
    lib.dlm_workspace_bytes.restype = ctypes.c_size_t
    lib.dlm_workspace_bytes_topk.argtypes = [i64, i64, i64, i64, i32, i32]
    lib.dlm_workspace_bytes_topk.restype = ctypes.c_size_t
    lib.dlm_workspace_init.argtypes = [vp, ctypes.c_size_t, vp]
    lib.dlm_workspace_init.restype = ctypes.c_int
    lib.dlm_last_error.argtypes = []
    lib.dlm_last_error.restype = ctypes.c_char_p
    lib.dlm_version.argtypes = []
    lib.dlm_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _check(status: int) -> None:
    if status != DLM_OK:
        raise DlmError(status, load().dlm_last_error().decode())


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream  # torch.cuda.Stream on ROCm wraps a hipStream_t


class StepPolicy:
    """Python side of ``dlm_policy``: shapes, per-sequence rules and launch context.

    ``seq`` is a list of ``(kind, threshold, decay, max_depth[, eos_token])``
    tuples or objects with those fields (``eos_token`` -1 when absent).  The C
    struct is built once and reused; only pointers change between calls.
    """

    def __init__(self, B: int, L: int, H: int, V: int, dtype: int, seq: Sequence, workspace=None,
                 workspace_bytes: Optional[int] = None, flags: int = 0, stream=None, out_conf=None, out_gap=None,
                 seq_done=None, topk: int = 0, out_topk_tokens=None, out_topk_prob=None):
        self._seq = (dlm_seq_policy * max(1, len(seq)))()
        for i, s in enumerate(seq):
            if hasattr(s, "kind"):
                k, t, d, m = s.kind, s.threshold, getattr(s, "decay", 0.0), getattr(s, "max_depth", 0)
                e = getattr(s, "eos_token", -1)
            else:
                k, t, d, m = s[:4]
                e = s[4] if len(s) > 4 else -1
            self._seq[i] = dlm_seq_policy(int(k), float(t), float(d), int(m), int(e))
        self.c = dlm_policy()
        self.c.B, self.c.L, self.c.H, self.c.V, self.c.dtype, self.c.flags = B, L, H, V, dtype, flags
        self.c.seq = ctypes.cast(self._seq, ctypes.POINTER(dlm_seq_policy)) if len(seq) else None
        self.set_workspace(workspace, workspace_bytes)
        self.c.stream = _stream_handle(stream)
        self.c.out_conf = _ptr(out_conf)
        self.c.out_gap = _ptr(out_gap)
        self.c.seq_done = _ptr(seq_done)
        self.set_topk(topk, out_topk_tokens, out_topk_prob)
        self._keep = (workspace, out_conf, out_gap, seq_done)

    def set_workspace(self, workspace, nbytes: Optional[int] = None) -> None:
        self.c.workspace = _ptr(workspace)
        if nbytes is None:
            nbytes = workspace.numel() * workspace.element_size() if workspace is not None and not isinstance(workspace, int) else 0
        self.c.workspace_bytes = nbytes

    def set_stream(self, stream) -> None:
        self.c.stream = _stream_handle(stream)

    def set_seq_done(self, seq_done=None) -> None:
        self.c.seq_done = _ptr(seq_done)

    def set_topk(self, topk: int = 0, out_topk_tokens=None, out_topk_prob=None) -> None:
        self.c.topk = int(topk)
        self.c.out_topk_tokens = _ptr(out_topk_tokens)
        self.c.out_topk_prob = _ptr(out_topk_prob)
        self._keep_topk = (out_topk_tokens, out_topk_prob)

    def set_head_events(self, begin=None, end=None) -> None:
        """Events recorded right before / after the vocabulary-head kernel (``head_events``):
        ``torch.cuda.Event(enable_timing=True)`` objects or raw ``hipEvent_t`` handles, or None."""
        def handle(ev):
            if ev is None or isinstance(ev, int):
                return ev or None
            if not ev.cuda_event:          # torch creates the event at its first record
                ev.record()
            return ev.cuda_event
        self.c.head_events[0] = handle(begin)
        self.c.head_events[1] = handle(end)
        self._keep_events = (begin, end)

    def set_outputs(self, out_conf=None, out_gap=None) -> None:
        self.c.out_conf = _ptr(out_conf)
        self.c.out_gap = _ptr(out_gap)


def dlm_decode_step(hidden, W_vocab, mask_state, credit_state, policy: StepPolicy, out_tokens, out_commit) -> None:
    _check(load().dlm_decode_step(_ptr(hidden), _ptr(W_vocab), _ptr(mask_state), _ptr(credit_state),
                                  ctypes.byref(policy.c), _ptr(out_tokens), _ptr(out_commit)))


def dlm_decode_step_noalloc(hidden, W_vocab, mask_state, credit_state, policy: StepPolicy, out_tokens,
                            out_commit) -> None:
    """dlm_decode_step with the library's static per-GPU scratch as workspace (policy's workspace ignored)."""
    _check(load().dlm_decode_step_noalloc(_ptr(hidden), _ptr(W_vocab), _ptr(mask_state), _ptr(credit_state),
                                          ctypes.byref(policy.c), _ptr(out_tokens), _ptr(out_commit)))


def dlm_decode_steps(hidden_steps, W_vocab, mask_state, credit_state, policy: StepPolicy, n_steps: int,
                     out_tokens_steps, out_commit_steps) -> None:
    _check(load().dlm_decode_steps(_ptr(hidden_steps), _ptr(W_vocab), _ptr(mask_state), _ptr(credit_state),
                                   ctypes.byref(policy.c), int(n_steps), _ptr(out_tokens_steps),
                                   _ptr(out_commit_steps)))


def dlm_token_stats(hidden, W_vocab, policy: StepPolicy, out_conf, out_tokens, out_gap=None) -> None:
    _check(load().dlm_token_stats(_ptr(hidden), _ptr(W_vocab), ctypes.byref(policy.c), _ptr(out_conf),
                                  _ptr(out_tokens), _ptr(out_gap)))


def dlm_commit(conf, tokens, mask_state, credit_state, policy: StepPolicy, out_commit) -> None:
    _check(load().dlm_commit(_ptr(conf), _ptr(tokens), _ptr(mask_state), _ptr(credit_state),
                             ctypes.byref(policy.c), _ptr(out_commit)))


def dlm_shard_stats(hidden, W_shard, v_begin: int, policy: StepPolicy, out_records) -> None:
    """out_records: [B][L] dlm_shard_record, e.g. a float32 tensor [B][L][4] (max, sum, id bits, second)."""
    _check(load().dlm_shard_stats(_ptr(hidden), _ptr(W_shard), int(v_begin), ctypes.byref(policy.c), _ptr(out_records)))


def dlm_merge_commit(records, n_shards: int, mask_state, credit_state, policy: StepPolicy, out_tokens,
                     out_commit) -> None:
    _check(load().dlm_merge_commit(_ptr(records), int(n_shards), _ptr(mask_state), _ptr(credit_state),
                                   ctypes.byref(policy.c), _ptr(out_tokens), _ptr(out_commit)))


def dlm_workspace_bytes(B: int, L: int, H: int, V: int, dtype: int) -> int:
    return int(load().dlm_workspace_bytes(B, L, H, V, dtype))


def dlm_workspace_bytes_topk(B: int, L: int, H: int, V: int, dtype: int, topk: int) -> int:
    return int(load().dlm_workspace_bytes_topk(B, L, H, V, dtype, topk))


def dlm_workspace_init(workspace, workspace_bytes: Optional[int] = None, stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check(load().dlm_workspace_init(_ptr(workspace), workspace_bytes, _stream_handle(stream)))


def dlm_last_error() -> str:
    return load().dlm_last_error().decode()


def dlm_version() -> str:
    return load().dlm_version().decode()
