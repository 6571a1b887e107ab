"""Device-memory helpers around the C ABI (torch supplies memory and streams only)."""
from __future__ import annotations

import numpy as np
import torch

from . import _native as nat


def torch_dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return nat.DLM_BF16
    if t.dtype == torch.float32:
        return nat.DLM_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    """numpy -> device tensor; uint16 arrays are bfloat16 bit patterns."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def new_credit(B: int, L: int, device="cuda") -> torch.Tensor:
    """``[B][L][4]`` dlm_credit_slot records as int32 pairs, all empty (token -1, credit 0)."""
    t = torch.zeros((B, L, nat.DLM_CREDIT_SLOTS, 2), dtype=torch.int32, device=device)
    t[..., 0] = -1
    return t


def credit_tokens(t: torch.Tensor) -> torch.Tensor:
    return t[..., 0]


def credit_values(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.float32)[..., 1]


def credit_from_numpy(tok: np.ndarray, val: np.ndarray, device="cuda") -> torch.Tensor:
    rec = np.empty(tok.shape + (2,), dtype=np.int32)
    rec[..., 0] = tok
    rec[..., 1] = np.asarray(val, dtype=np.float32).view(np.int32)
    return torch.from_numpy(rec).to(device)


class Decoder:
    """One decode step on device buffers it owns: workspace, outputs and diagnostics."""

    def __init__(self, W: torch.Tensor, B: int, L: int, seq, flags: int = 0, stream=None, diagnostics: bool = True,
                 topk: int = 0):
        V, H = W.shape
        self.W, self.B, self.L, self.H, self.V = W, B, L, H, V
        dev = W.device
        code = torch_dtype_code(W)
        nbytes = nat.dlm_workspace_bytes_topk(B, L, H, V, code, topk)
        if nbytes == 0:
            raise nat.DlmError(nat.DLM_ERR_SHAPE, f"unsupported shapes B={B} L={L} H={H} V={V}")
        self.workspace = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
        self.out_tokens = torch.empty((B, L), dtype=torch.int32, device=dev)
        self.out_commit = torch.empty((B, L), dtype=torch.uint8, device=dev)
        self.conf = torch.empty((B, L), dtype=torch.float32, device=dev) if diagnostics else None
        self.gap = torch.empty((B, L), dtype=torch.float32, device=dev) if diagnostics else None
        self.topk = topk
        self.topk_tokens = torch.empty((B, L, topk), dtype=torch.int32, device=dev) if topk else None
        self.topk_prob = torch.empty((B, L, topk), dtype=torch.float32, device=dev) if topk else None
        self.policy = nat.StepPolicy(B, L, H, V, code, seq, self.workspace, flags=flags, stream=stream,
                                     out_conf=self.conf, out_gap=self.gap, topk=topk,
                                     out_topk_tokens=self.topk_tokens, out_topk_prob=self.topk_prob)

    def step(self, hidden: torch.Tensor, mask: torch.Tensor, credit=None) -> None:
        nat.dlm_decode_step(hidden, self.W, mask, credit, self.policy, self.out_tokens, self.out_commit)

    def steps(self, hidden_steps: torch.Tensor, mask: torch.Tensor, credit, out_tokens: torch.Tensor,
              out_commit: torch.Tensor, out_topk_tokens=None, out_topk_prob=None) -> None:
        """hidden_steps[n] for step n; per-step outputs [n][B][L] (dlm_decode_steps), and with top-k on
        per-step exports [n][B][L][topk] (required: the library writes one export per step)."""
        n = hidden_steps.shape[0]
        if self.topk:
            if out_topk_tokens is None or out_topk_tokens.numel() < n * self.B * self.L * self.topk:
                raise ValueError(f"top-k is on: out_topk_tokens must hold [{n}][{self.B}][{self.L}][{self.topk}]")
            if out_topk_prob is not None and out_topk_prob.numel() < n * self.B * self.L * self.topk:
                raise ValueError(f"out_topk_prob must hold [{n}][{self.B}][{self.L}][{self.topk}]")
            self.policy.set_topk(self.topk, out_topk_tokens, out_topk_prob)
        try:
            nat.dlm_decode_steps(hidden_steps, self.W, mask, credit, self.policy, n, out_tokens, out_commit)
        finally:
            if self.topk:
                self.policy.set_topk(self.topk, self.topk_tokens, self.topk_prob)

    def token_stats(self, hidden: torch.Tensor, conf: torch.Tensor, tokens: torch.Tensor, gap=None) -> None:
        nat.dlm_token_stats(hidden, self.W, self.policy, conf, tokens, gap)
