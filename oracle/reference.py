"""Plain CPU reference of one masked-diffusion decode step -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  It shares no code with the HIP path
and imports nothing from it.  Inputs are plain numpy arrays; bfloat16 data
arrives as uint16 bit patterns and is widened here on its own.

What one step computes, and where it comes from.  The pages are four news
pages about dInfer; the mechanisms are only on the Traditional-Chinese
explainer of arXiv 2510.08666 hosted on 91haoming.cn ("the explainer"):

* the decoding-strategy component of the explainer decides whether to fix
  a position from how sure the model is about that position's text, which
  presupposes, per position, a candidate token and a confidence.  The
  candidate is the arg-max of the logits ``z = h W^T`` of the vocabulary
  head, the confidence the largest softmax probability ``1 / sum_v
  exp(z_v - max z)``;
* threshold decoding (same component, first strategy): fix at once every
  masked position whose confidence is high enough and leave the others
  for later iterations;
* hierarchical decoding (second strategy): split the regions still to be
  filled recursively into sub-regions and fix the centre of each region
  first;
* credit decoding (third strategy): keep, for every position and every
  candidate, a credit that grows when the candidate is chosen again with
  confidence; stable candidates then commit more easily;
* the diffusion-iteration manager paragraph: fixed-size blocks are handled
  in turn (the block of L positions is the unit of one step).

The pages give no number (threshold, decay, slot count, tie rule); those
come from the workload definitions and the readings listed in the design
notes (R1..R18): every row of the block goes through the head (R1); lowest
token id wins an arg-max tie (R2); ``conf >= tau`` commits (R3); forced picks
take the lowest position on ties (R4, R12, R15); an empty mask commits
nothing (R7); an even span's centre is ``(s + e) // 2`` (R8); credit is
updated before it is tested (R9); decay-then-add (R10); a candidate not in a
slot evicts the first empty slot, else the smallest credit, lowest slot on
ties (R11); the committed token is the current arg-max (R13); a span is split
only when its centre commits (R14); credit changes only on masked rows (R16);
``out_tokens`` holds the candidate of every row (R17); the optional top-k export ranks
float32-rounded logits with ties to the lower id and gives full-vocabulary probabilities (T1-T4).

Precision.  Logits and the softmax sum are float64 over the exact input
values (bfloat16 products are exact).  Where a float decides an integer the
decision is taken in the kernel's precision: the logits are rounded to
float32 before the arg-max / second-best, and confidences, credits and
scores are float32 values compared against float32 thresholds, with each
credit operation rounded to float32 as the state is stored in float32.

Pins (tests/test_oracle_*.py): closed forms (zero hidden state, two-token
vocabulary, hand-built logits with known softmax), brute-force loops on tiny
shapes, permutation and shift properties, exact ties, the planted-peak
limit, hand-worked commit sequences for all three strategies
(tests/golden/), and the block invariants (monotone mask, each position
committed once, at least one commit per step).
"""
from __future__ import annotations

from typing import Iterable, Sequence

import numpy as np

THRESHOLD, HIERARCHICAL, CREDIT = 0, 1, 2
SLOTS = 4          # tracked (token, credit) candidates per position
EMPTY = -1         # token id of an unused credit slot

_F32 = np.float32


# --------------------------------------------------------------------------------------------
# Inputs
# --------------------------------------------------------------------------------------------
def as_f64(x: np.ndarray) -> np.ndarray:
    """Exact float64 values of float32 data or of bfloat16 bit patterns (uint16)."""
    x = np.asarray(x)
    if x.dtype == np.float64:
        return x                      # already widened (lets callers widen a large W once)
    if x.dtype == np.uint16:
        # a bfloat16 value is the float32 whose upper half is the pattern
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if x.dtype == np.float32:
        return x.astype(np.float64)
    raise TypeError(f"unsupported input dtype {x.dtype}")


# --------------------------------------------------------------------------------------------
# LM head and per-position statistics
# --------------------------------------------------------------------------------------------
def lm_head_logits(hidden: np.ndarray, W: np.ndarray, vocab_chunk: int = 8192) -> np.ndarray:
    """``z[r, v] = sum_k h[r, k] * W[v, k]`` in float64 for every row ``r`` (R1: all rows).

    ``hidden`` is ``[M][H]``, ``W`` is ``[V][H]``; the matmul is a library
    step, done over vocabulary chunks only to bound memory.
    """
    h = as_f64(hidden)
    V = W.shape[0]
    z = np.empty((h.shape[0], V), dtype=np.float64)
    for v0 in range(0, V, vocab_chunk):
        z[:, v0:v0 + vocab_chunk] = h @ as_f64(W[v0:v0 + vocab_chunk]).T
    return z


def token_stats(hidden: np.ndarray, W: np.ndarray, row_chunk: int = 64) -> dict:
    """Candidate token, confidence and top-2 gap of every row.

    * ``tok``  = lowest token id among the maxima of the float32-rounded logits (R2);
    * ``gap``  = top logit minus the second-largest logit, counted with
      multiplicity (an exact tie gives 0; a one-token vocabulary gives +inf);
    * ``conf`` = ``1 / sum_v exp(z_v - max z)`` in float64, returned as float32:
      the largest softmax probability (R5).
    """
    hidden = np.asarray(hidden)
    H = W.shape[1]
    h2 = hidden.reshape(-1, H)
    M = h2.shape[0]
    conf = np.empty(M, dtype=np.float32)
    tok = np.empty(M, dtype=np.int64)
    gap = np.empty(M, dtype=np.float32)
    for r0 in range(0, M, row_chunk):
        z = lm_head_logits(h2[r0:r0 + row_chunk], W)
        rows = np.arange(z.shape[0])
        z32 = z.astype(np.float32)
        t = np.argmax(z32, axis=1)                     # first maximum = lowest id
        top = z32[rows, t]
        rest = z32.copy()
        rest[rows, t] = -np.inf
        second = rest.max(axis=1) if z.shape[1] > 1 else np.full(z.shape[0], -np.inf, np.float32)
        gap[r0:r0 + z.shape[0]] = (top.astype(np.float64) - second.astype(np.float64)).astype(np.float32)
        zmax = z.max(axis=1)
        S = np.exp(z - zmax[:, None]).sum(axis=1)
        conf[r0:r0 + z.shape[0]] = (1.0 / S).astype(np.float32)
        tok[r0:r0 + z.shape[0]] = t
    shape = hidden.shape[:-1]
    return {"conf": conf.reshape(shape), "tok": tok.reshape(shape), "gap": gap.reshape(shape)}


def shard_stats(hidden: np.ndarray, W_shard: np.ndarray, v_begin: int, row_chunk: int = 64) -> dict:
    """Softmax statistics of every row over one vocabulary shard (tokens ``v_begin ..
    v_begin + V_shard - 1``), the per-GPU half of the tensor-parallel head (explainer,
    system-level optimisations: the model is split over GPUs so a single request uses them all).

    * ``m``: the largest logit of the shard (float64), ``s = sum exp(z - m)`` over the shard;
    * ``tok``: the lowest global id among the shard's float32-rounded maxima (R2), ``top32`` that
      float32 maximum, ``second32`` the shard's second-largest float32 logit (with multiplicity).
    """
    hidden = np.asarray(hidden)
    H = W_shard.shape[1]
    h2 = hidden.reshape(-1, H)
    M = h2.shape[0]
    out = {"m": np.empty(M), "s": np.empty(M), "tok": np.empty(M, np.int64),
           "top32": np.empty(M, np.float32), "second32": np.empty(M, np.float32)}
    for r0 in range(0, M, row_chunk):
        z = lm_head_logits(h2[r0:r0 + row_chunk], W_shard)
        n = z.shape[0]
        rows = np.arange(n)
        z32 = z.astype(np.float32)
        t = np.argmax(z32, axis=1)
        rest = z32.copy()
        rest[rows, t] = -np.inf
        m = z.max(axis=1)
        out["m"][r0:r0 + n] = m
        out["s"][r0:r0 + n] = np.exp(z - m[:, None]).sum(axis=1)
        out["tok"][r0:r0 + n] = v_begin + t
        out["top32"][r0:r0 + n] = z32[rows, t]
        out["second32"][r0:r0 + n] = rest.max(axis=1) if z.shape[1] > 1 else -np.inf
    return out


def merge_shards(shards: Sequence[dict]) -> dict:
    """Statistics of the whole vocabulary from the shards' (in vocabulary order): the exchange
    step of the tensor-parallel head.  ``M = max m``, ``S = sum s_g exp(m_g - M)``, ``conf = 1/S``;
    the candidate is the lowest id among the shards whose float32 maximum is the largest; the
    runner-up logit is the larger of that shard's own runner-up and every other shard's maximum."""
    m = np.stack([d["m"] for d in shards])
    s = np.stack([d["s"] for d in shards])
    top = np.stack([d["top32"] for d in shards])
    sec = np.stack([d["second32"] for d in shards])
    tok = np.stack([d["tok"] for d in shards])
    G, M = m.shape
    Mx = m.max(axis=0)
    S = (s * np.exp(m - Mx[None, :])).sum(axis=0)
    conf = (1.0 / S).astype(np.float32)
    T = top.max(axis=0)
    out_tok = np.empty(M, np.int64)
    gap = np.empty(M, np.float32)
    for r in range(M):
        winners = [g for g in range(G) if top[g, r] == T[r]]
        w = min(winners, key=lambda g: tok[g, r])
        out_tok[r] = tok[w, r]
        second = max([float(sec[w, r])] + [float(top[g, r]) for g in range(G) if g != w])
        gap[r] = np.float32(float(T[r]) - second)
    return {"conf": conf, "tok": out_tok, "gap": gap}


def topk_candidates(hidden: np.ndarray, W: np.ndarray, k: int, row_chunk: int = 64) -> dict:
    """The ``k`` best candidates of every row and their softmax probabilities.

    The explainer's iteration-manager paragraph says the information of the candidates a step
    does not choose is carried into the next iteration, without saying in what form.  This is
    the data such a scheme starts from (readings T1-T4):

    * ``tok[r, i]``: the token with the i-th largest float32-rounded logit, ties to the lower
      id (the arg-max rule R2 extended), so ``tok[:, 0]`` is the candidate of
      :func:`token_stats`;
    * ``prob[r, i]`` = ``exp(z_tok - max z) / sum_v exp(z_v - max z)`` in float64, returned
      as float32: its softmax probability, so ``prob[:, 0]`` is the confidence;
    * when ``k > V`` the entries past ``V`` are token -1 with probability 0;
    * every row is ranked, masked or not (like the candidate of R17).
    """
    if k < 1:
        raise ValueError("k must be >= 1")
    hidden = np.asarray(hidden)
    H = W.shape[1]
    V = W.shape[0]
    h2 = hidden.reshape(-1, H)
    M = h2.shape[0]
    tok = np.full((M, k), -1, dtype=np.int64)
    prob = np.zeros((M, k), dtype=np.float32)
    kk = min(k, V)
    for r0 in range(0, M, row_chunk):
        z = lm_head_logits(h2[r0:r0 + row_chunk], W)
        z32 = z.astype(np.float32)
        # a stable sort of the negated logits keeps equal logits in ascending id order
        order = np.argsort(-z32, axis=1, kind="stable")[:, :kk]
        zmax = z.max(axis=1, keepdims=True)
        e = np.exp(z - zmax)
        S = e.sum(axis=1, keepdims=True)
        rows = np.arange(z.shape[0])[:, None]
        tok[r0:r0 + z.shape[0], :kk] = order
        prob[r0:r0 + z.shape[0], :kk] = (e[rows, order] / S).astype(np.float32)
    shape = hidden.shape[:-1] + (k,)
    return {"tok": tok.reshape(shape), "prob": prob.reshape(shape)}


# --------------------------------------------------------------------------------------------
# Commit strategies (one sequence: arrays of length L)
# --------------------------------------------------------------------------------------------
def _best(values: Sequence[float], positions: Sequence[int]) -> int:
    """Position of the largest value; the lowest position wins a tie."""
    best_p, best_v = None, None
    for p, v in sorted(zip(positions, values)):
        if best_v is None or _F32(v) > best_v:
            best_p, best_v = p, _F32(v)
    return best_p


def _masked(mask: np.ndarray) -> list:
    return [l for l in range(len(mask)) if mask[l]]


def commit_threshold(conf: np.ndarray, mask: np.ndarray, tau: float) -> np.ndarray:
    """Threshold decoding (explainer, decoding-strategy component, first strategy).

    Every masked position with ``conf >= tau`` (R3) is fixed; when none is,
    the single most confident masked position is (lowest position on ties,
    R4).  No masked position: nothing is fixed (R7).
    """
    L = len(conf)
    U = _masked(mask)
    C = [l for l in U if _F32(conf[l]) >= _F32(tau)]
    if not C and U:
        C = [_best([conf[l] for l in U], U)]
    out = np.zeros(L, dtype=bool)
    out[C] = True
    return out


def _runs(mask: np.ndarray) -> list:
    """Maximal runs ``(s, e)`` (inclusive) of masked positions, left to right."""
    runs, l, L = [], 0, len(mask)
    while l < L:
        if mask[l]:
            s = l
            while l + 1 < L and mask[l + 1]:
                l += 1
            runs.append((s, l))
        l += 1
    return runs


def commit_hierarchical(conf: np.ndarray, mask: np.ndarray, tau: float, max_depth: int = 0) -> np.ndarray:
    """Hierarchical decoding (explainer, decoding-strategy component, second strategy).

    The regions still to fill are the maximal masked runs.  A worklist
    takes a run ``(s, e)``, looks at its centre ``c = (s + e) // 2`` (R8) and,
    if ``conf[c] >= tau``, fixes ``c`` and puts the two halves ``(s, c-1)``
    and ``(c+1, e)`` back on the list; a run whose centre is not confident
    is left for a later iteration (R14).  ``max_depth > 0`` stops splitting
    below that depth (the runs themselves are depth 1).  If nothing was
    fixed, the most confident centre of a top-level run is (R15).
    """
    L = len(conf)
    out = np.zeros(L, dtype=bool)
    runs = _runs(mask)
    work = [(s, e, 1) for (s, e) in runs]
    while work:
        s, e, depth = work.pop()
        c = (s + e) // 2
        if _F32(conf[c]) >= _F32(tau):
            out[c] = True
            if max_depth == 0 or depth < max_depth:
                if s <= c - 1:
                    work.append((s, c - 1, depth + 1))
                if c + 1 <= e:
                    work.append((c + 1, e, depth + 1))
    if not out.any() and runs:
        centres = [(s + e) // 2 for (s, e) in runs]
        out[_best([conf[c] for c in centres], centres)] = True
    return out


def commit_credit(conf: np.ndarray, tok: np.ndarray, mask: np.ndarray,
                  slot_tok: np.ndarray, slot_cr: np.ndarray, decay: float, theta: float):
    """Credit decoding (explainer, decoding-strategy component, third strategy).

    For every masked position ``l`` (R16), with ``SLOTS`` tracked candidates:

    1. every slot's credit is multiplied by ``decay`` (R10);
    2. if the current candidate ``tok[l]`` holds a slot, ``conf[l]`` is added
       to that slot; otherwise it takes the first empty slot, else the slot
       with the smallest credit (lowest slot on ties), with credit
       ``0 + conf[l]`` (R11);
    3. ``score = conf * (1 + credit of tok[l])`` with the updated credit (R9).

    Masked positions with ``score >= theta`` are fixed with token ``tok[l]``
    (R13); if none is, the highest score is (lowest position on ties, R12).
    Returns ``(commit, slot_tok, slot_cr, score)``; the slot arrays are new.
    """
    L = len(conf)
    st = np.array(slot_tok, dtype=np.int32, copy=True)
    sc = np.array(slot_cr, dtype=np.float32, copy=True)
    score = np.full(L, -np.inf, dtype=np.float32)
    d = _F32(decay)
    U = _masked(mask)
    for l in U:
        c = _F32(conf[l])
        for i in range(SLOTS):
            sc[l, i] = _F32(sc[l, i] * d)
        held = [i for i in range(SLOTS) if st[l, i] == tok[l]]
        if held:
            i = held[0]
            sc[l, i] = _F32(sc[l, i] + c)
        else:
            empty = [i for i in range(SLOTS) if st[l, i] == EMPTY]
            if empty:
                i = empty[0]
            else:
                i = min(range(SLOTS), key=lambda j: (sc[l, j], j))
            st[l, i] = tok[l]
            sc[l, i] = _F32(_F32(0.0) + c)
        score[l] = _F32(c * _F32(_F32(1.0) + sc[l, i]))
    C = [l for l in U if score[l] >= _F32(theta)]
    if not C and U:
        C = [_best([score[l] for l in U], U)]
    out = np.zeros(L, dtype=bool)
    out[C] = True
    return out, st, sc, score


# --------------------------------------------------------------------------------------------
# The whole step
# --------------------------------------------------------------------------------------------
def _policy_fields(p) -> tuple:
    """(kind, threshold, decay, max_depth, eos_token); eos_token -1 = no end token."""
    if isinstance(p, dict):
        return (int(p["kind"]), float(p["threshold"]), float(p.get("decay", 0.0)), int(p.get("max_depth", 0)),
                int(p.get("eos_token", -1)))
    if hasattr(p, "kind"):
        return (int(p.kind), float(p.threshold), float(getattr(p, "decay", 0.0)), int(getattr(p, "max_depth", 0)),
                int(getattr(p, "eos_token", -1)))
    kind, thr, dec, depth = p[:4]
    return int(kind), float(thr), float(dec), int(depth), int(p[4]) if len(p) > 4 else -1


# Early stop (the explainer's engineering paragraph: once an end token appears in the generated
# text, the computation that would follow it is skipped).  Per sequence, an optional state:
RUNNING, FINISHED, EOS_IN_BLOCK = 0, 1, 2


def early_stop(commit: np.ndarray, tok: np.ndarray, mask_after: np.ndarray, eos: int, state: int):
    """Apply one step's end-token rule to one sequence (readings E2, E3).

    ``commit`` is the policy's commit set, ``mask_after`` the mask with those commits removed.
    When the step commits the end token, the text ends at the first such position e: every
    position after e that is still masked is committed too, and every position after e that
    this step commits (by the policy or as padding) carries the end token.  The state becomes
    EOS_IN_BLOCK, and FINISHED once the block has no masked position left.
    Returns (commit, tokens, mask_after, state) as new arrays.
    """
    commit, tok, mask_after = commit.copy(), tok.copy(), mask_after.copy()
    ends = [l for l in range(len(commit)) if commit[l] and tok[l] == eos]
    if ends:
        e = ends[0]
        for p in range(e + 1, len(commit)):
            if mask_after[p] or commit[p]:
                commit[p] = True
                tok[p] = eos
                mask_after[p] = False
        state = EOS_IN_BLOCK
    if state == EOS_IN_BLOCK and not mask_after.any():
        state = FINISHED
    return commit, tok, mask_after, state


def decode_step(hidden: np.ndarray, W: np.ndarray, mask: np.ndarray, policies: Iterable,
                credit_tok: np.ndarray | None = None, credit_val: np.ndarray | None = None,
                auto_advance: bool = False, stats: dict | None = None,
                seq_done: np.ndarray | None = None) -> dict:
    """One decode step over ``B`` sequences of ``L`` positions.

    ``hidden`` ``[B][L][H]``, ``W`` ``[V][H]`` (uint16 bf16 bits or float32),
    ``mask`` ``[B][L]`` (non-zero = still masked), one policy per sequence
    (``(kind, threshold, decay, max_depth)``, a dict or an object with those
    fields), credit state ``[B][L][SLOTS]`` (token, credit) when any policy is
    credit decoding.  With ``auto_advance`` a sequence whose mask is empty on
    entry starts a new block first (mask refilled, credit cleared), as the
    iteration manager moves to the next fixed-size block.  ``stats`` may pass
    precomputed :func:`token_stats` output.

    ``seq_done`` (``[B]``, RUNNING / FINISHED / EOS_IN_BLOCK) turns on early stop for the
    sequences whose policy names an end token (readings E1-E4): a FINISHED sequence commits
    nothing and keeps its state (no block advance either); otherwise :func:`early_stop` runs
    after the policy; a new block resets EOS_IN_BLOCK to RUNNING.

    Returns new arrays: ``tokens`` (candidate of every row, R17, or the end token where a
    position was padded after it), ``commit``, ``mask``, ``credit_tok``, ``credit_val``,
    ``conf``, ``gap``, ``score``, and ``seq_done`` when given.
    """
    hidden = np.asarray(hidden)
    B, L = hidden.shape[0], hidden.shape[1]
    policies = [_policy_fields(p) for p in policies]
    assert len(policies) == B
    st = token_stats(hidden, W) if stats is None else stats
    conf, tok, gap = st["conf"].reshape(B, L), st["tok"].reshape(B, L), st["gap"].reshape(B, L)
    new_mask = (np.asarray(mask).reshape(B, L) != 0).copy()
    if credit_tok is None:
        ctok = np.full((B, L, SLOTS), EMPTY, dtype=np.int32)
        cval = np.zeros((B, L, SLOTS), dtype=np.float32)
    else:
        ctok = np.array(credit_tok, dtype=np.int32, copy=True).reshape(B, L, SLOTS)
        cval = np.array(credit_val, dtype=np.float32, copy=True).reshape(B, L, SLOTS)
    commit = np.zeros((B, L), dtype=bool)
    score = np.full((B, L), -np.inf, dtype=np.float32)
    tok = tok.astype(np.int32).copy()
    done = None if seq_done is None else np.array(seq_done, dtype=np.uint8, copy=True).reshape(B)
    for b, (kind, thr, dec, depth, eos) in enumerate(policies):
        stopping = done is not None and eos >= 0
        if stopping and done[b] == FINISHED:
            continue                                  # E1: nothing more for this sequence
        if auto_advance and not new_mask[b].any():
            new_mask[b] = True
            ctok[b] = EMPTY
            cval[b] = 0.0
            if stopping:
                done[b] = RUNNING
        if kind == THRESHOLD:
            commit[b] = commit_threshold(conf[b], new_mask[b], thr)
        elif kind == HIERARCHICAL:
            commit[b] = commit_hierarchical(conf[b], new_mask[b], thr, depth)
        elif kind == CREDIT:
            commit[b], ctok[b], cval[b], score[b] = commit_credit(
                conf[b], tok[b], new_mask[b], ctok[b], cval[b], dec, thr)
        else:
            raise ValueError(f"unknown policy kind {kind}")
        new_mask[b] &= ~commit[b]
        if stopping:
            commit[b], tok[b], new_mask[b], done[b] = early_stop(commit[b], tok[b], new_mask[b], eos, int(done[b]))
    out = {
        "tokens": tok.astype(np.int32),
        "commit": commit.astype(np.uint8),
        "mask": new_mask.astype(np.uint8),
        "credit_tok": ctok,
        "credit_val": cval,
        "conf": conf.astype(np.float32),
        "gap": gap.astype(np.float32),
        "score": score,
    }
    if done is not None:
        out["seq_done"] = done
    return out
