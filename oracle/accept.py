"""LM-head argmax and greedy acceptance of a draft block (oracle; test
infrastructure only).

The pages: a drafter proposes a block of tokens and the target checks all of
them in one parallel forward pass ([de] §1; [fr] §1; [zh] abstract); the
acceptance criterion reads the logits after dequantization, which are kept
in high precision ([de] §2 "De-Quantisierung"; [it] §2 "Campionamento di
rifiuto"; [ja] §2.2 item 4); correct guesses are all validated at once and
on a wrong one the rest is rejected and decoding restarts ([fr] lay
summary, "Le Double Chef"); results are reported for greedy decoding, T=0
([ja] §4 main results).

Readings (pages silent or ambiguous):
* the logits read by acceptance are the fp32 dequantized values ``y32``;
* argmax breaks ties toward the lowest index (IEEE compare, so -0 == +0);
  inputs must be finite;
* rows are laid out ``[B*(G+1)][V]``: row ``b*(G+1)+i`` is the target's
  prediction after position i of sequence b (i = 0..G);
* accept_len[b] = the number of leading drafts that equal the target's
  argmax at their position; next_token[b] = the target's argmax at the first
  mismatch, or at position G when every draft matched.  The tokens emitted
  by one verify step are accept_len + 1.
"""
import numpy as np


def argmax_rows(y32) -> np.ndarray:
    """For each row, the lowest index whose value equals the row maximum."""
    y = np.asarray(y32, dtype=np.float32)
    if y.ndim != 2 or y.shape[1] == 0:
        raise ValueError("argmax_rows expects [R][V] with V > 0")
    if not np.all(np.isfinite(y)):
        raise ValueError("argmax_rows: logits must be finite")
    top = np.max(y, axis=1)
    hit = y == top[:, None]
    return np.argmax(hit, axis=1).astype(np.int32)  # first True per row


def greedy_accept(draft, target_argmax) -> tuple:
    """Greedy acceptance.

    ``draft`` is ``int32[B][G]``; ``target_argmax`` is ``int32[B*(G+1)]``.
    Returns ``(accept_len int32[B], next_token int32[B])``."""
    d = np.asarray(draft, dtype=np.int64)
    if d.ndim != 2:
        raise ValueError("draft must be [B][G]")
    B, G = d.shape
    a = np.asarray(target_argmax, dtype=np.int64).reshape(B, G + 1)
    accept_len = np.zeros(B, dtype=np.int32)
    next_token = np.zeros(B, dtype=np.int32)
    for b in range(B):
        n = 0
        while n < G and d[b, n] == a[b, n]:
            n += 1
        accept_len[b] = n
        next_token[b] = a[b, n]
    return accept_len, next_token


def verify_accept(logits, draft) -> tuple:
    """argmax of every row of ``logits[B*(G+1)][V]`` then greedy acceptance.
    Returns ``(argmax int32[B*(G+1)], accept_len int32[B], next_token int32[B])``."""
    am = argmax_rows(logits)
    al, nt = greedy_accept(draft, am)
    return am, al, nt
