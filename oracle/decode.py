"""Plain float64 definitions of the decode-side reductions that follow the
attention of a denoising step.

TEST INFRASTRUCTURE ONLY (see the package docstring): used by tests, the
smoke check and the CPU baseline of bench.py, never by the product path.

Citation keys (as in flashcache.py):
  [FD]  Flash-dLLM paper summary page, 方法步骤详情 step 2 (confidence of each
        masked window position, decoded at or above epsilon = 0.9, the rest form
        the search set) and step 3 (the verify forward: accepted in causal
        left-to-right order while the draft-view and mask-view predictions agree
        and the mask-view confidence is at least gamma = 0.8; the first failure
        stops acceptance); 前置知识 (the confidence is the maximum of the model's
        predicted distribution at the position).
  [FST] Fast-dLLM article (senqingzn.com), 并行解碼新策略 (confidence-aware
        parallel decoding):
        when no position reaches the threshold, the most confident one is
        decoded anyway, so every step makes progress.

Readings of points the pages leave open:
  * the distribution is the softmax of the position's full logits row (no
    temperature, no top-p): confidence = max softmax probability, and the
    decoded token is its argmax;
  * argmax ties go to the lowest token id; the forced decode takes the most
    confident row, ties to the lowest row;
  * "left to right" is increasing position within the sequence (one explainer
    page speaks of confidence order; the paper summary's causal order is
    followed because the verify mask is causal in position);
  * decisions are per sequence: rows cu[b] .. cu[b+1]-1 belong to sequence b.
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np


def confidence_argmax(logits: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per row: the argmax token (lowest id on ties) and the maximum softmax
    probability, 1 / sum_x exp(l_x - max l) ([FD] 方法步骤详情 step 2)."""
    z = np.asarray(logits, dtype=np.float64)
    idx = np.argmax(z, axis=1)                 # first occurrence: the lowest id
    m = z.max(axis=1, keepdims=True)
    conf = 1.0 / np.exp(z - m).sum(axis=1)
    return idx.astype(np.int64), conf


def confidence_commit(conf: np.ndarray, cu: Sequence[int], eps: float) -> Tuple[np.ndarray, np.ndarray]:
    """Rows decoded this step: confidence >= eps; a sequence with rows but none
    above the threshold decodes its most confident row ([FST] 并行解碼新策略).
    Returns (commit bool [R], count per sequence)."""
    conf = np.asarray(conf, dtype=np.float64)
    commit = conf >= eps
    n = np.zeros(len(cu) - 1, dtype=np.int64)
    for b in range(len(cu) - 1):
        r0, r1 = int(cu[b]), int(cu[b + 1])
        if r1 > r0 and not commit[r0:r1].any():
            commit[r0 + int(np.argmax(conf[r0:r1]))] = True
        n[b] = int(commit[r0:r1].sum())
    return commit, n


def verify_accept(draft: Sequence[int], pred: Sequence[int], conf: Sequence[float], cu: Sequence[int],
                  gamma: float) -> Tuple[np.ndarray, np.ndarray]:
    """Flash-Verify acceptance ([FD] 方法步骤详情 step 3): within each sequence,
    the search rows in position order are accepted while the draft equals the
    mask view's prediction and the mask view's confidence is >= gamma; the
    first row that fails ends the sequence's acceptance.  Returns (accept bool
    [R], accepted count per sequence)."""
    R = len(draft)
    accept = np.zeros(R, dtype=bool)
    n = np.zeros(len(cu) - 1, dtype=np.int64)
    for b in range(len(cu) - 1):
        for r in range(int(cu[b]), int(cu[b + 1])):
            if int(draft[r]) == int(pred[r]) and float(conf[r]) >= gamma:
                accept[r] = True
                n[b] += 1
            else:
                break
    return accept, n
