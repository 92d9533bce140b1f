"""Oracle for the expert-routing steps around the grouped MLP.  TEST INFRASTRUCTURE ONLY.

The pages ask for MoE kernels whose buffers are allocated up front, with no
dynamic shapes and no host read of the top-k expert ids (nvfp4-megamoe-kernel
performance audit, P8 item 5 and its note on `topk_ids.max().item()`), and for
grouped MUL_MAT_ID-style contractions (llama.cpp discussion, "Verified").  The
pages do not spell out the router; the plainest reading is used here:

* each token takes the k experts with the largest router logits, ties going
  to the lower expert id (softmax is strictly increasing, so these are the k
  largest router probabilities);
* the token's combine weights are the softmax restricted to its k experts,
  p_j = exp(l_j - m) / sum_i exp(l_i - m) over the chosen experts, m the
  largest chosen logit (float64);
* the (token, choice) pairs become slots sorted by (expert, token):
  group_offsets[e] is the number of slots whose expert is below e, a_rows[s]
  the token of slot s, slot_of[t, j] the slot of token t's j-th choice;
* the combine of per-slot outputs Y is y[t] = sum_j p_j * Y[slot_of[t, j]]
  (float64, choices in order).
"""
from dataclasses import dataclass

import numpy as np


@dataclass
class Routing:
    topk: np.ndarray            # int32 [T, k]: expert ids by decreasing logit (ties: lower id first)
    weights: np.ndarray         # float64 [T, k]: softmax over the chosen experts
    a_rows: np.ndarray          # int32 [T*k]: token of each slot
    group_offsets: np.ndarray   # int32 [E+1]
    slot_of: np.ndarray         # int32 [T, k]


def route(logits, k):
    """Top-k routing of logits [T, E] (float32) as defined in the module docstring."""
    logits = np.asarray(logits, dtype=np.float32)
    t, e = logits.shape
    if not 1 <= k <= e:
        raise ValueError("need 1 <= k <= E")
    if not np.all(np.isfinite(logits)):
        raise ValueError("logits must be finite")
    # rank experts by (-logit, id): lexsort takes its last key as the primary one
    ids = np.broadcast_to(np.arange(e), (t, e))
    order = np.lexsort((ids, -logits), axis=1)
    topk = order[:, :k].astype(np.int32)
    chosen = np.take_along_axis(logits, topk, axis=1).astype(np.float64)
    z = np.exp(chosen - chosen[:, :1])
    weights = z / z.sum(axis=1, keepdims=True)
    experts = topk.reshape(-1).astype(np.int64)
    tokens = np.repeat(np.arange(t, dtype=np.int64), k)
    slot_order = np.lexsort((tokens, experts))            # slot s holds pair slot_order[s]
    a_rows = tokens[slot_order].astype(np.int32)
    slot_of = np.empty(t * k, dtype=np.int32)
    slot_of[slot_order] = np.arange(t * k, dtype=np.int32)
    offsets = np.zeros(e + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(np.bincount(experts, minlength=e))
    return Routing(topk, weights, a_rows, offsets, slot_of.reshape(t, k))


def combine(y_slots, slot_of, weights):
    """y[t] = sum_j weights[t, j] * y_slots[slot_of[t, j]] in float64."""
    y_slots = np.asarray(y_slots, dtype=np.float64)
    slot_of = np.asarray(slot_of)
    weights = np.asarray(weights, dtype=np.float64)
    out = np.zeros((slot_of.shape[0], y_slots.shape[1]), dtype=np.float64)
    for j in range(slot_of.shape[1]):
        out += weights[:, j:j + 1] * y_slots[slot_of[:, j]]
    return out
