"""Dispatch ("grouped experts") for the CPU oracle.

TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
benchmark's CPU baseline; never by the product path.

The HunyuanImage-3.0 model-coverage page ("Model Class") converts the fused
expert projections to grouped experts: the routed (token, k) pairs are grouped
by expert so that each expert's rows form one contiguous block. The grouping
is defined here by library routines:

* counts[e]   = number of real (token, k) pairs routed to expert e (bincount);
* offsets     = exclusive prefix sum of counts, with offsets[E] = total pairs;
* slot order  = a stable sort of the flattened pairs by expert id, so inside
  one expert the pairs keep ascending (token, k) order;
* perm_token[s] = token of the pair in slot s; slot_of[t, k] = slot of (t, k),
  -1 for padding rows;
* valid_tok   = ascending list of real (non-padding) tokens, the rows the
  shared expert runs on.
"""
import numpy as np


def dispatch(topk_idx: np.ndarray, E: int):
    idx = np.asarray(topk_idx, np.int64)
    T, K = idx.shape
    flat = idx.reshape(-1)
    pairs = np.nonzero(flat >= 0)[0]
    ids = flat[pairs]
    if ids.size and (ids.min() < 0 or ids.max() >= E):
        raise ValueError("expert id out of range")
    counts = np.bincount(ids, minlength=E).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    order = np.argsort(ids, kind="stable")
    sorted_pairs = pairs[order]
    perm_token = (sorted_pairs // K).astype(np.int64)
    slot_of = np.full(T * K, -1, np.int64)
    slot_of[sorted_pairs] = np.arange(sorted_pairs.size)
    return {
        "counts": counts,
        "offsets": offsets,
        "perm_token": perm_token,
        "slot_of": slot_of.reshape(T, K),
    }


def valid_tokens(pad_mask: np.ndarray) -> np.ndarray:
    return np.nonzero(np.asarray(pad_mask) == 0)[0].astype(np.int64)
