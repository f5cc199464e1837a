"""Oracle: batch-B decode with union channel masks (test infrastructure only).

"Where Activation Sparsity and KV-Cache Sparsity Cross in LLM Decoding", §3.3
"Dispatch and batching" and §4.4 "Batching": a batch of B sequences shares
every weight read, while each sequence reads its own cache.  A sparse
projection then has to read every channel that at least one sequence of the
batch keeps: the union of the B masks, a fraction u_B of the channels.

What the batch computes is fixed by that description: sequence b's new
hidden state is exactly the single-sequence decode step of sequence b (its
own caches, position and mask, the shared weights).  The union only decides
which weight rows are read; a channel that sequence b dropped contributes
nothing to sequence b even when another sequence keeps it.  So the oracle is
the single-sequence step applied per sequence, plus the union of the masks.

Readings:
* one threshold per layer, shared by the batch (the per-layer CATS threshold);
  each sequence decides its own mask from its own float32 |a| (as in
  cats.cats_mask);
* u_B is the kept fraction of the union mask, per layer; for masks whose
  channels are kept independently with probability r, E[u_B] = 1 - (1 - r)^B
  (the pages measure 92% at B = 4 and 98.5% at B = 8 on real text, where
  channels are correlated across sequences).

Pins (tests/test_oracle_batch.py): B = 1 is the single-sequence step bit for
bit and its union is its mask; a sequence's result does not depend on the
other sequences; the union of identical masks is that mask, of disjoint masks
their sum; the Monte-Carlo union fraction of independent masks matches
1 - (1 - r)^B within its sampling error.
"""

from __future__ import annotations

import numpy as np

from . import step


def union_mask(masks) -> np.ndarray:
    """Channels kept by at least one sequence: OR over the first axis."""
    m = np.asarray(masks, dtype=bool)
    return np.any(m, axis=0)


def union_fraction(masks) -> float:
    return float(union_mask(masks).mean())


def independent_union_fraction(keep: float, batch: int) -> float:
    """E[u_B] when every channel of every sequence is kept independently
    with probability `keep`: one minus the chance that all B drop it."""
    return 1.0 - (1.0 - keep) ** batch


def decode_step_batch(seq_layers, hs, positions, *, kv_sparse, mlp_sparse, trace=None, **dims):
    """B sequences, one decode step each.

    seq_layers[b] is sequence b's list of step.Layer (weights shared across
    the batch, caches its own); hs[b] its hidden state; positions[b] its
    position.  Returns (new hidden states [B, d], per-layer union masks or
    None when the MLP is dense)."""
    outs, masks = [], []
    for b, (layers, h, pos) in enumerate(zip(seq_layers, hs, positions)):
        tr = []
        outs.append(step.decode_step(layers, h, pos, kv_sparse=kv_sparse, mlp_sparse=mlp_sparse,
                                     trace=tr, **dims))
        masks.append([t["mask"] for t in tr])
        if trace is not None:
            trace.append(tr)
    n_layers = len(masks[0])
    unions = [union_mask([masks[b][li] for b in range(len(masks))]) for li in range(n_layers)]
    return np.stack(outs), unions
