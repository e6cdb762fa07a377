"""Second formulations of the MoE layer, used only to pin the C oracle.

TEST INFRASTRUCTURE ONLY. Everything here is float64 numpy / scipy / torch-CPU
library calls, written the way the pages state the method rather than the way
the C oracle evaluates it:

* ``masked_softmax_gate``: the sparse-gating equation on the notion page, G(x) =
  Softmax(TopK(x . W_g)) with every non-top-K logit set to -inf, as a dense
  [T, E] matrix (top-K chosen with a stable argsort, lower index first on ties).
* ``softmax_topk_renorm_gate``: the ml-canon page's PyTorch snippet: softmax over
  all experts, keep the top 2, divide by their sum.
* ``dense_moe``: the notion page's output equation summed over ALL n experts,
  y = sum_i G(x)_i E_i(x), every expert evaluated densely (brute force).
* ``dense_swiglu``: one SwiGLU FFN, W2 (silu(W1 x) * (W3 x)), with
  silu(z) = z * expit(z), as matrix products.
"""
from __future__ import annotations

import numpy as np
from scipy.special import expit, softmax


def topk_sets(logits: np.ndarray, K: int) -> np.ndarray:
    """[T, K] expert ids: stable sort of -logits (lower index first on ties)."""
    return np.argsort(-logits, axis=1, kind="stable")[:, :K]


def masked_softmax_gate(logits: np.ndarray, K: int) -> np.ndarray:
    keep = topk_sets(logits, K)
    masked = np.full_like(logits, -np.inf)
    rows = np.arange(logits.shape[0])[:, None]
    masked[rows, keep] = logits[rows, keep]
    return softmax(masked, axis=1)


def softmax_topk_renorm_gate(logits: np.ndarray, K: int):
    """(idx, w) by softmax -> topk -> renormalise, in torch float64 on the CPU."""
    import torch

    l = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float64))
    w, idx = l.softmax(-1).topk(K, -1)
    w = w / w.sum(-1, keepdim=True)
    return idx.numpy(), w.numpy()


def dense_swiglu(x: np.ndarray, w1: np.ndarray, w3: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """x [n, d] -> [n, d] through one expert; all float64."""
    g = x @ w1.T
    u = x @ w3.T
    return (g * expit(g) * u) @ w2.T


def dense_moe(x: np.ndarray, w_g: np.ndarray, w1: np.ndarray, w3: np.ndarray,
              w2: np.ndarray, K: int) -> np.ndarray:
    """Brute force over all experts with the dense masked gate; float64 inputs."""
    G = masked_softmax_gate(x @ w_g, K)
    y = np.zeros_like(x)
    for i in range(w1.shape[0]):
        y += G[:, i:i + 1] * dense_swiglu(x, w1[i], w3[i], w2[i])
    return y
