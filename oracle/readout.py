"""Selective readout, Eq. (1), float64.

For question i with last-token hidden row ``h_i`` and option set ``O_i``:
``p_i(o) = exp(w_o^T h_i) / sum_{o' in O_i} exp(w_o'^T h_i)``
(Korean summary, §어떻게 동작하나; Flide: Accelerating Decision Inference with
Exact State Forking, §前置知识 and §方法步骤详情 — only question-final rows are
read out).  No bias and no temperature (the pages give none).

Pinned by tests/test_oracle_readout.py (one option, equal logits, a
hand-computed two-option case, and normalisation).
"""
from __future__ import annotations

import numpy as np


def option_probs(h: np.ndarray, w_rows: np.ndarray) -> np.ndarray:
    """Softmax over ``w_rows @ h``; h: [hidden], w_rows: [n_opt, hidden]."""
    z = np.asarray(w_rows, np.float64) @ np.asarray(h, np.float64)
    z = z - z.max()
    e = np.exp(z)
    return e / e.sum()
