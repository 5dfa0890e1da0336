"""The output side of a streamed step: embedding lookup, token cross-entropy on the
untied head's logits, and the sigmoid preference (DPO) loss over sequence log-prob sums.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Where these come from.  The vocab-sized embed_tokens and the untied lm_head share one
device slot in the layer stream, and the output head and its loss can run a chunk of
tokens at a time (the Soup deep dive, "Core feature: how layer streaming works" and the
``stream_loss_chunk`` key in "Streaming config keys").  The preference step compares
the adapted model with the same base run with the adapters switched off (the Soup 4 GB
article, "Memory-free reference model"; the 20B-RLHF article, step 3).  The pages give
no formula for the preference loss; the reading taken is the standard sigmoid form
with a temperature beta over sequence log-probability sums.

Definitions (fp64 throughout; logits arrive as the bf16 values the GPU holds):

  embedding       out[t] = table[ids[t]]
  log-softmax     lse_t = log sum_j exp(l[t, j]),  logp_t = l[t, label_t] - lse_t
  token loss      loss_t = -logp_t
  its gradient    dlogits[t, j] = g_t * (softmax_j(l[t]) - [j == label_t])
                  (g_t = d(objective)/d(loss_t): 1/T for a mean over T tokens)
  sequence sums   S_i = sum of logp_t over the tokens of sequence i
  DPO             m_p = beta * ((S_pol[chosen_p] - S_ref[chosen_p])
                                - (S_pol[rejected_p] - S_ref[rejected_p]))
                  L = mean_p -log sigmoid(m_p)
                  dL/dS_pol[chosen_p] = -beta * sigmoid(-m_p) / P,
                  dL/dS_pol[rejected_p] = +beta * sigmoid(-m_p) / P
"""
from __future__ import annotations

import numpy as np


def embed_gather(table_bits, ids):
    """Rows of the embedding table (bf16 bit patterns, [V, H]) for token ids [T]."""
    table_bits = np.asarray(table_bits)
    ids = np.asarray(ids, dtype=np.int64)
    if ids.size and (ids.min() < 0 or ids.max() >= table_bits.shape[0]):
        raise ValueError("token id out of range")
    return table_bits[ids]


def log_softmax_rows(logits):
    """Row-wise log-softmax in fp64, shifted by the row maximum."""
    l = np.asarray(logits, dtype=np.float64)
    m = l.max(axis=1, keepdims=True)
    lse = m + np.log(np.exp(l - m).sum(axis=1, keepdims=True))
    return l - lse, lse[:, 0]


def cross_entropy(logits, labels, grad_scale=None):
    """Token cross-entropy.  Returns (logp [T], loss [T], dlogits [T, V]) where
    dlogits[t] = grad_scale[t] * (softmax(l[t]) - onehot(label_t)); grad_scale defaults
    to 1/T (mean over the tokens)."""
    l = np.asarray(logits, dtype=np.float64)
    labels = np.asarray(labels, dtype=np.int64)
    T, V = l.shape
    if labels.shape != (T,) or (T and (labels.min() < 0 or labels.max() >= V)):
        raise ValueError("labels must be [T] ids in [0, V)")
    lp, _ = log_softmax_rows(l) if T else (np.zeros((0, V)), None)
    rows = np.arange(T)
    logp = lp[rows, labels] if T else np.zeros(0)
    g = np.full(T, 1.0 / max(T, 1)) if grad_scale is None else np.asarray(grad_scale, dtype=np.float64)
    d = np.exp(lp) if T else np.zeros((0, V))
    d[rows, labels] -= 1.0
    d *= g[:, None]
    return logp, -logp, d


def sequence_sums(values, seq_len: int):
    """Sums of consecutive runs of seq_len values (one per sequence)."""
    v = np.asarray(values, dtype=np.float64)
    if seq_len <= 0 or v.size % seq_len:
        raise ValueError("length must be a multiple of seq_len")
    return v.reshape(-1, seq_len).sum(axis=1)


def dpo_loss(pol_sums, ref_sums, beta: float):
    """Sigmoid DPO over P pairs; sums are ordered (chosen_0, rejected_0, chosen_1, ...).
    Returns (loss, dL/dpol_sums [2P])."""
    ps = np.asarray(pol_sums, dtype=np.float64).reshape(-1, 2)
    rs = np.asarray(ref_sums, dtype=np.float64).reshape(-1, 2)
    P = ps.shape[0]
    m = beta * ((ps[:, 0] - rs[:, 0]) - (ps[:, 1] - rs[:, 1]))
    # -log sigmoid(m) = log(1 + exp(-m)), written to stay finite for large |m|
    loss = np.mean(np.logaddexp(0.0, -m))
    sig_neg = 0.5 * (1.0 - np.tanh(0.5 * m))      # sigmoid(-m)
    g = np.empty((P, 2))
    g[:, 0] = -beta * sig_neg / P
    g[:, 1] = beta * sig_neg / P
    return loss, g.reshape(-1)


def dpo_token_scale(coef, seq_len: int):
    """Per-token gradient scale of the policy pass: d L / d loss_t = -dL/dS_i for the
    tokens of sequence i (loss_t = -logp_t)."""
    c = np.asarray(coef, dtype=np.float64)
    return np.repeat(-c, seq_len)
