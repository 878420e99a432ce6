"""Dense causal GQA softmax attention in fp64 (oracle side).

The paged consumer must compute the same logical attention whatever its
tiling, split or page order ("Paged KV Context Store" page, consumer rules),
so the oracle is that plain definition over K/V gathered in logical order:

  query token at position q, query head j, KV head h = floor(j / (Hq/H)):
      s_i  = (q_vec . k_i) * sm_scale          for i in [0, q]
      out  = sum_i softmax(s)_i * v_i           (fp64, max subtracted)

Readings (pages silent, the consuming header is not on them): contiguous GQA
grouping, sm_scale passed by the caller (1/sqrt(D) in every workload), no
soft-cap, window or bias.  Decode: the step token is appended first, so a
sequence with seq_len n attends [0, n).  Verify/prefill: chunk token i sits at
position n0+i and attends [0, n0+i].  An empty context gives a zero output.
"""

from __future__ import annotations

import numpy as np

from .codecs import bf16_to_f32
from .store import OracleStore


def attend(qvec: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float) -> np.ndarray:
    """One query vector [D] against K, V [n, D] -> fp64 [D]."""
    if K.shape[0] == 0:
        return np.zeros(qvec.shape[-1], dtype=np.float64)
    s = (K.astype(np.float64) @ qvec.astype(np.float64)) * float(sm_scale)
    w = np.exp(s - s.max())
    return (w @ V.astype(np.float64)) / w.sum()


def attend_many(Qm: np.ndarray, limits, K: np.ndarray, V: np.ndarray, sm_scale: float) -> np.ndarray:
    """Several query vectors against one K, V [n, D]: row r of Qm [m, D] attends
    keys [0, limits[r]) -> fp64 [m, D].  The definition of ``attend`` for each
    row (an empty range gives zeros); the scores of all rows come from one
    product, which only saves time at long contexts."""
    m = Qm.shape[0]
    lim = np.asarray(limits, dtype=np.int64).reshape(m)
    out = np.zeros((m, V.shape[-1]), dtype=np.float64)
    n = int(lim.max()) if m else 0
    if n == 0:
        return out
    s = (K[:n].astype(np.float64) @ Qm.astype(np.float64).T) * float(sm_scale)      # [n, m]
    visible = np.arange(n)[:, None] < lim[None, :]
    s = np.where(visible, s, -np.inf)
    live = lim > 0
    mx = np.where(live, s.max(axis=0, initial=-np.inf), 0.0)
    w = np.where(visible, np.exp(s - mx[None, :]), 0.0)
    out[live] = (w.T @ V[:n].astype(np.float64))[live] / w.sum(axis=0)[live, None]
    return out


def decode_dense(q_bf16: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float) -> np.ndarray:
    """q [Hq, D] bf16 bits, K/V [n, H, D] float -> fp64 [Hq, D] (last-token query)."""
    q = bf16_to_f32(q_bf16)
    Hq, H = q.shape[0], K.shape[1]
    g = Hq // H
    return np.stack([attend(q[j], K[:, j // g], V[:, j // g], sm_scale) for j in range(Hq)])


def causal_dense(q_bf16: np.ndarray, K: np.ndarray, V: np.ndarray, n0: int, sm_scale: float) -> np.ndarray:
    """q [T, Hq, D], K/V [>= n0+T, H, D] -> fp64 [T, Hq, D]; token i attends [0, n0+i]."""
    q = bf16_to_f32(q_bf16)
    T, Hq = q.shape[0], q.shape[1]
    g = Hq // K.shape[1]
    out = np.empty((T, Hq, q.shape[2]), dtype=np.float64)
    for i in range(T):
        n = n0 + i + 1
        for j in range(Hq):
            out[i, j] = attend(q[i, j], K[:n, j // g], V[:n, j // g], sm_scale)
    return out


def paged_decode(store: OracleStore, layer: int, rows, seq_lens, q_bf16: np.ndarray,
                 sm_scale: float) -> np.ndarray:
    """Decode for a compact batch: q [B, Hq, D]; batch entry b reads table row rows[b]."""
    B = len(rows)
    out = np.empty(q_bf16.shape, dtype=np.float64)
    for b in range(B):
        K, V = store.gather(layer, int(rows[b]), int(seq_lens[b]))
        out[b] = decode_dense(q_bf16[b], K, V, sm_scale)
    return out


def paged_decode_one(store: OracleStore, layer: int, row: int, seq_len: int, q_bf16_head: np.ndarray,
                     j: int, Hq: int, sm_scale: float) -> np.ndarray:
    """One (sequence, query head) decode output, gathering only its KV head."""
    h = j // (Hq // store.H)
    K, V = store.gather_head(layer, row, seq_len, h)
    return attend(bf16_to_f32(q_bf16_head), K, V, sm_scale)


def paged_verify(store: OracleStore, layer: int, rows, n0s, cu_q, q_bf16: np.ndarray,
                 sm_scale: float) -> np.ndarray:
    """Multi-token verify / prefill chunk: q [sum T, Hq, D]; token i of entry b at n0[b]+i."""
    out = np.empty(q_bf16.shape, dtype=np.float64)
    for b in range(len(rows)):
        a, e = int(cu_q[b]), int(cu_q[b + 1])
        if e == a:
            continue
        K, V = store.gather(layer, int(rows[b]), int(n0s[b]) + (e - a))
        out[a:e] = causal_dense(q_bf16[a:e], K, V, int(n0s[b]), sm_scale)
    return out


def paged_verify_one(store: OracleStore, layer: int, row: int, n0: int, i: int, q_bf16_head: np.ndarray,
                     j: int, Hq: int, sm_scale: float) -> np.ndarray:
    """One (chunk token i, query head j) verify output."""
    h = j // (Hq // store.H)
    K, V = store.gather_head(layer, row, n0 + i + 1, h)
    return attend(bf16_to_f32(q_bf16_head), K, V, sm_scale)
