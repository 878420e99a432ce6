"""Drive one workload through the oracle and through the device pool, in the same order.

History construction: roots in sequence order (open, map, append, commit),
then forks (fork at the source's frontier, map, append own history, commit).
Step: optional tail copy, map the step's tokens, one batched append of every
entry's new rows per layer, then decode (last token) or verify (the chunk).
"""

from __future__ import annotations

import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from oracle.pool import OraclePool
from oracle.store import OracleStore


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


# ------------------------------------------------------------------ oracle --
def build_oracle(wl, free_order=None, privatize=False, layers=None):
    layers = range(wl.layers) if layers is None else layers
    pool = OraclePool(wl.S, wl.C, wl.M, free_order=wl.free_order if free_order is None else free_order)
    st = OracleStore(pool, wl.profile, wl.H, wl.D, wl.layers, scale_bytes=wl.scale_bytes)
    sids = {}
    for b in wl.order():
        row = wl.table_rows[b]
        if wl.fork[b] is None or privatize:
            sids[b] = pool.open(row)
            n_inh = 0
        else:
            src, F = wl.fork[b]
            sids[b] = pool.fork(sids[src], F, row)
            n_inh = F
            if wl.hist[b] > F and F % 64:          # own history starts inside the shared tail
                _, info = pool.cow_tail(sids[b])
                st.cow_copy(*info)
        if wl.hist[b] > n_inh:
            assert pool.ensure_mapped(sids[b], wl.hist[b]) == ("OK", 0)
            for layer in layers:
                k, v = wl.logical_kv(layer, b, wl.hist[b])
                st.append(layer, row, n_inh, k[n_inh:], v[n_inh:])
        pool.commit(sids[b], wl.hist[b])
    for b in range(wl.B):                           # every tail copy before any write of the step
        if wl.cow[b]:
            _, info = pool.cow_tail(sids[b])
            if info is not None:
                st.cow_copy(*info)
    for b in range(wl.B):
        assert pool.ensure_mapped(sids[b], wl.hist[b] + wl.step[b]) == ("OK", 0)
        for layer in layers:
            k, v = wl.step_kv(layer, b)
            st.append(layer, wl.table_rows[b], wl.hist[b], k, v)
    return pool, st, sids


def oracle_pool_only(wl, free_order=None):
    """Block-table bookkeeping alone (cheap at any size)."""
    pool = OraclePool(wl.S, wl.C, wl.M, free_order=wl.free_order if free_order is None else free_order)
    sids = {}
    for b in wl.order():
        row = wl.table_rows[b]
        if wl.fork[b] is None:
            sids[b] = pool.open(row)
        else:
            sids[b] = pool.fork(sids[wl.fork[b][0]], wl.fork[b][1], row)
            if wl.hist[b] > wl.fork[b][1] and wl.fork[b][1] % 64:
                pool.cow_tail(sids[b])
        assert pool.ensure_mapped(sids[b], wl.hist[b])[0] == "OK"
        pool.commit(sids[b], wl.hist[b])
    for b in range(wl.B):
        if wl.cow[b]:
            pool.cow_tail(sids[b])
    for b in range(wl.B):
        assert pool.ensure_mapped(sids[b], wl.hist[b] + wl.step[b])[0] == "OK"
    return pool, sids


# ------------------------------------------------- oracle at full sizes --
PROFILE_KINDS = {"BF16": ("bf16", "bf16"), "INT8_G64": ("int8_g64",) * 2, "FP8_E4M3FN_ROW256": ("fp8_row",) * 2,
                 "NVFP4_G16": ("nvfp4_g16",) * 2, "K8V4": ("fp8_row", "nvfp4_g16")}


def oracle_logical(wl, layer, b, n):
    """Dequantized K, V float32 [n, H, D] of entry b's logical positions [0, n):
    the rows the workload wrote, through the oracle's codecs (the same values
    the oracle's store holds there; its planes are checked against the
    device's bit for bit elsewhere)."""
    from oracle import codecs as Q
    k, v = wl.logical_kv(layer, b, n)
    kind_k, kind_v = PROFILE_KINDS[wl.profile]
    K = Q.dequantize(kind_k, *Q.quantize(kind_k, k, wl.scale_bytes))
    V = Q.dequantize(kind_v, *Q.quantize(kind_v, v, wl.scale_bytes))
    return K.reshape(n, wl.H, wl.D), V.reshape(n, wl.H, wl.D)


def oracle_decode_all(wl, layer, seq_lens=None):
    """fp64 [B, Hq, D]: every decode output of the workload's step."""
    from oracle import attention as A
    from oracle import codecs as Q
    lens = wl.seq_lens if seq_lens is None else seq_lens
    q = Q.bf16_to_f32(wl.q(layer))
    g = wl.Hq // wl.H
    out = np.zeros((wl.B, wl.Hq, wl.D), dtype=np.float64)

    def entry(b):
        if lens[b] == 0:
            return
        K, V = oracle_logical(wl, layer, b, lens[b])
        for h in range(wl.H):
            out[b, h * g:(h + 1) * g] = A.attend_many(q[b, h * g:(h + 1) * g], [lens[b]] * g, K[:, h], V[:, h],
                                                       wl.sm_scale)

    # entries are independent; NumPy releases the interpreter lock in its loops
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        list(ex.map(entry, range(wl.B)))
    return out


def oracle_verify_rows(wl, layer, tokens):
    """fp64 outputs of chosen chunk tokens: tokens[b] lists token indices i of
    entry b (position hist[b] + i); returns {(b, i): [Hq, D]}."""
    from oracle import attention as A
    from oracle import codecs as Q
    q = Q.bf16_to_f32(wl.q(layer))
    g = wl.Hq // wl.H
    res = {}
    for b, toks in tokens.items():
        if not toks:
            continue
        toks = sorted(toks)
        n = wl.hist[b] + toks[-1] + 1
        rows = np.array([wl.cu_q[b] + i for i in toks])
        K, V = oracle_logical(wl, layer, b, n)
        for h in range(wl.H):
            Qm = q[rows][:, h * g:(h + 1) * g].reshape(-1, wl.D)
            lim = np.repeat([wl.hist[b] + i + 1 for i in toks], g)
            o = A.attend_many(Qm, lim, K[:, h], V[:, h], wl.sm_scale).reshape(len(toks), g, wl.D)
            for t, i in enumerate(toks):
                res.setdefault((b, i), np.zeros((wl.Hq, wl.D)))[h * g:(h + 1) * g] = o[t]
    return res


# ------------------------------------------------------------------ device --
from workloads.device_driver import build_device, device_decode, device_verify, plane_np  # noqa: E402,F401
