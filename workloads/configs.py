"""Workload shapes: the five named configurations and small randomized cases.

Readings taken where the workload descriptions leave a choice open:
* tiny decode: S is not given; C=1 with M=16 forces L=16, so S=1024.  The
  300-token history is 4 full pages plus 44 columns; the step appends token 300.
* 8-sequence decode (BF16 and INT8-G64): sequences 0-3 share the 4096-token
  prefix written by sequence 0 (forks at the aligned frontier 4096, so no
  copy); their post-step context is U[4097, 32768]; the others are private with
  context U[1, 32768].  INT8-G64 appends T ~ U[1, 64] tokens per sequence;
  sequences 0, 2, 4, 6 are placed so that their append crosses a page
  boundary; 1% of K/V elements are scaled by 20.
* K8V4 long context: every sequence holds 65535 tokens (1023 full pages and a
  63-column tail); sequence 1 is a fork of sequence 0 at 65535 that copies the
  shared tail before appending; every sequence then appends one token.
* verify/prefill: n0 = 2039*64 + {35, 1, 63, 17}; sequences 0-1 verify 5
  tokens, 2-3 prefill a 512-token chunk.
* one layer where the text gives no layer count.
More workloads, not among the named five: BF16 pages at head_dim 256 (the
K8V4 decode shapes; the verify/prefill mix with 16 query / 2 KV heads), and
the verify/prefill mix on quantized pools (INT8-G64 with config 5's shapes,
K8V4 with config 4's heads and head_dim at 64K contexts).
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

from .gen import bf16_normal, rng_for


@dataclass
class Workload:
    name: str
    profile: str
    C: int
    S: int
    M: int
    layers: int
    Hq: int
    H: int
    D: int
    seed: int
    hist: list                      # committed tokens per sequence before the step
    step: list                      # tokens appended by the step per sequence
    fork: list                      # None or (source sequence, frontier) per sequence
    cow: list                       # sequence copies its shared tail before the step
    mode: str = "decode"            # "decode" or "verify"
    outlier_frac: float = 0.0
    scale_mul: float = 1.0          # softmax scale = scale_mul / sqrt(D) (> 1: peaked distributions)
    scale_bytes: int = 4            # INT8-G64 / FP8-row scale planes: 4 (fp32) or 2 (binary16)
    table_rows: list = field(default_factory=list)
    free_order: np.ndarray | None = None

    def __post_init__(self):
        B = len(self.hist)
        r = rng_for(self.seed, 0)
        if self.free_order is None:
            self.free_order = r.permutation(self.M).astype(np.int32)
        if not self.table_rows:
            self.table_rows = [int(x) for x in r.permutation(self.C)[:B]]

    # ------------------------------------------------------------ shapes --
    @property
    def B(self) -> int:
        return len(self.hist)

    @property
    def sm_scale(self) -> float:
        return float(np.float32(self.scale_mul) / np.sqrt(np.float32(self.D)))

    @property
    def seq_lens(self) -> list:
        """Context each sequence attends after the step (decode)."""
        return [n + t for n, t in zip(self.hist, self.step)]

    @property
    def cu_q(self) -> list:
        out = [0]
        for t in self.step:
            out.append(out[-1] + t)
        return out

    def own_start(self, b: int) -> int:
        """First history position sequence b writes itself (forks inherit the rest)."""
        return 0 if self.fork[b] is None else self.fork[b][1]

    def order(self) -> list:
        """Sequences in history-construction order: roots, then forks."""
        roots = [b for b in range(self.B) if self.fork[b] is None]
        return roots + [b for b in range(self.B) if self.fork[b] is not None]

    # -------------------------------------------------------------- data --
    def hist_kv(self, layer: int, b: int, lo: int | None = None, hi: int | None = None):
        """bf16 K, V [n, H, D] for positions [lo, hi) of sequence b's own history.

        The history is generated in 1024-token blocks so any slice can be
        regenerated alone.
        """
        start = self.own_start(b)
        lo = start if lo is None else lo
        hi = self.hist[b] if hi is None else hi
        assert start <= lo <= hi <= self.hist[b]
        blk = 1024

        def one(c):
            a, e = max(lo, c * blk), min(hi, (c + 1) * blk)
            r = rng_for(self.seed, 1, layer, b, c)
            k = bf16_normal(r, (blk, self.H, self.D), self.outlier_frac)
            v = bf16_normal(r, (blk, self.H, self.D), self.outlier_frac)
            return k[a - c * blk:e - c * blk], v[a - c * blk:e - c * blk]

        blocks = list(range(lo // blk, (hi + blk - 1) // blk))
        if len(blocks) > 2:
            with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
                parts = list(ex.map(one, blocks))
        else:
            parts = [one(c) for c in blocks]
        ks, vs = [p[0] for p in parts], [p[1] for p in parts]
        if not ks:
            z = np.zeros((0, self.H, self.D), dtype=np.uint16)
            return z, z.copy()
        return np.concatenate(ks), np.concatenate(vs)

    def logical_kv(self, layer: int, b: int, n: int):
        """bf16 K, V [n, H, D] of sequence b's logical positions [0, n) (history + step)."""
        parts_k, parts_v = [], []
        src = b
        segs = []
        pos = min(n, self.hist[b])
        # walk fork chain backwards to collect inherited prefixes
        while True:
            s = self.own_start(src)
            if pos > s:
                segs.append((src, s, pos))
            if self.fork[src] is None:
                break
            pos = min(pos, s)
            src = self.fork[src][0]
        for (sb, a, e) in reversed(segs):
            k, v = self.hist_kv(layer, sb, a, e)
            parts_k.append(k)
            parts_v.append(v)
        if n > self.hist[b]:
            k, v = self.step_kv(layer, b)
            parts_k.append(k[: n - self.hist[b]])
            parts_v.append(v[: n - self.hist[b]])
        return np.concatenate(parts_k), np.concatenate(parts_v)

    def step_kv(self, layer: int, b: int):
        r = rng_for(self.seed, 2, layer, b)
        k = bf16_normal(r, (self.step[b], self.H, self.D), self.outlier_frac)
        v = bf16_normal(r, (self.step[b], self.H, self.D), self.outlier_frac)
        return k, v

    def step_kv_all(self, layer: int):
        ks, vs = zip(*(self.step_kv(layer, b) for b in range(self.B)))
        return np.concatenate(ks), np.concatenate(vs)

    def q(self, layer: int) -> np.ndarray:
        """Queries: decode [B, Hq, D] (the step's last token); verify [sum T, Hq, D]."""
        r = rng_for(self.seed, 3, layer)
        n = self.B if self.mode == "decode" else sum(self.step)
        return bf16_normal(r, (n, self.Hq, self.D))


def _cfg1() -> Workload:
    return Workload("tiny_bf16_decode_ctx300", "BF16", C=1, S=1024, M=16, layers=1, Hq=8, H=2, D=128,
                    seed=1001, hist=[300], step=[1], fork=[None], cow=[False])


def _decode8(k: int, profile: str, outliers: float, multi: bool) -> Workload:
    r = rng_for(1000 + k, 9)
    hist, step, fork = [], [], []
    for b in range(8):
        T = int(r.integers(1, 65)) if multi else 1
        if b in (0, 2, 4, 6) and multi:
            T = max(T, 2)
        lo = 4096 + T if b < 4 else T      # post-step context range
        ctx = int(r.integers(lo, 32769))
        n = ctx - T
        if multi and b in (0, 2, 4, 6):
            # move the frontier so the append crosses a page boundary
            off = 64 - int(r.integers(1, T))          # in [65 - T, 63]
            n = (n // 64) * 64 + off
            if n + T > 32768:
                n -= 64
            if b < 4 and n < 4096:
                n += 64 * ((4096 - n) // 64 + 1)
        hist.append(n)
        step.append(T)
        fork.append((0, 4096) if b in (1, 2, 3) else None)
    name = "bf16_decode_c8_ctx32k_32layers" if profile == "BF16" else "int8g64_decode_c8_ctx32k_32layers"
    return Workload(name, profile, C=8, S=32768, M=8 * 512, layers=32, Hq=32, H=8, D=128,
                    seed=1000 + k, hist=hist, step=step, fork=fork, cow=[False] * 8,
                    outlier_frac=outliers)


def _cfg4() -> Workload:
    fork = [None] * 8
    fork[1] = (0, 65535)
    cow = [False] * 8
    cow[1] = True
    return Workload("k8v4_decode_c8_ctx64k", "K8V4", C=8, S=65536, M=8 * 1024, layers=1, Hq=16, H=2,
                    D=256, seed=1004, hist=[65535] * 8, step=[1] * 8, fork=fork, cow=cow)


def _cfg5() -> Workload:
    n0 = [2039 * 64 + o for o in (35, 1, 63, 17)]
    return Workload("bf16_verify5_prefill512_c4_ctx128k", "BF16", C=4, S=131072, M=4 * 2048, layers=1,
                    Hq=32, H=8, D=128, seed=1005, hist=n0, step=[5, 5, 512, 512], fork=[None] * 4,
                    cow=[False] * 4, mode="verify")


def _cfg6() -> Workload:
    # the K8V4 long-context shapes on BF16 pages (head_dim 256, the size the
    # D256 payload table is written for): 65535-token histories, one token each
    fork = [None] * 8
    fork[1] = (0, 65535)
    cow = [False] * 8
    cow[1] = True
    return Workload("bf16_d256_decode_c8_ctx64k", "BF16", C=8, S=65536, M=8 * 1024, layers=1, Hq=16, H=2,
                    D=256, seed=1006, hist=[65535] * 8, step=[1] * 8, fork=fork, cow=cow)


def _cfg7() -> Workload:
    # the verify / prefill mix at head_dim 256 (16 query / 2 KV heads, as above)
    n0 = [2039 * 64 + o for o in (35, 1, 63, 17)]
    return Workload("bf16_d256_verify5_prefill512_c4_ctx128k", "BF16", C=4, S=131072, M=4 * 2048, layers=1,
                    Hq=16, H=2, D=256, seed=1007, hist=n0, step=[5, 5, 512, 512], fork=[None] * 4,
                    cow=[False] * 4, mode="verify")


def _cfg8() -> Workload:
    # the verify / prefill mix on an INT8-G64 pool (config 5's shapes)
    n0 = [2039 * 64 + o for o in (35, 1, 63, 17)]
    return Workload("int8g64_verify5_prefill512_c4_ctx128k", "INT8_G64", C=4, S=131072, M=4 * 2048, layers=1,
                    Hq=32, H=8, D=128, seed=1008, hist=n0, step=[5, 5, 512, 512], fork=[None] * 4,
                    cow=[False] * 4, mode="verify", outlier_frac=0.01)


def _cfg9() -> Workload:
    # the verify / prefill mix on a K8V4 pool (config 4's heads and head_dim, 64K contexts)
    n0 = [1015 * 64 + o for o in (35, 1, 63, 17)]
    return Workload("k8v4_verify5_prefill512_c4_ctx64k", "K8V4", C=4, S=65536, M=4 * 1024, layers=1, Hq=16, H=2,
                    D=256, seed=1009, hist=n0, step=[5, 5, 512, 512], fork=[None] * 4, cow=[False] * 4,
                    mode="verify")


WORKLOADS = {
    1: _cfg1,
    2: lambda: _decode8(2, "BF16", 0.0, False),
    3: lambda: _decode8(3, "INT8_G64", 0.01, True),
    4: _cfg4,
    5: _cfg5,
    6: _cfg6,
    7: _cfg7,
    8: _cfg8,
    9: _cfg9,
}


def get(k: int) -> Workload:
    return WORKLOADS[k]()


def small(seed: int, profile: str = "BF16", *, B: int = 3, C: int = 4, Hq: int = 8, H: int = 2,
          D: int = 128, S: int = 1024, layers: int = 1, mode: str = "decode", hist=None, step=None,
          fork=None, cow=None, outlier_frac: float = 0.0, M: int | None = None,
          scale_mul: float = 1.0, scale_bytes: int = 4) -> Workload:
    """A randomized small case (several pages, ragged tails) the oracle finishes in seconds."""
    r = rng_for(5000 + seed, 9)
    if hist is None:
        hist = [int(r.integers(0, S - 64)) for _ in range(B)]
    B = len(hist)
    if step is None:
        step = [1] * B if mode == "decode" else [int(r.integers(1, 40)) for _ in range(B)]
    fork = fork or [None] * B
    cow = cow or [False] * B
    L = -(-S // 64)
    return Workload(f"small{seed}_{profile}", profile, C=C, S=S, M=M or C * L, layers=layers, Hq=Hq, H=H,
                    D=D, seed=5000 + seed, hist=list(hist), step=list(step), fork=list(fork), cow=list(cow),
                    mode=mode, outlier_frac=outlier_frac, scale_mul=scale_mul, scale_bytes=scale_bytes)
