"""Plane storage written and read through the block table (oracle side).

Source: NInfer "Paged KV Context Store" maintainer page -- page-group diagram
(one page-group id selects slice g of every grouped plane), page-major order
[X, P, H, N] (C-order [M][H][P][X] here), P=64 translation (block =
position >> 6, offset = position & 63, page = block_table[block]), and the
tail-COW rule (copy the committed columns of the shared tail into a private
page group for every plane), the writer-cardinality rule (a write into a page
that several address spaces reference is refused), and the host replica's logical-order packed
layout (no device page ids or table holes; each page carries the payload of
every grouped plane of the pool; full pages are copied).

Planes are plain NumPy arrays indexed [g, h, o, x]; ``geometry.element_index``
is the equivalent flat-address form, pinned against this indexing in tests.
"""

from __future__ import annotations

import numpy as np

from . import codecs
from .geometry import P, PROFILE_SIDES, plane_schema
from .pool import OraclePool

_NP_DTYPE = {"bf16": np.uint16, "i8": np.int8, "e4m3fn": np.uint8, "e2m1x2": np.uint8,
             "u8_e4m3": np.uint8}


class OracleStore:
    def __init__(self, pool: OraclePool, profile: str, H: int, D: int, layers: int, scale_bytes: int = 4):
        """scale_bytes: 4 (fp32) or 2 (binary16) INT8-G64 / FP8-row scale planes."""
        if scale_bytes not in (2, 4):
            raise ValueError("scale planes are 4 or 2 bytes")
        self.pool, self.profile, self.H, self.D, self.layers = pool, profile, H, D, layers
        self.scale_bytes = scale_bytes
        self.kinds = PROFILE_SIDES[profile]
        self.schema = plane_schema(profile, D, scale_bytes=scale_bytes)
        self.planes = []
        for _ in range(layers):
            lp = {}
            for spec in self.schema:
                dt = (np.float32 if scale_bytes == 4 else np.uint16) if spec.kind == "scale" else _NP_DTYPE[spec.kind]
                lp[spec.role] = np.zeros((pool.M, H, P, spec.x_extent), dtype=dt)
            self.planes.append(lp)

    # ------------------------------------------------------------- write --
    def append(self, layer: int, row: int, pos0: int, k_bf16: np.ndarray, v_bf16: np.ndarray) -> None:
        """Quantize rows [T, H, D] and store them at positions pos0 .. pos0+T-1."""
        T = k_bf16.shape[0]
        lp = self.planes[layer]
        pos = pos0 + np.arange(T)
        blocks, offs = pos >> 6, pos & 63
        pages = self.pool.table[row, blocks]
        if np.any(pages < 0):
            raise ValueError("append into an unmapped logical block")
        # writer-cardinality rule: a page referenced by several address spaces
        # is immutable; its tail must be copied before a write
        if np.any(self.pool.refs[pages] > 1):
            raise ValueError("append into a page shared by several address spaces")
        for side, x in (("K", k_bf16), ("V", v_bf16)):
            code, scale = codecs.quantize(self.kinds[0 if side == "K" else 1], x, self.scale_bytes)
            lp[f"{side}_CODE"][pages, :, offs, :] = code
            if scale is not None:
                lp[f"{side}_SCALE"][pages, :, offs, :] = scale.reshape(T, self.H, -1)

    def cow_copy(self, src: int, dst: int, cols: int) -> None:
        """Copy columns [0, cols) of page group src into dst for every plane."""
        for lp in self.planes:
            for arr in lp.values():
                arr[dst, :, :cols, :] = arr[src, :, :cols, :]

    # -------------------------------------------------------------- read --
    def gather(self, layer: int, row: int, n: int) -> tuple[np.ndarray, np.ndarray]:
        """Dequantized K, V float32 [n, H, D] of logical positions [0, n) of a row."""
        lp = self.planes[layer]
        pos = np.arange(n)
        pages = self.pool.table[row, pos >> 6]
        if np.any(pages < 0):
            raise ValueError("read of an unmapped logical block")
        offs = pos & 63
        out = []
        for i, side in enumerate(("K", "V")):
            code = lp[f"{side}_CODE"][pages, :, offs, :]
            scale = lp[f"{side}_SCALE"][pages, :, offs, :] if f"{side}_SCALE" in lp else None
            out.append(codecs.dequantize(self.kinds[i], code, scale))
        return out[0], out[1]

    def gather_head(self, layer: int, row: int, n: int, h: int) -> tuple[np.ndarray, np.ndarray]:
        """Dequantized K, V float32 [n, D] of one KV head (cheaper for big contexts)."""
        lp = self.planes[layer]
        pos = np.arange(n)
        pages = self.pool.table[row, pos >> 6]
        if np.any(pages < 0):
            raise ValueError("read of an unmapped logical block")
        offs = pos & 63
        out = []
        for i, side in enumerate(("K", "V")):
            code = lp[f"{side}_CODE"][pages, h, offs, :]
            scale = lp[f"{side}_SCALE"][pages, h, offs, :] if f"{side}_SCALE" in lp else None
            out.append(codecs.dequantize(self.kinds[i], code, scale))
        return out[0], out[1]


    # ------------------------------------------------------- host replica --
    def replica_order(self) -> list:
        """(layer, PlaneSpec) in the order a replica page stores them: layers
        ascending, then K code, K scale, V code, V scale."""
        return [(layer, spec) for layer in range(self.layers) for spec in self.schema]

    def replica_page_bytes(self) -> int:
        return sum(self.H * P * spec.x_extent * spec.elem_bytes for _, spec in self.replica_order())

    def replica(self, sid: int) -> tuple[np.ndarray, int]:
        """Logical-order packed copy of an address space's committed pages:
        page i of the replica is logical block i, holding every plane's
        [H][64][X] slice of its page group (all 64 rows), planes in
        replica_order.  Returns (bytes, committed frontier)."""
        n = self.pool.frontier_of(sid)
        pages = self.pool.pages_of(sid)[: -(-n // P)]
        out = []
        for g in pages:
            for layer, spec in self.replica_order():
                out.append(np.ascontiguousarray(self.planes[layer][spec.role][g]).view(np.uint8).ravel())
        data = np.concatenate(out) if out else np.zeros(0, np.uint8)
        return data, n

    def restore(self, row: int, data: np.ndarray, frontier: int) -> int:
        """A new address space on `row` holding the replica's pages: map
        ceil(frontier / 64) page groups, write each page's payload into them,
        commit the frontier."""
        pool = self.pool
        n_pages = -(-frontier // P)
        pb = self.replica_page_bytes()
        if data.size < n_pages * pb:
            raise ValueError("replica shorter than its pages")
        sid = pool.open(row)
        st, _ = pool.ensure_mapped(sid, frontier)
        if st != "OK":
            pool.release(sid)
            raise ValueError(f"restore: {st}")
        for i, g in enumerate(pool.pages_of(sid)):
            off = i * pb
            for layer, spec in self.replica_order():
                arr = self.planes[layer][spec.role]
                nb = self.H * P * spec.x_extent * spec.elem_bytes
                arr[g] = data[off:off + nb].view(arr.dtype).reshape(arr.shape[1:])
                off += nb
        pool.commit(sid, frontier)
        return sid
