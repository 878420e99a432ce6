"""Plane storage written and read through the block table (oracle side).

Source: NInfer "Paged KV Context Store" maintainer page -- page-group diagram
(one page-group id selects slice g of every grouped plane), page-major order
[X, P, H, N] (C-order [M][H][P][X] here), P=64 translation (block =
position >> 6, offset = position & 63, page = block_table[block]), and the
tail-COW rule (copy the committed columns of the shared tail into a private
page group for every plane).

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
    def __init__(self, pool: OraclePool, profile: str, H: int, D: int, layers: int):
        self.pool, self.profile, self.H, self.D, self.layers = pool, profile, H, D, layers
        self.kinds = PROFILE_SIDES[profile]
        self.schema = plane_schema(profile, D, scale_bytes=4)
        self.planes = []
        for _ in range(layers):
            lp = {}
            for spec in self.schema:
                dt = np.float32 if spec.kind == "scale" else _NP_DTYPE[spec.kind]
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
        for side, x in (("K", k_bf16), ("V", v_bf16)):
            code, scale = codecs.quantize(self.kinds[0 if side == "K" else 1], x)
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
