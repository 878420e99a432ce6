"""Convenience owner of a pool's device memory (torch tensors) around the C ABI.

torch provides the device memory and the stream; every operation is one call
of the C entry point with the same name (``_abi``).  Nothing here computes
any part of the path.
"""

from __future__ import annotations

import torch

from . import _abi as abi

_PLANE_TORCH = {abi.KV_DT_BF16: torch.int16, abi.KV_DT_I8: torch.int8, abi.KV_DT_E4M3FN: torch.uint8,
                abi.KV_DT_E2M1X2: torch.uint8, abi.KV_DT_F32: torch.float32, abi.KV_DT_U8_E4M3: torch.uint8,
                abi.KV_DT_F16: torch.int16}
ROLE_NAMES = {abi.KV_ROLE_K_CODE: "K_CODE", abi.KV_ROLE_K_SCALE: "K_SCALE", abi.KV_ROLE_V_CODE: "V_CODE",
              abi.KV_ROLE_V_SCALE: "V_SCALE"}


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def ptr(t: torch.Tensor | None) -> int:
    return 0 if t is None else t.data_ptr()


def i32(vals, device) -> torch.Tensor:
    return torch.tensor([int(v) for v in vals], dtype=torch.int32, device=device)


class DevicePool:
    """Planes [M][H][64][X] per layer and role, the block table [C][L], and the pool handle."""

    def __init__(self, profile: str, H: int, D: int, layers: int, S: int, C: int, M: int, free_order=None,
                 host_only: bool = False, zero: bool = True, device: str = "cuda", scale_bytes: int = 4,
                 head_major: bool = False):
        """scale_bytes: 4 (fp32) or 2 (binary16) INT8-G64 / FP8-row scale planes.

        head_major: planes in the head-major order [X, P, N, H] (storage [H][M][64][X]);
        ``planes`` always holds [M][H][64][X] views of the storage.
        """
        self.profile, self.H, self.D, self.layers, self.S, self.C, self.M = profile, H, D, layers, S, C, M
        self.L = -(-S // 64)
        self.host_only = host_only
        self.head_major = head_major
        layout = abi.KV_LAYOUT_HEAD_MAJOR if head_major else abi.KV_LAYOUT_PAGE_MAJOR
        self.device = None if host_only else torch.device(device)
        schema = abi.kv_profile_planes(abi.KV_PROFILE[profile], D,
                                       abi.KV_DT_F16 if scale_bytes == 2 else abi.KV_DT_F32)
        self.geo = abi.KVPageGeometry(64, H, D, layers, S, C, M)
        self.planes: list[dict] = []
        descs = []
        alloc = torch.zeros if zero else torch.empty
        for layer in range(layers):
            lp = {}
            for p in schema:
                t = None
                if not host_only:
                    shape = (H, M, 64, p.x_extent) if head_major else (M, H, 64, p.x_extent)
                    t = alloc(shape, dtype=_PLANE_TORCH[p.dtype], device=self.device)
                lp[ROLE_NAMES[p.role]] = t.permute(1, 0, 2, 3) if (head_major and t is not None) else t
                descs.append(abi.KVPlaneDesc(layer, p.role, p.dtype, p.x_extent, p.elem_bytes, layout,
                                             ptr(t) or None))
            self.planes.append(lp)
        self.table = None if host_only else torch.empty((C, self.L), dtype=torch.int32, device=self.device)
        self.handle = abi.kv_pool_create(self.geo, descs, ptr(self.table) or None, free_order, self.stream)

    @property
    def stream(self) -> int:
        return 0 if self.host_only else _stream()

    def close(self) -> None:
        if self.handle:
            abi.kv_pool_destroy(self.handle)
            self.handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ------------------------------------------------------------- metadata --
    def stats(self):
        return abi.kv_pool_stats(self.handle)

    def table_host(self):
        return abi.kv_pool_table_host(self.handle, self.C * self.L)

    def refs(self, g: int) -> int:
        return abi.kv_pool_page_refs(self.handle, g)

    def open(self, row: int) -> int:
        return abi.kv_seq_open(self.handle, row, self.stream)

    def fork(self, src: int, frontier: int, row: int) -> int:
        return abi.kv_seq_fork(self.handle, src, frontier, row, self.stream)

    def ensure_mapped(self, seq: int, tokens: int) -> None:
        abi.kv_seq_ensure_mapped(self.handle, seq, tokens, self.stream)

    def commit(self, seq: int, frontier: int) -> None:
        abi.kv_seq_commit(self.handle, seq, frontier)

    def release(self, seq: int) -> None:
        abi.kv_seq_release(self.handle, seq, self.stream)

    def reserve(self, seq: int, pages: int) -> None:
        abi.kv_seq_reserve(self.handle, seq, pages)

    def trim(self, seq: int, provisional: int) -> None:
        abi.kv_seq_trim(self.handle, seq, provisional, self.stream)

    def commit_accepted(self, seq: int, produced: int, accepted: int, cancelled: bool = False) -> None:
        abi.kv_seq_commit_accepted(self.handle, seq, produced, accepted, cancelled, self.stream)

    def reservation(self, seq: int) -> int:
        return abi.kv_seq_reservation(self.handle, seq)

    def replica_page_bytes(self) -> int:
        return abi.kv_replica_page_bytes(self.handle)

    def offload(self, seq: int, host: torch.Tensor) -> tuple:
        """Committed pages of seq into a pinned host tensor (replica layout); (pages, frontier)."""
        if not host.is_pinned():
            raise ValueError("the replica buffer must be pinned host memory")
        return abi.kv_seq_offload(self.handle, seq, host.data_ptr(), host.numel() * host.element_size(),
                                  self.stream)

    def restore(self, row: int, host: torch.Tensor, frontier: int) -> int:
        """A new address space on row from a replica in a pinned host tensor."""
        if not host.is_pinned():
            raise ValueError("the replica buffer must be pinned host memory")
        return abi.kv_seq_restore(self.handle, row, host.data_ptr(), host.numel() * host.element_size(), frontier,
                                  self.stream)

    def info(self, seq: int):
        return abi.kv_seq_info(self.handle, seq)

    def cow_tail(self, seq: int) -> None:
        abi.kv_cow_tail_page(self.handle, seq, self.stream)

    # --------------------------------------------------------------- kernels --
    def append(self, layer: int, table_rows: torch.Tensor, pos0: torch.Tensor, cu: torch.Tensor, total: int,
               k: torch.Tensor, v: torch.Tensor) -> None:
        abi.kv_append(self.handle, layer, table_rows.numel(), ptr(table_rows), ptr(pos0), ptr(cu), total, ptr(k),
                      ptr(v), self.stream)

    def workspace(self, B: int, Hq: int, max_seq_len: int, max_q_len: int = 0) -> torch.Tensor:
        n = abi.paged_attn_workspace_bytes(self.handle, B, Hq, max_seq_len, max_q_len)
        # no initialization: every call writes the parts of it that it reads
        return torch.empty(max(n, 256), dtype=torch.uint8, device=self.device)

    def decode(self, layer: int, Hq: int, table_rows: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
               q: torch.Tensor, sm_scale: float, out: torch.Tensor, ws: torch.Tensor) -> None:
        abi.paged_attn_decode(self.handle, layer, table_rows.numel(), Hq, ptr(table_rows), ptr(seq_lens),
                              max_seq_len, ptr(q), sm_scale, ptr(out), ptr(ws), ws.numel(), self.stream)

    def decode_noalloc(self, layer: int, Hq: int, table_rows: torch.Tensor, seq_lens: torch.Tensor,
                       max_seq_len: int, q: torch.Tensor, sm_scale: float, out: torch.Tensor) -> None:
        """decode on the library's static scratch (no workspace)."""
        abi.paged_attn_decode_noalloc(self.handle, layer, table_rows.numel(), Hq, ptr(table_rows), ptr(seq_lens),
                                      max_seq_len, ptr(q), sm_scale, ptr(out), self.stream)

    def decode_plan(self, Hq: int, table_rows: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                    ws: torch.Tensor) -> None:
        """Work list of this batch state into ws (valid for every layer until the rows or lengths change)."""
        abi.paged_attn_decode_plan(self.handle, table_rows.numel(), Hq, ptr(table_rows), ptr(seq_lens), max_seq_len,
                                   ptr(ws), ws.numel(), self.stream)

    def step_graph(self, B: int, Hq: int, table_rows: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                   qs: list, sm_scale: float, outs: list, ws: torch.Tensor, ks: list | None = None,
                   vs: list | None = None, pos0: torch.Tensor | None = None, cu: torch.Tensor | None = None,
                   total_tokens: int | None = None) -> int:
        """One decode step of len(qs) layers captured as a HIP graph (handle); the
        tensors must stay alive and in place for the graph's lifetime."""
        return abi.kv_decode_step_graph_create(
            self.handle, B, Hq, max_seq_len, ptr(table_rows), ptr(seq_lens), [ptr(q) for q in qs], sm_scale,
            [ptr(o) for o in outs], ptr(ws), ws.numel(), None if ks is None else [ptr(k) for k in ks],
            None if vs is None else [ptr(v) for v in vs], ptr(pos0) if pos0 is not None else 0,
            ptr(cu) if cu is not None else 0, total_tokens)

    def graph_launch(self, graph: int) -> None:
        abi.kv_step_graph_launch(graph, self.stream)

    @staticmethod
    def graph_destroy(graph: int) -> None:
        abi.kv_step_graph_destroy(graph)

    def decode_run(self, layer: int, B: int, Hq: int, max_seq_len: int, q: torch.Tensor, sm_scale: float,
                   out: torch.Tensor, ws: torch.Tensor) -> None:
        abi.paged_attn_decode_run(self.handle, layer, B, Hq, max_seq_len, ptr(q), sm_scale, ptr(out), ptr(ws),
                                  ws.numel(), self.stream)

    def decode_append_run(self, layer: int, B: int, Hq: int, max_seq_len: int, k: torch.Tensor, v: torch.Tensor,
                          q: torch.Tensor, sm_scale: float, out: torch.Tensor, ws: torch.Tensor) -> None:
        """Append each entry's one step row at seq_len - 1, then decode (the matrix-core page streams)."""
        abi.paged_attn_decode_append_run(self.handle, layer, B, Hq, max_seq_len, ptr(k), ptr(v), ptr(q), sm_scale,
                                         ptr(out), ptr(ws), ws.numel(), self.stream)

    def verify(self, layer: int, Hq: int, table_rows: torch.Tensor, q_pos0: torch.Tensor, cu_q: torch.Tensor,
               total_q: int, max_q_len: int, max_seq_len: int, q: torch.Tensor, sm_scale: float, out: torch.Tensor,
               ws: torch.Tensor) -> None:
        abi.paged_attn_verify(self.handle, layer, table_rows.numel(), Hq, ptr(table_rows), ptr(q_pos0), ptr(cu_q),
                              total_q, max_q_len, max_seq_len, ptr(q), sm_scale, ptr(out), ptr(ws), ws.numel(),
                              self.stream)
