"""Page geometry, plane inventory and address translation (oracle side).

Source: NInfer "Paged KV Context Store" maintainer page --
  * capacity-geometry equations: L = ceil(S/P), M_min = max(L, C), M_max = C*L;
  * closed plane orders: page-major [X, P, H, N_physical] (first extent fastest);
  * X-extent list: code X=D; INT8-G64 scale X=D/64; FP8-E4M3FN-row256 scale
    X=1; NVFP4-G16 code packed U8 X=D/2 and U8 scale X=D/16;
  * address-translation equations: b = floor(p/P), o = p mod P,
    g = block_table[b], addr = base + d*nb0 + o*nb1 + h*nb2 + g*nb3;
  * D256 payload table (bytes per token and KV head);
  * PageBytes = sum over planes of PlaneBytesPerToken * P;
  * physical pages per backend (capacity of the selected backend): an MTP
    draft pool with window K holds M + C * ceil((K - 1) / P) pages, covering
    each active row's provisional lead of one speculative round.
"""

from __future__ import annotations

from dataclasses import dataclass

P = 64  # allocation granularity of every growing pool (granularity table)

PROFILES = ("BF16", "INT8_G64", "FP8_E4M3FN_ROW256", "NVFP4_G16", "K8V4")

# per-side storage kind of each closed profile (closed-profile paragraph:
# K8V4 is K = FP8-E4M3FN-row256 and V = NVFP4-G16, not a free combination)
PROFILE_SIDES = {
    "BF16": ("bf16", "bf16"),
    "INT8_G64": ("int8_g64", "int8_g64"),
    "FP8_E4M3FN_ROW256": ("fp8_row", "fp8_row"),
    "NVFP4_G16": ("nvfp4_g16", "nvfp4_g16"),
    "K8V4": ("fp8_row", "nvfp4_g16"),
}


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def logical_pages(S: int) -> int:
    """L: logical page capacity of one address space (capacity geometry)."""
    return ceil_div(S, P)


def m_bounds(S: int, C: int) -> tuple[int, int]:
    """(M_min, M_max) = (max(L, C), C*L) -- capacity geometry."""
    L = logical_pages(S)
    return max(L, C), C * L


def draft_pool_pages(M: int, C: int, K: int) -> int:
    """Physical pages of the MTP draft pool for draft window K >= 1 (backend
    capacity list): the Main pool's M plus one provisional lead of K - 1
    tokens per active row, in whole pages."""
    if K < 1:
        raise ValueError("draft window must be >= 1")
    return M + C * ceil_div(K - 1, P)


def explicit_capacity(k_main_tokens: int, S: int, C: int) -> int:
    """Explicit kv_capacity policy: M = ceil(K_main / P), K_main >= S, M in range."""
    if k_main_tokens < S:
        raise ValueError("K_main must be >= S")
    M = ceil_div(k_main_tokens, P)
    lo, hi = m_bounds(S, C)
    if not lo <= M <= hi:
        raise ValueError(f"M={M} outside [{lo}, {hi}]")
    return M


def check_geometry(*, page_size: int, S: int, C: int, M: int, H: int, D: int,
                   Hq: int | None = None, profile: str = "BF16") -> None:
    """Raise ValueError for geometry the pages rule out (or this library does not take)."""
    if page_size != P:
        raise ValueError("page size must be 64")
    if not 1 <= C <= 8:
        raise ValueError("max_concurrency must be in [1, 8]")
    if S < 1 or H < 1:
        raise ValueError("S and H must be positive")
    lo, hi = m_bounds(S, C)
    if not lo <= M <= hi:
        raise ValueError(f"M={M} outside [{lo}, {hi}]")
    if profile not in PROFILE_SIDES:
        raise ValueError("unknown profile")
    ksd, vsd = PROFILE_SIDES[profile]
    for kind in (ksd, vsd):
        g = {"bf16": 1, "int8_g64": 64, "fp8_row": 1, "nvfp4_g16": 16}[kind]
        if D % g or D % 2:
            raise ValueError(f"head_dim {D} not divisible by the {kind} group")
    if Hq is not None and (Hq < H or Hq % H):
        raise ValueError("query heads must be a multiple of KV heads")


@dataclass(frozen=True)
class PlaneSpec:
    role: str        # "K_CODE", "K_SCALE", "V_CODE", "V_SCALE"
    kind: str        # storage element kind
    x_extent: int    # X of the [X, P, H, N] order
    elem_bytes: int  # bytes of one X element


def side_planes(side: str, kind: str, D: int, scale_bytes: int = 4) -> list[PlaneSpec]:
    """Planes one side (K or V) of a profile resolves to (X-extent list)."""
    c, s = f"{side}_CODE", f"{side}_SCALE"
    if kind == "bf16":
        return [PlaneSpec(c, "bf16", D, 2)]
    if kind == "int8_g64":
        return [PlaneSpec(c, "i8", D, 1), PlaneSpec(s, "scale", D // 64, scale_bytes)]
    if kind == "fp8_row":
        return [PlaneSpec(c, "e4m3fn", D, 1), PlaneSpec(s, "scale", 1, scale_bytes)]
    if kind == "nvfp4_g16":
        return [PlaneSpec(c, "e2m1x2", D // 2, 1), PlaneSpec(s, "u8_e4m3", D // 16, 1)]
    raise ValueError(kind)


def plane_schema(profile: str, D: int, scale_bytes: int = 4) -> list[PlaneSpec]:
    """Per-layer plane schema of a closed profile (K planes then V planes)."""
    ks, vs = PROFILE_SIDES[profile]
    return side_planes("K", ks, D, scale_bytes) + side_planes("V", vs, D, scale_bytes)


def payload_bytes_per_token_head(profile: str, D: int, scale_bytes: int = 4) -> dict:
    """Physical bytes per token and KV head, split like the D256 payload table."""
    out = {"K_CODE": 0, "K_SCALE": 0, "V_CODE": 0, "V_SCALE": 0}
    for p in plane_schema(profile, D, scale_bytes):
        out[p.role] += p.x_extent * p.elem_bytes
    out["K"] = out["K_CODE"] + out["K_SCALE"]
    out["V"] = out["V_CODE"] + out["V_SCALE"]
    out["KV"] = out["K"] + out["V"]
    return out


def page_bytes(profile: str, D: int, H: int, layers: int, scale_bytes: int = 4) -> int:
    """PageBytes: bytes of one page group across every plane of every layer."""
    per_token = sum(p.x_extent * p.elem_bytes for p in plane_schema(profile, D, scale_bytes))
    return per_token * H * layers * P


def plane_shape(M: int, H: int, X: int) -> tuple[int, int, int, int]:
    """C-order shape of a page-major plane [X, P, H, N] (first extent fastest)."""
    return (M, H, P, X)


def element_index(d: int, o: int, h: int, g: int, X: int, H: int) -> int:
    """Element offset (in elements) of (d, o, h, g) in a page-major plane.

    With contiguous strides nb0 = 1, nb1 = X, nb2 = X*P, nb3 = X*P*H this is the
    address-translation equation of the page-major order.
    """
    nb0, nb1, nb2, nb3 = 1, X, X * P, X * P * H
    return d * nb0 + o * nb1 + h * nb2 + g * nb3


def element_index_head_major(d: int, o: int, h: int, g: int, X: int, M: int) -> int:
    """Element offset of (d, o, h, g) in a head-major plane [X, P, N, H].

    The head-major order swaps the head and page-group terms of the page-major
    equation: with contiguous strides nb0 = 1, nb1 = X, nb2 = X*P (the page
    group) and nb3 = X*P*M (the head).
    """
    nb0, nb1, nb2, nb3 = 1, X, X * P, X * P * M
    return d * nb0 + o * nb1 + g * nb2 + h * nb3


def translate(position: int, block_table_row) -> tuple[int, int, int]:
    """(b, o, g) for a logical position: b = floor(p/P), o = p mod P, g = table[b]."""
    b, o = divmod(position, P)
    return b, o, int(block_table_row[b])


def attention_pairs(reused: int, suffix: int) -> int:
    """Prefill attention work B*S + S(S+1)/2 ("Resource Scheduling and Context
    Cache" page, text-suffix prefill-work equation): B reused prefix tokens, S
    new suffix tokens, each new token attending itself and everything before."""
    return reused * suffix + suffix * (suffix + 1) // 2
