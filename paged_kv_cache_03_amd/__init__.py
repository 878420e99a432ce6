"""Paged KV context store hot path for MI355X (gfx950).

The product is ``libkvstore.so``: hand-written HIP kernels (quantizing append,
split-K paged decode, MFMA verify/prefill, tail COW) behind the C ABI in
``include/kvstore.h``.  ``_abi`` binds that ABI with ctypes under the same
names; ``device_pool.DevicePool`` owns torch device memory for a pool.  There
is no CPU fallback: importing fails if the library is not built.
"""

from . import _abi  # noqa: F401  (loads libkvstore.so or raises ImportError)
from ._abi import KVError  # noqa: F401
