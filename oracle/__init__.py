"""CPU oracle for the paged KV context store hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
(``paged_kv_cache_03_amd``, its HIP kernels and its C ABI) never imports it, and
this package imports nothing from the product: the two share no code, tables
or constants.  Inputs for both sides come from ``workloads`` (seeded generators
only, no arithmetic of the method).

What it computes, and where the pages define it (NInfer maintainer pages;
headings were lost in extraction, so passages are named by what they hold):

* ``geometry``  -- page geometry bounds, plane inventory, payload bytes,
  address translation.  "Paged KV Context Store" page: the capacity-geometry
  equations (L, M_min, M_max), the closed plane orders and X-extent list, the
  address-translation equations, the D256 payload table, the PageBytes
  equation, the P=64 translation.
* ``pool``      -- page-group allocator, address spaces, fork, tail COW, block
  table.  Same page: lease accounting equation, KVAddressSpace descriptor,
  device block-table matrix, ensure_mapped_to_tokens rules, Fork worked example
  (F=1000), writer-cardinality rules, finish/release rules.
* ``codecs``    -- the closed KV profiles' quantize/dequantize.  Same page:
  the closed-profile paragraph and X-extent list.  The exact rounding rules
  live in a header the pages do not contain; the reading used here is fp32
  arithmetic, round-half-even, saturating FP8/FP4, and fp32 or binary16
  INT8-G64 / FP8-row scales (the module docstring states each rule).
* ``store``     -- plane storage written and read through the block table.
* ``attention`` -- dense causal GQA softmax attention in fp64 over the
  logically gathered (dequantized) K/V: the plain definition of what the
  paged consumer must compute ("consumer rules": same logical attention,
  persistent codec and address contract whatever the tiling).

Every function is pinned by ``tests/test_oracle_*.py`` against values the
pages print (``tests/golden/``), closed forms, library routines and brute
force.  No function here is "parity unpinned".
"""

from . import geometry, codecs, pool, store, attention  # noqa: F401
