"""Block-sparse attention for one MI355X (gfx950): C-ABI library + thin Python binding.

* ``sparse_mask_load_amd.binding``   — ctypes binding of ``libsparse_attn.so`` (the
  entry points of ``include/sparse_attn.h``: ``sparse_attn_plan``, ``sparse_attn_fwd``,
  ``chunk_merge`` and the plan accessors).
* ``sparse_mask_load_amd.workloads`` — seeded synthetic inputs of the five workloads.
* ``sparse_mask_load_amd.build``     — builds the library in-tree with hipcc.

Importing this package loads nothing; the library is loaded on first use.
"""
