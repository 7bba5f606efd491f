"""MI355X (gfx950) paged-attention decode: a C-ABI HIP library plus a thin Python binding.

`paged_kv_cache_445_amd.pa` loads the compiled library (libpa.so) and raises if it is
missing; `paged_kv_cache_445_amd.workloads` builds seeded synthetic batches.
"""
