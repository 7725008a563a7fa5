"""QuoKA-style query-oriented KV selection + compacted attention for chunked
prefill on MI355X (gfx950): hand-written HIP kernels behind a C ABI
(include/kvsel.h, libkvsel.so) and a thin ctypes binding.

    from chunked_prefill_kv_amd import kvsel     # the C-ABI calls
    from chunked_prefill_kv_amd import gen       # seeded synthetic workloads
    from chunked_prefill_kv_amd import runner    # resident-tensor drivers
"""
