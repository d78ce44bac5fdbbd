"""MI355X-native hot path of Pre-hoc Sparsity (PrHS) sparse decode.

``sparse_top_kv_head_amd.prhs`` is the ctypes binding of the C-ABI library
``libprhs.so`` (HIP kernels for gfx950); ``sparse_top_kv_head_amd.synth``
builds the seeded synthetic workloads. The library is loaded on first use and
its absence is an error: there is no fallback path.
"""
