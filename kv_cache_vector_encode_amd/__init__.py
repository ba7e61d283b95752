"""MI355X-native rotation-preconditioned KV-cache codec (TurboQuant-style).

The compute path is the C-ABI library ``libtq`` (hand-written HIP for gfx950);
``kv_cache_vector_encode_amd.tq`` is a thin ctypes binding over it.
"""
