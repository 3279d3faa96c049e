"""MI355X (gfx950) DSA sparse-attention step: lightning indexer + Top-K +
sparse flash attention over a paged MLA latent cache.

``dsa`` is the ctypes binding of the C ABI (``include/dsa.h``, built into
``libdsa.so`` by ``build.build()``); ``inputs`` draws seeded synthetic inputs.
"""
