"""MI355X-native confidence-gated KV-cache eviction (CONF-KV, KVpop variant).

The decode step runs in hand-written HIP kernels for gfx950 behind the C ABI
declared in ``include/confkv.h`` (``libconfkv.so`` in this directory).
``confkv`` is the thin ctypes binding; ``synth`` holds the seeded synthetic
input generators. Importing this package loads nothing native; the binding
loads the library on first use and raises if it is missing.
"""
