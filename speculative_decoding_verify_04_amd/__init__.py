"""MI355X-native verify step of batched speculative sampling.

The compute lives in ``libspecverify.so`` (hand-written HIP kernels for gfx950
behind a C ABI, declared in ``include/specverify.h``).  ``api`` is a thin ctypes
binding over it; ``workloads`` builds seeded synthetic inputs.  Importing this
package does not load the library; the first call into ``api`` does, and fails
loudly if it has not been built.
"""
