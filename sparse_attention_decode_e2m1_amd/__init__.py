"""CSA2 compressed sparse attention decode with FP4 (E2M1) global KV, for
MI355X (gfx950).  The library is ``libcsa2.so`` (hand-written HIP kernels
behind a C ABI declared in ``include/csa2.h``); ``api`` is its thin ctypes
binding.  ``inputs`` is the seeded synthetic input generator."""
