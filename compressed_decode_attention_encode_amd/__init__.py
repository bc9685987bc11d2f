"""TurboQuant KV-cache encode and fused decode attention for AMD Instinct MI355X (gfx950).

The compute path lives in ``libtq.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/tq.h``).  :mod:`.tq` is a thin ctypes binding with the same
function names; :mod:`.workloads` draws the seeded synthetic inputs.
"""
