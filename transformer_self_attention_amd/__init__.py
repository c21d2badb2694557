"""RoPE + causal MHA/GQA attention for MI355X (gfx950): HIP kernels behind a C-ABI library.

``inputs`` draws the seeded synthetic workloads; ``lib`` is the thin ctypes binding to
``libattn.so`` (import it explicitly: it loads the HIP library and fails loudly when the
library is missing).
"""
