"""Float64 CPU oracle of the DiT denoiser block (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this package.  It shares no code with the GPU library.
"""
