"""CPU oracle of the TurboQuant-style KV-cache codec and its decode attention.

Test infrastructure only: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg, never by the library.  Written from the mlx-bun
TurboQuant design pages; it shares no code with the HIP path.
"""
