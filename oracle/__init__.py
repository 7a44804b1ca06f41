"""CPU oracle for the Lion Cub compressed-update step.

TEST INFRASTRUCTURE ONLY: imported by tests/, by __graft_entry__.smoke() and by
bench.py's CPU-baseline leg.  The GPU library and its Python binding never
import it.  See lco.h for the definitions and their sources.
"""
