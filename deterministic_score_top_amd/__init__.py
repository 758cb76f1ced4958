"""MI355X-native deterministic DSA indexer top-k scan.

The compute path is the HIP library `libdsa_indexer.so` (gfx950), reached
through the thin ctypes binding in `deterministic_score_top_amd.indexer`.
Importing the package loads nothing; the binding loads the library on first
use and raises if it is missing.
"""
