"""Indexer + top-k sparse attention for MI355X (gfx950).

The compute lives in the HIP library ``libdsa.so`` (C ABI declared in
include/dsa.h); ``binding`` marshals torch tensors into it.  ``synth`` draws
the seeded synthetic inputs.
"""
