"""INT4 single-token decode block for AMD MI355X (gfx950).

The compute path is the HIP library ``libi4d.so`` (C ABI in include/i4d.h);
``binding`` exposes its entry points to Python by the same names,
``device`` allocates GPU buffers with torch, ``synth`` draws the seeded
synthetic workloads.  Importing the package loads nothing; the first call
into ``binding`` loads the library and fails loudly if it is missing.
"""
__all__ = ["binding", "device", "synth"]
