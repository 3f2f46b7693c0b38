"""Speculative sampling hot path on MI355X (gfx950): verify pass + accept/resample.

The compute lives in the HIP library ``libspecdec.so`` (C ABI, declared in
``include/specdec.h``); ``binding`` marshals arguments to it with ctypes and
``synth`` draws seeded synthetic inputs.  Nothing here computes the method on the CPU.
"""
