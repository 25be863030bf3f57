"""Trellis-coded (EXL3-style) linear layers on MI355X (gfx950).

The compute path is the HIP library ``libtrellis.so`` behind a C ABI; the Python
binding in :mod:`trellis_coded_bit_amd.binding` only marshals arguments.
"""
__all__ = ["synth", "binding"]
