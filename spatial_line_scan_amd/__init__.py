"""MI355X-native GSPN four-direction line-scan propagation.

The compute path is a C-ABI shared library (``libgspn.so``, built from
``csrc/`` with hipcc for gfx950); ``spatial_line_scan_amd.gspn`` is its thin
ctypes binding.  Importing this package does not load the library; the first
call into ``gspn`` does, and raises if it is missing.
"""
__all__ = ["gspn", "inputs"]
