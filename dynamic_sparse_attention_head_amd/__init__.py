"""mmsa: modality-aware dynamic sparse-attention prefill on MI355X (gfx950).

The compute path is the HIP library libmmsa.so; `mmsa` is its thin ctypes
binding.  Importing this package loads nothing; the binding loads the library
on first use and raises if it is missing.
"""
