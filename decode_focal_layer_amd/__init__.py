"""libkvsel for MI355X: attention-score-guided KV token selection and sparse
decode attention (HIP kernels for gfx950 behind a C ABI).

Importing the package loads nothing; ``decode_focal_layer_amd.kvsel`` is the
Python binding of the C library.
"""
