"""Multipole Attention decode path for AMD MI355X (gfx950).

The HIP library libmpattn.so implements the C ABI of include/mpattn.h; the
Python binding is the submodule ``sparse_long_context_means_amd.mpattn``
(import it explicitly; the package itself loads nothing so that the build
step can run before the library exists).
"""
