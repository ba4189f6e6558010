"""libks for AMD MI355X: Kronecker-sparse (KS) matrix multiplication.

Y = X W^T where W has support I_a (x) 1_{b x c} (x) I_d and its a*b*c*d
nonzeros are stored as an (a, d, b, c) tensor (KS abstract page,
taxoreview.com "dblp:303/4794", first paragraph). The compute path is the
HIP library libks.so (C ABI in include/ks.h); ``libks`` is its ctypes
binding. Importing this package loads nothing; the first call does.
"""
from . import datagen  # noqa: F401  (seeded inputs; no KS arithmetic)

__all__ = ["datagen", "libks"]


def __getattr__(name):
    if name == "libks":
        import importlib
        return importlib.import_module(__name__ + ".libks")
    raise AttributeError(name)
