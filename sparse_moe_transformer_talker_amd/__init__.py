"""Talker MoE feed-forward layer for AMD Instinct MI355X (gfx950).

The compute lives in the HIP shared library ``libtalker_moe.so`` built from
``csrc/``; :mod:`.api` is a thin ctypes binding with the library's entry-point
names.  Importing this package loads nothing: :mod:`.inputs` (seeded synthetic
inputs) stays usable on machines without the library or a GPU.
"""

__version__ = "0.1.0"


def __getattr__(name):
    if name == "api":
        import importlib
        return importlib.import_module(".api", __name__)
    raise AttributeError(name)
