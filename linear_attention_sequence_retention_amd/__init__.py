"""MI355X-native RetNet multi-scale retention: HIP kernels behind a C ABI.

The compute lives in ``libretention.so`` (built from ``csrc/``); the Python
side only marshals arguments.  Import :mod:`.binding` for the entry points.
This package's ``__init__`` loads nothing so that the seeded input generator
(:mod:`.workloads`) can be imported without the library.
"""
