"""MI355X decode megakernel: one transformer-decoder decode step run as a
persistent task graph (C ABI in include/mk.h, kernels in csrc/).

Importing the package loads nothing; ``mk.lib()`` loads libmk.so on first
use and raises if it has not been built.
"""
