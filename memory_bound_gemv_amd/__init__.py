"""Batch-1 transformer decode on one MI355X: a persistent HIP kernel behind a
C-ABI (include/mbg.h).  ``_mbg`` is the ctypes binding with the C names;
``device_model`` holds the PyTorch plumbing (device memory, streams)."""
from . import _mbg  # noqa: F401  (fails loudly if libmbg.so is missing)
from ._mbg import MbgError  # noqa: F401
