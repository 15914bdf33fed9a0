"""Routed latent decode attention for MI355X (gfx950): Python binding of
libbasiskv.so, the C-ABI library of hand-written HIP kernels declared in
include/basiskv.h.  Importing raises if the library has not been built."""
from .basiskv import *  # noqa: F401,F403
from .basiskv import (Cache, Dims, Factors, BasisKVError, new_workspace,  # noqa: F401
                      workspace_bytes, LIB_PATH, EXPORTS)
