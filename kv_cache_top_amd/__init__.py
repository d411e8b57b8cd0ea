"""MI355X-native ParisKV decode path: coarse-to-fine KV-cache retrieval and
sparse GQA attention as hand-written HIP kernels behind a C ABI
(include/pariskv.h, libpariskv.so)."""
from . import _native  # noqa: F401  (raises ImportError when the library is not built)
from ._native import PkConfig, PkError, codebook, make_config  # noqa: F401
from .pariskv import ParisKV  # noqa: F401
