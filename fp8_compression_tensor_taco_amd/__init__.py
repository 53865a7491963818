"""MI355X-native TACO FP8 compression operator for tensor-parallel intermediate tensors.

Python face of libtaco (include/taco.h): ``compress``, ``decompress`` and
``decompress_sum`` over bf16 [tokens, hidden] GPU tensors.  The library is
loaded on first use and the calls raise if it is missing; there is no CPU path.
"""
from ._binding import (  # noqa: F401
    TACO_AMAX_FLOATS,
    TACO_AMAX_SLOTS,
    TACO_MAX_PARTS,
    TacoError,
    compress,
    compress_blockscale,
    compress_delayed,
    compress_int8,
    compress_noalloc,
    TACO_DEFAULT_BARRIER_POLLS,
    TACO_FLAG_TWO_PASS,
    is_single_pass,
    two_shot_allreduce,
    decompress,
    decompress_blockscale,
    decompress_int8,
    decompress_sum,
    decompress_sum_compress,
    library_path,
    load,
    num_scales,
    version,
    workspace_bytes,
    workspace_timed_out,
)

__all__ = [
    "TACO_AMAX_FLOATS", "TACO_AMAX_SLOTS", "TACO_DEFAULT_BARRIER_POLLS", "TACO_FLAG_TWO_PASS", "TACO_MAX_PARTS",
    "TacoError", "compress", "compress_blockscale", "compress_delayed", "compress_int8", "compress_noalloc", "decompress",
    "decompress_blockscale", "decompress_int8", "decompress_sum", "decompress_sum_compress", "is_single_pass",
    "library_path", "load", "num_scales", "two_shot_allreduce", "version", "workspace_bytes",
    "workspace_timed_out",
]
