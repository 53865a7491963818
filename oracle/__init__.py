"""fp64 CPU oracle for the TACO FP8 compression operator.

Test infrastructure only: see ``oracle/taco_oracle.py`` for what it computes and
which passages it follows.  Product code never imports this package.
"""
from .int8 import (  # noqa: F401
    compress_int8_block,
    compress_int8_tensor,
    decompress_int8,
    decompress_int8_f64,
    int8_scale,
    quantize_int8,
)
from .taco_oracle import (  # noqa: F401
    Q_MAX,
    ash_scale,
    bf16_bits_to_f64,
    block_energy,
    compress,
    compress_blockscale,
    compress_delayed,
    decompress,
    decompress_blockscale,
    decompress_blockscale_f64,
    decompress_f64,
    decompress_sum,
    decompress_sum_compress,
    ds_scale,
    e4m3_decode,
    e4m3_decode_code,
    e4m3_encode,
    e4m3_table,
    f64_to_bf16_bits,
    hadamard,
    hadamard_rotate,
    quantize,
    two_shot_allreduce,
)
