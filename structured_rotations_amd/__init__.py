"""HARP / randomized-Hadamard apply path for MI355X (gfx950).

The compute lives in libharp.so (C ABI: include/harp.h); `api` is its Python
binding.  `inputs` and `workloads` draw seeded synthetic inputs.
"""
from .api import (  # noqa: F401
    harp_apply, harp_apply_decode, harp_apply_decode_workspace, harp_apply_inverse, harp_apply_vjp,
    harp_apply_vjp_workspace, harp_theta_vjp, harp_block_count, harp_gauss_count, harp_group_count,
    harp_materialize_blocks, harp_materialize_blocks_q8, harp_quantize_theta, harp_rotate_weight, harp_rotate_weight_workspace, harp_theta_count,
    rht_compose,
)

__version__ = "0.1.0"
