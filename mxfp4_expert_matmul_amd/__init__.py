"""MI355X (gfx950) forward pass of one sparse Mixture-of-Experts layer with
MXFP4 expert weights, behind the C ABI declared in include/k3moe.h.

This package is argument marshalling only: every step of the layer runs in
the HIP kernels of libk3moe.so. Importing it does not need a GPU; calling
into the library does. If the library has not been built, every entry point
raises instead of falling back to anything else.
"""
from ._binding import (  # noqa: F401
    K3MOE_OK, K3MOE_EINVAL, K3MOE_ENOMEM, K3MOE_EHIP, K3MOE_EUNSUPPORTED,
    K3MOE_FLAG_BIAS_SELECT_ONLY, K3MOE_CACHE_DEVICE_PLAN,
    K3MoEError, Config, Layer, CachedLayer, load_library, library_path,
    k3moe_create, k3moe_destroy, k3moe_status_str, k3moe_workspace_bytes,
    k3moe_layer_forward, k3moe_layer_forward_noalloc, k3moe_route, k3moe_group, k3moe_experts_forward,
    k3moe_pack_mxfp4, k3moe_pack_mxfp4_from_host, k3moe_tiled_scale_bytes, pack_mxfp4,
    pack_mxfp4_from_host, pack_layer_weights, pack_layer_weights_from_host,
)
