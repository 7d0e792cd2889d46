"""MI355X-native routed Mixture-of-Experts layer (Qwen3.5-35B-A3B shape).

The compute lives in libmoe_hip.so (hand-written HIP kernels for gfx950,
C ABI in include/moe.h); ``_lib`` is its thin ctypes binding and
``layer.DeviceLayer`` holds a layer's weights in device memory.
"""
from ._lib import (MOE_PATH_AUTO, MOE_PATH_GEMV, MOE_PATH_MFMA, MOE_SB_MXFP4, MOE_WFMT_KQUANT,  # noqa: F401
                   MOE_WFMT_MXFP4, MoeError, make_desc,
                   moe_abi_version, moe_dequant, moe_layer_forward, moe_layer_forward_noalloc,
                   moe_layer_forward_range,
                   moe_layer_forward_shard,
                   moe_reduce_partials, moe_reduce_residual, moe_rmsnorm, moe_rmsnorm_apply,
                   moe_rmsnorm_sumsq, moe_route_bucket, moe_status_str, moe_workspace_bytes,
                   router_topk)
