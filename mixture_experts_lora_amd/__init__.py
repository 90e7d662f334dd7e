"""MI355X (gfx950) MoE expert layer with split LoRA.

The compute lives in the HIP library ``libmoe_lora.so`` (C ABI in
``include/moe_lora.h``); this package only loads it and marshals torch
tensors.  Importing the package does not load the library; the first call
does, and fails loudly if it has not been built.
"""
from .api import (  # noqa: F401
    ENGINE_ALL,
    ENGINE_DH,
    ENGINE_DOWN,
    ENGINE_DX,
    ENGINE_GATE_UP,
    ENGINE_RANK,
    PRODUCTS,
    SPLITK_1024,
    SPLITK_4096,
    STAGE32,
    TILE256,
    Dims,
    Grads,
    MergedWeights,
    MoELoRALayer,
    RouterGrads,
    Routing,
    Weights,
    autotune,
    backward,
    describe_engines,
    empty_grads,
    empty_router_grads,
    empty_routing,
    forward,
    forward_merged,
    forward_saved_bytes,
    get_engines,
    merge_lora,
    route,
    route_noalloc,
    route_workspace_bytes,
    set_engines,
    workspace_bytes,
)
from ._lib import MOE_BF16, MOE_F16, MoeError, load  # noqa: F401
from .autograd import moe_lora  # noqa: F401
