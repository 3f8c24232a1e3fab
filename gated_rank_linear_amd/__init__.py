"""gated_rank_linear_amd: Gated Subspace Inference (GSI) linear layers on MI355X (gfx950).

The compute path is libgsi (hand-written HIP kernels behind the C ABI in include/gsi.h); this
package only marshals arguments to it. Importing it without the built library raises.
"""
from ._binding import (GSI_BF16, GSI_F16, GSI_F32, GSI_OK, GSI_SITE_DENSE, GSI_SITE_GATED,  # noqa: F401
                       GSI_SITE_STATIC, LIB_PATH, SIGNATURES, STATUS_NAMES, GsiError, Layer, Stack, create_dense_layer,
                       create_layer, dtype_code, gsi_block_step, gsi_block_step_workspace_bytes, gsi_calibrate, gsi_decode_step, gsi_decode_step_devpos,
                       gsi_calibrate_workspace_bytes,
                       gsi_device_check,
                       gsi_forward, gsi_layer_aux_bytes, gsi_layer_create, gsi_layer_create_dense,
                       gsi_layer_create_workspace_bytes, gsi_stack_create,
                       gsi_stack_create_modes, gsi_stack_decode, gsi_stack_workspace_bytes, gsi_workspace_bytes,
                       gsi_workspace_status, layer_image, lib, new_workspace)
