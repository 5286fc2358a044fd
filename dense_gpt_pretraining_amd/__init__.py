"""One forward+backward pretraining step of the nanochat-style dense decoder
on an MI355X (gfx950), behind the C ABI of include/nc.h.

The HIP library libnc.so does every step of the computation; this package
only builds it (``build``) and binds it (``binding``).
"""
from .binding import (  # noqa: F401
    Model, NcError, make_config, nc_config, nc_forward_backward, nc_forward_loss,
    nc_init_params, nc_last_hip_error, nc_param_count, nc_param_layout, nc_status_string,
    nc_validate_tokens, nc_workspace_size, NC_BF16, NC_F32,
)
