"""One forward+backward pretraining step of the nanochat-style dense decoder
on an MI355X (gfx950), behind the C ABI of include/nc.h.

The HIP library libnc.so does every step of the computation; this package
only builds it (``build``) and binds it (``binding``).

The binding is imported on first use of any of its names, so that
``python -m dense_gpt_pretraining_amd.build`` works on a tree where the
library has not been built yet.  Using a name while libnc.so is missing
raises ImportError: there is no fallback.
"""
_EXPORTS = (
    "Model", "NcError", "make_config", "nc_config", "nc_forward_backward", "nc_forward_loss",
    "nc_forward_token_loss", "nc_init_params", "nc_last_hip_error", "nc_param_count",
    "nc_param_layout", "nc_status_string", "nc_validate_tokens", "nc_workspace_size",
    "NC_BF16", "NC_F32", "Optimizer", "make_optim_config", "nc_optim_step", "nc_optim_init",
    "nc_grad_accumulate", "nc_lr_multiplier", "Generator", "nc_prefill", "nc_decode_step",
)

__all__ = list(_EXPORTS)


def __getattr__(name):
    if name in _EXPORTS or name == "binding":
        import importlib
        b = importlib.import_module(".binding", __name__)
        return b if name == "binding" else getattr(b, name)
    raise AttributeError(f"module {__name__!r} has no attribute {name!r}")
