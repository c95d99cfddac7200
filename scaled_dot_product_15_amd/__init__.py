"""MI355X (gfx950) fused scaled dot-product attention, forward and backward.

The compute lives in a HIP C-ABI shared library (``libsdpa_mi355x.so``); this
package only marshals arguments to it.  Importing the package touches neither
the library nor the GPU; the first call of an entry point loads the library and
raises if it is missing.
"""
_API = ("attn_fwd", "attn_bwd", "attn_validate", "attn_fwd_workspace_size",
        "attn_bwd_workspace_size", "attn_bwd_ds_workspace_size", "attn_status_string", "debug_tile_map",
        "debug_mask_probe", "host_tile_map", "host_key_range", "host_query_range",
        "load_library", "AttnError", "Params", "make_params", "fwd_tile_shape")


def __getattr__(name):
    if name in _API:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
