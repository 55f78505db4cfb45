"""Paged KV-cache attention for AMD MI355X (gfx950).

The compute path is the C-ABI library libpagedkv.so (include/pa.h), built from
hand-written HIP kernels by `python -m paged_kv_cache_40_amd.build`.  This
package adds the torch-tensor binding (api.py, argument marshalling only) and
the host block manager that decides slots, sharing and copy-on-write pairs
(block_manager.py).  The binding loads the library on first use and raises if
it is not built; there is no other implementation to fall back to.
"""

from .block_manager import BlockManager, tables_to_array  # noqa: F401


def __getattr__(name):
    if name in ("pa_write_kv", "pa_decode", "pa_decode_ext", "pa_copy_blocks",
                "pa_swap_blocks", "pa_decode_workspace_bytes", "pa_strerror"):
        from . import api
        return getattr(api, name)
    raise AttributeError(name)
