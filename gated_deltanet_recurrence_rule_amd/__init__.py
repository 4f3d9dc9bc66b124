"""libgdn: the gated delta-rule scan on MI355X (gfx950), behind a C ABI.

    from gated_deltanet_recurrence_rule_amd import decode_step, prefill

Both calls go through libgdn.so (include/gdn.h); there is no CPU fallback.
"""
from .binding import GdnError, decode_step, load, prefill, prefill_workspace_size, version

__all__ = ["GdnError", "decode_step", "load", "prefill", "prefill_workspace_size", "version"]
