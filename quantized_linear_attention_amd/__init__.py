"""MI355X (gfx950) low-bit recurrent-state pool for gated Delta-rule decode.

Thin binding over the C ABI in include/stq.h (libstq.so, built in-tree by
``quantized_linear_attention_amd.build``).  Every function has the name of
the C entry point it marshals to; PyTorch supplies device memory and
streams only.  Import fails loudly when the HIP library is missing.
"""
from ._lib import (  # noqa: F401
    STQ_GATE_CHANNEL, STQ_GATE_HEAD, STQ_UNIT_HEAD, STQ_UNIT_ROW, StqError, library_path,
    make_desc, stq_decode_step, stq_pool_bytes, stq_pool_create, stq_pool_destroy,
    stq_pool_fetch, stq_pool_store, stq_requant_fixed_scales, stq_status_str,
    stq_allocate_bits, stq_decode_commit, stq_decode_readout, stq_prefill, stq_prefill_states, stq_window_flush,
)
