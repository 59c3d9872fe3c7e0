"""MI355X (gfx950) Direct-P FP4 attention forward.

The computation lives in the HIP library ``libattnfp4.so`` (C ABI in
``include/attn_fp4.h``); this package is its thin ctypes binding plus the
seeded synthetic-input generators (``synth``).
"""

from ._binding import (  # noqa: F401
    AttnError, LIB_PATH, OUT_BF16, OUT_F32, V_FP8, V_MXFP4, EXPORTS, Workspace,
    bwd_fp8, decode_directp, decode_fp8pv, fwd_bf16, fwd_directp, fwd_directp_noalloc, fwd_directp_efq, fwd_directp_efq_mxqk, fwd_directp_mxqk, fwd_fp8pv, fwd_fp8pv_mxqk, fwd_fp8pv_cast, fwd_fp8pv_cast_mxqk, load_library, make_fwd_args, probe_issue_rates, quant_mxfp4, quant_nvfp4, quant_v, quant_v_cache, v_cols,
)
