"""CPU oracle for the NVFP4 W4A4 hot path.

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import it.  The GPU library never does.
"""
from .nvfp4_ref import (  # noqa: F401
    BLOCK, E2M1_MAGNITUDES, E4M3_TABLE, GIVEN, NVFP4, PER_ROW, PER_TENSOR,
    dequantize, dequantize_f32, e2m1_decode, e2m1_rne_sat, e4m3_decode, e4m3_rne_sat,
    fused_segments, fused_shared_scale, gemm, global_scale, nvfp4_bytes, pack_codes,
    quantize, unpack_codes,
)
