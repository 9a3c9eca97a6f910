"""w4mi: weight-only 4-bit dequantize-and-multiply, y = x . dequant(W)^T, on
AMD MI355X (gfx950).

The compute lives in libw4mi.so (hand-written HIP, C ABI in include/w4mi.h);
``binding`` marshals torch-ROCm tensors into it. ``synth`` draws the seeded
synthetic operands. Importing the package loads nothing; the first call into
``binding`` loads the library and fails if it has not been built.
"""
from .binding import (  # noqa: F401
    W4Error,
    qmm_affine4,
    qmm_id_q4_0,
    qmm_id_q4_0_scratch_bytes,
    qmm_lut4,
    qmv_affine4,
    w4_unpack_affine,
    w4_unpack_lut,
    w4_unpack_q4_0,
)
