"""Plain, slow CPU oracle for the NVFP4 block-scaled MoE layer.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute anything under ``oracle/``: only the tests, the smoke check in
``__graft_entry__.py`` and the ``cpu_baseline`` leg of ``bench.py`` use it.
The oracle shares no code, tables or helpers with the HIP library; the two
meet only through the seeded input generators, which hold none of the
method's arithmetic.

Everything floating point here is float64 (NumPy), except where the method
fixes a float32 step (the quantizer's scale and division steps), which is
emulated exactly with ``np.float32`` scalars/arrays.

Modules
  nvfp4  -- E2M1 / E4M3 code tables, unpacking, dequantize, quantize.
  mxfp4  -- the MXFP4 variant (group 32, UE8M0 scales): dequantize, quantize.
  mxfp8  -- block-scaled FP8 (MXFP8: E4M3 elements, UE8M0 per 32): dequantize,
            quantize.
  moe    -- router, permutation, grouped GEMM, SwiGLU, unpermute-reduce,
            FP8 activation round trip, the whole MoE layer (W4A16 / W4A4 /
            MXFP4).

Parity status of each function is stated in its docstring; every function
here is pinned by a ``-m "not gpu"`` test against something other than
itself (closed forms, an independent library cast, exact rational brute
force, invariants).
"""
from . import nvfp4, mxfp4, mxfp8, moe  # noqa: F401
