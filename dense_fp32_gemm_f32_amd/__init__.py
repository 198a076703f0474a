"""MI355X (gfx950) dense row-major fp32 GEMM: C = A x B with fp32 accumulation.

The product path is the HIP shared library ``libgemm_f32.so`` built from
``csrc/`` and reached through the C ABI declared in ``include/gemm_f32.h``;
``binding`` marshals torch tensors into it.  Nothing here falls back to a CPU
or PyTorch computation: if the library is missing, the binding raises.
"""
__all__ = ["binding", "inputs"]
