"""MLA chunked prefill and absorbed decode for AMD Instinct MI355X (gfx950).

The computation lives in libmla.so (hand-written HIP kernels behind the C ABI of
include/mla.h); `binding` marshals torch tensors into its calls.
"""
