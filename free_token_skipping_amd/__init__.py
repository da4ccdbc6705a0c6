"""SPTS prefill hot path on AMD Instinct MI355X (gfx950).

libspts.so (HIP kernels behind the C ABI of include/spts.h) does all the
computation; `capi` is its thin ctypes binding and `pipeline` strings the
calls together into one SPTS layer and the MSDP stack.  PyTorch supplies
device memory and streams only.
"""
