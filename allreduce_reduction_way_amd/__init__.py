"""MI355X-native share of a small-message bf16 allreduce (fp32 accumulate).

The compute path is the C-ABI library ``libar.so`` (hand-written HIP for
gfx950, declared in ``include/ar.h``); :mod:`allreduce_reduction_way_amd.ar`
is its thin ctypes binding.  PyTorch only allocates device memory and
supplies streams.  The binding loads the library on first use and raises if
it is not built: there is no CPU fallback.
"""
__all__ = ["ar", "inputs", "workloads"]
