"""MI355X-native 2-bit routed-MoE block (ds4 / DeepSeek-V4-Flash shapes).

The compute lives in ``libds4moe.so`` (hand-written HIP kernels for gfx950
behind a C ABI, declared in ``include/ds4moe.h``).  This package is a thin
ctypes binding: it marshals torch device tensors and streams into that ABI.
"""
