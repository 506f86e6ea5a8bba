"""MI355X-native hybrid compressed attention (DeepSeek-V4 CSA + HCA).

The compute path is the HIP library ``libcsa.so`` (hand-written gfx950
kernels behind the C ABI in ``include/csa.h``); ``binding`` marshals torch
tensors into that ABI and nothing else.
"""
