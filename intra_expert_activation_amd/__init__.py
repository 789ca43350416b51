"""MI355X-native routed-MoE SwiGLU expert FFN with intra-expert activation sparsity.

The compute path is the C-ABI library ``libmoesparse.so`` (hand-written HIP for
gfx950); ``intra_expert_activation_amd.moe`` is its thin ctypes binding.  The
library is loaded on first use and an ImportError-free import of this package
never falls back to anything else: every call raises if the library is missing.
"""
