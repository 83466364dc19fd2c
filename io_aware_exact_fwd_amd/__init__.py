"""MI355X-native tiled exact attention (FlashAttention forward and backward).

The compute path is the HIP library ``libfa_mi355x.so`` built from ``csrc/``;
this package only marshals arguments to its C ABI.
"""
