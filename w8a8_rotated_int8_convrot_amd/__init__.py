"""INT8 ConvRot linear layer for AMD MI355X (gfx950).

The layer rotates the bf16 activation along K with the orthogonal block
rotation baked into the tensorwise-int8 weight, quantizes it to int8 per
token, multiplies int8 x int8 into int32 on the MFMA units and dequantizes
with act_scale * weight_scale (+bias) to bf16.  All of it runs in the HIP
library ``libconvrot.so`` (C ABI in ``include/convrot.h``); the submodule
``binding`` marshals torch tensors into that ABI, ``synth`` draws the seeded
synthetic inputs and ``build`` compiles the library.  Submodules are imported
explicitly (``from w8a8_rotated_int8_convrot_amd import binding``).
"""
