"""INT8 ConvRot linear layer for AMD MI355X (gfx950).

The layer rotates the bf16 activation along K with the orthogonal block
rotation baked into the tensorwise-int8 weight, quantizes it to int8 per
token, multiplies int8 x int8 into int32 on the MFMA units and dequantizes
with act_scale * weight_scale (+bias) to bf16.  All of it runs in the HIP
library ``libconvrot.so`` (C ABI in ``include/convrot.h``); ``binding``
marshals torch tensors into that ABI.  The binding is imported lazily so
that ``synth`` (the seeded input generator) loads without the library.
"""

__all__ = ["binding", "synth"]


def __getattr__(name):
    if name == "binding":
        from . import binding
        return binding
    raise AttributeError(name)
