"""MI355X-native sparse mixture-of-experts FFN layer forward.

The compute path is the C-ABI library ``libmoe.so`` (hand-written HIP for
gfx950); ``binding`` marshals torch tensors into it.
"""
