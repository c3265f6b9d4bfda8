"""MI355X-native grouped top-k W4A16 MoE FFN (LFM2.5-24B-A2B expert shape).

The compute path is the C-ABI library ``libmoe_w4a16.so`` (HIP kernels for
gfx950); ``packed_bit_expert_amd.moe`` is its thin ctypes binding.  Importing
this package loads nothing; the binding loads the library on first use and
raises if it is missing.
"""
