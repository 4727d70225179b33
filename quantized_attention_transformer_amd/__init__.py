"""SageAttention 8-bit attention forward for MI355X (gfx950).

The compute lives in the HIP library ``libsage.so`` built from ``csrc/``;
``quantized_attention_transformer_amd.sage`` is its thin Python binding.
Importing the package does not load the library.
"""
