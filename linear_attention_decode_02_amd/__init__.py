"""MI355X-native fused single-token KDA decode step.

``kda_decode`` (in ``linear_attention_decode_02_amd.kda``) is the Python
binding of the C-ABI library ``libkda_decode.so`` built from ``csrc/``;
``synth`` draws seeded synthetic inputs.  Submodules are imported on use so
that the input generator can be used without loading the HIP library.
"""
