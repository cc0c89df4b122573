"""MI355X-native verification stage of tree speculative sampling.

The compute path is the HIP library built from csrc/ (C ABI in
include/specverify.h); `speculative_decoding_tree_amd.lib` is the thin Python
binding over it. `synth` draws seeded synthetic inputs. Importing this package
loads nothing; the binding loads the library on first use and raises if it is
missing.
"""
__version__ = "0.1.0"
