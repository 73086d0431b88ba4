"""MI355X-native TQ2_0 ternary decode matvec.

The C ABI (include/tq2.h) lives in libtq2.so, built from csrc/ by build.py;
`ternary_packed_weight_amd.tq2` is its ctypes binding (import it explicitly;
it loads the GPU library).  `ternary_packed_weight_amd.synth` holds the
seeded synthetic inputs and loads nothing.
"""
