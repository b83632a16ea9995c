"""MI355X-native gated delta rule: chunkwise forward (WY / UT transform) and recurrent
decode, as hand-written HIP kernels for gfx950 behind a C ABI (include/gdn.h)."""
