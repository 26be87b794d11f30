"""MI355X-native (gfx950) hot path of an AdaLN diffusion-transformer block.

The compute lives in `libdit.so` (hand-written HIP kernels behind a C ABI,
declared in include/dit.h).  `diffusion_transformer_amd.lib` is the thin
ctypes binding; nothing is loaded at package import, so `synth` (seeded
inputs) can be used without the library.
"""
