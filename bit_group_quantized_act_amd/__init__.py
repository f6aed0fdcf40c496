"""MI355X-native W4A8 linear layer: 4-bit group-quantized weights x int8 group-quantized
activations, as hand-written HIP kernels for gfx950 behind a small C ABI (``libw4a8.so``).

``synth`` holds the seeded input generators.  The binding to the C ABI is added beside it.
"""
