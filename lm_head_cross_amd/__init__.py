"""MI355X (gfx950) flash-CCE ORPO head: HIP kernels behind a C ABI, with a thin Python binding.

`lm_head_cross_amd.head` holds the binding (fwd / loss / bwd); `lm_head_cross_amd.synth` draws
seeded synthetic inputs. Importing the package does not load the shared library.
"""
