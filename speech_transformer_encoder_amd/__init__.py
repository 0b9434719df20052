"""MI355X-native forward pass of the Whisper-style pre-LN encoder block (gfx950 HIP kernels).

The compute lives in ``libwhisper_enc.so`` (built from ``csrc/``) behind a C ABI declared in
``include/whisper_enc.h``; ``binding`` exposes the same entry points to Python with argument
marshalling only.  ``synth`` draws the seeded synthetic workloads.
"""
