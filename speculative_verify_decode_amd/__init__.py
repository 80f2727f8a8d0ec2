"""MI355X (gfx950) verify-decode layer step: HIP kernels behind a C ABI (libsdverify.so).

``speculative_verify_decode_amd.binding`` loads the library and exposes its entry points;
``speculative_verify_decode_amd.synth`` generates seeded synthetic inputs.
"""
