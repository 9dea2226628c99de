"""MI355X-native VeriCache draft/verify attention path.

``vc`` is the thin binding over the HIP library ``libvc.so`` (C ABI in include/vc.h);
``synth`` draws the seeded synthetic inputs; ``harness`` drives whole rounds on the GPU.
"""
