"""MI355X-native DSpark draft / schedule / verify hot path.

The compute path is the HIP library ``libdspark.so`` (C ABI declared in ``include/dspark.h``);
``draft_head_verification_amd.dspark`` is its thin ctypes binding.  ``synth`` draws the seeded
synthetic workloads used by the tests and the benchmark.
"""
