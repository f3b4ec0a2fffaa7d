"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

Holds the workload configurations and the generators of synth_recipe.md:
expert blobs, activations, router matrices (host C and device HIP twins) and
Zipf-routed logits (numpy).  None of the MoE layer's arithmetic lives here.
"""
from .configs import CONFIGS, Config, config_by_name  # noqa: F401
from .gen import (HostGen, DevGen, zipf_logits, zipf_popularity, build_libs,  # noqa: F401
                  host_lib_path, dev_lib_path)
