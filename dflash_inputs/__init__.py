"""Seeded synthetic inputs for the DFlash drafter hot path.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It holds workload shapes and seeded random draws only: none of the
method's arithmetic (no fusion, projection, attention, norm or argmax) lives
here.  Every tensor is drawn from numpy's PCG64 seeded by
``SeedSequence([base_seed, config_id, tensor_id, chunk])`` so that any tensor
(or any 4M-element chunk of one) can be regenerated independently.
"""
from .configs import CONFIGS, Config, get_config, shrink
from .gen import Inputs, bf16_round_f32, build_target_logits_np, build_target_np

__all__ = ["CONFIGS", "Config", "get_config", "shrink", "Inputs",
           "bf16_round_f32", "build_target_logits_np", "build_target_np"]
