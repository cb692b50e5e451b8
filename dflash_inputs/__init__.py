"""Seeded synthetic inputs for the DFlash drafter hot path.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It holds workload shapes and seeded random draws only: none of the
method's arithmetic (no fusion, projection, attention, norm or argmax) lives
here.  Every tensor is drawn from numpy's PCG64 seeded by
``SeedSequence([base_seed, cid, tensor_id, chunk])`` (cid: the workload's id) so that any tensor
(or any 4M-element chunk of one) can be regenerated independently.
"""
from .configs import (BATCH16_RAGGED, DEEP8_B4_N8192, LONG_CTX_N32768, QWEN3_8B_N2048, TINY_F32, WORKLOADS, Config,
                      shrink)
from .gen import Inputs, bf16_round_f32, build_target_logits_np, build_target_np

__all__ = ["TINY_F32", "QWEN3_8B_N2048", "LONG_CTX_N32768", "BATCH16_RAGGED", "DEEP8_B4_N8192", "WORKLOADS",
           "Config", "shrink", "Inputs",
           "bf16_round_f32", "build_target_logits_np", "build_target_np"]
