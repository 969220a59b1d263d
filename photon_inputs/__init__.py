"""Seeded synthetic inputs shared by the CPU oracle and the HIP path.

This module holds shapes and random numbers only: the five model/workload
configurations, the seeded weight generator, the seeded prompt generator and a
seeded stand-in for a decode state (cached keys and values, the last top
output) that tests inject into both sides.
It holds none of the method's arithmetic, so both the oracle and the GPU
binding may import it without sharing any computation.

Model shape: PHOTON paper record (ACL 2026 long paper, "PHOTON: Hierarchical
Autoregressive Modeling for Lightspeed and Memory-Efficient Language
Generation"), abstract; PHOTON explainer (mokumoku.ipfde.com, Fujitsu PHOTON
vertical scan), module table and the hierarchy-shape paragraph under it
(L = 2 levels, C1 = C2 = 4 main setting, C1 = C2 = 2 quality setting).
"""
from .configs import PhotonConfig, VanillaConfig, vanilla_of, Workload, CONFIGS, WORKLOADS, get
from .gen import (weight_names, weight_shapes, gen_weights, gen_prompts, gen_decode_state,
                  bf16_bits, MATRIX_STD)

__all__ = ["PhotonConfig", "VanillaConfig", "vanilla_of", "Workload", "CONFIGS", "WORKLOADS", "get",
           "weight_names", "weight_shapes", "gen_weights", "gen_prompts", "gen_decode_state",
           "bf16_bits", "MATRIX_STD"]
