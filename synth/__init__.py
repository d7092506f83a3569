"""Seeded synthetic inputs for the HSTU layer.

This module is shared by the fp64 oracle's tests and by the HIP path's tests
and benchmark.  It holds input construction only (lengths, timestamps, random
tensors, bf16 input quantisation) and none of the layer's arithmetic: no
projection, bucketing, attention, normalisation or gating happens here.
"""
from .configs import CONFIGS, Config, get_config
from .gen import (AttnInputs, Inputs, LayerWeights, bf16_round, make_attn_inputs,
                  make_inputs, make_lengths, sub_batch)

__all__ = ["CONFIGS", "Config", "get_config", "Inputs", "LayerWeights",
           "bf16_round", "make_inputs", "make_lengths", "sub_batch", "AttnInputs",
           "make_attn_inputs"]
