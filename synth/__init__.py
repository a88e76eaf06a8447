"""Seeded synthetic inputs for the LSA layer (keys, values, queries, projection).

This package builds input tensors only.  It holds no step of the attention
method itself, so both the CPU oracle and the HIP path can consume what it
makes without sharing any of the method's arithmetic.
"""

from .topics import WORKLOADS, LayerConfig, get_config, layer_inputs, decode_inputs, random_lr_lists

__all__ = ["WORKLOADS", "LayerConfig", "get_config", "layer_inputs", "decode_inputs", "random_lr_lists"]
