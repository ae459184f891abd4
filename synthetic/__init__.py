"""Seeded synthetic inputs for the activation-sparse FFN step.

This package produces weights, biases, tokens and per-layer thresholds with the
structure the PowerInfer and KAIROX pages measure (power-law activation, temporal
locality of successive tokens, co-activated groups of 32 neurons).  It holds none
of the step's own arithmetic: no predictor, no gate, no sparse product, no TAM.
Both the HIP path and the fp64 oracle consume what it produces.
"""
from .configs import CONFIGS, FFNConfig, scaled  # noqa: F401
from .gen import (LAYER_COS, Layer, make_layer, make_layer_chain, make_tokens, seed_for,  # noqa: F401
                  storage_numpy, threshold_for, threshold_for_share, layer_threshold, zipf_profile,
                  quantize_q4)
