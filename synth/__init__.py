"""Seeded synthetic inputs for LB-ADMM layers and calibration activations.

This package draws random numbers only. It holds none of the method's
arithmetic (no preconditioning, no init scale, no ADMM step), so the CPU
oracle and the HIP path can both take their inputs from it without sharing
any computation.
"""
from .activations import CALIB_TOKENS, make_activations
from .layers import WORKLOADS, Workload, LayerInputs, make_layer, make_tiny

__all__ = ["WORKLOADS", "Workload", "LayerInputs", "make_layer", "make_tiny",
           "CALIB_TOKENS", "make_activations"]
