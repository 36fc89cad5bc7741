"""Seeded synthetic workloads shared by the oracle and the GPU path (inputs only)."""
from .configs import (ModelConfig, SOFTMAX, LINEAR, WORKLOADS, SMALL_CASES, get,
                      tensor_names, tensor_shape, LAYER_TENSORS, hybrid_kinds)
from .generate import make_weights, make_tensor, make_prompt, weight_bytes

__all__ = ["ModelConfig", "SOFTMAX", "LINEAR", "WORKLOADS", "SMALL_CASES", "get",
           "tensor_names", "tensor_shape", "LAYER_TENSORS", "hybrid_kinds",
           "make_weights", "make_tensor", "make_prompt", "weight_bytes"]
