"""Seeded synthetic inputs for the routed-expert MoE layer.

This package holds no arithmetic of the layer itself: it only draws inputs
(features, routing ids and weights, FP8 expert weights with their block
scales) with the shapes and distributions of the Kimi-K2 workloads. Both the
oracle side and the HIP side of a test receive the same arrays from here.
"""
from .configs import CONFIGS, Config, config_by_name
from .gen import (make_routing, make_x_bits, make_experts_host, make_experts_device,
                  make_shared_host, make_shared_device, experts_to_host, Workload, make_workload)

__all__ = ["CONFIGS", "Config", "config_by_name", "make_routing", "make_x_bits",
           "make_experts_host", "make_experts_device", "make_shared_host", "make_shared_device",
           "experts_to_host", "Workload", "make_workload"]
