"""Seeded synthetic inputs shared by the CPU oracle's tests and the GPU path."""
from .synthetic import (WORKLOADS, Workload, bf16_bits_to_f32, custom_workload, f32_to_bf16_bits,
                        make_w, make_x, outlier_channels, to_f32, to_torch, workload)

__all__ = ["WORKLOADS", "Workload", "bf16_bits_to_f32", "custom_workload", "f32_to_bf16_bits",
           "make_w", "make_x", "outlier_channels", "to_f32", "to_torch", "workload"]
