"""Seeded synthetic inputs for the activation-sparse gated FFN workloads.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the FFN's arithmetic, so the CPU oracle and the HIP path can
both take their inputs from here without sharing any of the method's code.
"""
from .inputs import CONFIGS, Workload, make_inputs, config_summary

__all__ = ["CONFIGS", "Workload", "make_inputs", "config_summary"]
