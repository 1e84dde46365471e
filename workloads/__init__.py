"""Seeded synthetic inputs for the ForwardPass attention step.

This package only draws random numbers and lays out geometry (row offsets,
slots, positions, page tables, mask bitmaps, channel counts). It holds none
of the step's arithmetic: no RoPE, no attention, no fold or readout logic.
Both the CPU oracle and the GPU path consume the same arrays from here.
"""

from .gen import (  # noqa: F401
    FOLD_ALL,
    FOLD_CHANNEL,
    Pass,
    RunAhead,
    Workload,
    bf16_bits_from_f32,
    Lora,
    make_append_mix,
    make_config,
    make_empty_pass,
    make_explicit,
    make_window_decode,
    make_lora,
    make_random,
    make_run_ahead,
    split_pass,
    CONFIG_NAMES,
)
