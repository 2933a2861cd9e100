"""Seeded synthetic inputs for the KDA recurrent-state path.

This package only draws random inputs (Gaussian vectors, gates, initial
states, acceptance counts) and rounds them to their storage types.  It holds
none of the recurrence's arithmetic; both the fp64 oracle (``oracle/``) and
the HIP path consume exactly what it produces.
"""

from .kda_inputs import (  # noqa: F401
    CONFIGS,
    ConfigSpec,
    accepted_counts,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    initial_state,
    raw_token_inputs,
    token_inputs,
)
