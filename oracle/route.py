"""Activation-format routing by timestep bucket.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: the Chameleon article, "the format is chosen by the value
distribution": calibration splits the sampling trajectory into ten intervals
and writes a table from which each layer reads its activation format for the
current stage; concatenated-feature convolutions (channel ranges up to 163x
apart) are forced to MXFP8.  "Plans should add calibration": at inference the
routing is a table read.

Readings: bucket = min(B - 1, floor(B * step / num_steps)) for step in
[0, num_steps); the table is row-major [layers][B] of format identifiers.
Filling the table (calibration) needs a trained model and captions and is
not part of this library.
"""

from __future__ import annotations


def bucket(step: int, num_steps: int, n_buckets: int = 10) -> int:
    if num_steps <= 0 or not 0 <= step < num_steps:
        raise ValueError("step must lie in [0, num_steps)")
    return min(n_buckets - 1, (n_buckets * step) // num_steps)


def act_format(table, n_buckets: int, layer: int, step: int, num_steps: int):
    return table[layer * n_buckets + bucket(step, num_steps, n_buckets)]
