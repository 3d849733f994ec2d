"""Cache-size arithmetic from the pages.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

* ThinK page, preliminaries on KV-cache optimisation: a batch of B prompts of
  S tokens on a model with L layers, N heads and head dimension D holds
  2 * B * S * L * N * D cache elements.
* ThinK page, magnitude-based pruning: T = floor((1 - lambda) D) channels kept.
"""

import math


def kv_cache_bytes(B, S, L, N, D, elem_bytes):
    return 2 * B * S * L * N * D * elem_bytes


def think_channels(D, lam):
    return int(math.floor((1.0 - lam) * D))


def think_total_fraction(D, lam):
    """Fraction of the full K+V cache left when only keys are pruned to T channels."""
    return (think_channels(D, lam) + D) / (2.0 * D)
