"""Seeded synthetic inputs for the GNN-layer hot path.

This package only draws random graphs, feature matrices, weights and upstream
gradients.  It holds none of the layer's arithmetic: no normalisation, no
aggregation, no transform.  Both the CPU oracle and the HIP path take their
inputs from here, so the two never share anything else.
"""
from .graphs import *  # noqa: F401,F403
from .configs import CONFIGS, make_config  # noqa: F401
