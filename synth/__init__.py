"""Seeded synthetic inputs for the DFlash drafter hot path.

This module is shared by the oracle-side tests, the GPU parity tests, the
bench and the smoke run. It holds the workload shapes and the random draws
only: none of the method's arithmetic (fusion, projection, attention,
verification) lives here.

Recipe (one per workload, all seeded):

* target hidden states: N(0, 1), one array per fused target layer;
* projection matrices, embedding and LM head: N(0, 0.02^2);
* RMSNorm gains: 1;
* anchor token: uniform over 0..V-2 (V-1 is the mask token);
* target logits for greedy verification: N(0, 1) per entry, then "planted"
  so that the target's argmax agrees with the drafted block for the first
  ``a`` positions and disagrees at position ``a`` (``plant_agreement``);
* agreement lengths: tau = min(G, block_size) with G ~ Geometric(0.25) on
  {1, 2, ...}, a = tau - 1;
* ragged context lengths for the batched workload: uniform integers in
  [512, 4096];
* candidate-selector tables (DFlash 2): hidden projection N(0, 1/D),
  predecessor and successor codes N(0, 0.3^2), rank 256.
* dynamic two-tap conv (DFlash 2): base kernel N(0, 0.5^2), projection
  N(0, 1/D), 16 channels per group, input rows N(0, 1) in fp32; the same
  draws for the two instances of every draft layer (make_conv_layers).

Floating-point draws are made in fp32 and rounded once to bf16 (round to
nearest even, torch's conversion) where the tensor is stored in bf16; the
same bf16 values are handed to both the GPU path and the oracle.
"""
from .configs import CONFIGS, DraftConfig, target_layer_ids_rule  # noqa: F401
from .gen import (  # noqa: F401
    make_weights,
    make_selector,
    make_conv,
    make_conv_layers,
    make_feats,
    make_anchor,
    make_target_logits,
    plant_agreement,
    planted_taus,
    ragged_lengths,
    seed_for,
)
