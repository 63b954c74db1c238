"""Seeded synthetic workloads shared by the tests, the bench and the oracle checks."""
from .configs import WORKLOADS, BY_ID, layout_counts, n_tokens, shrink
from .gen import adaptive_inputs, joint_inputs, normal_tensors, sparse_inputs, upstream_grad
