"""Seeded synthetic inputs shared by the tests, the bench and the oracle.

This package holds workload shapes and input generators only (token ids,
lengths, labels, candidate lists).  It contains none of the method's
arithmetic: no forward pass, no estimator, no update and no random-direction
stream.
"""
from .configs import CONFIGS, ModelCfg, Workload, get
from .inputs import Batch, make_batch

__all__ = ["CONFIGS", "ModelCfg", "Workload", "get", "Batch", "make_batch"]
