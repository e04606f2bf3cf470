"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This package draws random numbers and rounds them to a storage dtype. It holds
none of the selective-scan arithmetic: neither the oracle nor the HIP library
imports anything else from the other, and this is the one module both sides'
callers share.
"""
from .inputs import (  # noqa: F401
    CONFIGS,
    BackboneConfig,
    LayerConfig,
    RecurrenceConfig,
    ScanConfig,
    backbone_inputs,
    layer_inputs,
    recurrence_inputs,
    round_bf16,
    round_storage,
    scan_inputs,
)
