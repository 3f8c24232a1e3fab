"""Seeded synthetic GSI workloads (shapes in `configs`, inputs in `generate`).

Input generation only: nothing here projects, gates or multiplies by W. Both the HIP path's tests
and the oracle consume what this package produces; neither is imported here.
"""
from .configs import CONFIGS, Config, Site, SlowPlan, get  # noqa: F401
from .generate import (PLAN_MARGIN, SiteInputs, orthonormal_columns, planned_ratios, site_basis,  # noqa: F401
                       site_inputs, site_tokens, site_weight, store, token_steps)
