"""Seeded synthetic workloads (input infrastructure; no arithmetic of the method)."""
from .configs import CONFIGS, ORDER, GLOBAL, LOCAL, RETRIEVAL, DENSE, CLASS_NAMES  # noqa: F401
from .generate import Layout, make_layout, custom_layout, free_list, unit_values, seq_queries, score_values  # noqa: F401
