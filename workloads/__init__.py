"""Seeded synthetic decode workloads shared by the tests, the bench and the smoke check.

This package generates inputs only (shapes, lengths, page tables, random values); it holds no
part of the attention arithmetic, so both the HIP library and the CPU oracle can consume it.
"""
from .configs import CONFIGS, DecodeConfig, config, default_scale  # noqa: F401
from .generate import (Workload, make_workload, relabel_pages, subset_rows,  # noqa: F401
                       unshare_prefix, fill_normal, draw_lengths, rope_tables)
