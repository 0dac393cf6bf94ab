"""Seeded synthetic workloads shaped like the pages' settings (shapes and
input generators only; no arithmetic of the method)."""
from .configs import C0, C1, C2, C3, C4, CONFIGS, FocalDecode, WindowSelect, BudgetDecode, budget, small
