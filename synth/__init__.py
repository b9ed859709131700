"""Seeded synthetic inputs shared by the CPU oracle and the HIP library's tests and benchmark."""
from .workloads import WORKLOADS, ORDER, Workload  # noqa: F401
from .gen import generate, redraw_q_token, to_bf16_bits, bf16_to_f32, tree_masks, tree_parents  # noqa: F401
