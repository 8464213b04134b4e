"""Benchmark of the union-path SwitchGLU-q4 MoE layer on one MI355X (filled in below)."""


def expert_bytes(H: int, I: int) -> int:
    """Bytes of one expert's gate, up and down matrices: 4-bit codes plus a bf16
    scale and a bf16 bias per group of 64 inputs (the size the mlx issue
    "gather_qmm at M=1 streams 4-bit expert weights..." counts per expert)."""
    per_matrix = H * I // 2 + (H * I // 64) * 2 * 2
    return 3 * per_matrix
