"""MoE layer benchmark on one MI355X (filled in with the HIP path)."""


def layer_flops(slots: int, hidden: int, inter: int) -> int:
    """Useful FLOPs of the expert FFN for ``slots`` routed token slots:
    gate+up is a [slots,H]x[H,2I] GEMM (2*H*2I flops per slot) and down a
    [slots,I]x[I,H] GEMM (2*I*H per slot): 6*H*I per slot."""
    return 6 * slots * hidden * inter
