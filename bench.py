"""Benchmark of the W4A16 decode path (placeholder: the full benchmark follows)."""


def gbps(nbytes: float, seconds: float) -> float:
    """Effective bandwidth in GB/s (GB = 1e9 B): bytes moved / time."""
    return nbytes / seconds / 1e9
