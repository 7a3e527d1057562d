"""Block partition of the token sequence (oracle; test infrastructure only).

PARK's abstract speaks of query blocks and key blocks without fixing their
shape.  Reading used here: a block is a run of ``B`` consecutive tokens in
the (frame, height, width) raster order; query and key blocks share one
partition; the last block holds the ``N mod B`` leftover tokens when ``B``
does not divide ``N``.
"""


def num_blocks(n: int, b: int) -> int:
    return -(-n // b)


def block_bounds(j: int, n: int, b: int):
    """Token range ``[lo, hi)`` of block ``j``."""
    lo = j * b
    return lo, min(n, lo + b)
