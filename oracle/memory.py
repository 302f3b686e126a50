"""The pages' analytic memory model: score-matrix size, tile counts, score
tile and working-set bytes, materialisation ratio (P2 Q1-Q3), and the on-chip
budget rows (P1 §1.2).  Written from the formulas the pages state; sizes that
are not positive raise ValueError, the convention P2 uses throughout.  Test
infrastructure only (see the package docstring).
"""


def _positive(*vals):
    if any(v <= 0 for v in vals):
        raise ValueError("sizes must be positive")


def score_bytes(seq_len, batch=1, heads=1, dtype_bytes=2):
    """Bytes of a materialised score tensor: batch * heads * N^2 * bytes
    (P2 Q1; a capacity figure, not measured traffic)."""
    _positive(seq_len, batch, heads, dtype_bytes)
    return batch * heads * seq_len * seq_len * dtype_bytes


def tiles_1d(seq_len, tile):
    """Tiles along one sequence axis, ceil(N / tile) (P2 Q2)."""
    _positive(seq_len, tile)
    return -(-seq_len // tile)


def score_tiles(seq_len, tile):
    """Query-tile x key-tile pairs, tiles_1d squared (P2 Q2)."""
    return tiles_1d(seq_len, tile) ** 2


def score_tile_bytes(tile, dtype_bytes=2):
    """Bytes of one tile x tile score block (P2 Q2)."""
    _positive(tile, dtype_bytes)
    return tile * tile * dtype_bytes


def working_set_bytes(tile, head_dim, dtype_bytes=2):
    """P2 Q2's teaching working set: Q, K, V blocks (3 t d), one score block
    (t^2) and one output block (t d), times the element size.  The row
    statistics are not part of this model."""
    _positive(tile, head_dim, dtype_bytes)
    return (4 * tile * head_dim + tile * tile) * dtype_bytes


def tile_tradeoff(seq_len, tile, head_dim=128, dtype_bytes=2):
    """Tile pair count, score tile bytes and working set for one tile size
    (P2 Q3)."""
    return dict(tile_count=score_tiles(seq_len, tile),
                score_tile_bytes=score_tile_bytes(tile, dtype_bytes),
                working_set_bytes=working_set_bytes(tile, head_dim, dtype_bytes))


def materialization_ratio(seq_len, tile, dtype_bytes=2):
    """Full score matrix over one score tile, N^2 / t^2 (P2 Q3)."""
    _positive(seq_len, tile, dtype_bytes)
    return score_bytes(seq_len, dtype_bytes=dtype_bytes) / score_tile_bytes(tile, dtype_bytes)


def sram_budget(block_q, block_k, d, elem_bytes=2):
    """On-chip budget rows of P1 §1.2: the Q, K, V, S and O blocks at
    ``elem_bytes`` each, and the row statistics at 8 bytes per query row (two
    fp32 numbers: running max and running sum).  Returns a dict of rows and
    their total in bytes."""
    _positive(block_q, block_k, d, elem_bytes)
    rows = dict(Q_block=block_q * d * elem_bytes,
                K_block=block_k * d * elem_bytes,
                V_block=block_k * d * elem_bytes,
                S_block=block_q * block_k * elem_bytes,
                O_block=block_q * d * elem_bytes,
                stats=block_q * 8)
    rows["total"] = sum(rows.values())
    return rows


def sram_formula_as_printed(B, d):
    """The closed form the P1 §1.2 table prints on its total line, taken at
    face value as 2*(2*B*d + B^2) bytes.  Kept only so a test can show it does
    not match the table's own rows (the printed total is garbled)."""
    return 2 * (2 * B * d + B * B)
