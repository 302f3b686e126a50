"""Tile bookkeeping of the block algorithm: which (query-block, key-block)
pairs a launch computes, skips or masks, the P1 §2.2 glyph figure, and the
P1 §2.1 HBM traffic model.  Integer arithmetic only.  Test infrastructure
only (see the package docstring); page tags are defined there.
"""


def _ceil_div(a, b):
    return -(-a // b)


def _check_pos(**kw):
    for name, val in kw.items():
        if val <= 0:
            raise ValueError(f"{name} must be positive, got {val}")


def _tile_class(q0, q1, k0, k1, block_k, causal):
    """Class of the tile covering query rows [q0, q1] and key rows [k0, k1]
    (inclusive).  A tile whose first key lies after its last query is never
    touched under a causal mask (P1 §2.2, fully-above-diagonal blocks are
    skipped); a computed tile that reaches past the diagonal needs the element
    mask on chip (P1 §2.2, blocks crossing the diagonal); a computed tile
    shorter than the block is the ragged tail (P2 Q2 counts tiles with a
    ceiling, so the last one can be partial).  Precedence: causal-masked, then
    ragged, then full."""
    if causal and k0 > q1:
        return "skipped"
    if causal and k1 > q0:
        return "causal_masked"
    if k1 - k0 + 1 < block_k:
        return "ragged"
    return "full"


def block_counts(N, block_q, block_k, causal):
    """Counts of computed / full / causal_masked / ragged / skipped tiles for
    one head of length N (query and key lengths equal).  ``computed`` is the
    sum of full, causal_masked and ragged; ``computed + skipped`` is the number
    of tile pairs ceil(N/block_q) * ceil(N/block_k).  Multiply by B*H for a
    launch."""
    _check_pos(N=N, block_q=block_q, block_k=block_k)
    counts = dict(computed=0, full=0, causal_masked=0, ragged=0, skipped=0)
    for i in range(_ceil_div(N, block_q)):
        q0, q1 = i * block_q, min((i + 1) * block_q, N) - 1
        for j in range(_ceil_div(N, block_k)):
            k0, k1 = j * block_k, min((j + 1) * block_k, N) - 1
            c = _tile_class(q0, q1, k0, k1, block_k, causal)
            counts[c] += 1
            if c != "skipped":
                counts["computed"] += 1
    return counts


def block_pattern(N, block_q, block_k, causal):
    """Boolean matrix ``[query block][key block]``: True where the tile is
    computed (not skipped)."""
    _check_pos(N=N, block_q=block_q, block_k=block_k)
    out = []
    for i in range(_ceil_div(N, block_q)):
        q0, q1 = i * block_q, min((i + 1) * block_q, N) - 1
        row = []
        for j in range(_ceil_div(N, block_k)):
            k0, k1 = j * block_k, min((j + 1) * block_k, N) - 1
            row.append(_tile_class(q0, q1, k0, k1, block_k, causal) != "skipped")
        out.append(row)
    return out


def causal_figure(N, block):
    """The P1 §2.2 glyph grid (N=8, B=2 on the page) rebuilt from the causal
    block pattern.  The page prints one line per block pair and one glyph per
    single index; read with lines = key blocks and glyph columns = query
    indices, glyph (r, c) is filled iff key block r is computed for the query
    block holding query c.  (Read the other way -- lines as query blocks --
    the printed grid would be the upper triangle and let query 0 see key 7,
    which the page's own text on the lower-triangular mask rules out.)

    Returns a list of strings, '■' computed and '□' skipped."""
    pat = block_pattern(N, block, block, True)         # [q block][k block]
    lines = []
    for r in range(_ceil_div(N, block)):               # key block
        lines.append("".join("■" if pat[c // block][r] else "□"
                             for c in range(N)))
    return lines


def traffic(N, d, block_q, block_k, elem_bytes, causal=False, mode="tiled"):
    """Bytes moved between HBM and the chip for one head under the pages'
    cacheless model (P1 §2.1 table; P3, six transfers vs. two).

    mode "standard": Q, K, V read once; S written then read back; P written
    then read back; O written (the page lists S and P as read-and-write rows).
    mode "tiled": each query block read once; each computed tile reads its K
    block and V block; each output block written once; S and P stay on chip.

    Returns a dict with per-operand reads/writes, their totals, and the LSE
    bytes (4 per row, fp32) on a line of their own, since the page's table has
    no row for the saved statistics."""
    _check_pos(N=N, d=d, block_q=block_q, block_k=block_k, elem_bytes=elem_bytes)
    e = elem_bytes
    row = d * e
    rd, wr = {}, {}
    if mode == "standard":
        rd = dict(Q=N * row, K=N * row, V=N * row, S=N * N * e, P=N * N * e, O=0)
        wr = dict(Q=0, K=0, V=0, S=N * N * e, P=N * N * e, O=N * row)
    elif mode == "tiled":
        kr = 0
        for i in range(_ceil_div(N, block_q)):
            q0, q1 = i * block_q, min((i + 1) * block_q, N) - 1
            for j in range(_ceil_div(N, block_k)):
                k0, k1 = j * block_k, min((j + 1) * block_k, N) - 1
                if _tile_class(q0, q1, k0, k1, block_k, causal) != "skipped":
                    kr += (k1 - k0 + 1) * row
        rd = dict(Q=N * row, K=kr, V=kr, S=0, P=0, O=0)
        wr = dict(Q=0, K=0, V=0, S=0, P=0, O=N * row)
    else:
        raise ValueError(f"unknown mode {mode!r}")
    return dict(reads=rd, writes=wr, read_total=sum(rd.values()),
                write_total=sum(wr.values()), lse_write=4 * N)
