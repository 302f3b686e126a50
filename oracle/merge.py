"""Blocked softmax of one vector with the merge step of P3's worked example
("Softmax 的分块计算": [1,2,3,4] split into [1,2] and [3,4]).  Test
infrastructure only (see the package docstring).
"""

import math


def blocked_softmax(x, sizes):
    """Softmax of ``x`` computed block by block and merged.

    For each block: its local maximum, the local numerators exp(x_i - m_b)
    and their sum (the local denominator).  Then the global maximum M is the
    largest local maximum, each block's denominator is multiplied by the
    correction exp(m_b - M) and the corrected denominators are added; the
    softmax value of an element is its local numerator times its block's
    correction over the merged denominator.  This is P3's worked example
    (local maxima, local numerators and denominators, global maximum, the
    factor exp(2-4) for the first block) written for any split.

    Returns a dict with ``local_max``, ``local_num`` (lists per block),
    ``local_sum``, ``global_max``, ``correction``, ``merged_sum``,
    ``softmax`` (list) and ``lse`` (= M + ln merged_sum).
    """
    x = [float(t) for t in x]
    if sum(sizes) != len(x) or any(s <= 0 for s in sizes):
        raise ValueError("block sizes must be positive and cover x")
    blocks, at = [], 0
    for s in sizes:
        blocks.append(x[at:at + s])
        at += s
    local_max = [max(b) for b in blocks]
    local_num = [[math.exp(t - m) for t in b] for b, m in zip(blocks, local_max)]
    local_sum = [math.fsum(n) for n in local_num]
    gmax = max(local_max)
    corr = [math.exp(m - gmax) for m in local_max]
    merged = math.fsum(s * c for s, c in zip(local_sum, corr))
    soft = [n * c / merged for nums, c in zip(local_num, corr) for n in nums]
    return dict(local_max=local_max, local_num=local_num, local_sum=local_sum,
                global_max=gmax, correction=corr, merged_sum=merged,
                softmax=soft, lse=gmax + math.log(merged))
