"""CPU models of the 64-lane cross-lane primitives, lane by lane.

dpp_reduce() follows the DPP sequence the production kernels use, written
from the DPP pattern definitions: quad_perm [1,0,3,2] pairs lane i with
i ^ 1 and [2,3,0,1] with i ^ 2; row_half_mirror reverses each 8-lane half
row, row_mirror each 16-lane row; row_bcast:15 gives rows 1 and 3 the value of
lane 15 of the row before; row_bcast:31 gives rows 2 and 3 the value of lane
31. Lanes a masked step does not write receive the identity. The result is
lane 63. Because the pairing is fixed, a float64 sum through this model is
bit-identical to the GPU's.

shfl_down() is the simulator page's rule ("simt_lab.py", section 4,
Block.shfl_down): lane i takes lane i + offset's value, and keeps its own when
i + offset is past the wave.
"""

WAVE = 64


def _step(v, src, combine, identity, rows=None):
    out = []
    for i in range(WAVE):
        moved = identity if (rows is not None and i // 16 not in rows) else v[src(i)]
        out.append(combine(v[i], moved))
    return out


def dpp_reduce(values, combine, identity):
    v = list(values)
    assert len(v) == WAVE
    v = _step(v, lambda i: i ^ 1, combine, identity)
    v = _step(v, lambda i: i ^ 2, combine, identity)
    v = _step(v, lambda i: (i & ~7) | (7 - (i & 7)), combine, identity)
    v = _step(v, lambda i: (i & ~15) | (15 - (i & 15)), combine, identity)
    v = _step(v, lambda i: (i // 16 - 1) * 16 + 15, combine, identity, rows={1, 3})
    v = _step(v, lambda i: 31, combine, identity, rows={2, 3})
    return v[63]


def shfl_down(values, offset):
    v = list(values)
    return [v[i + offset] if i + offset < WAVE else v[i] for i in range(WAVE)]


def add(a, b):
    return a + b


def max_rule(a, b):
    """The running value a is replaced only by a strictly greater b."""
    return b if b > a else a
