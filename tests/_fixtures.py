"""Test-side helpers: golden-file parsing and input construction.

Packing an integer matrix into words is how a test *builds* an input from a
rule; the golden hand cases fix the nibble order independently of it.
"""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_cases(fname):
    cases, cur = [], None
    with open(os.path.join(GOLDEN, fname)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(" ")
            if key == "case":
                cur = {"name": rest, "src": [], "dst": []}
            elif key == "end":
                cases.append(cur)
                cur = None
            elif key in ("src", "dst"):
                cur[key].append([int(w, 16) for w in rest.split()])
            else:
                cur[key] = rest
    return cases


def words(hexlist):
    return np.array([int(w, 16) for w in hexlist.split()], dtype=np.uint32).view(np.int32)


def pack_rows(q):
    """int matrix [R, C] with entries 0..15 -> int32 [R, C/8], nibble j = column 8w+j."""
    q = np.asarray(q, dtype=np.uint32)
    R, C = q.shape
    assert C % 8 == 0
    out = np.zeros((R, C // 8), dtype=np.uint32)
    for j in range(8):
        out |= (q[:, j::8] & 0xF) << np.uint32(4 * j)
    return out.view(np.int32)


def unpack_rows(w):
    """Inverse of pack_rows."""
    w = np.asarray(w).view(np.uint32)
    R, C8 = w.shape
    q = np.zeros((R, C8 * 8), dtype=np.int64)
    for j in range(8):
        q[:, j::8] = (w >> np.uint32(4 * j)) & 0xF
    return q



def oracle_gemm_columns(a, b_kn8, scales, qzeros, G, zp_bias=8):
    """The oracle's full product over column slices on the host's cores
    (identical to one oracle.gemm call)."""
    import oracle
    return oracle.gemm_columns(a, b_kn8, scales, qzeros, G, zp_bias)
