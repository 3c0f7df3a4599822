"""Routing bookkeeping and packing.  TEST INFRASTRUCTURE ONLY (see package header).

[GEMM-modes] sec. 4.2-4.3: each (token t, slot r) with an expert id is one
assignment; assignments are grouped by expert into a packed buffer, keeping
token order within an expert; m_indices maps packed row -> expert and
output_index maps (t, r) -> packed row.  Sec. 4.6: with 128-row alignment each
expert's segment is its count rounded up to a multiple of 128 (empty experts
take no rows), segments follow in expert order, padding rows carry no data and
still carry their expert in m_indices; routes with a negative id are skipped.

[AsymGEMM] "Token Layout Protocols": the masked layout gives expert g the fixed
slice starting at g * max_m of a [G, max_m, K] buffer, with masked_m[g] valid
rows.

[CuTeDSL] (MoE dispatch): count the tokens per expert, give each token a unique
index within its expert, copy into (optionally padded) buffers.

Readings taken where the pages are silent:
  * order within an expert is the assignment order i = t*k + r (the page's
    worked example keeps token order; the atomic allocation it describes in
    sec. 4.6 is not used, so the layout is deterministic);
  * ids >= E are skipped and flagged (DEV_ID_RANGE); negative ids are skipped;
  * masked layout: an expert with more than max_m assignments keeps its first
    max_m (in assignment order); the rest get output_index -1 and DEV_CAPACITY;
  * counts[e] is the number of rows placed in expert e's segment (clipped to
    max_m for the masked layout);
  * m_indices rows past the packed total (contiguous) are -1; in the masked
    layout row r belongs to expert r // max_m.
"""

from __future__ import annotations

import numpy as np

DEV_ID_RANGE = 1 << 0
DEV_CAPACITY = 1 << 1

CONTIGUOUS = "contiguous"
MASKED = "masked"


def packed_rows_cap(T: int, k: int, E: int, align: int) -> int:
    """Upper bound on the contiguous packed rows, known before routing.

    Every assignment takes a row and each non-empty expert pads at most
    align-1 rows; at most min(E, T*k) experts are non-empty.
    """
    R = T * k
    cap = R + min(E, R) * (align - 1)
    return ((cap + align - 1) // align) * align


def route(topk_ids: np.ndarray, E: int, layout: str = CONTIGUOUS, align: int = 128,
          max_m: int = 0, rows_cap: int | None = None) -> dict:
    """Plain-loop routing over assignments in order i = t*k + r.

    Returns a dict with counts[E], seg_offsets[E+1] (segment starts; last entry is
    the packed total, or E*max_m for the masked layout), output_index[T, k],
    m_indices[rows_cap], m_packed and the status bits.

    Pinned by: the page's worked example (unaligned and 128-aligned) and
    invariants checked against an independent stable sort.
    """
    ids = np.asarray(topk_ids).astype(np.int64)
    T, k = ids.shape
    flat = ids.reshape(-1)
    status = 0

    # 1. count assignments per expert
    total = [0] * E
    for i in range(flat.size):
        e = int(flat[i])
        if e < 0:
            continue
        if e >= E:
            status |= DEV_ID_RANGE
            continue
        total[e] += 1

    # 2. segment starts
    starts = [0] * (E + 1)
    if layout == CONTIGUOUS:
        run = 0
        for e in range(E):
            starts[e] = run
            run += -(-total[e] // align) * align
        starts[E] = run
        m_packed = run
        if rows_cap is None:
            rows_cap = packed_rows_cap(T, k, E, align)
        counts = list(total)
    elif layout == MASKED:
        if max_m < 1:
            raise ValueError("masked layout needs max_m >= 1")
        for e in range(E + 1):
            starts[e] = e * max_m
        m_packed = E * max_m
        rows_cap = E * max_m if rows_cap is None else rows_cap
        counts = [min(c, max_m) for c in total]
        if any(c > max_m for c in total):
            status |= DEV_CAPACITY
    else:
        raise ValueError(layout)

    # 3. rank within expert (assignment order) -> packed row
    seen = [0] * E
    output_index = np.full(flat.size, -1, dtype=np.int32)
    for i in range(flat.size):
        e = int(flat[i])
        if e < 0 or e >= E:
            continue
        rho = seen[e]
        seen[e] += 1
        if layout == MASKED and rho >= max_m:
            continue
        output_index[i] = starts[e] + rho

    # 4. packed row -> expert
    m_indices = np.full(rows_cap, -1, dtype=np.int32)
    for e in range(E):
        hi = starts[e + 1]
        for r in range(starts[e], min(hi, rows_cap)):
            m_indices[r] = e

    return {
        "counts": np.array(counts, dtype=np.int32),
        "seg_offsets": np.array(starts, dtype=np.int32),
        "output_index": output_index.reshape(T, k),
        "m_indices": m_indices,
        "m_packed": m_packed,
        "rows_cap": rows_cap,
        "status": status,
    }


def pack_rows(payload: np.ndarray, output_index: np.ndarray, rows_cap: int, fill=None):
    """Copy token rows into packed rows: packed[output_index[t, r]] = payload[t].

    payload: [T, ...] any dtype.  Rows that no assignment targets keep ``fill``
    (default zeros); callers compare only rows named by output_index.
    """
    payload = np.asarray(payload)
    T, k = output_index.shape
    out = np.zeros((rows_cap,) + payload.shape[1:], dtype=payload.dtype)
    if fill is not None:
        out[...] = fill
    for t in range(T):
        for r in range(k):
            p = int(output_index[t, r])
            if p >= 0:
                out[p] = payload[t]
    return out
