"""Closed-form composed dense buffer (TEST INFRASTRUCTURE ONLY).

The compose moves bytes only, so what it reaches has a plain definition
(page d63fbd4, commit "current rows written straight into staging": prefix
pages come from the KV pool, all current pages from the staging, the result
is slot-dense with each request's prefix span abutting its current span; the
staging span is zeroed first, so the rows of a last current page past the
request's tokens stay zero; page 0d87bc5, commit "canonical prefix/current
slot spans": prefix span then current span per request).

For request r with P_r prefix pages, c_r current tokens and the page ids it
lists (prefix pages first, then current pages), dense row k_r + j, where
k_r is the number of dense rows of all earlier requests, holds

    pool row  page[j // PS] * PS + j % PS     for j <  PS * P_r
    current row  t_r + (j - PS * P_r)         for 0 <= j - PS * P_r < c_r
    zero bytes                                 up to the page boundary

with t_r the number of current rows of all earlier requests.  Rows are
opaque byte strings.  This module does not use the plan at all.
"""
import numpy as np


def dense(pool_rows, cur_rows, prefix_pages, cur_tokens, req_pages, page_size):
    """pool_rows: uint8 [n_pool_pages*PS, RB]; cur_rows: uint8 [T, RB].

    Returns the composed dense buffer, uint8 [S*PS, RB]."""
    PS = int(page_size)
    RB = pool_rows.shape[1]
    out = []
    page_cursor = 0   # position in req_pages (request-major)
    token_cursor = 0  # position in cur_rows
    for P, c in zip(prefix_pages, cur_tokens):
        P, c = int(P), int(c)
        C = -(-c // PS)
        for k in range(P):
            page = int(req_pages[page_cursor + k])
            out.append(pool_rows[page * PS:(page + 1) * PS])
        page_cursor += P + C
        if C:
            block = np.zeros((C * PS, RB), dtype=np.uint8)
            block[:c] = cur_rows[token_cursor:token_cursor + c]
            out.append(block)
        token_cursor += c
    if not out:
        return np.zeros((0, RB), dtype=np.uint8)
    return np.concatenate(out, axis=0)
