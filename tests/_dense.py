"""Independent dense references used to pin the oracle (tests only).

Nothing here pages anything: it is textbook softmax attention on dense K/V
written with numpy/scipy library routines, plus a scatter of dense rows into a
page pool driven by the ledger's own placement.
"""
import numpy as np
from scipy.special import softmax

from oracle.ledger import PageAllocator, RequestPages


def dense_attention_rows(q, K, V, scale, visible):
    """q [R, D], K/V [N, D] float64; visible[r] = number of leading keys row r
    sees.  Returns [R, D] with zero rows where nothing is visible."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    out = np.zeros((q.shape[0], V.shape[1]))
    logits = (q @ K.T) * scale                     # [R, N]
    for r in range(q.shape[0]):
        n = int(visible[r])
        if n > 0:
            out[r] = softmax(logits[r, :n]) @ V[:n]
    return out


def scatter_with_ledger(rng, dense_k, dense_v, page_size, num_pages_extra, garbage,
                        appends=None):
    """Place per-request dense K/V [B][H_kv, n_b, D] into a page pool.

    Token placement comes from ``RequestPages(policy="fill_tail")`` appends (one
    cache per request, one shared pool); physical ids are then relabelled by a
    seeded permutation of the pool.  Returns (key_pages, value_pages,
    block_table, context_lens) with garbage in every unwritten slot.
    """
    B = len(dense_k)
    Hkv, D = dense_k[0].shape[0], dense_k[0].shape[2]
    pool = PageAllocator(page_size)
    caches = [RequestPages(pool, "fill_tail") for _ in range(B)]
    placements = [[] for _ in range(B)]
    # interleave requests' appends so their pages are not contiguous
    for b in range(B):
        n = dense_k[b].shape[1]
        chunks = appends[b] if appends is not None else _random_chunks(rng, n)
        assert sum(chunks) == n
        placements[b] = chunks
    pending = [list(c) for c in placements]
    for b in range(B):
        placements[b] = []
    while any(pending):
        for b in range(B):
            if pending[b]:
                placements[b].extend(caches[b].append(pending[b].pop(0)))
    used = pool.fresh_count
    num_pages = used + num_pages_extra
    relabel = rng.permutation(num_pages)
    kp = np.full((num_pages, Hkv, page_size, D), garbage, dtype=np.float64)
    vp = np.full((num_pages, Hkv, page_size, D), garbage, dtype=np.float64)
    max_pages = max(1, max(len(c.pages) for c in caches))
    bt = np.full((B, max_pages), -1, dtype=np.int32)
    for b in range(B):
        for t, (page, slot) in enumerate(placements[b]):
            kp[relabel[page], :, slot, :] = dense_k[b][:, t, :]
            vp[relabel[page], :, slot, :] = dense_v[b][:, t, :]
        row = caches[b].block_table_row(max_pages)
        bt[b] = [relabel[p] if p >= 0 else -1 for p in row]
    cl = np.array([c.context_len() for c in caches], dtype=np.int32)
    return kp, vp, bt, cl


def _random_chunks(rng, n):
    chunks = []
    while n > 0:
        c = int(rng.integers(1, min(n, 7) + 1))
        chunks.append(c)
        n -= c
    return chunks
