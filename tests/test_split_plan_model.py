"""Host model of the bf16 prefill's key-split planner (the integer rules every
workgroup of the kernel applies to the context lengths): over random shapes
and slot counts, the pieces of each (request, tile) pair cover its keys
exactly, split pieces use fewer than 0.8 of the workspace slots, the grid
(one workgroup per pair and kv head plus half the slots) has a workgroup for
every piece, and the longest-first dispatch order hands every piece to
exactly one workgroup.  Constants are read from the kernel source."""
import math
import os
import re

import numpy as np

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "paged_kv_cache_96_amd", "csrc", "pa_prefill.hip")


def _constants():
    text = open(SRC).read()
    bn = int(re.search(r"constexpr int kBN = (\d+);", text).group(1))
    mult = int(re.search(r"constexpr int kMinPieceKeys = (\d+) \* kBN;", text).group(1))
    return bn, mult * bn


BN, MIN_PIECE = _constants()


def plan(ctx, qlen, G, Hkv, causal, S, packed=False, L=None):
    """Pieces of one call: list of (workgroup order key, pair, head, piece,
    k0, k1, split) and the grid size.  With packed rows a tile with no row
    to write is a pair of the fifth class (ordered after all others); L
    bounds the rows of a request (default: the longest)."""
    nt = -(-(G * (L or max(qlen))) // 128) if qlen else 0
    keys, empty = [], []
    for b in range(len(ctx)):
        for tr in range(nt):
            t = nt - 1 - tr
            rho0, last = t * 128, min(t * 128 + 128, G * qlen[b]) - 1
            keys.append(0 if last < rho0 else (ctx[b] - qlen[b] + last // G + 1 if causal else ctx[b]))
            empty.append(packed and last < rho0)
    work = np.float32(sum(-(-k // BN) for k in keys)) * np.float32(Hkv)
    target = np.float32(0.4) * np.float32(max(2, S))
    blocks = min(math.ceil(float(np.float32(work / target))), 1 << 24)
    P = max(MIN_PIECE, blocks * BN)
    pieces, slots = [], 0
    for q, k in enumerate(keys):
        ln = k
        if k > P:
            n0 = -(-k // P)
            ln = (-(-k // n0) + BN - 1) // BN * BN
        n = -(-k // ln) if k > ln else 1
        cls = 0 if 4 * ln >= 3 * P else 1 if 2 * ln >= P else 2 if 4 * ln >= P else 3
        if empty[q]:
            cls = 4
        for g in range(Hkv):
            for sp in range(n):
                pieces.append(((cls, q, g, sp), q, g, sp, sp * ln, min(k, sp * ln + ln), n > 1))
        if n > 1:
            slots += Hkv * n
    grid = len(keys) * Hkv + max(1, S // 2)
    return keys, P, pieces, slots, grid


def _shapes(seed):
    r = np.random.default_rng(seed)
    B = int(r.integers(1, 40))
    G = int(r.integers(1, 9))
    Hkv = int(r.choice([1, 2, 4, 8]))
    L = int(r.choice([1, 16, 100, 512, 2048]))
    qlen = [int(v) for v in r.integers(0, L + 1, B)] if r.random() < 0.3 else [L] * B
    ctx = [q + int(r.integers(0, 40000 if r.random() < 0.3 else 3000)) for q in qlen]
    S = int(r.choice([2, 3, 5, 10, 64, 5 * 256, 5 * 304, 2048]))
    return ctx, qlen, G, Hkv, bool(r.random() < 0.8), S


def test_split_plan_bounds_and_coverage():
    checked = 0
    for seed in range(300):
        ctx, qlen, G, Hkv, causal, S = _shapes(seed)
        if len(ctx) * -(-(G * max(qlen)) // 128) > 2048:
            continue  # more pairs than the split plans over: the call runs unsplit
        _check(ctx, qlen, G, Hkv, causal, S)
        checked += 1
    assert checked > 200


def _check(ctx, qlen, G, Hkv, causal, S):
    keys, P, pieces, slots, grid = plan(ctx, qlen, G, Hkv, causal, S)
    assert P % BN == 0 and P >= MIN_PIECE
    assert slots <= 0.8 * S + 1e-6 * S, (slots, S)
    assert len(pieces) <= grid, (len(pieces), grid)
    # every pair and head: pieces tile [0, k) in order, interior bounds on the BN grid
    by = {}
    for _, q, g, sp, k0, k1, _ in pieces:
        by.setdefault((q, g), []).append((sp, k0, k1))
    for (q, g), ps in by.items():
        ps.sort()
        assert ps[0][1] == 0 and ps[-1][2] == keys[q]
        for (_, a0, a1), (_, b0, _) in zip(ps, ps[1:]):
            assert a1 == b0 and a1 % BN == 0 and a1 > a0
    # dispatch order: workgroup i takes the i-th piece of the class-major,
    # pair-ordered list; the rest of the grid finds no piece
    order = sorted(pieces, key=lambda x: x[0])
    assert len({x[0] for x in order}) == len(order)


def test_c3_and_c5_like_plans_split_the_long_tiles():
    # four 512-row chunks after prefixes up to 2048 (G 7, 4 kv heads), 5 slots per CU
    keys, P, pieces, slots, grid = plan([1662 + 512, 512, 900 + 512, 40 + 512], [512] * 4, 7, 4,
                                        True, 5 * 256)
    assert any(k > P for k in keys) and 0 < slots <= 0.8 * 1280
    # one long prompt of 16384 rows: no tile is longer than P, nothing splits
    keys, P, pieces, slots, grid = plan([16384], [16384], 7, 4, True, 5 * 256)
    assert max(keys) <= P and slots == 0 and len(pieces) == len(keys) * 4


def test_packed_grid_bound_covers_every_piece_with_rows():
    """Packed rows of known total T: the grid of floor(G T / 128) + (requests
    with rows) pairs per kv head plus half the slots (ragged prefill part:
    requests of two rows or more) still reaches every piece that has rows,
    because the pairs without rows are dispatched last."""
    r = np.random.default_rng(7)
    checked = 0
    for _ in range(400):
        B = int(r.integers(1, 64))
        G = int(r.integers(1, 9))
        Hkv = int(r.choice([1, 2, 4, 8]))
        L = int(r.choice([2, 16, 100, 256, 600]))
        ragged = r.random() < 0.5
        # a ragged call's prefill part sees the one-row requests as rowless
        qlen = [int(v) for v in r.integers(0, L + 1, B)]
        if ragged:
            qlen = [q if q >= 2 else 0 for q in qlen]
        ctx = [q + int(r.integers(0, 5000)) for q in qlen]
        S = int(r.choice([2, 10, 64, 5 * 256]))
        nt = -(-(G * L) // 128)
        if B * nt > 2048 or not any(qlen):
            continue
        keys, P, pieces, slots, grid = plan(ctx, qlen, G, Hkv, True, S, packed=True, L=L)
        T = sum(qlen) + (sum(1 for q in qlen if q == 0) if ragged else 0)  # one-row requests
        with_rows = min(B, T // 2 if ragged else T)
        pairs = min(B * nt, G * T // 128 + with_rows)
        bound = pairs * Hkv + max(1, S // 2)
        order = sorted(pieces, key=lambda x: x[0])
        with_work = [i for i, x in enumerate(order) if x[0][0] < 4]
        assert not with_work or with_work[-1] < bound, (with_work[-1], bound)
        checked += 1
    assert checked > 200
