"""Host model of the balanced decode schedule (pa_decode.hip run_segment,
pa_reduce.hip balanced_waves, BalancedSplit in pa_internal.h): the steps of
every row block, each preceded by kUnitSetupSteps setup positions, are laid
out request-major and cut into equal runs, one per wave.  Checked over random
shapes: every step of every row block is walked exactly once, a piece's slot
(row block + wave) is unique and below the workspace's slots, and the waves
the merge expects for a row block (w0 .. w1 from the same formulas) are
exactly the waves that walked it.  The constants are read from the header."""
import math
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _const(name):
    with open(os.path.join(ROOT, "paged_kv_cache_96_amd", "csrc", "pa_internal.h")) as f:
        m = re.search(rf"constexpr int {name} = (\d+);", f.read())
    return int(m.group(1))


SETUP = _const("kUnitSetupSteps")
MIN_STEPS = _const("kBalancedMinSteps")
WAVE_FACTOR = _const("kBalancedWaveFactor")


def _waves(grid_waves, T, units, S):
    if T <= 0:
        return 0
    return min(grid_waves, (T + MIN_STEPS - 1) // MIN_STEPS, S - units,
               math.isqrt(WAVE_FACTOR * units * T))


def _walk(ctx, U, step, grid_waves, S):
    n = [(c + step - 1) // step for c in ctx]
    R = [0]
    for nb in n:
        R.append(R[-1] + U * (nb + SETUP if nb > 0 else 0))
    T, units = R[-1], len(ctx) * U
    Wa = _waves(grid_waves, T, units, S)
    begin = lambda v: v * T // Wa  # noqa: E731
    wave_of = lambda t: ((t + 1) * Wa - 1) // T  # noqa: E731
    walked, slots, pieces = {}, set(), {}
    for v in range(Wa):
        t, e = begin(v), begin(v + 1)
        while t < e:
            b = max(i for i in range(len(ctx)) if R[i] <= t)
            nu = n[b] + SETUP
            u = (t - R[b]) // nu
            row0 = R[b] + u * nu + SETUP
            if t < row0:
                t = row0
                continue
            j0 = t - row0
            j1 = min(n[b], j0 + (e - t))
            unit = b * U + u
            for j in range(j0, j1):
                assert (unit, j) not in walked
                walked[(unit, j)] = v
            w0, w1 = wave_of(row0), wave_of(row0 + n[b] - 1)
            assert w0 <= v <= w1
            assert unit + v not in slots and unit + v < S
            slots.add(unit + v)
            pieces.setdefault(unit, set()).add(v)
            t += j1 - j0
    return n, R, Wa, walked, pieces, wave_of


@pytest.mark.parametrize("seed", range(6))
def test_balanced_split_covers_every_step_once_with_unique_slots(seed):
    rng = np.random.default_rng(seed)
    for _ in range(40):
        B = int(rng.integers(1, 30))
        U = int(rng.integers(1, 12))
        ctx = [int(rng.choice([0, rng.integers(1, 3000)], p=[0.2, 0.8])) for _ in range(B)]
        grid_waves = int(rng.integers(1, 1500))
        S = B * U + int(rng.integers(1, 1500))
        n, R, Wa, walked, pieces, wave_of = _walk(ctx, U, 16, grid_waves, S)
        if Wa == 0:
            assert sum(n) == 0
            continue
        for b in range(B):
            before = sum(U * (n[c] + SETUP if n[c] > 0 else 0) for c in range(b))
            assert before == R[b]
            for u in range(U):
                unit = b * U + u
                if n[b] == 0:
                    assert unit not in pieces
                    continue
                assert all((unit, j) in walked for j in range(n[b]))
                # the merge's view (pa_reduce balanced_waves)
                row0 = before + u * (n[b] + SETUP) + SETUP
                w0 = wave_of(row0)
                count = wave_of(row0 + n[b] - 1) - w0 + 1
                assert pieces[unit] == set(range(w0, w0 + count))


def test_setup_positions_move_steps_away_from_multi_piece_runs():
    # with setup positions, a run that starts a new row block inside it walks
    # fewer steps than a run inside one long row block
    ctx = [16 * 40] * 8
    n, R, Wa, walked, pieces, _ = _walk(ctx, 2, 16, 24, 10_000)
    per_wave = {}
    for (unit, j), v in walked.items():
        per_wave.setdefault(v, []).append(unit)
    multi = [len(u) for v, u in per_wave.items() if len(set(u)) > 1]
    single = [len(u) for v, u in per_wave.items() if len(set(u)) == 1]
    assert multi and single and max(multi) <= min(single)


@pytest.mark.parametrize("B,U,keys", [(1, 8, 16384), (2, 8, 4096), (4, 8, 4096), (1, 8, 32768),
                                      (3, 16, 9000)])
def test_piece_cap_bounds_waves_and_pieces_per_row_block(B, U, keys):
    # a small batch over long contexts: the grid and the slot count would allow
    # hundreds of pieces per row block; the cap keeps Wa^2 <= factor * units * T
    # (runs of at least pieces / factor steps) and still walks every step once
    ctx = [keys - 37 * b for b in range(B)]
    n, R, Wa, walked, pieces, _ = _walk(ctx, U, 16, 8192, B * U + 1280)
    units, T = B * U, R[-1]
    assert Wa == min(math.isqrt(WAVE_FACTOR * units * T), (T + MIN_STEPS - 1) // MIN_STEPS, 1280)
    assert Wa * Wa <= WAVE_FACTOR * units * T
    assert len(walked) == U * sum(n)
    per_unit = sum(len(p) for p in pieces.values()) / units
    steps_per_run = T / Wa
    assert per_unit <= WAVE_FACTOR * steps_per_run + 2

