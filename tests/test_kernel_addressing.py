"""CPU models of the kernels' address arithmetic (no GPU).

Each model repeats, in Python, the index expressions a kernel uses for its global
loads, its stores and its LDS slots, for every workgroup, wave and lane of a launch,
and checks that every access stays inside its buffer and that every LDS slot a lane
reads was written with the data it expects. The launch-shape constants are read from
the HIP sources, so a change there is checked here. A model that disagrees with its
kernel is a bug in one of them: both are written from the same description in the
kernel's comments.
"""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_quantized_weight_q8_amd", "csrc")
K_BATCH_MAX, K_STEP_K, K_TILE_ROWS = 16, 64, 16


def batch_shapes():
    src = open(os.path.join(CSRC, "batch.hip")).read()
    shapes = {}
    for name in ("WideSplitShape", "SplitShape", "WholeShape"):
        m = re.search(rf"using {name} = Shape<(\d+), (\d+), (\d+), (\d+)>;", src)
        assert m, name
        shapes[name] = tuple(int(v) for v in m.groups())
    wide = int(re.search(r"kWideSplitTiles = (\d+);", src).group(1))
    split = int(re.search(r"kSplitTiles = (\d+);", src).group(1))
    max_k = re.search(r"kMaxK = ([^;]+);", src)
    return shapes, wide, split, max_k


SHAPES, WIDE_TILES, SPLIT_TILES, _ = batch_shapes()


def shape_for(n):
    tiles = (n + K_TILE_ROWS - 1) // K_TILE_ROWS
    if tiles <= WIDE_TILES:
        return SHAPES["WideSplitShape"]
    return SHAPES["SplitShape"] if tiles <= SPLIT_TILES else SHAPES["WholeShape"]


def batch_staging(N, K, B, W, S, TK):
    """The staged activation: codes swizzled per vector, scales [block][vector], and each
    wave's weight scales; every read slot holds what the consuming lane expects."""
    nb = K // 32
    codes_area = K_BATCH_MAX * TK
    dx_area = (TK // 32) * K_BATCH_MAX * 4
    wsc_tile = K_TILE_ROWS * (TK // 32) * 4
    k0 = 0
    while k0 < K:
        kt = min(K - k0, TK)
        nbt, cpv = kt // 32, kt // 16
        rowc16 = (cpv + 15) & ~15
        steps = (kt + K_STEP_K - 1) // K_STEP_K
        written = {}
        for p in range(B * rowc16):
            b = p // rowc16
            c = (p - b * rowc16) ^ (b & 15)
            bb, cc = min(b, B - 1), (c if c < cpv else 0)
            src = bb * K + k0 + 16 * cc
            assert 0 <= src and src + 16 <= B * K
            assert 16 * p + 16 <= codes_area
            written[p] = (bb, cc)
        for t in range(nbt * K_BATCH_MAX):
            blk, b = divmod(t, K_BATCH_MAX)
            assert min(b, B - 1) * nb + k0 // 32 + blk < B * nb
            assert 4 * t + 4 <= dx_area
        for st in range(steps):
            hi = st * K_STEP_K + 32 < kt
            assert 2 * st < nbt and (not hi or 2 * st + 1 < nbt)
            for j in range(16):
                for q in range(4):
                    if j < B and (q < 2 or hi):
                        c = 4 * st + q
                        assert c < cpv
                        assert written[j * rowc16 + (c ^ j)] == (j, c)
        for split in range(S):
            sb, se = steps * split // S, steps * (split + 1) // S
            nbw = 2 * (se - sb)
            assert K_TILE_ROWS * 4 * 2 * sb + 4 * K_TILE_ROWS * nbw <= wsc_tile
            blk0 = k0 // 32 + 2 * sb
            for t in range(K_TILE_ROWS * nbw):
                bo = t % nbw
                assert (blk0 + bo if blk0 + bo < nb else blk0) < nb
        k0 += TK


def batch_rows(N, K, B, W, S):
    """Weight rows as a wave-uniform base plus a 32-bit lane offset, clamped for rows past N
    (including a tile wholly past N); outputs and residuals [B][N]."""
    nb = K // 32
    tiles = (N + K_TILE_ROWS - 1) // K_TILE_ROWS
    tpg = W // S
    groups = (tiles + tpg - 1) // tpg
    for g in range(groups):
        for wave in range(W):
            tile = wave // S
            row0 = (g * tpg + tile) * K_TILE_ROWS
            rbase = row0 if row0 < N else N - 1
            for j in range(16):
                row = row0 + j
                jr = (row if row < N else N - 1) - rbase
                assert 0 <= jr < 16
                assert jr * K < 2**32
                if K:
                    assert rbase * K + jr * K + K <= N * K
                    assert rbase * nb + jr * nb + nb <= N * nb
                for b in range(16):
                    if row < N and b < B:
                        assert b * N + row < B * N  # the stored output
                # the residuals every lane requests up front: vectors 4q..4q+3 of its row,
                # clamped to vector B-1 and row N-1
                rr = row if row < N else N - 1
                for q in range(4):
                    for r in range(4):
                        b = 4 * q + r if 4 * q + r < B else B - 1
                        assert 0 <= b * N + rr < B * N


BATCH_CASES = [(16, 64, 1), (17, 96, 3), (100, 1024, 16), (1024, 2048, 8), (300, 3584, 5), (33, 5120, 16),
               (4111, 160, 2), (7168, 1024, 16), (1030, 2048, 6), (1, 96, 1), (15, 96, 16), (4097, 96, 16),
               (40001, 96, 5), (64, 2080, 7), (64, 4128, 16), (32785, 64, 16), (1, 64, 16), (1024, 3584, 16)]


@pytest.mark.parametrize("n,k,b", BATCH_CASES)
def test_batch_kernel_addressing(n, k, b):
    W, S, P, TK = shape_for(n)
    batch_rows(n, k, b, W, S)
    # staging is independent of N: check every shape on this K and B
    for W_, S_, P_, TK_ in SHAPES.values():
        batch_staging(n, k, b, W_, S_, TK_)


def test_batch_shape_constants_are_consistent():
    for W, S, P, TK in SHAPES.values():
        assert W % S == 0 and 1 <= W <= 16
        assert TK % K_STEP_K == 0 and (TK // 16) % 16 == 0
        lds = 16 + (TK // 32) * K_BATCH_MAX * 4 + K_BATCH_MAX * TK + (W // S) * K_TILE_ROWS * (TK // 32) * 4
        assert lds <= 160 * 1024
        assert W * 64 * 4 * 4 <= K_BATCH_MAX * TK  # split partial sums fit the code area


# --------------------------------------------------------------------------- stream_kernel


def stream_constants():
    src = open(os.path.join(CSRC, "batch.hip")).read()
    m = re.search(r"using StreamShape = Shape<(\d+), (\d+), (\d+), (\d+)>;", src)
    assert m
    wpu = int(re.search(r"kStreamWavesPerUnit = (\d+);", src).group(1))
    units = int(re.search(r"kUnits = (\d+);", src).group(1))
    return tuple(int(v) for v in m.groups()), wpu, units


def stream_model(N, K, B):
    """The streaming form of the tiled layout: every tile taken by exactly one wave, every
    consumed step reading the weights requested for it P requests earlier, every request,
    scale chunk and residual inside its buffer, every scale read from LDS written first."""
    (W, S, P, TK), wpu, units = stream_constants()
    steps = (K + K_STEP_K - 1) // K_STEP_K
    assert steps in (8, 16) and steps % P == 0 and steps * K_STEP_K <= TK
    nb = K // 32
    ntiles = (N + K_TILE_ROWS - 1) // K_TILE_ROWS
    code_bytes = ntiles * K_TILE_ROWS * steps * K_STEP_K
    scale_elems = ntiles * K_TILE_ROWS * nb
    target = units * wpu
    per_wave = (ntiles + target - 1) // target
    groups = ((ntiles + per_wave - 1) // per_wave + W - 1) // W
    GW = groups * W
    scale_bytes = K_TILE_ROWS * (TK // 32) * 2
    lds = 16 + (TK // 32) * K_BATCH_MAX * 4 + K_BATCH_MAX * TK + W * scale_bytes
    assert lds <= 160 * 1024
    covered = []
    for gw in range(GW):
        nt = (ntiles - 1 - gw) // GW + 1 if gw < ntiles else 0
        assert nt <= per_wave
        tiles = [gw + i * GW for i in range(nt)]
        covered += tiles
        t0 = gw if nt > 0 else ntiles - 1
        requests = [(t0, p) for p in range(P)]
        scale_tiles = [t0]
        for i, t in enumerate(tiles):
            more = i + 1 < nt
            tn = tiles[i + 1] if more else t
            scale_tiles.append(tn)
            for st in range(steps):
                requests.append((t, st + P) if st + P < steps else (tn, st + P - steps if more else steps - 1))
        consumed = [(t, st) for t in tiles for st in range(steps)]
        assert requests[:len(consumed)] == consumed
        for t, st in requests:
            assert 0 <= t < ntiles and 0 <= st < steps
            assert (t * steps + st) * 1024 + 16 * 63 + 16 <= code_bytes
        for t in scale_tiles:
            for lane in range(64):
                sl = lane if lane < 2 * nb else 0
                assert t * nb * K_TILE_ROWS + 8 * sl + 8 <= scale_elems
        # LDS: lanes < 2 nb write 16 bytes each (elements [0, 16 nb)); step st reads blocks
        # 2 st and, when present, 2 st + 1 of row j
        assert 32 * nb <= scale_bytes
        for st in range(steps):
            hi = st * K_STEP_K + 32 < K
            for j in range(16):
                for blk in ([2 * st, 2 * st + 1] if hi else [2 * st]):
                    assert blk * K_TILE_ROWS + j < 16 * nb
        for t in tiles:
            for j in range(16):
                row = t * K_TILE_ROWS + j
                rr = row if row < N else N - 1
                for q in range(4):
                    for r in range(4):
                        b = 4 * q + r if 4 * q + r < B else B - 1
                        assert 0 <= b * N + rr < B * N
    assert sorted(covered) == list(range(ntiles)), "every tile exactly once"


@pytest.mark.parametrize("n,k,b", [(32785, 1024, 16), (2049 * 16, 512, 1), (40000, 992, 5), (36017, 480, 16),
                                   (65536, 1024, 3), (151936, 1024, 16), (1 << 20, 512, 2)])
def test_stream_kernel_addressing(n, k, b):
    stream_model(n, k, b)


# --------------------------------------------------------------------------- gemv_kernel


def gateup_epilogue(F, K):
    """Workgroup b owns gate rows 32b..32b+31 (waves 0..7, 4 rows each) and the same up rows
    (waves 8..15); the stacked row space is [gate (F) | up (F)]; LDS s_gu[64]; outputs
    qa[32b + j] and da[b]."""
    n_total = 2 * F
    seen = set()
    for blk in range(F // 32):
        gu_slots = set()
        for wave in range(16):
            row0 = 32 * blk + 4 * wave if wave < 8 else n_total // 2 + 32 * blk + 4 * (wave - 8)
            for i in range(4):
                g = row0 + i
                assert g < n_total
                part, local = (0, g) if g < F else (1, g - F)
                assert 0 <= local < F
                assert local * K + K <= F * K  # the row's bytes within its part
                seen.add(g)
                slot = (0 if wave < 8 else 32) + 4 * (wave & 7) + i
                assert 0 <= slot < 64
                gu_slots.add(slot)
                # gate row j pairs with up row j in the same slot offset
                assert slot % 32 == local % 32 and local // 32 == blk
        assert gu_slots == set(range(64))
        for lane in range(64):
            j = lane & 31
            if lane < 32:
                assert 32 * blk + j < F
        assert blk < F // 32
    assert seen == set(range(n_total))


@pytest.mark.parametrize("f,k", [(32, 32), (64, 96), (3584, 1024), (96, 16384), (4096 + 32, 64)])
def test_gateup_epilogue_addressing(f, k):
    gateup_epilogue(f, k)


def fused_prologue_loads(K, threads, passes, two):
    """Every lane loads x (and the second input: gamma, or the up half of [gate | up]) at
    e < K ? e : K - 4, so with K >= 32 all loads are in bounds and the values used are
    exactly those with e < K; block sums and codes go to LDS index e >> 5 < K / 32."""
    assert K >= 32 and K % 32 == 0
    xlen = 2 * K if two == "silu" else K
    used = set()
    for t in range(threads):
        for p in range(passes):
            e = 4 * t + p * 4 * threads
            ec = e if e < K else K - 4
            assert 0 <= ec and ec + 4 <= K
            if two == "silu":
                assert K + ec + 4 <= xlen
            if e - (t & 7) * 4 < K:  # the 8-lane group of the block is in range
                assert e < K
                assert (e >> 5) < K // 32
                used.update(range(e, e + 4))
        # the reload loop past the register passes
        e = 4 * t + passes * 4 * threads
        while e < K:
            assert e + 4 <= K and (e >> 5) < K // 32
            used.update(range(e, e + 4))
            e += 4 * threads
    assert used == set(range(K))


def launch_passes(k, threads):
    """Activation passes the f32-input GEMV launch picks: one when one pass of 4 values per thread
    covers K, two when two do, else four (the gate+up epilogue launch: one, else four)."""
    return 1 if k <= 4 * threads else 2 if k <= 8 * threads else 4


@pytest.mark.parametrize("k", [32, 96, 1024, 2048, 2080, 3584, 4096, 16384])
@pytest.mark.parametrize("waves", [4, 8, 16])
@pytest.mark.parametrize("two", [None, "norm", "silu"])
def test_fused_prologue_addressing(k, waves, two):
    for passes in (1, 2, 4):  # the launch's choice and the other templates, all valid for any K
        fused_prologue_loads(k, waves * 64, passes, two)
    assert launch_passes(k, waves * 64) in (1, 2, 4)


def weight_batch_items(K, R, kbatch=4, chunk=1024):
    """The first weight batch of an f32-input launch: item j reads chunk min(j / R, nchunk - 1)
    of row j % R (clamped, so that every load is issued), lanes past the row end read offset 0;
    items past the last chunk are skipped when consumed, so each real (row, chunk) is consumed
    exactly once."""
    nchunk = (K + chunk - 1) // chunk
    assert nchunk >= 1
    consumed = []
    for j in range(kbatch):
        c_real = j // R
        c = c_real if c_real < nchunk else nchunk - 1
        for lane in range(64):
            off = c * chunk + 16 * lane
            o = off if off < K else 0
            assert 0 <= o and o + 16 <= K  # the 16 bytes lie inside the row
        if c_real < nchunk:
            consumed.append((j % R, c_real))
    expect = [(r, c) for c in range(min(nchunk, kbatch // R)) for r in range(R)]
    assert sorted(consumed) == sorted(expect)


@pytest.mark.parametrize("k", [32, 96, 1024, 2048, 3584, 5120])
@pytest.mark.parametrize("r", [1, 2, 4])
def test_first_weight_batch_addressing(k, r):
    weight_batch_items(k, r)


def row_batch_schedule(nchunk, cb):
    """The main loop of a wave's rows, batch by batch: cur holds the batch at chunk 0 on
    entry; each trip requests the next batch into nxt, consumes cur, requests the one after
    into cur, consumes nxt; then the last one or two batches. Returns the (kind, buffer, c0)
    events in program order."""
    ev = [("load", "cur", 0)] if nchunk > 0 else []
    c0 = 0
    while c0 + 2 * cb < nchunk:
        ev += [("load", "nxt", c0 + cb), ("use", "cur", c0), ("load", "cur", c0 + 2 * cb), ("use", "nxt", c0 + cb)]
        c0 += 2 * cb
    if c0 + cb < nchunk:
        ev += [("load", "nxt", c0 + cb), ("use", "cur", c0), ("use", "nxt", c0 + cb)]
    elif c0 < nchunk:
        ev += [("use", "cur", c0)]
    return ev


@pytest.mark.parametrize("cb", [1, 2, 4, 8])
def test_row_batch_schedule(cb):
    """Every chunk of the row is consumed exactly once, from the buffer that holds it; a
    buffer is refilled only after its batch was consumed; at most two batches are in flight;
    every load of a batch is in bounds (chunks past the end re-read the last one), and only
    the row's last batch re-reads."""
    for nchunk in range(0, 24):
        held, pending, consumed, rereads = {}, set(), [], 0
        for kind, b, c0 in row_batch_schedule(nchunk, cb):
            if kind == "load":
                assert b not in pending, "a buffer refilled before its batch was consumed"
                assert 0 <= c0 < nchunk
                items = [c0 + i for i in range(cb)]
                clamped = [c if c < nchunk else nchunk - 1 for c in items]
                assert all(0 <= c < nchunk for c in clamped)
                rereads += sum(c >= nchunk for c in items)
                held[b] = c0
                pending.add(b)
                assert len(pending) <= 2
            else:
                assert held.get(b) == c0 and b in pending
                pending.discard(b)
                consumed += [c for c in range(c0, c0 + cb) if c < nchunk]
        assert consumed == list(range(nchunk))
        assert not pending
        assert rereads == (0 if nchunk == 0 else (-nchunk) % cb)


def test_row_batch_schedule_matches_source():
    src = open(os.path.join(CSRC, "q8gemv.hip")).read()
    assert "for (; c0 + 2 * CB < nchunk; c0 += 2 * CB) {" in src
    assert "load_batch<DT, R, !FUSED, true>(rows, x, dx, c0 + CB, nchunk, row_bytes, lane_off, nxt);" in src
    assert "load_batch<DT, R, !FUSED, true>(rows, x, dx, c0 + 2 * CB, nchunk, row_bytes, lane_off, cur);" in src
    assert "if (c0 + CB < nchunk) {" in src
    assert "} else if (c0 < nchunk) {" in src


def test_fused_prologue_constants():
    src = open(os.path.join(CSRC, "q8gemv.hip")).read()
    assert re.search(r"constexpr int kXPasses = XP;", src)
    assert "constexpr bool one_pass(int64_t K, int threads) { return K <= 4 * (int64_t)threads; }" in src
    assert "constexpr bool two_passes(int64_t K, int threads) { return K <= 8 * (int64_t)threads; }" in src
    assert re.search(r"constexpr int kMaxFusedK = 16384;", src)
    assert "e < K ? e : K - 4" in src
    assert "const bool real = c0 + j / R < nchunk;" in src
    assert "const int64_t c = real ? c0 + j / R : nchunk - 1;" in src
