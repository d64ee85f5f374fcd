"""Seeded input generators: known answers and recipe invariants (CPU only)."""
import numpy as np

import synth


def test_splitmix64_known_answers():
    # Published SplitMix64 outputs for state 0 (Steele, Lea & Flood 2014; the
    # reference implementation's first three outputs).
    w = synth.splitmix64(0, np.arange(3, dtype=np.uint64))
    assert [int(v) for v in w] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_streams_are_deterministic_and_distinct():
    k1 = synth.layer_key(7, 0, "gate", 3)
    k2 = synth.layer_key(7, 0, "up", 3)
    a = synth.q2k_blocks(k1, 100)
    b = synth.q2k_blocks(k1, 100)
    c = synth.q2k_blocks(k2, 100)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c)
    # a block range drawn from an offset equals the slice of the full draw
    assert np.array_equal(synth.q2k_blocks(k1, 10, start_block=37), a[37:47])
    q = synth.q41_blocks(k1, 50)
    assert np.array_equal(synth.q41_blocks(k1, 5, start_block=20), q[20:25])


def test_q2k_recipe_fields():
    blk = synth.q2k_blocks(synth.stream_key(1), 20000)
    assert blk.shape == (20000, 84)
    nib = np.concatenate([blk[:, :16] & 15, blk[:, :16] >> 4]).ravel()
    assert abs(nib.mean() - 7.5) < 0.05                      # U{0..15}
    codes = np.stack([(blk[:, 16:80] >> s) & 3 for s in (0, 2, 4, 6)]).ravel()
    assert abs(codes.mean() - 1.5) < 0.01                    # U{0..3}
    d = blk[:, 80:84].copy().view("<f2").astype(np.float64)
    assert (d >= 0).all()
    # |N(0, 0.01)|: mean 0.01*sqrt(2/pi), second moment 1e-4
    assert abs(d.mean() - 0.01 * np.sqrt(2 / np.pi)) < 2e-4
    assert abs((d ** 2).mean() - 1e-4) < 4e-6


def test_q41_recipe_fields():
    blk = synth.q41_blocks(synth.stream_key(2), 20000)
    assert blk.shape == (20000, 20)
    dm = blk[:, 0:4].copy().view("<f2").astype(np.float64)
    assert (dm[:, 0] >= 0).all()
    # m = -7.5 |N(0, 0.01)|: the block minimum, centring d*q + m near zero
    assert (dm[:, 1] <= 0).all()
    assert abs(dm[:, 1].mean() + 7.5 * 0.01 * np.sqrt(2 / np.pi)) < 2e-3
    assert abs((dm[:, 1] ** 2).mean() - 56.25e-4) < 3e-4
    w_mean = (dm[:, 0] * 7.5 + dm[:, 1]).mean()
    assert abs(w_mean) < 2e-3
    nib = np.concatenate([blk[:, 4:] & 15, blk[:, 4:] >> 4]).ravel()
    assert abs(nib.mean() - 7.5) < 0.05


def test_quantile_tables_monotone():
    half, mtab = synth.f16_tables()
    h = half.view(np.float16).astype(np.float64)
    m = mtab.view(np.float16).astype(np.float64)
    assert (np.diff(h) >= 0).all() and (np.diff(m) <= 0).all()
    assert h[0] >= 0 and (m <= 0).all()
    assert np.allclose(m, (-7.5 * h.astype(np.float16).astype(np.float64)), rtol=1e-3, atol=1e-6)


def test_normal_and_bf16_recipe():
    x = synth.x_f32(synth.stream_key(3), 64, 4096)
    assert x.dtype == np.float32
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    xb = synth.bf16_bits_from_f32(x)
    back = (xb.astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.abs(back - x) <= np.abs(x) * 2.0 ** -8)


def test_zipf_logits_skew():
    lg = synth.logits_zipf(synth.stream_key(4), 4096, 256)
    top = np.argsort(-lg, axis=1, kind="stable")[:, :6]
    load = np.bincount(top.ravel(), minlength=256)
    assert load.sum() == 4096 * 6
    srt = np.sort(load)[::-1]
    assert srt[0] > 2000 and np.median(load) < 60           # heavy head, light tail


def test_tile_cover_tokens_covers_every_group_and_position():
    """The GPU tests' sample of tokens at the 4096-token chunk: every 16-pair
    group of every m-tile and every position of a tile holds a pair of a
    chosen token (checked here by brute force on a small routing)."""
    import oracle
    from helpers import tile_cover_tokens
    T, E, k, tm = 300, 8, 6, 128
    lg = synth.logits_zipf(synth.stream_key(77), T, E)
    ids, _ = oracle.route(lg, k)
    chosen = set(tile_cover_tokens(ids, E, tm).tolist())
    _, offsets, pairs = oracle.group(ids, E)
    cells, positions = set(), set()
    need_cells, need_positions = set(), set()
    for e in range(E):
        for i in range(offsets[e], offsets[e + 1]):
            local = i - offsets[e]
            cell = (e, local // tm, (local % tm) // 16)
            need_cells.add(cell)
            need_positions.add(local % tm)
            if pairs[i] // k in chosen:
                cells.add(cell)
                positions.add(local % tm)
    assert cells == need_cells and positions == need_positions
    assert len(chosen) < T
