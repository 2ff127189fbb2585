"""The compaction's 4-byte word mover for rows whose byte width is 2 modulo 4,
checked on the CPU with the kernel's own index arithmetic.

Such rows (q8_0 at head_dim 32, 96, 160 and 224) sit on 2-byte boundaries only.
The launch moves them in 2-byte pieces while those fit 256-row chunks (rows up
to 64 bytes), else in 4-byte words (96, 160 and 224).  A task splits its chunk of CR
destination rows into 16-row groups, each contiguous in memory (a paged block,
or 16 consecutive rows of a contiguous unit), and moves each group's byte span
in aligned 4-byte words: lane l of the group's W = 256 / CR wavefronts takes
words l + 64 v, l + 64 v + 64 W, ... (v its wavefront within the group), at
most 8 per lane.  Each half of a word is the 2-byte half of the aligned source
word that holds it (one load when both halves come from one aligned source
word); the word is stored whole when both halves move, else as its one moving
half.  The model below replays that arithmetic (the lane's first word split
into row and byte once, later words stepped by 4 x 64 W bytes, as on the
device) over contiguous units at both alignments and shuffled paged blocks,
and requires:
  - every moved destination byte written exactly once, with its source byte;
  - nothing else written (rows that stay, rows past the kept count, other
    chunks' and other units' spans);
  - every load an aligned word that holds a byte of a moved source row;
  - the chunk size the launch picks leaving no word of a span uncovered.
Two plausible mistakes must fail on the same inputs (the test is not vacuous):
always taking the lower half of a loaded word, and storing whole words when
only one half moves.
"""
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "kv_cache_eviction_tria_amd", "csrc", "tria_compact.hip")
BLOCK = 16        # rows per group (paged block)
THREADS = 1024    # the word mover runs with every thread of the workgroup
ITEMS = 8         # words per lane
WIDTHS = (34, 102, 170, 238)  # q8_0 rows at head_dim 32, 96, 160, 224
WORDS = 1         # the kernel's piece code for 4-byte words


def piece_code(rb):
    """The launch's choice for an array of rb-byte rows: the widest of 16, 8, 4, 2
    bytes dividing rb, and words for 2-byte pieces that would not fit 256 rows."""
    pw = next(w for w in (16, 8, 4, 2) if rb % w == 0)
    return WORDS if pw == 2 and 256 * (rb // 2) > THREADS * ITEMS else pw


def chunk_rows(rb, other_rb=256, other_pw=16):
    """The launch's chunk size for a word-moved array of rb bytes beside another
    array of other_rb bytes moved in other_pw-byte pieces."""
    for rows in (256, 128, 64):
        waves = (THREADS // 64) // (rows // BLOCK)
        if 4 * rb + 1 > ITEMS * 64 * waves:
            continue
        if rows * (other_rb // other_pw) > THREADS * ITEMS:
            continue
        return rows
    return None


def move_chunk(mem, orig, rb, src_row, grp_row, cr, written, moved_src, mistake=None):
    """One task: every wavefront and lane as the kernel runs them."""
    groups = cr // BLOCK
    wpg = (THREADS // 64) // groups
    step = 64 * wpg
    for w in range(THREADS // 64):
        g = w // wpg
        g0 = g * BLOCK
        if grp_row[g] < 0:
            continue
        G = grp_row[g] * rb
        ga, span = G & 3, BLOCK * rb
        for lane in range(64):
            j0 = (w % wpg) * 64 + lane
            p0 = 4 * j0 - ga            # span byte of half 0 of the first word, >= -2
            r = -1 if p0 < 0 else p0 // rb
            off = p0 - r * rb
            dr, doff = divmod(4 * step, rb)
            for k in range(ITEMS):
                p = p0 + 4 * step * k
                if p >= span:
                    break
                assert (r, off) == ((-1, rb - 2) if p < 0 else divmod(p, rb))
                s0 = src_row[g0 + r] if r >= 0 else -1
                r1, off1 = (r + 1, 0) if off + 2 == rb else (r, off + 2)
                s1 = -1 if p + 2 >= span else (s0 if r1 == r else src_row[g0 + r1])
                a0 = s0 * rb + off if s0 >= 0 else -1
                a1 = s1 * rb + off1 if s1 >= 0 else -1
                m0, m1 = a0 >= 0, a1 >= 0
                one = m0 and m1 and r1 == r and a0 % 4 == 0
                r, off = r + dr, off + doff
                if off >= rb:
                    r, off = r + 1, off - rb
                lo = hi = np.zeros(4, np.uint8)  # registers start at zero
                for which, a, flag in ((0, a0, m0), (1, a1, m1 and not one)):
                    if not flag:
                        continue
                    word = orig[(a & ~3):(a & ~3) + 4]
                    # the aligned word holds a byte of a moved source row
                    assert moved_src[(a & ~3):(a & ~3) + 4].any(), (rb, a)
                    if which == 0:
                        lo = word
                    else:
                        hi = word
                upper0 = bool(a0 & 2) and mistake != "lower_half"
                upper1 = bool(a1 & 2) and mistake != "lower_half"
                h0 = lo[2:4] if upper0 else lo[0:2]
                x = lo if one else hi
                h1 = x[2:4] if upper1 else x[0:2]
                if not (m0 or m1):
                    continue
                W = (G & ~3) + 4 * (j0 + step * k)
                for h, val, moves in ((0, h0, m0), (1, h1, m1)):
                    if not moves and mistake != "whole_words":
                        continue
                    for i in range(2):
                        b = W + 2 * h + i
                        written[b] += 1
                        mem[b] = val[i]


def run_units(rb, layout, seed, mistake=None):
    rng = np.random.default_rng(seed)
    cr = chunk_rows(rb)
    assert cr is not None and (4 * rb + 1) <= ITEMS * 64 * ((THREADS // 64) // (cr // BLOCK))
    n_units = 3
    ns = [int(x) for x in rng.integers(cr // 2, 3 * cr, size=n_units)]
    if layout == "paged":
        max_blocks = max((n + BLOCK - 1) // BLOCK for n in ns)
        perm = rng.permutation(n_units * max_blocks)
        table = perm.reshape(n_units, max_blocks)  # unit u's logical block -> physical block

        def phys(u, r):
            return int(table[u, r // BLOCK]) * BLOCK + r % BLOCK
        total = n_units * max_blocks * BLOCK
    else:
        cap = max(ns) + (1 if layout == "contiguous_odd" else 0)  # odd cap: spans on 2 mod 4

        def phys(u, r):
            return u * cap + r
        total = n_units * cap
    orig = rng.integers(0, 256, size=total * rb + 8, dtype=np.int64).astype(np.uint8)
    mem = orig.copy()
    written = np.zeros(len(mem), np.int64)
    expect = orig.copy()
    moved_dst = np.zeros(len(mem), bool)
    moved_src = np.zeros(len(mem), bool)
    plans = []
    for u, n in enumerate(ns):
        kept = int(rng.integers(1, n))
        stay = int(rng.integers(0, kept)) if rng.random() < 0.5 else 0  # rows that stay
        keep = np.concatenate([np.arange(stay),
                               np.sort(rng.choice(np.arange(stay, n), size=kept - stay,
                                                  replace=False))])
        for d in range(kept):
            s = int(keep[d])
            if s > d:
                pd, ps = phys(u, d), phys(u, s)
                expect[pd * rb:pd * rb + rb] = orig[ps * rb:ps * rb + rb]
                moved_dst[pd * rb:pd * rb + rb] = True
                moved_src[ps * rb:ps * rb + rb] = True
        plans.append((u, n, kept, keep))
    for u, n, kept, keep in plans:
        for d0 in range(0, kept, cr):
            src_row = np.full(cr, -1, np.int64)
            for i in range(cr):
                d = d0 + i
                if d < kept and d < int(keep[d]) < n:
                    src_row[i] = phys(u, int(keep[d]))
            grp_row = [phys(u, d0 + BLOCK * g) if d0 + BLOCK * g < kept else -1
                       for g in range(cr // BLOCK)]
            move_chunk(mem, orig, rb, src_row, grp_row, cr, written, moved_src, mistake)
    return mem, expect, written, moved_dst


@pytest.mark.parametrize("rb", WIDTHS)
@pytest.mark.parametrize("layout", ["contiguous_even", "contiguous_odd", "paged"])
def test_word_mover_is_the_exact_gather(rb, layout):
    for seed in range(3):
        mem, expect, written, moved_dst = run_units(rb, layout, seed)
        assert np.array_equal(written[moved_dst], np.ones(int(moved_dst.sum()), np.int64)), \
            "a moved byte not written exactly once"
        assert not written[~moved_dst].any(), "a byte outside the moved rows was written"
        assert np.array_equal(mem, expect)


@pytest.mark.parametrize("mistake", ["lower_half", "whole_words"])
def test_a_planted_mistake_fails(mistake):
    with pytest.raises(AssertionError):
        for seed in range(3):
            mem, expect, written, moved_dst = run_units(102, "contiguous_odd", seed, mistake)
            assert not written[~moved_dst].any()
            assert np.array_equal(mem, expect)


def test_piece_codes_of_the_q8_widths():
    """Words exactly for the q8_0 widths 2 modulo 4 above 64 bytes."""
    rbs = [34 * hd // 32 for hd in range(32, 257, 32)]
    assert [piece_code(rb) for rb in rbs] == [2, 4, WORDS, 8, WORDS, 4, WORDS, 16]


def test_chunk_rows_of_the_widths():
    """hd 32 and 96 take 256-row chunks, hd 160 and 224 take 128 (V fp16 beside)."""
    assert [chunk_rows(rb) for rb in WIDTHS] == [256, 256, 128, 128]
    assert [chunk_rows(rb, other_rb=2 * hd) for rb, hd in zip(WIDTHS, (32, 96, 160, 224))] == \
        [256, 256, 128, 128]


def test_the_kernel_uses_the_modelled_constants():
    src = open(SRC).read()
    assert re.search(r"struct HalfMove \{.*?static constexpr int kItems = 8;", src, re.S)
    assert "kWavesPerGroup = (kMaxFlowThreads / 64) / kGroups" in src
    assert "kStep = 64 * kWavesPerGroup" in src
    assert "constexpr int kMaxFlowThreads = 1024;" in src
    assert "if (pk == kWords || pv == kWords) threads = kMaxFlowThreads;" in src
    assert "constexpr int kWords = 1;" in src
    assert re.search(r"return pw == 2 && 4 \* kChunkRows \* \(rb / 2\) > \(int64_t\)"
                     r"kMaxFlowThreads \* kItems \? kWords", src)
    assert "4 * rb + 1 > (int64_t)kItems * 64 * waves" in src
