"""A host-side model of the copy, wait, barrier and read order of every kernel
whose waits leave LDS-DMA copies in flight: the two that carry their LDS ring
from one output tile into the next (the BF16 256 x 256 kernel and the
microscaled FP4 kernel, three tiles per workgroup), the 64 x 64 long-K kernel,
whose B units arrive in parts over four steps, and the whole-step rings of
the 64 x 64 kernel and of the split-K kernel's A and B copying waves; every
step count up to 40 (60 for the long-K kernel).

The only ordering assumed of the hardware is the one the kernels rely on: a
wave's LDS-DMA copies complete in the order it issued them, while its stores
and register loads may complete before or after any of them. So a wait for
"at most N outstanding vector-memory operations" proves complete exactly the
copies issued before the last N copies; a wait for zero proves all. Every wave
runs the same sequence, so a unit (one step's tile of an operand, copied in
parts by every wave) is visible to all waves after a barrier that follows the
wait proving it complete in each.

Checked for every event:
  * a fragment read reads a unit that is visible and still in its slot;
  * a copy overwrites a slot only after a barrier that follows every read of
    the unit it held (each barrier follows the wave's wait for its own reads);
  * every wait bound stays within the counter's 63.

The sequences are written from the kernels' step bodies; the constants they
use are compared with the headers' below, so a change to either side fails
here until the model is updated with it.
"""
import os
import re

import pytest

CSRC = os.path.join(os.path.dirname(__file__), "..", "dense_gemm_14_amd", "csrc")


def _src(name):
    with open(os.path.join(CSRC, name)) as f:
        return f.read()


class Wave:
    """Events of one wave, checked as they are issued."""

    def __init__(self, slots):
        self.copies = []          # units of the copies issued, in order
        self.proven = 0           # copies proven complete: a prefix of self.copies
        self.visible = set()      # units every wave's copies of which are complete and behind a barrier
        self.content = [None] * slots
        self.parts = {}           # unit -> copies it takes in all (issued over one or several steps)
        self.last_read = {}       # unit -> sequence number of its last read
        self.seq = 0
        self.barrier_seq = -1
        self.reads_waited_seq = -1

    def tick(self):
        self.seq += 1
        return self.seq

    def copy(self, unit, slot, parts, total=None):
        self.parts[unit] = parts if total is None else total
        held = self.content[slot]
        if held is not None and held != unit:
            r = self.last_read.get(held, -1)
            assert r < self.barrier_seq and r < self.reads_waited_seq, \
                "copy of %s into slot %d while %s may still be read" % (unit, slot, held)
            self.visible.discard(held)
        self.content[slot] = unit
        self.copies += [unit] * parts
        self.tick()

    def wait(self, n):
        assert 0 <= n <= 63
        self.proven = max(self.proven, len(self.copies) - n)
        self.tick()

    def wait_reads(self):
        self.reads_waited_seq = self.tick()

    def barrier(self):
        done = self.copies[:self.proven]
        pending = set(self.copies[self.proven:])
        for s, u in enumerate(self.content):
            if u is not None and u not in pending and done.count(u) == self.parts[u]:
                self.visible.add(u)
        self.barrier_seq = self.tick()

    def read(self, unit, slot):
        assert self.content[slot] == unit, "read of %s from slot %d, which holds %s" % (unit, slot, self.content[slot])
        assert unit in self.visible, "read of %s before every wave's copies of it are proven complete" % (unit,)
        self.last_read[unit] = self.tick()


# ---- BF16 256 x 256 kernel ---------------------------------------------------

BF16_UNIT_COPIES = 8   # 1 KiB copies per wave and unit (one step's 256-row tile of A or of B)
BF16_SLOTS = 5


def test_bf16_constants_match_the_kernel():
    s = _src("gemm_bf16.hpp")
    assert "constexpr int UNIT_COPIES = %d;" % BF16_UNIT_COPIES in s
    assert "constexpr int SLOTS = %d;" % BF16_SLOTS in s
    # the step's copy wait, skipped at a tile's first step; the epilogue waits for all
    assert re.search(r"if constexpr \(!first\)\s*wait_copies_le<UNIT_COPIES>\(\);\s*lds_barrier\(\);", s)
    assert "wait_all_copies();\n        const int ln" in s
    # A copies of step s + 2 before the barrier into ring[4], B copies after it into ring[0]
    assert "mma2_copies(p, 0, Int<(p - a_copy_at(0)) / a_step>{}, ring[4], ks_off, tail);" in s
    assert "mma2_copies(p, 1, Int<(p - b0) / b_step>{}, ring[0], ks_off, tail);" in s
    assert "read_a(ring[2], i);" in s and "read_b(ring[3], j);" in s
    assert "read_a(ring[0], i);" in s and "read_b(ring[1], 7);" in s
    assert re.search(r"ring\[0\] = ring\[2\];\s*ring\[1\] = ring\[3\];\s*ring\[2\] = ring\[4\];\s*"
                     r"ring\[3\] = r0;\s*ring\[4\] = r1;", s)


def bf16_run(nk, tiles, b_copy_ring=0):
    w = Wave(BF16_SLOTS)
    A = lambda t, k: ("A", t, k)
    B = lambda t, k: ("B", t, k)
    ring = list(range(BF16_SLOTS))   # ring[x]: slot of unit 2 s + x during step s
    # prologue of the first tile: A0, B0, A1, B1 into slots 0..3, all waited for
    for u, unit in enumerate((A(0, 0), B(0, 0), A(0, 1), B(0, 1))):
        w.copy(unit, u, BF16_UNIT_COPIES)
    w.wait(0)
    w.barrier()
    for j in range(7):
        if j < 4:
            w.read(A(0, 0), ring[0])
        w.read(B(0, 0), ring[1])
    for t in range(tiles):
        for s in range(nk):
            kt, ks = (t, s + 2) if s + 2 < nk else (t + 1, s + 2 - nk)   # what this step's copies fetch
            nt, nx = (t, s + 1) if s + 1 < nk else (t + 1, 0)            # the step read after the barrier
            # first half: this step's A blocks 4..7 and B block 7; A copies of step s + 2
            w.copy(A(kt, ks), ring[4], BF16_UNIT_COPIES)
            w.read(B(t, s), ring[1])
            for _ in range(4):
                w.read(A(t, s), ring[0])
            w.wait_reads()
            if s != 0:
                w.wait(BF16_UNIT_COPIES)
            w.barrier()
            # second half: B copies of step s + 2; the next step's A blocks 0..3 and B blocks 0..6
            w.copy(B(kt, ks), ring[b_copy_ring], BF16_UNIT_COPIES)
            for _ in range(4):
                w.read(A(nt, nx), ring[2])
            for _ in range(7):
                w.read(B(nt, nx), ring[3])
            ring = [ring[2], ring[3], ring[4], ring[0], ring[1]]
        # epilogue: every copy first, then the stores (not copies: not ordered against them)
        w.wait(0)
        w.tick()
    return w


@pytest.mark.parametrize("nk", range(4, 41))
def test_bf16_order(nk):
    """K > 192 (at least four steps) always takes this kernel."""
    bf16_run(nk, tiles=3)


def _fails_with_looser_waits(run, nk):
    """The model itself: with every nonzero wait one copy looser, a read must
    come before its unit is proven complete."""
    orig = Wave.wait

    def loose(self, n):
        return orig(self, n + 1 if n else n)
    Wave.wait = loose
    try:
        with pytest.raises(AssertionError, match="before every wave"):
            run(nk, 2)
    finally:
        Wave.wait = orig


def test_bf16_model_catches_a_looser_wait():
    w = bf16_run(8, 2)
    assert w.proven == len(w.copies)
    _fails_with_looser_waits(bf16_run, 8)


def test_bf16_model_catches_a_slot_still_to_be_read():
    """B copies into the slot of the next step's A tile, which the second
    half of the step still reads."""
    with pytest.raises(AssertionError, match="which holds|may still be read"):
        bf16_run(8, 2, b_copy_ring=2)


# ---- microscaled FP4 kernel -----------------------------------------------------

MX_COPIES = 4        # code copies per wave and step
MX_STAGES = 4
MX_SCALE_STEPS = 4   # steps per scale block
MX_SCALE_SLOTS = 2


def test_mx_constants_match_the_kernel():
    s = _src("gemm_mxfp4.hpp")
    assert "constexpr int COPIES = %d;" % MX_COPIES in s
    assert "constexpr int STAGES = %d;" % MX_STAGES in s
    assert "constexpr int SCALE_STEPS = %d;" % MX_SCALE_STEPS in s
    assert re.search(r"wait_reads\(\);\s*wait_copies_le<COPIES \* \(STAGES - 3\)>\(\);", s)
    assert "if constexpr (t % 4 == 1 && t < 4 * COPIES)\n                        copy_one(k + STAGES - 1, copy_stage, t / 4);" in s
    assert "if constexpr (block_start)\n                    copy_scales((k >> 2) + 1);" in s
    assert "copy_scales(0);" in s and "wait_copies_le<COPIES * (STAGES - 3)>();\n                lds_barrier();" in s


def mx_run(nk, tiles):
    """Stage k % 4 holds step k's codes; scale slot (blocks before + b) % 2 holds block b."""
    w = Wave(MX_STAGES + MX_SCALE_SLOTS)
    C = lambda t, k: ("codes", t, k)
    S = lambda t, b: ("scales", t, b)
    nb = nk // MX_SCALE_STEPS
    sslot = lambda t, b: MX_STAGES + ((t * nb + b) % MX_SCALE_SLOTS)

    def unit_of(t, k):            # step k of tile t, or of the next tile past the end
        return (t, k) if k < nk else (t + 1, k - nk)

    def sunit(t, b):
        return (t, b) if b < nb else (t + 1, b - nb)

    bound = MX_COPIES * (MX_STAGES - 3)
    # prologue of the first tile: scale block 0, steps 0..2
    w.copy(S(0, 0), sslot(0, 0), 1)
    for k in range(3):
        w.copy(C(0, k), k % MX_STAGES, MX_COPIES)
    w.wait(bound)
    w.barrier()
    for _ in range(3 + 4):
        w.read(C(0, 0), 0)
        w.read(S(0, 0), sslot(0, 0))
    for t in range(tiles):
        for k in range(nk):
            w.wait_reads()
            w.wait(bound)
            w.barrier()
            ct, ck = unit_of(t, k + 1)
            cur_s = S(t, k // MX_SCALE_STEPS)
            nxt_s = S(*sunit(t, (k + 1) // MX_SCALE_STEPS)) if k + 1 < nk else S(t + 1, 0)
            nxt_slot = sslot(*sunit(t, (k + 1) // MX_SCALE_STEPS)) if k + 1 < nk else sslot(t + 1, 0)
            for tt in range(32):
                g = tt >> 2
                if tt % 4 == 0:
                    if g < 5:
                        w.read(C(t, k), k % MX_STAGES)
                        w.read(cur_s, sslot(t, k // MX_SCALE_STEPS))
                    else:
                        w.read(C(ct, ck), (k + 1) % MX_STAGES)
                        w.read(nxt_s, nxt_slot)
                if tt % 4 == 2 and g < 4:
                    w.read(C(ct, ck), (k + 1) % MX_STAGES)
                    w.read(nxt_s, nxt_slot)
                if tt % 4 == 1 and tt < 4 * MX_COPIES:
                    ut, uk = unit_of(t, k + MX_STAGES - 1)
                    w.copy(C(ut, uk), (k + MX_STAGES - 1) % MX_STAGES, 1, total=MX_COPIES)
            if k % MX_SCALE_STEPS == 0:
                bt, bb = sunit(t, k // MX_SCALE_STEPS + 1)
                w.copy(S(bt, bb), sslot(bt, bb), 1)
        # epilogue: bias loads and stores only (not copies)
        w.tick()
    return w


@pytest.mark.parametrize("nk", range(4, 41, 4))
def test_mx_order(nk):
    """K % 512 == 0: the step count is a multiple of four."""
    mx_run(nk, tiles=3)


def test_mx_model_catches_a_looser_wait():
    _fails_with_looser_waits(mx_run, 8)


def test_mx_wait_counting_stores_would_not_prove_the_next_step():
    """The earlier first-step bound (one step's copies plus the 16 epilogue
    stores) proves nothing about step 1 once stores may complete first."""
    w = Wave(MX_STAGES)
    for k in range(3):
        w.copy(("codes", 1, k), k, MX_COPIES)
    w.wait(MX_COPIES + 16)
    assert w.proven == 0
    w.wait(MX_COPIES)
    assert w.copies[:w.proven] == [("codes", 1, 0)] * MX_COPIES + [("codes", 1, 1)] * MX_COPIES


# ---- BF16 64 x 64 long-K kernel ---------------------------------------------------

SL_A_SLOTS = 8       # A ring: one step per unit
SL_B_SLOTS = 3       # B ring: SUPER steps per unit (512-byte rows)
SL_SUPER = 4
SL_A_COPIES = 2      # per wave and step
SL_B_COPIES = 2      # per wave and step (one part of a B unit)


def sl_wait_left(phase):
    return 22 if phase == 0 else 18 if phase == 3 else 24


def test_small_long_constants_match_the_kernel():
    s = _src("gemm_bf16_small_long.hpp")
    assert "constexpr int A_SLOTS = %d;" % SL_A_SLOTS in s
    assert "static constexpr int SLOTS = %d;" % SL_B_SLOTS in s
    assert "constexpr int A_COPIES = %d;" % SL_A_COPIES in s
    assert "constexpr int B_COPIES = %d;" % SL_B_COPIES in s
    assert "static_assert(SUPER == %d," % SL_SUPER in s
    assert "static constexpr int wait_left(int phase) { return phase == 0 ? 22 : phase == 3 ? 18 : 24; }" in s
    assert re.search(r"copy_b\(s / SUPER \+ B_SLOTS - 1, Int<phase>\{\}\);\s*copy_a\(s \+ A_SLOTS - 1\);\s*"
                     r"wait_reads\(\);\s*wait_copies_left<BS::wait_left\(phase\)>\(\);\s*lds_barrier\(\);", s)
    assert "wait_copies_left<BS::wait_left(SUPER - 1)>();" in s


def small_long_run(nk):
    """One tile (each tile starts from drained rings): the prologue issues what
    steps -8 .. -1 would have, then step s copies part s % 4 of B unit s / 4 + 2
    and the A tile of step s + 7 (past K as zeros, still issued), waits, and
    after the barrier reads step s + 1."""
    w = Wave(SL_A_SLOTS + SL_B_SLOTS)
    A = lambda s: ("A", s)
    B = lambda j: ("B", j)
    aslot = lambda s: s % SL_A_SLOTS
    bslot = lambda j: SL_A_SLOTS + j % SL_B_SLOTS

    def copy_b(j):
        w.copy(B(j), bslot(j), SL_B_COPIES, total=SL_SUPER * SL_B_COPIES)

    def copy_a(s):
        w.copy(A(s), aslot(s), SL_A_COPIES)

    def read_step(s):
        for _ in range(4):
            w.read(A(s), aslot(s))
            w.read(B(s // SL_SUPER), bslot(s // SL_SUPER))

    w.wait_reads()
    w.wait(0)
    w.barrier()
    for t in range(-SL_SUPER * (SL_B_SLOTS - 1), 0):
        unit = (t - t % SL_SUPER) // SL_SUPER + SL_B_SLOTS - 1
        if unit >= 0:
            copy_b(unit)
        if t + SL_A_SLOTS - 1 >= 0:
            copy_a(t + SL_A_SLOTS - 1)
    w.wait(sl_wait_left(SL_SUPER - 1))
    w.barrier()
    read_step(0)
    for s in range(nk):
        copy_b(s // SL_SUPER + SL_B_SLOTS - 1)
        copy_a(s + SL_A_SLOTS - 1)
        w.wait_reads()
        w.wait(sl_wait_left(s % SL_SUPER))
        w.barrier()
        read_step(s + 1)
    w.wait_reads()
    w.wait(0)
    return w


@pytest.mark.parametrize("nk", range(1, 61))
def test_small_long_order(nk):
    small_long_run(nk)


def test_small_long_model_catches_a_looser_wait():
    _fails_with_looser_waits(lambda nk, tiles: small_long_run(nk), 12)


# ---- rings of whole-step units: the 64 x 64 kernel and the split-K kernel ----------

def ring_run(nk, stages, copies, wait_bound, tiles):
    """A wave that copies one unit of `copies` parts per step, `stages` - 1
    steps ahead, into a ring of `stages` slots; every tile starts from a
    drained ring. Step s copies step s + stages - 1 (past K as zeros, still
    issued) into the slot of step s - 1, waits, and after the barrier reads
    step s + 1."""
    w = Wave(stages)
    ahead = stages - 1
    for t in range(tiles):
        U = lambda s: ("step", t, s)
        w.wait_reads()
        w.wait(0)
        w.barrier()
        for s in range(ahead):
            w.copy(U(s), s % stages, copies)
        w.wait(wait_bound)
        w.barrier()
        w.read(U(0), 0)
        for s in range(nk):
            w.copy(U(s + ahead), (s + ahead) % stages, copies)
            w.wait_reads()
            w.wait(wait_bound)
            w.barrier()
            w.read(U(s + 1), (s + 1) % stages)
        w.tick()   # epilogue stores
    return w


def test_small_and_splitk_constants_match_the_kernels():
    s = _src("gemm_bf16_small.hpp")
    assert "constexpr int STAGES = 10;" in s and "constexpr int COPIES = 4;" in s
    assert s.count("wait_copies_le<COPIES * (STAGES - 2)>();") == 2
    assert "copy(s + STAGES - 1, Int<3>{});\n            wait_reads();" in s
    k = _src("gemm_bf16_splitk.hpp")
    assert "constexpr int A_STAGES = 3;" in k and "constexpr int B_STAGES = 7;" in k
    assert "constexpr int COPIES = 4;" in k
    assert re.search(r"if \(copies_b\)\s*wait_copies_le<COPIES \* \(B_STAGES - 2\)>\(\);\s*else\s*"
                     r"wait_copies_le<COPIES \* \(A_STAGES - 2\)>\(\);", k)
    assert "copy_step(ls + stages - 1);\n        // this wave's reads of step ls and its copies of step ls + 1 are done\n        wait_reads();\n        wait_next();" in k


@pytest.mark.parametrize("nk", range(1, 41))
@pytest.mark.parametrize("stages", [10, 3, 7])   # the 64 x 64 ring; split-K's A and B rings
def test_ring_order(nk, stages):
    ring_run(nk, stages, 4, 4 * (stages - 2), tiles=2)


def test_ring_model_catches_a_looser_wait():
    _fails_with_looser_waits(lambda nk, tiles: ring_run(nk, 7, 4, 20, tiles), 12)
