"""The extend kernel's hand-counted load schedule, checked on the host.

extend_kernel loads K/V rows and page-table entries straight into LDS with
inline-assembly loads and waits for them with count-based waits (`s_waitcnt
vmcnt(k)`: every vector-memory op of the wavefront except the last k issued has
completed).  This test reads the schedule's constants from the kernel source,
replays one wavefront's op stream in the order the kernel issues it, and
checks that
  * every wait covers the op it guards (ring entries before they are read,
    the next tile's rows before the barrier that hands them to every
    wavefront),
  * no LDS stage and no ring slot is overwritten before its last reader,
  * every iteration issues exactly kOpsPerTile ops (the wait counts assume it).
A planted error in each wait count must be caught."""
import pathlib
import re

import pytest

SRC = pathlib.Path(__file__).resolve().parent.parent / "paged_kv_attention_08_amd" / "csrc" / "extend.hip"
COMMON = SRC.parent / "common.hpp"


def constants():
    """The integer constexprs of common.hpp and extend.hip, evaluated in order."""
    env = {}
    for path in (COMMON, SRC):
        for name, expr in re.findall(r"^constexpr int (\w+) = ([^;]+);", path.read_text(), re.M):
            env[name] = eval(expr.replace("/", "//"), {}, dict(env))
    return env


def source():
    return SRC.read_text()


def test_source_has_the_replayed_structure():
    """The program replayed below, as the kernel source writes it."""
    s = source()
    assert re.search(r"load_entries\(0\);\s*load_entries\(1\);\s*load_entries\(2\);\s*"
                     r'asm volatile\("s_waitcnt vmcnt\(0\)"', s)
    assert re.search(r"read_entries\(0\);\s*issue\(-3\);\s*issue\(-2\);\s*issue\(-1\);\s*finish\(\);", s)
    assert "load_entries(n + kEntryLead);" in s
    assert "const int m = n + kRowLead;" in s
    assert 'asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kWaitEntries) : "memory");\n    read_entries(n + kRowLead + 1);' in s
    assert 's_waitcnt vmcnt(%0) lgkmcnt(0)\\n\\ts_barrier" ::"n"(kWaitRows)' in s
    # per iteration: one entry load, then kLoads x (K row load, V row load)
    issue = s[s.index("auto issue = [&](int n)"):s.index("auto finish = [&]()")]
    assert issue.count("lds_load16(") == 2 and "for (int u = 0; u < kLoads; ++u)" in issue
    assert s.count("lds_load4(") == 2 and s.count("lds_load4(pt_row") == 1  # the helper and its one call
    assert re.search(r"key_tile\(n \+ 3, std::integral_constant<int, 3>\{\}\);", s)  # 4 stages unrolled


class Wave:
    """One wavefront's vector-memory ops in issue order, with their state."""

    def __init__(self):
        self.ops = []        # (kind, tile)
        self.done = []       # completion flags
        self.errors = []

    def issue(self, kind, tile):
        self.ops.append((kind, tile))
        self.done.append(False)

    def wait(self, k):
        for i in range(max(0, len(self.ops) - k)):
            self.done[i] = True

    def complete(self, kind, tile):
        idx = [i for i, op in enumerate(self.ops) if op == (kind, tile)]
        return bool(idx) and all(self.done[i] for i in idx)


def replay(c, n_tiles, wait_entries=None, wait_rows=None):
    """Replays the kernel's schedule for n_tiles key tiles; returns the list of
    violations found."""
    S, R = c["kStages"], c["kRingSlots"]
    lead_rows, lead_entries = c["kRowLead"], c["kEntryLead"]
    w_ent = c["kWaitEntries"] if wait_entries is None else wait_entries
    w_rows = c["kWaitRows"] if wait_rows is None else wait_rows
    w = Wave()
    errors = w.errors
    ring = {}          # slot -> tile whose entries it holds
    ring_read = set()  # tiles whose entries were read from the ring
    stage = {}         # stage -> tile whose rows it holds (rows issued)
    barriers_after = {}  # tile -> whether the barrier ending its iteration passed
    ent_regs = None

    def load_entries(t):
        slot = t % R
        old = ring.get(slot)
        if old is not None and old not in ring_read:
            errors.append(f"ring slot {slot}: entries of tile {old} overwritten by tile {t} before they were read")
        ring[slot] = t
        w.issue("E", t)

    def read_entries(t):
        nonlocal ent_regs
        if not w.complete("E", t):
            errors.append(f"entries of tile {t} read before their load completed")
        if ring.get(t % R) != t:
            errors.append(f"ring slot of tile {t} holds tile {ring.get(t % R)}")
        ring_read.add(t)
        ent_regs = t

    def issue(n):
        load_entries(n + lead_entries)
        m = n + lead_rows
        if ent_regs != m:
            errors.append(f"rows of tile {m} issued from the entries of tile {ent_regs}")
        st = m % S
        old = stage.get(st)
        if old is not None and old >= 0 and not barriers_after.get(old, False) and old != m:
            errors.append(f"stage {st}: rows of tile {m} issued before every wavefront finished tile {old}")
        stage[st] = m
        for _ in range(c["kLoads"]):
            w.issue("K", m)
            w.issue("V", m)
        w.wait(w_ent)
        read_entries(n + lead_rows + 1)

    def finish(n_next):
        w.wait(w_rows)
        if n_next < n_tiles and not (w.complete("K", n_next) and w.complete("V", n_next)):
            errors.append(f"barrier before tile {n_next} passed with its rows still in flight")

    # prologue
    for t in range(lead_entries - lead_rows):
        load_entries(t)
    w.wait(0)
    read_entries(0)
    for n in range(-lead_rows, 0):
        before = len(w.ops)
        issue(n)
        if len(w.ops) - before != c["kOpsPerTile"]:
            errors.append("an issue step does not issue kOpsPerTile ops")
    finish(0)
    for n in range(n_tiles):
        before = len(w.ops)
        issue(n)
        if len(w.ops) - before != c["kOpsPerTile"]:
            errors.append("an issue step does not issue kOpsPerTile ops")
        if stage.get(n % S) != n:
            errors.append(f"tile {n} computed from stage {n % S} holding tile {stage.get(n % S)}")
        finish(n + 1)
        barriers_after[n] = True
    w.wait(0)
    return errors


@pytest.mark.parametrize("n_tiles", [1, 2, 3, 4, 5, 7, 8, 9, 13, 64])
def test_schedule_holds(n_tiles):
    c = constants()
    assert c["kOpsPerTile"] == 1 + 2 * c["kLoads"]
    errs = replay(c, n_tiles)
    assert not errs, errs[:5]


def test_planted_wait_errors_are_caught():
    """One op too few waited for, at either wait, must be reported."""
    c = constants()
    assert replay(c, 9, wait_entries=c["kWaitEntries"] + 1)
    assert replay(c, 9, wait_rows=c["kWaitRows"] + 1)
    # stricter waits stay correct (only slower)
    assert not replay(c, 9, wait_entries=c["kWaitEntries"] - 1, wait_rows=c["kWaitRows"] - 1)


def test_planted_lead_errors_are_caught():
    """Entries loaded too far ahead for the ring, or rows too far ahead for
    the stages, must be reported."""
    c = dict(constants())
    bad = dict(c, kEntryLead=c["kRowLead"] + c["kRingSlots"] + 1)
    assert replay(bad, 12)
    bad = dict(c, kRowLead=c["kStages"], kEntryLead=c["kStages"] + 3)
    assert replay(bad, 12)


def test_lds_layout_constants():
    """The byte budget and the immediate-offset reach the kernel relies on:
    every operand read is a per-lane base plus a 16-bit immediate holding the
    stage and key-block offsets."""
    c = constants()
    assert c["kTileBytes"] == c["kKeyTile"] * c["kHeadDim"] * 2
    assert c["kLdsBytes"] <= 160 * 1024
    last_stage = (c["kStages"] - 1) * c["kTileBytes"]
    assert last_stage + 8192 <= 65535          # K: stage + second 32-key block
    assert last_stage + 8192 + 4096 <= 65535   # V: stage + 32-key block + 16-key half
