"""The one-launch factorisation's schedule, checked on the CPU.

ispa_absorb_solve factorises G + lambda I in one launch for one layer with d <= 2048: work-group 0
carries the diagonal blocks, work-groups 1 and 2 bring the next row up to it one and two panels
behind, and the other work-groups take the trailing updates, the identity-part updates, the final
T_r B_rc blocks and the R / P blocks from a queue ordered by panel.  They exchange blocks through
device memory with a version number per block.  This file restates that protocol (which agent
waits for which versions, and which versions it reads and writes) and runs it under random
interleavings and worker counts, checking that it never deadlocks, that every read finds exactly
the version it expects (no block is overwritten before its last reader has read it), and that every
block ends at its final version.  It also checks that the queue's task count is the sum of the
per-panel counts.  It is a model of the protocol in kv_cache_attention_ispa_amd/csrc/solve.hip
(psweep_kernel); the GPU tests check the kernel's results bit for bit against the per-panel path.
"""
import random

import pytest

CHAIN = 6   # A-task entries per panel that belong to work-groups 0-2 (rows p+1 .. p+3)


def n_a(m):
    return m * (m + 1) // 2 - CHAIN if m * (m + 1) // 2 > CHAIN else 0


def count(nP, p):
    m = nP - 1 - p
    return n_a(m) + m * (p + 1) + p


def rp_count(n_rp, share, p):
    left = n_rp - p * share
    return 0 if left <= 0 else min(left, share)


def tri_decode(q):
    r = 0
    while (r + 1) * (r + 2) // 2 <= q:
        r += 1
    return r, q - r * (r + 1) // 2


def tasks(nP, n_rp):
    share = -(-n_rp // nP)
    out = []
    for p in range(nP):
        m = nP - 1 - p
        for q in range(n_a(m)):
            ii, jj = tri_decode(q + CHAIN)
            out.append(("A", p, p + 1 + ii, p + 1 + jj))
        for q in range(m * (p + 1)):
            out.append(("B", p, p + 1 + q // (p + 1), q % (p + 1)))
        for c in range(p):
            out.append(("F", p, p, c))
        for q in range(rp_count(n_rp, share, p)):
            out.append(("RP", p, p * share + q, 0))
    assert len(out) == sum(count(nP, p) + rp_count(n_rp, share, p) for p in range(nP))
    return out


class Schedule:
    def __init__(self, nP, workers, rng):
        self.nP, self.rng = nP, rng
        nT = nP
        self.n_rp = nT * nT + nT * (nT + 1) // 2
        self.queue = tasks(nP, self.n_rp)
        self.next = 0
        self.held = [None] * workers
        self.done = 0
        self.rp_done = set()
        self.tflag = 0          # T_k and X slot k published for k < tflag
        self.verA, self.verB, self.memA, self.memB = {}, {}, {}, {}
        self.wg0, self.wg1, self.wg2 = 0, 1, 2

    def vA(self, i, j):
        return self.verA.get((i, j), 0)

    def vB(self, i, c):
        return self.verB.get((i, c), 0)

    def read_a(self, i, j, v, who):
        if v:   # version 0 is G itself
            got = self.memA.get((i, j), 0)
            assert got == v, f"{who}: A({i},{j}) expected version {v}, memory holds {got}"

    def read_b(self, i, c, v, who):
        got = self.memB.get((i, c), 0)
        assert got == v, f"{who}: B({i},{c}) expected version {v}, memory holds {got}"

    def write_a(self, i, j, v, flag=True):
        self.memA[(i, j)] = v
        if flag:
            self.verA[(i, j)] = v

    # work-group 0, step k: reads (k+1, k) and (k+1, k+1) at version k (work-group 1's), factors,
    # publishes T_k and X_{k+1}
    def step_wg0(self):
        k = self.wg0
        if k >= self.nP:
            return False
        if k + 1 < self.nP:
            if k >= 1 and self.vA(k + 1, k + 1) < k:
                return False
            self.read_a(k + 1, k, k, "wg0")
            self.read_a(k + 1, k + 1, k, "wg0")
        self.tflag = k + 1
        self.wg0 += 1
        return True

    # work-group 1, round k: panel k-1 on (k+1, k), (k+1, k+1)
    def step_wg1(self):
        k = self.wg1
        r = k + 1
        if r >= self.nP:
            return False
        if self.tflag < k or (k >= 2 and self.vA(r, r) < k - 1):
            return False
        for c in (k - 1, k, r):
            self.read_a(r, c, k - 1, "wg1")
        self.write_a(r, k, k)
        self.write_a(r, r, k)
        self.wg1 += 1
        return True

    # work-group 2, round k: panel k-2 on (k+1, k-1 .. k+1) from the workers' versions k-2
    def step_wg2(self):
        k = self.wg2
        r = k + 1
        if r >= self.nP:
            return False
        if self.tflag < k - 1:
            return False
        if k >= 3 and not all(self.vA(r, c) >= k - 2 for c in (k - 2, k - 1, k, r)):
            return False
        for c in (k - 2, k - 1, k, r):
            self.read_a(r, c, k - 2, "wg2")
        for c in (k - 1, k, r):
            self.write_a(r, c, k - 1)
        self.wg2 += 1
        return True

    def step_worker(self, w):
        t = self.held[w]
        if t is None:
            if self.next >= len(self.queue):
                return False
            self.held[w] = self.queue[self.next]
            self.next += 1
            return True
        kind, p, i, j = t
        who = f"task {t}"
        if kind == "A":
            if not (self.tflag >= p + 1 and self.vA(i, p) >= p and self.vA(j, p) >= p and self.vA(i, j) >= p):
                return False
            self.read_a(i, p, p, who)
            self.read_a(j, p, p, who)
            self.read_a(i, j, p, who)
            self.write_a(i, j, p + 1)
        elif kind == "B":
            c = j
            if not (self.tflag >= p + 1 and self.vA(i, p) >= p):
                return False
            if c < p and not (self.vB(p, c) >= p - c and self.vB(i, c) >= p - c):
                return False
            self.read_a(i, p, p, who)
            if c < p:
                self.read_b(p, c, p - c, who)
                self.read_b(i, c, p - c, who)
            self.memB[(i, c)] = self.verB[(i, c)] = p - c + 1
        elif kind == "F":
            c = j
            if not (self.tflag >= p + 1 and self.vB(p, c) >= p - c):
                return False
            if p > c:
                self.read_b(p, c, p - c, who)
        else:
            assert i not in self.rp_done
            self.rp_done.add(i)
        self.held[w] = None
        self.done += 1
        return True

    def run(self):
        agents = ["wg0", "wg1", "wg2"] + list(range(len(self.held)))
        while True:
            self.rng.shuffle(agents)
            if not any(getattr(self, "step_" + a)() if isinstance(a, str) else self.step_worker(a) for a in agents):
                break
        stuck = f"wg0 {self.wg0} wg1 {self.wg1} wg2 {self.wg2} tasks {self.done}/{len(self.queue)}"
        assert self.wg0 == self.nP and self.done == len(self.queue), "deadlock: " + stuck
        assert self.wg1 + 1 >= self.nP and self.wg2 + 1 >= self.nP, "deadlock: " + stuck
        assert self.rp_done == set(range(self.n_rp))
        for i in range(self.nP):
            for j in range(1, i):
                assert self.memA.get((i, j), 0) == j, f"A({i},{j}) ends at version {self.memA.get((i, j), 0)}"
            for c in range(i):
                assert self.memB.get((i, c), 0) == i - c


@pytest.mark.parametrize("nP", [1, 2, 3, 4, 5, 6, 7, 9, 12, 16, 24, 32])
def test_schedule_never_deadlocks_and_reads_exact_versions(nP):
    rng = random.Random(1000 + nP)
    for workers in (1, 2, 5, 40, 253):
        for _ in range(3):
            Schedule(nP, workers, rng).run()


def test_planted_mistake_is_caught():
    """The check has teeth: a work-group 1 that publishes (k+1, k) one version early lets a worker
    read a block before its last update, which the model reports."""
    class Early(Schedule):
        def step_wg1(self):
            k = self.wg1
            r = k + 1
            if r >= self.nP or self.tflag < k:
                return False
            self.verA[(r, k)] = k   # flag set before the block is written
            return super().step_wg1()
    with pytest.raises(AssertionError):
        for seed in range(20):
            Early(8, 40, random.Random(seed)).run()
