"""A host model of the one-launch step's schedule (query_aware_kv_amd/csrc/
step.hip): an ordered ticket queue, per-row estimate counters whose last
finisher runs the row's Top-K and raises a ready flag, attention items that
wait for their row's flag, per-row attention counters whose last finisher
merges the row, and last-one-out reset of the queue.

Workgroups are threads; a semaphore with fewer slots than workgroups plays
the hardware dispatcher (a workgroup holds its slot until it exits), so the
model covers grids larger than what fits on the device at once.  Random
delays shuffle the interleavings.  Checked: every run ends, each row's
Top-K runs once and only after all its counted estimate items, every
attention item starts after its row's Top-K, each row is merged once after
all its splits, and the control words are zero again at the end.
"""
import random
import threading
import time

import pytest

EST_ITEM_PAGES = 64
ATTN_WAVES = 4


class Model:
    def __init__(self, lens, hkv, max_pages, k, ppw, grid, resident, seed):
        self.rng = random.Random(seed)
        self.lens, self.hkv, self.mp, self.k = lens, hkv, max_pages, k
        self.rows = len(lens) * hkv
        self.est_items = -(-max_pages // EST_ITEM_PAGES)
        self.attn_items = -(-k // (ATTN_WAVES * ppw))
        self.n_est = self.rows * self.est_items
        self.n_attn = self.rows * self.attn_items
        self.grid, self.slots = grid, threading.Semaphore(resident)
        self.lock = threading.Lock()
        self.ticket = self.exited = 0
        self.est_done = [0] * self.rows
        self.ready = [0] * self.rows
        self.attn_done = [0] * self.rows
        self.events = []          # (kind, row, detail) in completion order
        self.est_finished = [0] * self.rows
        self.attn_finished = [0] * self.rows

    def atomic_add(self, arr, i, v=1):
        with self.lock:
            old = arr[i]
            arr[i] += v
            return old

    def log(self, *e):
        with self.lock:
            self.events.append(e)

    def pause(self):
        if self.rng.random() < 0.3:
            time.sleep(self.rng.random() * 1e-4)

    def row_pages(self, row):
        L = self.lens[row // self.hkv]
        return min(-(-L // 16), self.mp) if L > 0 else 0

    def est_item(self, t):
        row, blk = divmod(t, self.est_items)
        counted = max(1, -(-self.row_pages(row) // EST_ITEM_PAGES))
        self.pause()
        if blk >= counted:
            return
        with self.lock:
            self.est_finished[row] += 1
        if self.atomic_add(self.est_done, row) != counted - 1:
            return
        with self.lock:   # Top-K only after every counted item of the row
            assert self.est_finished[row] == counted
        self.log("topk", row)
        self.pause()
        self.est_done[row] = 0
        self.ready[row] = 1

    def attn_item(self, t):
        row, split = divmod(t, self.attn_items)
        spins = 0
        while self.ready[row] == 0:
            spins += 1
            assert spins < 2_000_000, "wait did not end"
            time.sleep(1e-6)
        self.log("attn", row, split)
        self.pause()
        if self.attn_items == 1:
            self.log("merge", row)
            self.ready[row] = 0
            return
        with self.lock:
            self.attn_finished[row] += 1
        if self.atomic_add(self.attn_done, row) != self.attn_items - 1:
            return
        with self.lock:
            assert self.attn_finished[row] == self.attn_items
        self.log("merge", row)
        self.attn_done[row] = 0
        self.ready[row] = 0

    def workgroup(self):
        with self.slots:
            total = self.n_est + self.n_attn
            while True:
                with self.lock:
                    t = self.ticket
                    self.ticket += 1
                if t >= total:
                    break
                if t < self.n_est:
                    self.est_item(t)
                else:
                    self.attn_item(t - self.n_est)
            with self.lock:      # last one out resets the queue
                self.exited += 1
                if self.exited == self.grid:
                    self.ticket = self.exited = 0

    def run(self):
        ths = [threading.Thread(target=self.workgroup) for _ in range(self.grid)]
        for th in ths:
            th.start()
        for th in ths:
            th.join(timeout=60)
            assert not th.is_alive(), "a workgroup never finished"


@pytest.mark.parametrize("seed", range(12))
def test_schedule_model(seed):
    rng = random.Random(seed)
    B = rng.randint(1, 4)
    hkv = rng.choice([1, 2, 4])
    mp = rng.choice([3, 64, 65, 200])
    lens = [rng.choice([0, 1, 16, 17, rng.randint(1, mp * 16)]) for _ in range(B)]
    k = rng.choice([1, 4, 8, 40])
    ppw = rng.choice([1, 2])
    m = Model(lens, hkv, mp, k, ppw, grid=rng.randint(1, 24),
              resident=rng.randint(1, 6), seed=seed)
    for _ in range(2):   # two calls through the same control words
        m.events = []
        m.run()
        topk = [e[1] for e in m.events if e[0] == "topk"]
        merge = [e[1] for e in m.events if e[0] == "merge"]
        assert sorted(topk) == list(range(m.rows))
        assert sorted(merge) == list(range(m.rows))
        first_topk = {}
        for i, e in enumerate(m.events):
            if e[0] == "topk":
                first_topk[e[1]] = i
            elif e[0] == "attn":
                assert e[1] in first_topk, "attention before its Top-K"
        assert m.ticket == 0 and m.exited == 0
        assert m.est_done == [0] * m.rows and m.attn_done == [0] * m.rows
        assert m.ready == [0] * m.rows
        m.est_finished = [0] * m.rows
        m.attn_finished = [0] * m.rows
