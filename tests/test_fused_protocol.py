"""CPU model of the fused kernel's producer/consumer protocol (one team).

The fused forward kernel (csrc/kda_fused.hip) passes chunk records from P
producer workgroups to NCW consumer workgroups through a ring of R slots:

  producer p, items i = p, p + P, ...:  wait until min(progress) >= i - R + 1;
      write the record of item i into slot i % R (many separate stores);
      ready[i % R] = i + 1.
  consumer: wait ready[0]; read both halves of item 0; for each item i:
      progress = i (items < i fully read); use the U half of item i;
      wait ready[(i+1) % R] == i + 2 and read the U half of item i + 1;
      use the S half of item i; read the S half of item i + 1;
      at the end progress = n.

Threads stand in for workgroups, with random delays between every step and
between the stores of one record.  The model checks that every value a
consumer reads belongs to the item it expects (a slot is never overwritten
before every consumer has read it), that the run finishes (no deadlock) for
any ring of at least two slots (one slot deadlocks: the consumer looks one
item ahead), and that a bounded wait turns a stuck producer, or that
deadlock, into an error instead of a hang.
"""

import random
import threading
import time

import pytest

PARTS = 6      # stores per record half


class Team:
    def __init__(self, n_items, P, R, NCW, seed, stuck_item=None, max_polls=None):
        self.n, self.P, self.R, self.NCW = n_items, P, R, NCW
        self.rng = random.Random(seed)
        self.slots = [[-1] * (2 * PARTS) for _ in range(R)]
        self.ready = [0] * R
        self.prog = [0] * NCW
        self.errors = []
        self.err_bits = 0
        self.stuck_item = stuck_item
        self.max_polls = max_polls
        self.lock = threading.Lock()

    def pause(self):
        time.sleep(self.rng.random() * 2e-4)

    def wait(self, cond, who):
        polls = 0
        while not cond():
            polls += 1
            if self.max_polls is not None and polls > self.max_polls:
                with self.lock:
                    self.err_bits |= 2 if who == "consumer" else 4
                return False
            time.sleep(1e-5)
        return True

    def producer(self, p):
        dead = False
        for i in range(p, self.n, self.P):
            if i == self.stuck_item:
                return  # a producer that never delivers
            if i >= self.R and not dead:
                if not self.wait(lambda: min(self.prog) >= i - self.R + 1, "producer"):
                    dead = True
            slot = self.slots[i % self.R]
            for k in range(2 * PARTS):   # the record is many separate stores
                slot[k] = i
                self.pause()
            self.ready[i % self.R] = i + 1

    def consumer(self, w):
        dead = False

        def wait_ready(i):
            nonlocal dead
            if not dead and not self.wait(lambda: self.ready[i % self.R] == i + 1, "consumer"):
                dead = True

        def read_half(i, half):
            s = self.slots[i % self.R]
            vals = []
            for k in range(half * PARTS, (half + 1) * PARTS):
                vals.append(s[k])
                self.pause()
            return vals

        if self.n == 0:
            return
        wait_ready(0)
        u, s_half = read_half(0, 0), read_half(0, 1)
        for i in range(self.n):
            if i > 0:
                self.prog[w] = i
            if not dead and u != [i] * PARTS:
                self.errors.append(("U half", w, i, u))
            self.pause()
            if i + 1 < self.n:
                wait_ready(i + 1)
                u = read_half(i + 1, 0)
            if not dead and s_half != [i] * PARTS:
                self.errors.append(("S half", w, i, s_half))
            if i + 1 < self.n:
                s_half = read_half(i + 1, 1)
        self.prog[w] = self.n

    def run(self, timeout=60.0):
        threads = [threading.Thread(target=self.producer, args=(p,), daemon=True) for p in range(self.P)]
        threads += [threading.Thread(target=self.consumer, args=(w,), daemon=True) for w in range(self.NCW)]
        self.rng.shuffle(threads)
        for t in threads:
            t.start()
        deadline = time.time() + timeout
        for t in threads:
            t.join(max(0.0, deadline - time.time()))
        return not any(t.is_alive() for t in threads)


@pytest.mark.parametrize("n_items,P,R,NCW,seed", [
    (60, 12, 12, 4, 1),   # the dense layout: 12 producers, 12 slots, 4 consumers
    (37, 12, 12, 4, 2),   # ragged item count
    (40, 6, 3, 2, 3),     # fewer slots than producers
    (25, 4, 2, 3, 4),     # two slots, the fewest the protocol allows
    (5, 12, 12, 4, 5),    # fewer items than producers
    (0, 3, 3, 2, 6),      # nothing to do
])
def test_protocol_delivers_every_item_intact_without_deadlock(n_items, P, R, NCW, seed):
    team = Team(n_items, P, R, NCW, seed)
    assert team.run(), "deadlock"
    assert team.errors == []
    assert team.prog == [n_items] * NCW and team.err_bits == 0


def test_a_single_slot_would_deadlock_and_the_bounded_waits_report_it():
    # With one slot, the producer of item i + 1 waits for item i to be read
    # while the consumer waits for item i + 1 before finishing item i: the
    # kernel therefore requires R >= 2 (its layout never picks fewer).
    team = Team(25, 4, 1, 3, 4, max_polls=2000)
    assert team.run(timeout=120.0)
    assert team.err_bits != 0


def test_bounded_waits_turn_a_stuck_producer_into_an_error():
    team = Team(30, 4, 4, 2, 7, stuck_item=9, max_polls=2000)
    assert team.run(timeout=120.0), "a stuck producer must not hang the team"
    assert team.err_bits & 2          # the consumers' wait for item 9 timed out
