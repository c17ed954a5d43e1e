"""A second, independent formulation of the expert-cache policy (tests only).

Where the oracle keeps one "last miss" time per expert and one stamp per
slot, this keeps the full history: every miss time of an expert since its
last reset, and every use time of a slot since its current owner arrived.
Admission asks whether any remembered miss lies inside the window; a slot's
stamp is the latest use in its history. The miss log is a list of
(t, layer, expert) tuples sorted as tuples. Slow (quadratic), for small
random traces.
"""
from __future__ import annotations


class PolicyRef:
    def __init__(self, L, E, S, k, window=64, admit=2):
        self.L, self.E, self.S, self.k, self.window, self.admit = L, E, S, k, window, admit
        self.seed(None)

    def seed(self, freq):
        self.where = {}  # (layer, e) -> slot
        self.owner = [[None] * self.S for _ in range(self.L)]
        self.uses = [[[] for _ in range(self.S)] for _ in range(self.L)]
        self.misses_since_reset = {}
        self.counts = [[0] * self.E for _ in range(self.L)]
        if freq is not None:
            for layer in range(self.L):
                order = sorted(range(self.E), key=lambda e: (-int(freq[layer][e]), e))
                for s, e in enumerate(order[: self.S]):
                    self.where[(layer, e)] = s
                    self.owner[layer][s] = e
        self.clock = 1
        self.log = []
        self.step_tokens = 0
        self.hits = 0
        self.last_log = []

    def forward(self, layer, ids):
        T = len(ids)
        for t in range(T):
            clk = self.clock + t
            for e in ids[t]:
                e = int(e)
                self.counts[layer][e] += 1
                if (layer, e) in self.where:
                    self.uses[layer][self.where[(layer, e)]].append(clk)
                    self.hits += 1
                else:
                    self.log.append((clk, layer, e))
        self.step_tokens = max(self.step_tokens, T)

    def _stamp(self, layer, s):
        return max(self.uses[layer][s]) if self.uses[layer][s] else 0

    def step(self):
        entries = sorted(self.log)
        adm = ev = 0
        admissions = []
        for (t, layer, e) in entries:
            if (layer, e) in self.where:
                continue
            hist = self.misses_since_reset.setdefault((layer, e), [])
            if self.admit == 1:
                ok = True
            else:
                ok = any(t - tp < self.window for tp in hist)
                if not ok:
                    hist.append(t)
            if not ok or self.S == 0:
                continue
            free = [s for s in range(self.S) if self.owner[layer][s] is None]
            evicted = -1
            if free:
                victim = min(free)
            else:
                victim = max(range(self.S), key=lambda s: (-self._stamp(layer, s), s))
                evicted = self.owner[layer][victim]
                del self.where[(layer, evicted)]
                self.misses_since_reset[(layer, evicted)] = []
                ev += 1
            self.owner[layer][victim] = e
            self.where[(layer, e)] = victim
            self.uses[layer][victim] = [t]
            self.misses_since_reset[(layer, e)] = []
            adm += 1
            admissions.append((layer, e, victim, evicted))
        stats = dict(hits=self.hits, misses=len(self.log), admissions=adm, evictions=ev, tokens=self.step_tokens)
        self.last_log = [(t << 32) | (layer << 12) | e for (t, layer, e) in entries]
        self.last_admissions = admissions
        self.log = []
        self.hits = 0
        self.clock += self.step_tokens
        self.step_tokens = 0
        return stats

    def table(self):
        return [[self.where.get((layer, e), -1) for e in range(self.E)] for layer in range(self.L)]

    def stamps(self):
        return [[self._stamp(layer, s) for s in range(self.S)] for layer in range(self.L)]
