"""A second, independent formulation of the expert-cache policy (tests only).

Where the oracle keeps one "last miss" time per expert and one stamp per
slot, this keeps the full history: every miss time of an expert since its
last reset, and every use time of a slot since its current owner arrived.
Admission asks whether any remembered miss lies inside the window; a slot's
stamp is the latest use in its history. The miss log is a list of
(t, layer, expert) tuples sorted as tuples. Slow (quadratic), for small
random traces.

Swap budget and lead: admissions past the budget, or with every slot held
by a pending admission, count as one more remembered miss; an admission
with a lead waits in a pending list (owning its slot, not in the table)
until the step it is due at closes.
"""
from __future__ import annotations


class PolicyRef:
    """pool="layer": S slots per layer; pool="global": one pool of S slots that
    every layer draws from (owners are (layer, expert) pairs)."""

    def __init__(self, L, E, S, k, window=64, admit=2, pool="layer", budget=0, lead=0):
        self.L, self.E, self.S, self.k, self.window, self.admit = L, E, S, k, window, admit
        self.pool = pool
        self.budget, self.lead = budget, lead
        self.G = 1 if pool == "global" else L
        self.seed(None)

    def _group(self, layer):
        return 0 if self.pool == "global" else layer

    def seed(self, freq):
        self.where = {}  # (layer, e) -> slot
        self.pending = {}  # (layer, e) -> (slot, step at whose close it enters the table)
        self.nstep = 0
        self.owner = [[None] * self.S for _ in range(self.G)]  # (layer, e) or None
        self.uses = [[[] for _ in range(self.S)] for _ in range(self.G)]
        self.misses_since_reset = {}
        self.counts = [[0] * self.E for _ in range(self.L)]
        if freq is not None:
            for g in range(self.G):
                layers = range(self.L) if self.pool == "global" else [g]
                cands = [(layer, e) for layer in layers for e in range(self.E)]
                cands.sort(key=lambda le: (-int(freq[le[0]][le[1]]), le[0], le[1]))
                for s, le in enumerate(cands[: self.S]):
                    self.where[le] = s
                    self.owner[g][s] = le
        self.clock = 1
        self.log = []
        self.step_tokens = 0
        self.hits = 0
        self.last_log = []

    def forward(self, layer, ids):
        T = len(ids)
        g = self._group(layer)
        for t in range(T):
            clk = self.clock + t
            for e in ids[t]:
                e = int(e)
                self.counts[layer][e] += 1
                if (layer, e) in self.where:
                    self.uses[g][self.where[(layer, e)]].append(clk)
                    self.hits += 1
                else:
                    self.log.append((clk, layer, e))
        self.step_tokens = max(self.step_tokens, T)

    def _stamp(self, g, s):
        return max(self.uses[g][s]) if self.uses[g][s] else 0

    def step(self):
        entries = sorted(self.log)
        adm = ev = 0
        admissions = []
        for (t, layer, e) in entries:
            if (layer, e) in self.where or (layer, e) in self.pending:
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
            g = self._group(layer)
            free = [s for s in range(self.S) if self.owner[g][s] is None]
            held = {s for (s, _) in self.pending.values()} if self.pool == "global" else {
                s for (lay, _e), (s, _) in self.pending.items() if lay == layer}
            takeable = [s for s in range(self.S) if s not in held]
            if (not free and not takeable) or (self.budget and adm == self.budget):
                hist.append(t)
                continue
            evicted = (-1, -1)
            if free:
                victim = min(free)
            else:
                victim = max(takeable, key=lambda s: (-self._stamp(g, s), s))
                evicted = self.owner[g][victim]
                del self.where[evicted]
                self.misses_since_reset[evicted] = []
                ev += 1
            self.owner[g][victim] = (layer, e)
            if self.lead:
                self.pending[(layer, e)] = (victim, self.nstep + self.lead)
            else:
                self.where[(layer, e)] = victim
            self.uses[g][victim] = [t]
            self.misses_since_reset[(layer, e)] = []
            adm += 1
            admissions.append((layer, e, victim) + tuple(evicted))
        for le, (s, due) in list(self.pending.items()):
            if due <= self.nstep:
                self.where[le] = s
                del self.pending[le]
        self.nstep += 1
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
        return [[self._stamp(g, s) for s in range(self.S)] for g in range(self.G)]
