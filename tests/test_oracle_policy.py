"""Pins of the oracle's cache-policy simulation (CPU only).

  * hand traces worked out from the rules (window edge, victim choice, ties,
    full and empty pools, batch steps);
  * invariants on random traces (hypothesis);
  * agreement with an independent history-based formulation
    (tests/_policy_ref.py) on random traces;
  * statistics of the generated routing (first pick follows the Zipf
    popularity; the hot set moves at a rotation).
"""
import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st
from scipy import stats as sstats

import oracle
from tests._policy_ref import PolicyRef
from workload import Workload, frequency_table, rank_permutation, zipf_logits, zipf_popularity


def _run(pol, picks_per_step, layer=0):
    out = []
    for ids in picks_per_step:
        pol.forward(layer, np.array(ids, np.int32).reshape(-1, pol.k))
        out.append(pol.step())
    return out


def _seeded(E=4, S=2, k=1, freq=(9, 5, 1, 0), window=64, admit=2):
    pol = oracle.Policy(1, E, S, k, window=window, admit_misses=admit)
    pol.seed(np.array([freq], np.uint32))
    return pol


def test_seed_order_count_desc_id_asc():
    pol = oracle.Policy(2, 6, 3, 1)
    pol.seed(np.array([[5, 9, 9, 0, 5, 1], [0, 0, 0, 0, 0, 0]], np.uint32))
    t = pol.tables()
    assert t["table"][0].tolist() == [2, 0, 1, -1, -1, -1]  # 9(id1), 9(id2), 5(id0)
    assert t["table"][1].tolist() == [0, 1, 2, -1, -1, -1]  # all equal: lowest ids
    assert t["stamps"].max() == 0 and pol.clock == 1


def test_second_miss_inside_window_admits():
    pol = _seeded()
    steps = [[2]] + [[0]] * 62 + [[2]]  # expert 2 misses at t=1 and t=64; expert 0 hit at t=2..63
    st = _run(pol, steps)
    assert st[0]["misses"] == 1 and st[0]["admissions"] == 0
    assert st[-1] == dict(hits=0, misses=1, admissions=1, evictions=1, tokens=1)
    t = pol.tables()
    # slot 0 (expert 0) was used at t=63, slot 1 (expert 1) never: slot 1 is the victim
    assert t["table"][0].tolist() == [0, -1, 1, -1]
    assert t["stamps"][0].tolist() == [63, 64]
    assert pol.last_log().tolist() == [(64 << 32) | 2]
    assert pol.last_admissions().tolist() == [[0, 2, 1, 0, 1]]
    assert pol.clock == 65


def test_second_miss_outside_window_only_remembers():
    pol = _seeded()
    steps = [[2]] + [[0]] * 63 + [[2]]  # t=1 and t=65: 65 - 1 = 64 is not < 64
    st = _run(pol, steps)
    assert all(s["admissions"] == 0 for s in st)
    t = pol.tables()
    assert t["table"][0].tolist() == [0, 1, -1, -1]
    assert t["last_miss"][0].tolist() == [0, 0, 65, 0]
    # a third miss at t=66 is inside the window of the one at 65
    st = _run(pol, [[2]])
    assert st[0]["admissions"] == 1


def test_untouched_seeded_slots_leave_highest_index_first():
    pol = _seeded(E=5, S=3, freq=(9, 5, 3, 0, 0))
    st = _run(pol, [[3], [3], [4], [4]])
    t = pol.tables()
    # all stamps 0 at the first admission: tie -> highest slot (2, expert 2);
    # then stamps are [0, 0, 2]: tie between 0 and 1 -> slot 1 (expert 1)
    assert [s["admissions"] for s in st] == [0, 1, 0, 1]
    assert t["table"][0].tolist() == [0, -1, -1, 2, 1]
    assert t["stamps"][0].tolist() == [0, 4, 2]


def test_eviction_forgets_last_miss_and_admission_clears_it():
    pol = _seeded(E=4, S=1, freq=(5, 0, 0, 0))
    _run(pol, [[1], [1]])  # expert 1 admitted at t=2, evicting expert 0
    t = pol.tables()
    assert t["table"][0].tolist() == [-1, 0, -1, -1] and t["last_miss"][0].tolist() == [0, 0, 0, 0]
    _run(pol, [[0]])  # one miss of 0 at t=3: remembered
    assert pol.tables()["last_miss"][0].tolist() == [3, 0, 0, 0]
    _run(pol, [[0]])  # t=4: admitted, evicting 1
    t = pol.tables()
    assert t["table"][0].tolist() == [0, -1, -1, -1] and t["last_miss"][0].tolist() == [0, 0, 0, 0]


def test_full_pool_never_misses_and_empty_pool_never_admits():
    rng = np.random.default_rng(3)
    trace = [rng.choice(6, size=(2, 3), replace=False).tolist() for _ in range(4)]
    trace = [[rng.permutation(6)[:3].tolist() for _ in range(2)] for _ in range(40)]
    full = oracle.Policy(1, 6, 6, 3)
    full.seed(np.ones((1, 6), np.uint32))
    empty = oracle.Policy(1, 6, 0, 3)
    empty.seed(None)
    for ids in trace:
        full.forward(0, np.array(ids, np.int32))
        empty.forward(0, np.array(ids, np.int32))
        a, b = full.step(), empty.step()
        assert a["misses"] == 0 and a["hits"] == 6
        assert b["misses"] == 6 and b["admissions"] == 0 and b["hits"] == 0


def test_batch_step_two_tokens_same_expert():
    pol = _seeded()
    pol.forward(0, np.array([[2], [2]], np.int32))  # clocks 1 and 2 in one step
    st = pol.step()
    assert st == dict(hits=0, misses=2, admissions=1, evictions=1, tokens=2)
    assert pol.last_log().tolist() == [(1 << 32) | 2, (2 << 32) | 2]
    assert pol.tables()["stamps"][0].tolist() == [0, 2]
    assert pol.clock == 3


def test_admit_every_miss_mode_is_lru():
    pol = _seeded(admit=1)
    st = _run(pol, [[2], [3], [0]])
    assert [s["admissions"] for s in st] == [1, 1, 1]
    # t=1: stamps tie -> slot 1 (expert 1 out), 2 in with stamp 1; t=2: stamps
    # [0, 1] -> slot 0 (expert 0 out), 3 in with stamp 2; t=3: expert 0 misses
    # again, stamps [2, 1] -> slot 1 (expert 2 out)
    assert pol.tables()["table"][0].tolist() == [1, -1, -1, 0]


def test_layers_are_independent_and_log_packs_layer():
    pol = oracle.Policy(3, 8, 2, 2)
    pol.seed(np.tile(np.arange(8, 0, -1, dtype=np.uint32), (3, 1)))
    pol.forward(2, np.array([[7, 0]], np.int32))
    pol.forward(0, np.array([[5, 6]], np.int32))
    pol.step()
    assert pol.last_log().tolist() == [(1 << 32) | (0 << 12) | 5, (1 << 32) | (0 << 12) | 6,
                                       (1 << 32) | (2 << 12) | 7]


def _random_trace(draw_rng, L, E, k, steps, tmax):
    trace = []
    for _ in range(steps):
        T = int(draw_rng.integers(1, tmax + 1))
        trace.append([(layer, [draw_rng.permutation(E)[:k].tolist() for _ in range(T)]) for layer in range(L)])
    return trace


@settings(max_examples=60, deadline=None)
@given(seed=st.integers(0, 2**31 - 1), L=st.integers(1, 3), E=st.integers(2, 12), tmax=st.integers(1, 4),
       window=st.sampled_from([2, 5, 64]), admit=st.sampled_from([1, 2]), seeded=st.booleans(),
       pool=st.sampled_from(["layer", "global"]), budget=st.sampled_from([0, 0, 1, 2]),
       lead=st.sampled_from([0, 0, 1, 2]))
def test_agrees_with_history_formulation(seed, L, E, tmax, window, admit, seeded, pool, budget, lead):
    rng = np.random.default_rng(seed)
    k = int(rng.integers(1, E + 1))
    S = int(rng.integers(0, (E if pool == "layer" else L * E) + 1))
    freq = rng.integers(0, 5, size=(L, E)).astype(np.uint32) if seeded else None
    a = oracle.Policy(L, E, S, k, window=window, admit_misses=admit, pool=pool, swaps_per_step=budget,
                      swap_lead=lead)
    b = PolicyRef(L, E, S, k, window=window, admit=admit, pool=pool, budget=budget, lead=lead)
    a.seed(freq)
    b.seed(freq)
    cum_adm = cum_miss = 0
    for step in _random_trace(rng, L, E, k, 30, tmax):
        for layer, ids in step:
            a.forward(layer, np.array(ids, np.int32))
            b.forward(layer, ids)
        sa, sb = a.step(), b.step()
        assert sa == sb
        ta = a.tables()
        assert ta["table"].tolist() == b.table()
        assert ta["stamps"].tolist() == b.stamps()
        assert a.last_log().tolist() == b.last_log
        assert [tuple(r) for r in a.last_admissions().tolist()] == b.last_admissions
        # invariants: the table is a bijection onto the used slots of each
        # pool, owners agree with it, stamps never run ahead of the clock,
        # hits + misses = picks, two misses per admission
        for g in range(1 if pool == "global" else L):
            layers = range(L) if pool == "global" else [g]
            res = {(layer, e): s for layer in layers for e, s in enumerate(ta["table"][layer]) if s >= 0}
            assert len(set(res.values())) == len(res) <= S
            assert all(ta["owner_layer"][g][s] == layer and ta["owner"][g][s] == e for (layer, e), s in res.items())
            # an owner outside the table is an admission waiting for its lead
            assert all(o == -1 or ta["table"][ol][o] >= 0 or lead > 0
                       for ol, o in zip(ta["owner_layer"][g], ta["owner"][g]))
        assert ta["stamps"].size == 0 or ta["stamps"].max() < a.clock
        T = max(len(ids) for _, ids in step)
        assert sa["hits"] + sa["misses"] == sum(len(ids) for _, ids in step) * k
        assert sa["tokens"] == T
        if budget:
            assert sa["admissions"] <= budget
        cum_adm += sa["admissions"]
        cum_miss += sa["misses"]
        if admit == 2:
            assert cum_adm <= cum_miss // 2
    assert a.counts().tolist() == b.counts


def test_swap_budget_defers_the_rest_of_a_step():
    pol = oracle.Policy(1, 6, 3, 2, swaps_per_step=1)
    pol.seed(np.array([[9, 8, 7, 0, 0, 0]], np.uint32))
    pol.forward(0, [[3, 4]])
    pol.step()  # t=1: first misses of e3, e4
    pol.forward(0, [[3, 4]])
    st = pol.step()  # t=2: both qualify; the budget admits e3 only and e4 remembers t=2
    assert st["admissions"] == 1
    assert pol.last_admissions().tolist() == [[0, 3, 2, 0, 2]]
    assert pol.tables()["last_miss"][0].tolist() == [0, 0, 0, 0, 2, 0]
    pol.forward(0, [[4, 0]])  # t=3: e4's miss is inside the window of t=2; e0 hits (stamp 3)
    st = pol.step()  # e4 takes slot 1 (stamp 0; slot 2 holds e3 at 2), evicting e1
    assert st["admissions"] == 1 and pol.tables()["table"][0].tolist() == [0, -1, -1, 2, 1, -1]


def test_swap_lead_keeps_the_expert_cold_and_its_slot_reserved():
    pol = oracle.Policy(1, 6, 2, 2, swap_lead=1)
    pol.seed(np.array([[5, 4, 0, 0, 0, 0]], np.uint32))  # e0 -> 0, e1 -> 1
    pol.forward(0, [[2, 3]])
    pol.step()  # t=1: first misses of e2, e3
    pol.forward(0, [[1, 5]])
    pol.step()  # t=2: e1 hits (slot 1 stamped 2); first miss of e5
    pol.forward(0, [[2, 3]])
    st = pol.step()  # t=3: e2 takes slot 0 (stamp 0), e3 slot 1; both owners evicted now, both pending
    assert st["admissions"] == 2 and st["evictions"] == 2
    t = pol.tables()
    assert t["table"][0].tolist() == [-1] * 6
    assert t["owner"][0].tolist() == [2, 3] and t["stamps"][0].tolist() == [3, 3]
    # t=4: e2 still misses (logged, skipped by the walk); e5 qualifies but every
    # slot is held by a pending admission, so it is refused and remembers t=4
    pol.forward(0, [[2, 5]])
    st = pol.step()
    assert st["misses"] == 2 and st["admissions"] == 0
    assert pol.last_log().tolist() == [(4 << 32) | 2, (4 << 32) | 5]
    t = pol.tables()
    assert t["table"][0].tolist() == [-1, -1, 0, 1, -1, -1]  # the lead ended with this step: both flip in
    assert t["last_miss"][0].tolist() == [0, 0, 0, 0, 0, 4]
    pol.forward(0, [[2, 3]])
    assert pol.step()["hits"] == 2


def test_preheat_leaves_pending_admissions_alone():
    pol = oracle.Policy(1, 5, 2, 1, swap_lead=2)
    pol.seed(np.array([[5, 4, 0, 0, 0]], np.uint32))  # e0 -> 0, e1 -> 1
    for e in (2, 2):
        pol.forward(0, [[e]])
        pol.step()  # t=2: e2 admitted into slot 1 (stamp 0, highest index), pending
    assert pol.tables()["owner"][0].tolist() == [0, 2]
    # e2 is no candidate and slot 1 no victim: e3 displaces e0, e4 finds no slot
    adm = pol.preheat(0, [0, 0, 9, 5, 3], max_experts=2)
    assert adm.tolist() == [[0, 3, 0, 0, 0]]
    assert pol.tables()["table"][0].tolist() == [-1, -1, -1, 0, -1]


def test_swap_lead_zero_is_the_plain_policy():
    rng = np.random.default_rng(3)
    a = oracle.Policy(2, 10, 4, 2)
    b = oracle.Policy(2, 10, 4, 2, swaps_per_step=0, swap_lead=0)
    freq = rng.integers(0, 9, size=(2, 10)).astype(np.uint32)
    a.seed(freq)
    b.seed(freq)
    for _ in range(40):
        for layer in range(2):
            ids = np.stack([rng.permutation(10)[:2] for _ in range(2)]).astype(np.int32)
            a.forward(layer, ids)
            b.forward(layer, ids)
        assert a.step() == b.step()
        assert a.tables()["table"].tolist() == b.tables()["table"].tolist()


def test_first_pick_follows_zipf():
    wl = Workload("zipf-pin", 950, 1, 64, 4, 32, 32, tokens=1, steps=40000, zipf_s=1.1)
    z = zipf_logits(wl)[:, 0, 0]
    ids, _ = oracle.route(z, 1)
    perm = rank_permutation(wl, 0, 0)
    p = zipf_popularity(64, 1.1)
    observed = np.bincount(ids[:, 0], minlength=64)[perm]  # by rank
    chi2, pval = sstats.chisquare(observed, p * observed.sum())
    assert pval > 1e-4, (chi2, pval)


def test_rotation_moves_the_hot_set():
    wl = Workload("rot-pin", 951, 1, 512, 8, 32, 32, tokens=1, steps=1024, zipf_s=1.1, rotation=512)
    z = zipf_logits(wl)[:, 0, 0]
    ids, _ = oracle.route(z, 8)
    top_before = np.argsort(-np.bincount(ids[:512].ravel(), minlength=512), kind="stable")[:8]
    top_after = np.argsort(-np.bincount(ids[512:].ravel(), minlength=512), kind="stable")[:8]
    assert set(top_before) == set(rank_permutation(wl, 0, 0)[:8]) or len(
        set(top_before) & set(rank_permutation(wl, 0, 0)[:16])) >= 6
    assert len(set(top_before) & set(top_after)) <= 2
    # the frequency table is drawn from the epoch-0 popularity
    f = frequency_table(wl)[0]
    assert f.sum() == 1024 * 8 and int(np.argmax(f)) == int(rank_permutation(wl, 0, 0)[0])


def test_global_pool_seeds_across_layers():
    # counts: (1,1)=9 first, then the 5s by layer, then expert: (0,0), (0,2); (1,0) misses out
    pol = oracle.Policy(2, 3, 3, 1, pool="global")
    pol.seed(np.array([[5, 1, 5], [5, 9, 0]], np.uint32))
    t = pol.tables()
    assert t["table"].tolist() == [[1, -1, 2], [-1, 0, -1]]
    assert t["owner_layer"].tolist() == [[1, 0, 0]] and t["owner"].tolist() == [[1, 0, 2]]


def test_global_pool_evicts_across_layers():
    pol = oracle.Policy(2, 3, 3, 1, pool="global")
    pol.seed(np.array([[5, 1, 5], [5, 9, 0]], np.uint32))
    # t=1: layer 0 hits (0,2) in slot 2; layer 1 misses expert 2 (remembered)
    pol.forward(0, [[2]])
    pol.forward(1, [[2]])
    assert pol.step() == dict(hits=1, misses=1, admissions=0, evictions=0, tokens=1)
    # t=2: same picks; (1,2) misses again inside the window and is admitted.
    # slots 0 and 1 were never used (stamp 0): the tie goes to the higher
    # index, slot 1, whose owner is layer 0's expert 0
    pol.forward(0, [[2]])
    pol.forward(1, [[2]])
    assert pol.step() == dict(hits=1, misses=1, admissions=1, evictions=1, tokens=1)
    t = pol.tables()
    assert t["table"].tolist() == [[-1, -1, 2], [-1, 0, 1]]
    assert t["stamps"].tolist() == [[0, 2, 2]]
    assert pol.last_admissions().tolist() == [[1, 2, 1, 0, 0]]
    # with a pool per layer the same trace evicts inside layer 1 instead
    per = oracle.Policy(2, 3, 2, 1)
    per.seed(np.array([[5, 1, 5], [5, 9, 0]], np.uint32))
    for _ in range(2):
        per.forward(0, [[2]])
        per.forward(1, [[2]])
        per.step()
    assert per.last_admissions().tolist() == [[1, 2, 1, 1, 0]]


@settings(max_examples=25, deadline=None)
@given(seed=st.integers(0, 2**31 - 1), E=st.integers(2, 10), window=st.sampled_from([2, 64]))
def test_global_pool_of_one_layer_is_the_layer_pool(seed, E, window):
    rng = np.random.default_rng(seed)
    k = int(rng.integers(1, E + 1))
    S = int(rng.integers(0, E + 1))
    freq = rng.integers(0, 5, size=(1, E)).astype(np.uint32)
    a = oracle.Policy(1, E, S, k, window=window, pool="global")
    b = oracle.Policy(1, E, S, k, window=window)
    a.seed(freq)
    b.seed(freq)
    for step in _random_trace(rng, 1, E, k, 25, 3):
        for layer, ids in step:
            a.forward(layer, np.array(ids, np.int32))
            b.forward(layer, np.array(ids, np.int32))
        assert a.step() == b.step()
        ta, tb = a.tables(), b.tables()
        assert ta["table"].tolist() == tb["table"].tolist() and ta["stamps"].tolist() == tb["stamps"].tolist()
        assert a.last_log().tolist() == b.last_log().tolist()


def test_preheat_admits_the_cold_experts_a_prompt_used():
    pol = oracle.Policy(1, 6, 3, 1)
    pol.seed(np.array([[9, 8, 7, 0, 0, 0]], np.uint32))  # slots: e0 -> 0, e1 -> 1, e2 -> 2
    pol.forward(0, [[0]])  # t=1: stamp of slot 0 = 1
    pol.step()             # clock 2
    # the prompt used e1 (resident, 5 pairs) and e3, e4, e5 (cold: 3, 3, 1 pairs).
    # e1's stamp rises to 2. e3 (then e4: ties go to the lower id) displaces the
    # owner with the smallest (pass count, stamp): e2 (0, 0) in slot 2, then e0 (0, 1)
    adm = pol.preheat(0, [0, 5, 0, 3, 3, 1], max_experts=2)
    assert adm.tolist() == [[0, 3, 2, 0, 2], [0, 4, 0, 0, 0]]
    t = pol.tables()
    assert t["table"][0].tolist() == [-1, 1, -1, 2, 0, -1]
    assert t["stamps"][0].tolist() == [2, 2, 2]
    # e5 (1 pair) finds only owners used as much or more (3, 5, 3): nothing changes
    assert pol.preheat(0, [0, 5, 0, 3, 3, 1], max_experts=5).size == 0
    assert pol.tables()["table"][0].tolist() == [-1, 1, -1, 2, 0, -1]


def test_preheat_lets_a_busier_cold_expert_displace_a_lightly_used_one():
    pol = oracle.Policy(1, 5, 2, 1)
    pol.seed(np.array([[3, 2, 0, 0, 0]], np.uint32))  # e0 -> 0, e1 -> 1
    # the pass used all residents (e0: 1 pair, e1: 6) and the cold e3 (4 pairs):
    # e3 displaces e0, the owner with the fewest pairs; e4 (2 pairs) cannot
    # displace e3 (4) or e1 (6)
    adm = pol.preheat(0, [1, 6, 0, 4, 2], max_experts=3)
    assert adm.tolist() == [[0, 3, 0, 0, 0]]
    assert pol.tables()["table"][0].tolist() == [-1, 1, -1, 0, -1]


def test_preheat_fills_free_slots_and_respects_the_limit():
    pol = oracle.Policy(2, 5, 2, 2)
    pol.seed(None)  # every slot free
    adm = pol.preheat(1, [4, 0, 4, 7, 0], max_experts=5)  # at most S = 2: e3, then e0 (tie with e2)
    assert adm.tolist() == [[1, 3, 0, -1, -1], [1, 0, 1, -1, -1]]
    t = pol.tables()
    assert t["table"][1].tolist() == [1, -1, -1, 0, -1] and t["stamps"][1].tolist() == [1, 1]
    assert (t["table"][0] == -1).all()  # another layer's pool is untouched
    assert pol.preheat(0, [0, 0, 0, 0, 0], max_experts=5).size == 0
    # the admitted experts hit on the next step; the stamps then follow the clock
    pol.forward(1, [[3, 0]])
    assert pol.step()["hits"] == 2


def test_preheat_in_a_global_pool_evicts_unused_layers_first():
    pol = oracle.Policy(2, 3, 2, 1, pool="global")
    pol.seed(np.array([[5, 0, 0], [4, 0, 0]], np.uint32))  # slot 0 = (0,0), slot 1 = (1,0)
    pol.forward(0, [[0]])  # t=1: layer 0's expert stamped
    pol.step()
    adm = pol.preheat(1, [0, 2, 0], max_experts=1)  # layer 1's unused (1,0) goes, not layer 0's
    assert adm.tolist() == [[1, 1, 1, 1, 0]]
    assert pol.tables()["table"].tolist() == [[0, -1, -1], [-1, 1, -1]]
