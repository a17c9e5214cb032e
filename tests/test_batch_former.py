"""The adapter-aware batch former: the oracle pinned to the pages (hand-worked
cases, the 38% figure of the distinct-adapter cap, the cap's bound on any
queue), invariants, planted mistakes, and the library's native former
against the oracle, bit for bit (host code: runs without a GPU)."""
import json
import os

import numpy as np
import pytest

import oracle.batch_former as bf
import oracle.costmodel as cm

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
CASES = json.load(open(os.path.join(GOLDEN, "batch_former_cases.json")))["cases"]
FIGURES = {f["id"]: f for f in json.load(open(os.path.join(GOLDEN, "pages_figures.json")))["figures"]}


def _expand(v):
    return list(eval(v, {"range": range})) if isinstance(v, str) else list(v)  # "range(n)" only


def _args(c):
    return dict(max_batch=c["max_batch"], max_distinct=c["max_distinct"], min_batch=c["min_batch"],
                reserved_tail=c["reserved_tail"], waited_ms=c.get("waited_ms"), max_wait_ms=c.get("max_wait_ms"))


@pytest.mark.parametrize("case", CASES, ids=[c["id"] for c in CASES])
def test_hand_worked_cases(case):
    assert bf.form_batch(_expand(case["adapters"]), **_args(case)) == _expand(case["expect"])


def test_cap_32_gives_the_pages_38_percent():
    """All-modules rank 64 at batch 128: every request on its own adapter costs
    +151% of the base read; the cap of 32 (4 of them tail slots) bounds it at
    38% ("6. Deep Dive A", "The adapter-aware scheduler")."""
    q = list(range(128))
    fifo = q[:128]
    capped = bf.form_batch(q, max_batch=128, max_distinct=32, min_batch=32, reserved_tail=4)
    for got, fig in ((bf.distinct_adapters(q, fifo), "extra_all_r64_b128_pct"),
                     (bf.distinct_adapters(q, capped), "extra_all_r64_cap32_pct")):
        pct = 100 * cm.extra_decode_bytes_fraction(64, cm.ALL_MODULES, got)
        assert abs(pct - FIGURES[fig]["printed"]) <= FIGURES[fig]["tol"], (fig, got, pct)


def random_queue(rng, n, slots, s=1.1, base_frac=0.05):
    p = 1.0 / np.arange(1, slots + 1) ** s
    ids = rng.permutation(slots)[rng.choice(slots, size=n, p=p / p.sum())]
    ids[rng.random(n) < base_frac] = -1
    return ids.astype(np.int32)


def random_params(rng, n):
    md = int(rng.integers(0, 40))
    return dict(max_batch=int(rng.integers(1, max(2, n + 8))), max_distinct=md,
                min_batch=int(rng.integers(0, 64)), reserved_tail=int(rng.integers(0, 8)))


def test_cap_bounds_distinct_adapters_on_any_queue():
    """With min_batch <= max_distinct, tail and fill together admit at most
    max_distinct adapters, whatever the traffic ("Cap it at 32 and the worst
    case is bounded regardless of traffic shape")."""
    rng = np.random.default_rng(11)
    for _ in range(300):
        n = int(rng.integers(0, 600))
        q = random_queue(rng, n, int(rng.integers(1, 400)), s=float(rng.uniform(0.0, 2.0)))
        prm = random_params(rng, n)
        prm["min_batch"] = min(prm["min_batch"], prm["max_distinct"])
        out = bf.form_batch(list(q), **prm)
        assert bf.distinct_adapters(list(q), out) <= prm["max_distinct"]


def check_invariants(q, out, max_batch, max_distinct, min_batch, reserved_tail, waited_ms=None, max_wait_ms=None):
    n = len(q)
    assert len(out) == len(set(out)) and all(0 <= i < n for i in out) and len(out) <= max_batch
    urgent = [i for i in range(n) if waited_ms is not None and waited_ms[i] > max_wait_ms][:max_batch]
    assert out[:len(urgent)] == urgent
    rest = out[len(urgent):]
    left = [i for i in range(n) if i not in set(urgent)]
    single = [i for i in left if q[i] >= 0 and sum(1 for j in left if q[j] == q[i]) == 1]
    tail = single[:max(0, min(reserved_tail, max_distinct, max_batch - len(urgent)))]
    assert rest[:len(tail)] == tail
    fill = rest[len(tail):]
    left2 = [i for i in left if i not in set(tail)]
    key = {i: (q[i] if q[i] >= 0 else -1) for i in left2}
    members = {}
    for i in left2:
        members.setdefault(key[i], []).append(i)
    # the fill is a sequence of whole groups (the last may be cut where the batch is full),
    # each taken oldest first, in descending size
    runs, sizes = [], []
    for i in fill:
        if not runs or key[i] != runs[-1][0]:
            runs.append((key[i], []))
        runs[-1][1].append(i)
    seen = set()
    for r, (k, got) in enumerate(runs):
        assert k not in seen
        seen.add(k)
        assert got == members[k][:len(got)]
        if r < len(runs) - 1:
            assert len(got) == len(members[k])
        elif len(got) < len(members[k]):
            assert len(out) == max_batch
        sizes.append(len(members[k]))
    assert sizes == sorted(sizes, reverse=True)
    # stopped early only when the cap and the minimum batch allowed it
    if len(out) < max_batch and len(seen) < len(members):
        n_adapters = sum(1 for k in seen if k >= 0)
        assert n_adapters >= max_distinct - len(tail) and len(out) >= min_batch


def test_invariants_on_random_queues():
    rng = np.random.default_rng(12)
    for _ in range(200):
        n = int(rng.integers(0, 200))
        q = list(random_queue(rng, n, int(rng.integers(1, 120))))
        prm = random_params(rng, n)
        if rng.random() < 0.5:
            prm["waited_ms"] = list(rng.uniform(0, 400, size=n))
            prm["max_wait_ms"] = 300.0
        check_invariants(q, bf.form_batch(q, **prm), **prm)


# --------------------------------------------------------------- planted mistakes

SRC = open(bf.__file__).read()
MUTATIONS = {
    "smallest_group_first": ("records.sort(key=lambda r: (-r[0], r[1]))", "records.sort(key=lambda r: (r[0], r[1]))"),
    "newest_group_first_on_ties": ("records.sort(key=lambda r: (-r[0], r[1]))",
                                   "records.sort(key=lambda r: (-r[0], -r[1]))"),
    "tail_takes_shared": ("count[adapters[i]] == 1", "count[adapters[i]] >= 1"),
    "budget_ignores_tail": ("adapter_budget = max_distinct - tail", "adapter_budget = max_distinct"),
    "no_min_batch": ("big_enough = len(batch) >= min_batch", "big_enough = True"),
    "newest_first": ("for i in members[:min(size, room)]:", "for i in members[::-1][:min(size, room)]:"),
    "base_only_counts": ("adapters_admitted += 1 if key >= 0 else 0", "adapters_admitted += 1"),
    "deadline_inclusive": ("if waited_ms[i] > max_wait_ms:", "if waited_ms[i] >= max_wait_ms:"),
    "tail_not_capped": ("if tail >= min(reserved_tail, max_distinct) or", "if tail >= reserved_tail or"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    old, new = MUTATIONS[name]
    assert SRC.count(old) == 1, name
    ns = {}
    exec(compile(SRC.replace(old, new), "mutant_batch_former", "exec"), ns)
    caught = False
    for c in CASES:
        if ns["form_batch"](_expand(c["adapters"]), **_args(c)) != _expand(c["expect"]):
            caught = True
    assert caught, f"no pin catches {name}"


# --------------------------------------------------------------- native former

lg = pytest.importorskip("adapter_gemv_amd")


def _native_or_skip():
    try:
        lg.host_lib()
    except lg.LoraError as e:  # pragma: no cover - library not built
        pytest.skip(str(e))


@pytest.mark.parametrize("case", CASES, ids=[c["id"] for c in CASES])
def test_native_hand_worked_cases(case):
    _native_or_skip()
    a = _args(case)
    got = lg.form_batch(_expand(case["adapters"]), a["max_batch"], a["max_distinct"], a["min_batch"],
                        a["reserved_tail"], a["waited_ms"], a["max_wait_ms"] or 0.0)
    assert list(got) == _expand(case["expect"])


def test_native_matches_oracle_on_random_queues():
    _native_or_skip()
    rng = np.random.default_rng(13)
    for t in range(1500):
        n = int(rng.integers(0, 2000 if t % 50 == 0 else 300))
        q = random_queue(rng, n, int(rng.integers(1, 600)), s=float(rng.uniform(0.0, 2.0)),
                         base_frac=float(rng.choice([0.0, 0.05, 0.5])))
        prm = random_params(rng, n)
        w = None
        if rng.random() < 0.4:
            w = rng.uniform(0, 400, size=n).astype(np.float32)
        want = bf.form_batch(list(q), **prm, waited_ms=None if w is None else list(w),
                             max_wait_ms=None if w is None else 250.0)
        got = lg.form_batch(q, prm["max_batch"], prm["max_distinct"], prm["min_batch"], prm["reserved_tail"],
                            w, 250.0)
        assert list(got) == want, (t, n, prm)


def test_native_errors():
    _native_or_skip()
    for bad in (dict(max_batch=0), dict(max_distinct=-1), dict(min_batch=-1), dict(reserved_tail=-2)):
        prm = dict(max_batch=4, max_distinct=2, min_batch=0, reserved_tail=0) | bad
        with pytest.raises(lg.LoraError, match="LORA_ERR_SHAPE"):
            lg.form_batch(np.arange(5), **prm)
    assert list(lg.form_batch(np.zeros(0, np.int32), 4, 2)) == []
