"""CPU model of the encoder's top-stream placement walk (k_encode, top-last
layout): the status words, the 64-wide look-back, its waits and its give-up
rule, run under a simulated dispatcher.  No GPU; the model is written from the
protocol's description, not from the kernel's code.

What it pins:
- every wave that places its payload computes the exact offset of its top
  stream (the sum of the aligned sizes of the tensor's earlier top streams);
- with in-order dispatch per XCD, a limited number of slots and arbitrary
  coding times, no wave ever waits on a wave that cannot run (no give-up with
  a generous bound);
- a status that never arrives ends every wait behind it at the bound, and the
  waves that give up leave their payload to the packing pass;
- the 128-entry launch gives up at once on a chunk left to the 256-entry
  launch, which then places every chunk behind it.
"""
import random

import pytest

AGG, INC, LATER = 1, 2, 3


def top_prefix(st, g, f, wait_later):
    """One look-back attempt of the wave for chunk g (first chunk of its
    tensor: f < g) over the status list st, as the kernel's loop body:
    returns ("done", bytes), ("wait", None) or ("give_up", None)."""
    acc, hi = 0, g
    while True:
        span = hi - f
        nin = min(span, 64)
        lanes = [st[hi - 1 - l] if l < nin else (0, 0) for l in range(64)]
        inc = [l for l in range(nin) if lanes[l][0] == INC]
        last = inc[0] if inc else nin - 1
        need = range(last + 1)
        if not wait_later and any(lanes[l][0] == LATER for l in need):
            return "give_up", None
        if any(lanes[l][0] not in (AGG, INC) for l in need):
            return "wait", None
        acc += sum(lanes[l][1] for l in need)
        if inc or span <= 64:
            return "done", acc
        hi -= 64


class Wave:
    def __init__(self, pair, chunks, code_time):
        self.pair = pair
        self.chunks = chunks          # the chunk indices it codes (its "mine")
        self.left = code_time         # simulated coding steps
        self.phase = "code"
        self.waited = 0
        self.result = {}


def run_launch(tensor_of, first_of, sizes, coded, st, pairs, large, tab256, limit, rng, slots=24, xcds=8,
               never=()):
    """Simulate one encoder launch.  pairs: pair index -> chunk indices;
    coded: chunks whose top stream the encoder codes; large: chunks of the
    256-entry launch; never: chunks whose wave never publishes (a stuck
    predecessor).  Returns {chunk: offset or None (left to packing)}."""
    queues = [[p for p in range(len(pairs)) if p % xcds == x] for x in range(xcds)]
    running = [[] for _ in range(xcds)]
    out = {}
    while any(queues) or any(running):
        for x in range(xcds):  # in-order dispatch per XCD into free slots
            while queues[x] and len(running[x]) < slots:
                p = queues[x].pop(0)
                mine = [c for c in pairs[p] if c in coded and (c in large) == tab256]
                if not tab256:  # the 128-entry launch marks what it leaves to the 256-entry one
                    for c in pairs[p]:
                        if c in coded and c in large:
                            st[c] = (LATER, 0)
                running[x].append(Wave(p, mine, rng.randint(1, 40)))
        for x in range(xcds):
            for wv in list(running[x]):
                if rng.random() < 0.5:
                    continue  # arbitrary interleaving
                if wv.phase == "code":
                    wv.left -= 1
                    if wv.left > 0:
                        continue
                    for c in wv.chunks:
                        if c in never:
                            continue
                        st[c] = (INC if c == first_of[c] else AGG, sizes[c])
                    wv.phase = "walk"
                    wv.todo = [c for c in wv.chunks if c not in never]
                    continue
                # walk: one attempt per step for the first chunk still to place
                c = wv.todo[0]
                prev = wv.result.get(c - 1) if (c - 1) in wv.chunks else None
                if c == first_of[c]:
                    state, pre = "done", 0
                elif prev is not None and tensor_of[c - 1] == tensor_of[c]:
                    state, pre = "done", prev + sizes[c - 1]
                else:
                    state, pre = top_prefix(st, c, first_of[c], tab256)
                if state == "wait":
                    wv.waited += 1
                    if wv.waited > limit:
                        state = "give_up"
                    else:
                        continue
                if state == "done":
                    wv.result[c] = pre
                    if c != first_of[c]:
                        st[c] = (INC, pre + sizes[c])
                    out[c] = pre
                else:
                    out[c] = None
                wv.todo.pop(0)
                if not wv.todo:
                    running[x].remove(wv)
            for wv in list(running[x]):
                if wv.phase == "walk" and not wv.todo:
                    running[x].remove(wv)
    return out


def make_case(rng, ntensors=5, maxchunks=300, p_coded=0.9, p_large=0.0):
    counts = [rng.randint(1, maxchunks) for _ in range(ntensors)]
    tensor_of, first_of = [], []
    for j, k in enumerate(counts):
        f = len(tensor_of)
        tensor_of += [j] * k
        first_of += [f] * k
    K = len(tensor_of)
    sizes = [16 * rng.randint(0, 4096) for _ in range(K)]
    coded = {c for c in range(K) if rng.random() < p_coded}
    large = {c for c in coded if rng.random() < p_large}
    # k_scan part 1: settled top streams published, coded ones unknown
    st = [(0, 0) if c in coded else (INC if c == first_of[c] else AGG, sizes[c]) for c in range(K)]
    pairs = [list(range(2 * p, min(2 * p + 2, K))) for p in range((K + 1) // 2)]
    truth = [0] * K
    for c in range(K):
        truth[c] = 0 if c == first_of[c] else truth[c - 1] + sizes[c - 1]
    return tensor_of, first_of, sizes, coded, large, st, pairs, truth


@pytest.mark.parametrize("seed", range(12))
def test_every_placed_offset_is_exact_and_nobody_gives_up(seed):
    rng = random.Random(seed)
    tensor_of, first_of, sizes, coded, large, st, pairs, truth = make_case(rng, p_large=0.15 * (seed % 3))
    placed = {}
    for tab256 in (False, True):
        out = run_launch(tensor_of, first_of, sizes, coded, st, pairs, large, tab256, limit=10**6, rng=rng,
                         slots=rng.choice([1, 3, 24]))
        for c, v in out.items():
            if v is not None:
                assert v == truth[c], (c, v, truth[c])
                placed[c] = v
    # the 256-entry launch places everything (it never gives up on kStLater
    # chunks, which are its own); the 128-entry launch only gives up behind them
    for c in coded:
        if c in large or not any(d in large for d in range(first_of[c], c)):
            assert c in placed, c


def test_later_chunk_stops_the_first_launch_at_once():
    rng = random.Random(5)
    tensor_of, first_of, sizes, coded, large, st, pairs, truth = make_case(rng, ntensors=1, maxchunks=200,
                                                                          p_coded=1.0)
    K = len(tensor_of)
    large = {K // 2}
    out = run_launch(tensor_of, first_of, sizes, coded, st, pairs, large, False, limit=10**6, rng=rng)
    assert all(out[c] is None for c in range(K // 2 + 1, K) if c in out)
    assert all(out[c] == truth[c] for c in range(0, K // 2))
    out2 = run_launch(tensor_of, first_of, sizes, coded, st, pairs, large, True, limit=10**6, rng=rng)
    assert out2 == {K // 2: truth[K // 2]}
    # the statuses now hold every inclusive count a later walk needs
    state, pre = top_prefix(st, K - 1, 0, True)
    assert state == "done" and pre == truth[K - 1]


def test_missing_status_ends_every_wait_at_the_bound():
    rng = random.Random(9)
    tensor_of, first_of, sizes, coded, large, st, pairs, truth = make_case(rng, ntensors=2, maxchunks=150,
                                                                          p_coded=1.0)
    stuck = first_of[-1] + 3  # a chunk of the second tensor never publishes its size
    out = run_launch(tensor_of, first_of, sizes, coded, st, pairs, set(), False, limit=50, rng=rng,
                     never={stuck})
    for c, v in out.items():
        if tensor_of[c] == tensor_of[stuck] and c > stuck:
            assert v is None  # gave up: left to the packing pass
        else:
            assert v == truth[c]


def test_window_walk_crosses_many_windows():
    K = 1000
    sizes = [16 * (i % 7) for i in range(K)]
    st = [(INC, sizes[0])] + [(AGG, sizes[c]) for c in range(1, K)]
    state, pre = top_prefix(st, K - 1, 0, False)
    assert state == "done" and pre == sum(sizes[:K - 1])
    st[500] = (INC, sum(sizes[:501]))  # a nearer inclusive count ends the walk early
    st[400] = (0, 0)                   # ... so a gap behind it does not matter
    assert top_prefix(st, K - 1, 0, False) == ("done", sum(sizes[:K - 1]))
    st[600] = (0, 0)
    assert top_prefix(st, K - 1, 0, False) == ("wait", None)
    st[600] = (LATER, 0)
    assert top_prefix(st, K - 1, 0, False) == ("give_up", None)
    assert top_prefix(st, K - 1, 0, True) == ("wait", None)
