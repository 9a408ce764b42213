"""A CPU model of the inter-workgroup counter protocols kept in the workspace
header, run across consecutive calls on one workspace (test infrastructure:
it models the protocols, it runs no kernel).

Workgroups are Python generators that yield at every global-memory operation
(an atomic, a load or a store of a header word), and a seeded scheduler
interleaves them in arbitrary orders, so every interleaving the hardware can
produce for these operations is a candidate.  Each call checks three things:
the header words it relies on are zero when it starts, every work item is done
exactly once, and every index derived from a counter value stays below the
item count.

Protocols modelled:
  arrival   -- every workgroup publishes its result and adds one to a counter;
               the one that sees N - 1 reads all results and resets the
               counter (the prefill grouping kernel, the fused router top-k);
  claim     -- the prefill's fused routing and grouping: each token's picks
               claim places in their slots with atomic adds on per-slot claim
               words, every workgroup arrives, and the last one reads the
               claims as the counts and resets the claim words and the
               arrival counter;
  exit      -- items in a static order, a bounded wait per dependent item that
               on expiry raises the error word and carries on, and an exit
               counter whose last arriver resets every per-call counter (the
               general decode kernel's gate/up and slice counters);
  ticket    -- a reconstruction of the removed variant of the general decode
               kernel: items drawn from a global ticket counter, the next
               ticket drawn while the current item runs (its weights are
               requested at once), the counter reset by the workgroup that
               draws the last losing ticket, and an expired wait that leaves
               the item loop;
  ticket_fixed -- the same with the reset done by the last workgroup to exit
               (an exit path every workgroup takes, expired waits included) and
               every ticket-derived index clamped to the item count.

The reconstruction shows two flaws, one for each recorded symptom of the
removed variant.  Its reset trigger (the last losing ticket) is drawn at the
start of a workgroup's last item, so the reset can zero the counts that items
still running wait on: rows go missing, and counts left non-zero spoil the
next call.  And it requested an item's weights before comparing the ticket
with the item count: every call reads past the end of the item list, further
and further once the counter is stale, which on the device is an address past
the weight matrix.  The fixed protocol and the protocols in use pass every
scenario."""
import random

import pytest

# header words (u32 offsets) of the kernels, as declared in csrc/kernels.h and
# csrc/prefill.h; the general decode kernel's per-group and per-slice counters
WS_ERR, WS_EXIT, WS_ARRIVE, WS_EPOCH, WS_PF_ARRIVE, WS_ROUTER_ARRIVE = 0, 1, 2, 3, 4, 5
WS_GU, WS_DN = 16, 16 + 1024
WS_PF_CLAIM, PF_MAX_SLOTS = 2048, 1024 + 1    # claim word of slot s: WS_PF_CLAIM + s
WS_HEADER_WORDS = 16384 // 4
DEC_MAX_DIM, DEC_S2, DEC_MAX_T, MAX_TOPK = 8192, 64, 16, 32


class Mem:
    """The workspace header: u32 words, all zero in a fresh workspace."""

    def __init__(self):
        self.w = {}

    def ld(self, i):
        assert 0 <= i < WS_HEADER_WORDS, i
        return self.w.get(i, 0)

    def st(self, i, v):
        assert 0 <= i < WS_HEADER_WORDS, i
        self.w[i] = v & 0xFFFFFFFF

    def add(self, i, v):
        old = self.ld(i)
        self.st(i, old + v)
        return old


class Call:
    """What one call observed."""

    def __init__(self, n_items):
        self.done = [0] * n_items
        self.bad_index = []
        self.stale_start = []
        self.wrong_last = False


def run(wgs, rng):
    """Interleave the workgroup generators at random until all have finished."""
    live = list(wgs)
    while live:
        g = rng.choice(live)
        try:
            next(g)
        except StopIteration:
            live.remove(g)


# ---------------------------------------------------------------- protocols
def arrival_call(mem, call, G, word, expire):
    """G workgroups publish a count and arrive; the last one builds the plan."""
    results = {}

    def wg(w):
        if mem.ld(word) >= G:
            call.stale_start.append(w)
        yield
        results[w] = w + 1                       # its count, stored before the arrival
        yield
        prev = mem.add(word, 1)
        yield
        if prev == G - 1:
            if len(results) != G:
                call.wrong_last = True           # a "last" arriver that is not the last
            for v in range(G):
                call.done[v] += 1 if v in results else 0
            mem.st(word, 0)
            yield
    return [wg(w) for w in range(G)]


def exit_call(mem, call, G, n_gu, n_dn, expire):
    """Static item order: gate/up items then down items that wait (bounded) on
    their gate/up count; every workgroup arrives at the exit, the last resets."""
    total = n_gu + n_dn
    if any(mem.ld(WS_GU + j) for j in range(1)) or mem.ld(WS_EXIT):
        call.stale_start.append(-1)

    def wg(w):
        item = w
        while item < total:
            if item < n_gu:
                call.done[item] += 1
                yield
                mem.add(WS_GU, 1)
                yield
            else:
                spins = 0
                while mem.ld(WS_GU) < n_gu:
                    if expire or spins > 50:
                        mem.st(WS_ERR, 1)
                        break
                    spins += 1
                    yield
                call.done[item] += 1
                yield
            item += G
        old = mem.add(WS_EXIT, 1)
        yield
        if old == G - 1:
            mem.st(WS_GU, 0)
            mem.st(WS_EXIT, 0)
            yield
    return [wg(w) for w in range(G)]


def ticket_call(mem, call, G, n_gu, n_dn, expire, fixed):
    """Items drawn from a ticket counter; the next ticket is drawn, and its
    item's weights requested, while the current item runs."""
    total = n_gu + n_dn
    TKT = WS_ARRIVE
    if mem.ld(TKT) != 0:
        call.stale_start.append(mem.ld(TKT))

    def request(t):
        # the weight rows of item t: an index into the item list
        idx = min(t, total - 1) if fixed else t
        if not 0 <= idx < total:
            call.bad_index.append(t)

    def wg(w):
        t = mem.add(TKT, 1)
        yield
        while t < total:
            nxt = mem.add(TKT, 1)
            yield
            request(nxt)
            if t >= n_gu:
                spins, ok = 0, True
                while mem.ld(WS_GU) < n_gu:
                    if expire or spins > 50:
                        mem.st(WS_ERR, 1)
                        ok = False
                        break
                    spins += 1
                    yield
                if not ok and not fixed:
                    return                       # the removed variant left the item loop here
            call.done[t] += 1
            yield
            if t < n_gu:
                mem.add(WS_GU, 1)
                yield
            t = nxt
        if fixed:
            old = mem.add(WS_EXIT, 1)
            yield
            if old == G - 1:
                mem.st(TKT, 0)
                mem.st(WS_GU, 0)
                mem.st(WS_EXIT, 0)
                yield
        elif t == total + G - 1:                 # the last losing ticket resets
            mem.st(TKT, 0)
            mem.st(WS_GU, 0)
            yield
    return [wg(w) for w in range(G)]


def claim_call(mem, call, G, expire, n_slots=5, tokens_per_wg=2, picks=2):
    """Workgroup w routes tokens 2w, 2w + 1; pick r of token t is slot
    (t + 1 + 2r) % n_slots (distinct per token).  A claimed place at or past
    the token count is recorded as a bad index (the kernel compares it before
    forming an address); the last arriver checks the counts and that no place
    was handed out twice, then resets every claim word and the counter."""
    T = G * tokens_per_wg
    slot_of = lambda t, r: (t + 1 + 2 * r) % n_slots
    if mem.ld(WS_PF_ARRIVE) or any(mem.ld(WS_PF_CLAIM + s) for s in range(n_slots)):
        call.stale_start.append(-1)
    places = {}

    def wg(w):
        for j in range(tokens_per_wg):
            t = w * tokens_per_wg + j
            for r in range(picks):
                s = slot_of(t, r)
                p = mem.add(WS_PF_CLAIM + s, 1)
                yield
                if p >= T:
                    call.bad_index.append(p)
                    continue
                places[(s, p)] = places.get((s, p), 0) + 1
                call.done[t * picks + r] += 1
        prev = mem.add(WS_PF_ARRIVE, 1)
        yield
        if prev == G - 1:
            counts = [mem.ld(WS_PF_CLAIM + s) for s in range(n_slots)]
            want = [sum(slot_of(t, r) == s for t in range(T) for r in range(picks)) for s in range(n_slots)]
            if counts != want or any(v != 1 for v in places.values()):
                call.wrong_last = True
            for s in range(n_slots):
                mem.st(WS_PF_CLAIM + s, 0)
                yield
            mem.st(WS_PF_ARRIVE, 0)
            yield
    return [wg(w) for w in range(G)]


PROTOCOLS = {
    "arrival": lambda mem, call, G, expire: arrival_call(mem, call, G, WS_PF_ARRIVE, expire),
    "router_arrival": lambda mem, call, G, expire: arrival_call(mem, call, G, WS_ROUTER_ARRIVE, expire),
    "exit": lambda mem, call, G, expire: exit_call(mem, call, G, 6, 4, expire),
    "ticket": lambda mem, call, G, expire: ticket_call(mem, call, G, 6, 4, expire, False),
    "ticket_fixed": lambda mem, call, G, expire: ticket_call(mem, call, G, 6, 4, expire, True),
    "claim": lambda mem, call, G, expire: claim_call(mem, call, G, expire),
}
N_ITEMS = {"arrival": None, "router_arrival": None, "exit": 10, "ticket": 10, "ticket_fixed": 10, "claim": 32}


def one_call(name, mem, rng, G=8, expire=False):
    call = Call(N_ITEMS[name] or G)
    run(PROTOCOLS[name](mem, call, G, expire), rng)
    return call


def healthy(call, expire):
    """Every item once, nothing stale, no index out of range (an expired call
    may skip work; it reports the error word instead)."""
    ok = not call.stale_start and not call.bad_index and not call.wrong_last
    return ok and (expire or all(d == 1 for d in call.done))


# ---------------------------------------------------------------- scenarios
SCENARIOS = {
    # consecutive calls on one workspace
    "consecutive": [False] * 5,
    # a call whose waits all expire (the spin-limit hook), then normal calls
    "after_expired_wait": [True, False, False, False],
    # a captured launch replayed: the host clears nothing between replays
    "graph_replay": [False] * 6,
}


@pytest.mark.parametrize("scenario", sorted(SCENARIOS))
@pytest.mark.parametrize("name", ["arrival", "router_arrival", "exit", "claim", "ticket_fixed"])
def test_protocols_in_use_hold(name, scenario):
    for seed in range(40):
        rng = random.Random(seed)
        mem = Mem()
        for expire in SCENARIOS[scenario]:
            call = one_call(name, mem, rng, expire=expire)
            assert healthy(call, expire), (name, scenario, seed, call.__dict__)


def test_interleaved_kernels_share_one_header():
    """Calls of every protocol in use, interleaved on one workspace: each
    keeps to its own header words, so none sees another's counts."""
    for seed in range(40):
        rng = random.Random(seed)
        mem = Mem()
        for _ in range(3):
            for name in rng.sample(["arrival", "router_arrival", "exit", "claim", "ticket_fixed"], 5):
                call = one_call(name, mem, rng, expire=rng.random() < 0.3)
                assert not call.stale_start and not call.bad_index and not call.wrong_last, (name, seed)


def test_removed_ticket_variant_races_in_ordinary_calls():
    """With the next ticket drawn at the start of a workgroup's last item, the
    last losing ticket -- the variant's reset trigger -- can be drawn while
    other workgroups still run items: the reset zeroes the gate/up count that
    their down items wait on (the wait expires and the item is dropped: output
    rows missing), and gate/up items finishing after it leave the count
    non-zero for the next call."""
    lost = stale = 0
    for seed in range(40):
        rng = random.Random(seed)
        mem = Mem()
        for _ in range(4):
            call = one_call("ticket", mem, rng)
            lost += any(d == 0 for d in call.done)
            stale += bool(call.stale_start) or mem.ld(WS_GU) != 0
    assert lost > 0 and stale > 0, (lost, stale)


def test_removed_ticket_variant_requests_past_the_end():
    """Every workgroup's last draw is a losing ticket, and the variant issued
    that item's weight loads before comparing the ticket with the item count:
    with n items and G workgroups, a clean call requests items up to
    n + G - 1.  The recorded case had n = 10 items (six gate/up and four down
    slices of the fixed expert) and 256 workgroups: requests up to item 265,
    rows far past the end of the expert's weights -- an illegal address
    wherever that memory is not mapped, so the same call can read garbage in
    one process and fault in another."""
    total, G = 10, 8
    reach = 0
    for seed in range(40):
        call = one_call("ticket", Mem(), random.Random(seed), G=G)
        assert call.bad_index and min(call.bad_index) >= total
        reach = max(reach, max(call.bad_index))
    assert reach == total + G - 1
    # the fixed protocol clamps every such index (and still does every item once)
    for seed in range(40):
        call = one_call("ticket_fixed", Mem(), random.Random(seed), G=G)
        assert not call.bad_index and all(d == 1 for d in call.done)


def test_removed_ticket_variant_after_an_expired_wait():
    """A wait that expired left the item loop, so a workgroup that held the
    reset trigger never drew it: the next call on the workspace starts from a
    stale ticket count and loses rows."""
    stale = lost = 0
    for seed in range(40):
        rng = random.Random(seed)
        mem = Mem()
        one_call("ticket", mem, rng, expire=True)
        nxt = one_call("ticket", mem, rng)
        stale += bool(nxt.stale_start)
        lost += sum(nxt.done) < 10
    assert stale > 0 and lost > 0, (stale, lost)


def test_header_word_map_fits_and_does_not_overlap():
    """Every counter a kernel may touch, at the largest shapes the decode path
    accepts, lies inside the header, and no two kernels share a word."""
    n_groups = DEC_MAX_T * MAX_TOPK + 1
    n_slices = (DEC_MAX_DIM + DEC_S2 - 1) // DEC_S2
    gu = set(range(WS_GU, WS_GU + n_groups))
    dn = set(range(WS_DN, WS_DN + n_slices))
    singles = {WS_ERR, WS_EXIT, WS_ARRIVE, WS_EPOCH, WS_PF_ARRIVE, WS_ROUTER_ARRIVE}
    assert len(singles) == 6
    assert not (gu & dn) and not (gu & singles) and not (dn & singles)
    claims = set(range(WS_PF_CLAIM, WS_PF_CLAIM + PF_MAX_SLOTS))
    assert not (claims & (gu | dn | singles))
    assert max(gu | dn | singles | claims) < WS_HEADER_WORDS
    assert n_groups <= 1024 and WS_GU + 1024 <= WS_DN


def test_model_words_are_the_kernels_words():
    """The header words modelled here are the ones the kernel sources declare."""
    import os
    import re
    src = ""
    d = os.path.join(os.path.dirname(__file__), "..", "block_scaled_bit_moe_amd", "csrc")
    for f in ("kernels.h", "prefill.h", "decodeT_impl.h"):
        src += open(os.path.join(d, f)).read()
    found = dict((n, int(v)) for n, v in re.findall(r"constexpr (?:int|size_t) (WS_\w+) = (\d+)", src))
    want = {"WS_ERR": WS_ERR, "WS_EXIT": WS_EXIT, "WS_ARRIVE": WS_ARRIVE, "WS_EPOCH": WS_EPOCH,
            "WS_PF_ARRIVE": WS_PF_ARRIVE, "WS_ROUTER_ARRIVE": WS_ROUTER_ARRIVE, "WS_GU": WS_GU,
            "WS_PF_CLAIM": WS_PF_CLAIM,
            "WS_HEADER": WS_HEADER_WORDS * 4}
    for n, v in want.items():
        assert found.get(n) == v, (n, found.get(n), v)
    assert re.search(r"constexpr int WS_DN = 16 \+ 1024;", src) and WS_DN == 16 + 1024
