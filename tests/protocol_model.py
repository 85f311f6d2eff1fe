"""A CPU model of the walk's cross-workgroup selection protocol (Fig. 8 as an
all-gather), for testing its step tags, walk parities, line clearing and
watchdog under arbitrary interleavings.  Test infrastructure; it shares no
code with the library and models the protocol, not the kernel's code.

Protocol (one walk of `steps` steps over G workers, groups of 16, 8 copies):
  * at walk start, worker g clears its own first-level lines of the other
    parity, and the workers together clear the other parity's second-level
    lines;
  * at step t, worker g stores key | tag(t + 1) into first-level line
    [par][t & 1][g];
  * the leader of group r (worker r < 16) polls its members' lines until all
    carry tag t + 1, then stores the group maximum into second-level line
    [par][t & 1][copy][r] of every copy;
  * every worker polls the 16 group lines of its copy (g % 8) until all carry
    tag t + 1 and takes their maximum;
  * a wait that exceeds the watchdog latches a time-out and the worker stops.
The walk's last act advances the epoch, so the next walk uses the other parity.

Workers are generators; a seeded scheduler runs one step of a random runnable
worker at a time, so every interleaving the seed picks is a legal schedule.
"""
import random

TAG_SHIFT = 57
KEY_MASK = (1 << 50) - 1
GROUPS = 16
COPIES = 8


class Memory:
    """The control block: first- and second-level lines, both parities."""

    def __init__(self, G):
        self.G = G
        self.l1 = [[[0] * G for _ in range(2)] for _ in range(2)]
        self.l2 = [[[[0] * GROUPS for _ in range(COPIES)] for _ in range(2)] for _ in range(2)]
        self.epoch = 0
        self.err = None


def worker(mem, g, steps, keys, seen, par, watchdog, skip_clear=False, never_arrive_step=None):
    """One workgroup's walk; yields at every memory action (a scheduling point)."""
    G = mem.G
    q = par ^ 1
    if not skip_clear:
        for s in range(2):
            mem.l1[q][s][g] = 0
            yield
        for i in range(g, 2 * COPIES * GROUPS, G):   # the other parity's group lines, spread over the workers
            s, rest = divmod(i, COPIES * GROUPS)
            c, r = divmod(rest, GROUPS)
            mem.l2[q][s][c][r] = 0
            yield
    grp = g % GROUPS
    for t in range(steps):
        want = t + 1
        tag = want << TAG_SHIFT
        if never_arrive_step == t:
            return
        mem.l1[par][t & 1][g] = tag | keys[t][g]
        yield
        if g < GROUPS:
            members = list(range(grp, G, GROUPS))
            waited = 0
            while True:
                vals = []
                for m in members:
                    vals.append(mem.l1[par][t & 1][m])
                    yield
                if all(v >> TAG_SHIFT == want for v in vals):
                    break
                waited += 1
                if waited > watchdog:
                    mem.err = mem.err or "timeout"
                    return
            best = max(v & KEY_MASK for v in vals)
            for c in range(COPIES):
                mem.l2[par][t & 1][c][grp] = tag | best
                yield
        ngr = min(G, GROUPS)
        waited = 0
        while True:
            vals = []
            for r in range(ngr):
                vals.append(mem.l2[par][t & 1][g % COPIES][r])
                yield
            if all(v >> TAG_SHIFT == want for v in vals):
                break
            waited += 1
            if waited > watchdog:
                mem.err = mem.err or "timeout"
                return
        seen[t][g] = max(v & KEY_MASK for v in vals)
    if g == 0:
        mem.epoch += 1


def run_walk(mem, keys, rng, watchdog=10_000, skip_clear=False, never_arrive=None):
    """Run one walk to completion under a random schedule.  keys[t][g]: the
    key worker g publishes at step t.  never_arrive=(g, t): that worker
    stops before publishing at step t.  Returns seen[t][g] (None where a
    worker did not finish the step)."""
    G = mem.G
    steps = len(keys)
    par = mem.epoch & 1
    seen = [[None] * G for _ in range(steps)]
    gens = {}
    for g in range(G):
        nas = never_arrive[1] if never_arrive and never_arrive[0] == g else None
        gens[g] = worker(mem, g, steps, keys, seen, par, watchdog, skip_clear, nas)
    live = list(gens)
    while live:
        g = rng.choice(live)
        try:
            next(gens[g])
        except StopIteration:
            live.remove(g)
    return seen


def random_keys(rng, steps, G, ties=False):
    """Distinct (or, with ties, often equal) positive keys below the tag bits."""
    out = []
    for _ in range(steps):
        if ties:
            base = rng.randrange(1, 1 << 20)
            out.append([(base << 18) | rng.choice([5, 9, 200]) for _ in range(G)])
        else:
            out.append([rng.randrange(1, 1 << 50) for _ in range(G)])
    return out
