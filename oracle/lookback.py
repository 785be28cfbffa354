"""Float64 simulator of the single-pass decoupled look-back scan protocol.
Test infrastructure only.

Follows "Selective-scan CUDA kernels", sections "The problem" (the affine
combine is associative but not commutative) and "The five kernels" (each tile
publishes its local aggregate under flag A, walks back until it meets a
predecessor's inclusive prefix under flag P, then publishes its own P; tiles
are claimed in order from a counter so a waiting tile's predecessors are
always already claimed; the warp variant inspects a window of predecessors at
once).

The simulator runs the protocol with any element type and combine, under a
seeded random interleaving of the tiles' steps, so a reordered or swapped
combine shows up as a wrong answer.  A tile whose predecessors never publish
is reported as a deadlock after a step bound instead of spinning forever.
"""
from __future__ import annotations

import random

EMPTY, AGG, INC = 0, 1, 2


class Deadlock(RuntimeError):
    pass


def lookback_scan(elements, combine, identity, tile, window=64, seed=0,
                  resident=8, max_steps=10_000_000, swap_combine=False,
                  never_publish=None):
    """Inclusive scan of ``elements`` (one chain) through simulated tiles.

    ``combine(first, second)`` composes two elements, ``first`` earlier in the
    sequence.  Returns the list of inclusive prefixes.  ``swap_combine`` runs
    the deliberately broken variant that calls combine(later, earlier) in the
    look-back and in the final apply; ``never_publish`` names a tile that
    stalls, to exercise the deadlock bound.
    """
    def comb(first, second):
        return combine(second, first) if swap_combine else combine(first, second)

    rng = random.Random(seed)
    n = len(elements)
    ntiles = -(-n // tile)
    status = [EMPTY] * ntiles
    agg = [None] * ntiles
    inc = [None] * ntiles
    out = [None] * n
    next_claim = 0
    active = {}  # tile -> state dict
    steps = 0
    done = 0

    def local_scan(t):
        lo, hi = t * tile, min((t + 1) * tile, n)
        acc = None
        pref = []
        for i in range(lo, hi):
            acc = elements[i] if acc is None else combine(acc, elements[i])
            pref.append(acc)
        return pref

    while done < ntiles:
        steps += 1
        if steps > max_steps:
            raise Deadlock(f"no progress after {max_steps} steps; waiting tiles {sorted(active)}")
        while len(active) < resident and next_claim < ntiles:
            active[next_claim] = {"phase": 0}
            next_claim += 1
        t = rng.choice(sorted(active))
        st = active[t]
        if st["phase"] == 0:
            st["local"] = local_scan(t)
            if t == never_publish:
                st["phase"] = 9
                continue
            if t == 0:
                inc[0] = st["local"][-1]
                status[0] = INC
                st["prefix"] = None
                st["phase"] = 2
            else:
                agg[t] = st["local"][-1]
                status[t] = AGG
                st["phase"] = 1
                st["look"] = t - 1
                st["acc"] = None  # combination of AGGs already walked, earliest first
        elif st["phase"] == 1:
            # inspect up to `window` predecessors at once, nearest first
            lo = max(st["look"] - window + 1, 0)
            view = list(range(st["look"], lo - 1, -1))
            flags = [status[p] for p in view]
            resolved = False
            acc = st["acc"]
            for p, f in zip(view, flags):
                if f == EMPTY:
                    break  # a predecessor has not published yet: retry later
                if f == INC:
                    prefix = inc[p] if acc is None else comb(inc[p], acc)
                    resolved = True
                    break
                acc = agg[p] if acc is None else comb(agg[p], acc)
            else:
                # the whole window held aggregates: keep them and walk further back
                st["acc"] = acc
                st["look"] = lo - 1
                continue
            if resolved:
                st["prefix"] = prefix
                inc[t] = comb(prefix, st["local"][-1])
                status[t] = INC
                st["phase"] = 2
        elif st["phase"] == 2:
            lo = t * tile
            for k, v in enumerate(st["local"]):
                out[lo + k] = v if st["prefix"] is None else comb(st["prefix"], v)
            del active[t]
            done += 1
        else:  # stalled tile
            continue
    return out


def lookback_scan_halves(pairs, combine, tile, window=64, seed=0, resident=8, check_tags=True,
                         max_steps=10_000_000, anchor=None):
    """The look-back protocol of ``lookback_scan`` with each status word
    written and read as two halves, (tag, a) and (tag, b), where a and b are
    the two parts of the scalar recurrence's affine pair and the tag is the
    word's kind (0 unpublished, AGG, INC).

    A writer stores the two halves in two separate steps, and a tile's
    inclusive prefix later overwrites its aggregate in place; a reader loads
    the halves of its window in two separate steps.  Any interleaving can
    therefore show a reader one half of one publication and the other half of
    another (a torn read).  With ``check_tags`` a word counts only when both
    halves carry the same nonzero tag (otherwise it is read as not yet
    published and polled again); ``check_tags=False`` is the broken variant
    that trusts the first half's tag, which a torn read corrupts.

    ``anchor``: the anchored form of the protocol.  Tiles whose index is a
    multiple of ``anchor`` (anchors) publish only their inclusive prefix; the
    others publish only their aggregate.  Tile t looks back exactly to the
    anchor a = anchor * ((t - 1) // anchor), takes its inclusive prefix and
    folds the aggregates of tiles a + 1 .. t - 1, nearest first.  Which
    predecessors had published when a tile looked back then changes nothing in
    the combine order, so every interleaving gives the same values to the
    last bit (with the nearest-prefix form, the grouping follows the timing).
    ``anchor`` must not exceed ``window``, so one window reaches the anchor.
    """
    if anchor is not None and not 1 <= anchor <= window:
        raise ValueError("anchor must be in [1, window]")
    rng = random.Random(seed)
    n = len(pairs)
    ntiles = -(-n // tile)
    halves = [[(EMPTY, None), (EMPTY, None)] for _ in range(ntiles)]
    out = [None] * n
    next_claim = 0
    active = {}
    steps = 0
    done = 0

    def local_scan(t):
        acc = None
        pref = []
        for i in range(t * tile, min((t + 1) * tile, n)):
            acc = pairs[i] if acc is None else combine(acc, pairs[i])
            pref.append(acc)
        return pref

    while done < ntiles:
        steps += 1
        if steps > max_steps:
            raise Deadlock(f"no progress after {max_steps} steps; waiting tiles {sorted(active)}")
        while len(active) < resident and next_claim < ntiles:
            active[next_claim] = {"phase": "scan"}
            next_claim += 1
        t = rng.choice(sorted(active))
        st = active[t]
        ph = st["phase"]
        if ph == "scan":
            st["local"] = local_scan(t)
            st["prefix"] = None
            if anchor is not None and t > 0 and t % anchor == 0:
                # an anchor publishes nothing before its look-back
                st["phase"] = "read0"
                st["look"] = t - 1
                st["acc"] = None
                continue
            st["pub"] = (INC if t == 0 else AGG, st["local"][-1], "half0")
            st["phase"] = "publish"
        elif ph == "publish":  # one half per step
            kind, val, which = st["pub"]
            if which == "half0":
                halves[t][0] = (kind, val[0])
                st["pub"] = (kind, val, "half1")
            else:
                halves[t][1] = (kind, val[1])
                if kind == INC or (anchor is not None and st["prefix"] is not None):
                    st["phase"] = "apply"
                else:
                    st["phase"] = "read0"
                    st["look"] = t - 1
                    st["acc"] = None
        elif ph == "read0":  # first halves of the window, nearest first
            lo = max(st["look"] - window + 1, 0)
            if anchor is not None:
                lo = anchor * (st["look"] // anchor)  # exactly back to the anchor
            st["view"] = list(range(st["look"], lo - 1, -1))
            st["w0"] = [halves[p][0] for p in st["view"]]
            st["phase"] = "read1"
        elif ph == "read1":  # second halves, at a later step
            w1 = [halves[p][1] for p in st["view"]]
            acc = st["acc"]
            resolved = False
            retry = False
            for p, (t0, a), (t1, b) in zip(st["view"], st["w0"], w1):
                kind = (t0 if t0 == t1 else EMPTY) if check_tags else t0
                if anchor is not None and p % anchor == 0 and kind != INC:
                    kind = EMPTY  # an anchor counts only once it holds its inclusive prefix
                if kind == EMPTY:
                    retry = True
                    break
                val = (a, b)
                if kind == INC:
                    prefix = val if acc is None else combine(val, acc)
                    resolved = True
                    break
                acc = val if acc is None else combine(val, acc)
            if resolved:
                st["prefix"] = prefix
                if anchor is not None and t % anchor != 0:
                    st["phase"] = "apply"  # only anchors publish an inclusive prefix
                else:
                    st["pub"] = (INC, combine(prefix, st["local"][-1]), "half0")
                    st["phase"] = "publish"
            elif retry:
                st["phase"] = "read0"  # poll again from the same place
            else:
                st["acc"] = acc
                st["look"] = st["view"][-1] - 1
                st["phase"] = "read0"
        elif ph == "apply":
            lo = t * tile
            for k, v in enumerate(st["local"]):
                out[lo + k] = v if st["prefix"] is None else combine(st["prefix"], v)
            del active[t]
            done += 1
    return out
