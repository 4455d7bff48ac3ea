"""Host-side model of the attention kernel's two-group phase schedule.

The fused kernel runs two 4-wave groups per work-group half a tile apart,
with a work-group barrier after every phase and K/V tiles double-buffered in
LDS (csrc/attn_kernel.hip, the kernel's schedule comment). This test replays,
in Python, the phase sequence each group executes -- the same peeling of the
first pair, the two-at-a-time steady loop, the masked last tile and the idle
pairs -- and checks for every tile count a launch can see:

* both groups arrive at the same number of barriers, of the same kinds in the
  same order (a mismatch would hang the work-group);
* the loads of pair t are issued once each: K(t+1) by group 0 in the pair's
  first phase, V(t) by group 1 in its second phase (each group during its
  matrix phase, or in an idle pair where it has none);
* every LDS read finds the tile it expects in its buffer, and no load in
  flight targets a buffer that is being read;
* each group reads every K and V tile it attends to exactly once, in order.

It models the schedule only (no arithmetic), so it runs without a GPU.
"""
import pytest

BQ = BKV = 128


def tiles_for(q_tile, nk, causal):
    kv_end = min(nk, (q_tile + 1) * BQ) if causal else nk
    return (kv_end + BKV - 1) // BKV


def group_events(grp, n, n_wg):
    """Events of one group: ('load_k', t) for K(t+1), ('load_v', t) for V(t),
    ('read_k', t), ('read_v', t), ('bar',), ('barw',)."""
    ev = []
    bar, barw = ('bar',), ('barw',)
    own = 'load_k' if grp == 0 else 'load_v'    # group 0 loads K(t+1), group 1 V(t)

    def x(t, pv, qk):
        if pv:
            ev.append(('read_v', t - 1))
        if qk:
            ev.append(('read_k', t))

    def pair(t, first, second):
        # a group issues its load of pair t in its own phase of the pair: the
        # first for group 0, the second for group 1
        if grp == 0:
            ev.append((own, t))
        first()
        ev.append(bar)
        if grp == 1:
            ev.append((own, t))
        second()
        ev.append(barw)

    nothing = lambda: None
    if grp == 0:                                   # pair t: X(t) | Y(t)
        if n > 0:
            pair(0, lambda: x(0, False, True), nothing)
            t = 1
            while t + 1 <= n - 2:
                for tt in (t, t + 1):
                    pair(tt, lambda tt=tt: x(tt, True, True), nothing)
                t += 2
            if t <= n - 2:
                pair(t, lambda: x(t, True, True), nothing)
            if n >= 2:
                pair(n - 1, lambda: x(n - 1, True, True), nothing)
            pair(n, lambda: x(n, True, False), nothing)
    else:                                          # pair t: Y(t-1) | X(t)
        if n > 0:
            pair(0, nothing, lambda: x(0, False, True))
            t = 1
            while t + 1 <= n - 1:
                for tt in (t, t + 1):
                    pair(tt, nothing, lambda tt=tt: x(tt, True, True))
                t += 2
            if t <= n - 1:
                pair(t, nothing, lambda: x(t, True, True))
            # the last pair: PV(n-1) only; a live group 1 walks every tile of
            # the work-group (n == n_wg), so there is no V(n) to load
            assert n == n_wg
            ev.append(bar)
            x(n, True, False)
            ev.append(barw)
    for t in range(n + (1 if n > 0 else 0), n_wg + 1):
        pair(t, nothing, nothing)
    return ev


def check_work_group(nq, nk, causal, qp):
    live = [(2 * qp + g) * BQ < nq for g in (0, 1)]
    ns = [tiles_for(2 * qp + g, nk, causal) if live[g] else 0 for g in (0, 1)]
    n_wg = tiles_for(2 * qp + 1, nk, causal) if live[1] else tiles_for(2 * qp, nk, causal)
    evs = [group_events(g, ns[g], n_wg) for g in (0, 1)]
    kinds = [[e[0] for e in ev if e[0] in ('bar', 'barw')] for ev in evs]
    assert kinds[0] == kinds[1], "groups must meet the same barriers"
    phases = []
    for ev in evs:
        ph = [[]]
        for e in ev:
            ph[-1].append(e)
            if e[0] in ('bar', 'barw'):
                ph.append([])
        phases.append(ph[:-1])
    kbuf = {0: 0, 1: None}                          # K(0) is staged before the first phase
    vbuf = {0: None, 1: None}
    pending = []
    issued_k, issued_v = [], []
    for p in range(len(kinds[0])):
        lk = [[e[1] for e in phases[g][p] if e[0] == 'load_k'] for g in (0, 1)]
        lv = [[e[1] for e in phases[g][p] if e[0] == 'load_v'] for g in (0, 1)]
        assert lk[1] == [] and lv[0] == [], "K loads by group 0, V loads by group 1"
        assert lk[0] == ([p // 2] if p % 2 == 0 else []), "K(t+1) in pair t's first phase"
        assert lv[1] in ([], [p // 2]) if p % 2 == 1 else lv[1] == [], "V(t) in pair t's second phase"
        issued_k += lk[0]
        issued_v += lv[1]
        for t in lk[0]:
            if t + 1 < n_wg:
                pending.append(('k', (t + 1) & 1, t + 1))
        for t in lv[1]:
            if t < n_wg:
                pending.append(('v', t & 1, t))
        for g in (0, 1):
            for e in phases[g][p]:
                if e[0] in ('read_k', 'read_v'):
                    kind, t = e[0][-1], e[1]
                    buf = kbuf if kind == 'k' else vbuf
                    assert buf[t & 1] == t, (kind, t, buf)
                    assert not any(pk == kind and pb == (t & 1) for pk, pb, _ in pending), "read of a buffer being loaded"
        if kinds[0][p] == 'barw':                  # loads have landed
            for kind, b, t in pending:
                (kbuf if kind == 'k' else vbuf)[b] = t
            pending = []
    assert issued_k == list(range(n_wg + 1)), "every pair's K load is issued once"
    assert [t for t in issued_v if t < n_wg] == list(range(n_wg)), "every V tile is loaded once, in order"
    for g in (0, 1):
        assert [e[1] for e in evs[g] if e[0] == 'read_k'] == list(range(ns[g]))
        assert [e[1] for e in evs[g] if e[0] == 'read_v'] == list(range(ns[g]))


SHAPES = [(nq, nk, False) for nq in (1, 100, 128, 129, 255, 256, 257, 300, 640, 1000, 4096)
          for nk in (1, 7, 128, 129, 300, 1000, 4096)]
SHAPES += [(n, n, True) for n in (1, 65, 127, 128, 129, 255, 256, 257, 333, 384, 512, 640, 1000, 4096, 8192)]
SHAPES += [(32768, 32768, False), (32768, 32768, True), (16384, 16384, False)]
# a sequence of a packed batch can have queries but no keys: both groups idle
SHAPES += [(nq, 0, c) for nq in (1, 200, 300) for c in (False, True)]


@pytest.mark.parametrize("nq,nk,causal", SHAPES)
def test_phase_schedule_is_consistent(nq, nk, causal):
    n_qp = (nq + 2 * BQ - 1) // (2 * BQ)
    for qp in range(n_qp):
        check_work_group(nq, nk, causal, qp)


def test_model_catches_a_missing_barrier(monkeypatch):
    """The check fails when one group skips a phase (the kind of slip that hangs)."""
    orig = group_events

    def broken(grp, n, n_wg):
        ev = orig(grp, n, n_wg)
        if grp == 1:
            i = ev.index(('bar',))
            ev = ev[:i] + ev[i + 1:]
        return ev
    monkeypatch.setitem(globals(), "group_events", broken)
    with pytest.raises(AssertionError):
        check_work_group(1000, 1000, False, 0)


def test_model_catches_a_late_value_load(monkeypatch):
    """The check fails when group 1 issues V(t) a phase late (after the wait
    that should have landed it): group 0 would read a buffer still loading."""
    orig = group_events

    def late(grp, n, n_wg):
        ev = orig(grp, n, n_wg)
        if grp == 1:
            i = next(i for i, e in enumerate(ev) if e[0] == 'load_v' and e[1] == 1)
            j = ev.index(('barw',), i)
            ev = ev[:i] + ev[i + 1:j + 1] + [ev[i]] + ev[j + 1:]
        return ev
    monkeypatch.setitem(globals(), "group_events", late)
    with pytest.raises(AssertionError):
        check_work_group(1000, 1000, False, 0)
