"""Oracle of the service-aware profile selection.

Test infrastructure: only the tests, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may use anything under oracle/.  Plain Python in float64,
written from "KVServe: Service-Aware KV Cache Compression for Communication-
Efficient Disaggregated LLM Serving":

  Sec. 3.1   profile (cr_p, s_p); s_p = (1/s_enc + 1/s_dec)^-1
  Sec. 3.2   Eq. 1: T_p = T_model + V/s_p + V/(B cr_p); T_0 = T_model + V/B;
             Eq. 2-3: feasible set and arg-min
  Sec. 6.1   Eq. 5 (Theorem 6.1): B*_p = (1 - 1/cr_p) s_p;
             Eq. 6 (Theorem 6.2): lines 1/s_p + x/cr_p in x = 1/B, optimal
             profile = lower envelope, piecewise constant in x
  Sec. 6.2   candidate set (envelope optimum + neighbours), EWMA residual
             (Eq. 7), corrected latency (Eq. 8), epsilon-greedy, guardrails
             (predicted T <= T_SLO with a fallback; cooldown after more than K
             violations in the last M uses)

Readings where the page is open (the same ones the library takes): raw
transfer is the envelope line (intercept 0, slope 1, id RAW); intervals are
closed on the left; equal lines keep the lowest id; candidates are the
interval's profile and the adjacent envelope intervals' profiles in envelope
order; residuals start at 0; environment = (bucket, envelope interval of the
request's bandwidth); the k-th choose call draws outputs 2k and 2k+1 of
splitmix64 seeded with `seed`, explores when at least two candidates are
feasible and (out_2k >> 11) / 2^53 < epsilon, then takes candidate
out_{2k+1} mod n of the other n feasible candidates (envelope order); the
greedy choice is the lowest corrected latency, ties to the earlier envelope
position; a violation is an observed time above T_SLO; cooldown: the next
cooldown_len choose calls, per profile, history cleared.
"""
from __future__ import annotations

RAW = -1
_M64 = (1 << 64) - 1


def splitmix64(seed: int, n: int) -> int:
    """Output n (0-based) of splitmix64 (Steele, Lea and Flood, OOPSLA 2014)
    started at state `seed`: the state advances by the golden-ratio constant
    before each output, so output n mixes seed + (n + 1) * gamma."""
    z = (seed + (n + 1) * 0x9E3779B97F4A7C15) & _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def harmonic(s_enc: float, s_dec: float) -> float:
    """Sec. 3.1: the throughput at which V bytes take V/s_enc + V/s_dec."""
    return 1.0 / (1.0 / s_enc + 1.0 / s_dec)


def break_even(cr: float, s_enc: float, s_dec: float) -> float:
    """Eq. 5."""
    return (1.0 - 1.0 / cr) * harmonic(s_enc, s_dec)


def jct(profile, bandwidth: float, volume: float, t_model: float) -> float:
    """Eq. 1; profile = (id, bucket, cr, s_enc, s_dec) or None for raw transfer."""
    if profile is None:
        return t_model + volume / bandwidth
    _, _, cr, se, sd = profile
    return t_model + volume / harmonic(se, sd) + volume / (bandwidth * cr)


def lines_of(profiles, bucket):
    """Eq. 6 lines (id, intercept 1/s_p, slope 1/cr_p) of a bucket, raw first."""
    out = [(RAW, 0.0, 1.0)]
    for pid, b, cr, se, sd in profiles:
        if b == bucket:
            out.append((pid, 1.0 / se + 1.0 / sd, 1.0 / cr))   # codec seconds per byte
    return out


def argmin_line(lines, x):
    best = None
    for pid, a, b in lines:
        y = a + b * x
        if best is None or y < best[0] or (y == best[0] and pid < best[1]):
            best = (y, pid)
    return best[1]


def envelope(profiles, bucket):
    """Theorem 6.2 by enumeration: every pairwise intersection at x >= 0 is a
    possible breakpoint; between consecutive ones the minimizing line is
    constant and is read off at the midpoint (past the last one, at a point
    beyond it).  Returns (ids, x_from)."""
    ls = lines_of(profiles, bucket)
    pts = {0.0}
    for i in range(len(ls)):
        for j in range(i + 1, len(ls)):
            (_, a1, b1), (_, a2, b2) = ls[i], ls[j]
            if b1 != b2:
                x = (a2 - a1) / (b1 - b2)
                if x >= 0.0:
                    pts.add(x)
    pts = sorted(pts)
    ids, xs = [], []
    for k, x0 in enumerate(pts):
        probe = (x0 + pts[k + 1]) / 2 if k + 1 < len(pts) else (2 * x0 + 1.0)
        pid = argmin_line(ls, probe)
        if not ids or ids[-1] != pid:
            ids.append(pid)
            xs.append(x0)
    return ids, xs


def interval_of(xs, bandwidth):
    x = 1.0 / bandwidth
    k = 0
    for i, x0 in enumerate(xs):
        if x0 <= x:
            k = i
    return k


class Selector:
    """Sec. 6.2 controller state, one step per call."""

    def __init__(self, profiles, fallback_id=RAW, alpha=0.2, epsilon=0.1, cooldown_k=2, cooldown_m=8,
                 cooldown_len=16, seed=0):
        self.profiles = {p[0]: tuple(p) for p in profiles}
        self.plist = [tuple(p) for p in profiles]
        self.fallback = fallback_id
        self.alpha, self.epsilon = alpha, epsilon
        self.K, self.M, self.L = cooldown_k, cooldown_m, cooldown_len
        self.seed = seed
        self.calls = 0
        self.res = {}        # (bucket, interval, id) -> [residual, uses]
        self.hist = {}       # id -> list of recent violation flags (newest last)
        self.until = {}      # id -> first choose call it may take part in again

    def draw(self, n: int) -> int:
        return splitmix64(self.seed, n)

    def _profile(self, pid):
        return None if pid == RAW else self.profiles[pid]

    def choose(self, bucket, bandwidth, volume, t_model, t_slo):
        ids, xs = envelope(self.plist, bucket)
        i = interval_of(xs, bandwidth)
        k = self.calls
        self.calls += 1
        feas = []
        for j in range(max(0, i - 1), min(len(ids) - 1, i + 1) + 1):
            pid = ids[j]
            if k < self.until.get(pid, 0):
                continue
            pred = jct(self._profile(pid), bandwidth, volume, t_model)
            if not pred <= t_slo:
                continue
            r = self.res.get((bucket, i, pid), [0.0, 0])[0]
            feas.append((pid, pred, pred + r))
        if not feas:
            return self.fallback, jct(self._profile(self.fallback), bandwidth, volume, t_model)
        g = 0
        for j in range(1, len(feas)):
            if feas[j][2] < feas[g][2]:
                g = j
        pick = g
        if len(feas) >= 2:
            u = self.draw(2 * k)
            if (u >> 11) / 2.0 ** 53 < self.epsilon:
                others = [j for j in range(len(feas)) if j != g]
                pick = others[self.draw(2 * k + 1) % len(others)]
        return feas[pick][0], feas[pick][1]

    def observe(self, bucket, bandwidth, volume, t_model, t_slo, pid, observed):
        ids, xs = envelope(self.plist, bucket)
        i = interval_of(xs, bandwidth)
        st = self.res.setdefault((bucket, i, pid), [0.0, 0])
        delta = observed - jct(self._profile(pid), bandwidth, volume, t_model)
        st[0] = (1.0 - self.alpha) * st[0] + self.alpha * delta      # Eq. 7
        st[1] += 1
        h = self.hist.setdefault(pid, [])
        h.append(observed > t_slo)
        del h[:-self.M]
        if sum(h) > self.K:
            self.until[pid] = self.calls + self.L
            h.clear()

    def state(self, bucket, bandwidth, pid):
        ids, xs = envelope(self.plist, bucket)
        i = interval_of(xs, bandwidth)
        r, n = self.res.get((bucket, i, pid), [0.0, 0])
        return r, n, max(0, self.until.get(pid, 0) - self.calls)
