"""The tree kernel's multi-node schedule, modelled on the CPU, against a plain heap.

The kernel expands up to p frontier nodes per request per step, takes a
frontier entry only if fewer than N + 1 taken records precede it in the total
order (score desc, depth asc, token asc, parent's order asc), compacts its
record set when full, and ranks the records at the end.  This model follows
the same schedule step for step (batches that do not end inside a group of
equal keys, the acceptance test, pruning with tau, the frontier cut after N + 1
entries outside a tie group, compaction, the recursive comparator for equal
keys) on random trees with many exact ties, and checks
that it returns exactly the tree of the one-node-at-a-time heap.  It shares no
code with the kernel or with the oracle; the GPU parity tests check the kernel.
"""
import heapq
import random

import pytest


def seq_build(children, N):
    # children(path) -> list of (m, lp); path = tuple of m; total order (score desc, depth asc, m asc, parent asc)
    heap = []
    out = [((), 0.0, -1, 0)]  # (path, score, parent, depth)
    for m, lp in children(()):
        heapq.heappush(heap, (-(0.0 + lp), 1, m, 0, (m,)))
    while heap and len(out) < N + 1:
        negs, d, m, par, path = heapq.heappop(heap)
        i = len(out)
        out.append((path, -negs, par, d))
        if i < N:
            for mm, lp in children(path):
                heapq.heappush(heap, (-(-negs + lp), d + 1, mm, i, path + (mm,)))
    return out

def model_build(children, N, p, qmax, D):
    xcap = N + 1 + 2 * qmax
    # record: dict(U, par, path, score, depth, m, expanded)
    def U(score, depth, m):
        return (score, -depth, -m)       # larger = earlier
    rec = [dict(U=U(0.0, 0, -1), par=-1, path=(), score=0.0, depth=0, m=-1)]
    def rec_better(x, y):
        for _ in range(40):
            if x == y or x < 0 or y < 0: return False
            if rec[x]['U'] != rec[y]['U']: return rec[x]['U'] > rec[y]['U']
            x, y = rec[x]['par'], rec[y]['par']
        return False
    # frontier entries: (U, par, m, path, score, depth); key order = (U, par, m) desc
    front = []
    tau = None
    def key(f): return (f[0], f[1], f[2])
    def entry_better(f, g):
        if f[0] != g[0]: return f[0] > g[0]
        return rec_better(f[1], g[1])
    ex = [0]
    steps = 0
    while True:
        steps += 1
        assert steps <= N + 1, "too many steps"
        # expand
        new = []
        for y in ex:
            r = rec[y]
            for mm, lp in children(r['path']):
                s = r['score'] + lp
                new.append((U(s, r['depth'] + 1, mm), y, mm, r['path'] + (mm,), s, r['depth'] + 1))
        # merge with tau pruning
        if tau is not None:
            front = [f for f in front if f[0] >= tau]
            new = [f for f in new if f[0] >= tau]
        front = sorted(front + new, key=key, reverse=True)
        # keep N + 1 entries unless entry N + 1 shares entry N's U: the rest
        # have N + 1 entries of greater U ahead of them and are never taken
        if len(front) > N + 1 and front[N + 1][0] != front[N][0]:
            front = front[:N + 1]
        # pop
        ex = []
        stop = False
        rounds = 0
        while not stop:
            rounds += 1
            assert rounds < 10000
            if len(rec) + qmax > xcap:
                if ex: break
                # compaction
                rank = [sum(1 for y in range(len(rec)) if rec[y]['U'] > rec[x]['U'] or (rec[y]['U'] == rec[x]['U'] and y != x and rec_better(rec[y]['par'], rec[x]['par']))) for x in range(len(rec))]
                rN = rank.index(N)
                tauN = rec[rN]['U']
                tau = tauN if tau is None or tauN > tau else tau
                front = [f for f in front if f[0] >= tauN]
                for f in front: assert rank[f[1]] <= N
                newrec = [None] * (N + 1)
                for x in range(len(rec)):
                    if rank[x] <= N:
                        r = dict(rec[x]); r['par'] = rank[r['par']] if r['par'] >= 0 else -1
                        newrec[rank[x]] = r
                front = [(f[0], rank[f[1]], f[2], f[3], f[4], f[5]) for f in front]
                front.sort(key=key, reverse=True)
                rec[:] = newrec
            q = min(len(front), qmax, xcap - len(rec))
            special = False
            if q > 0 and q < len(front) and front[q - 1][0] == front[q][0]:
                u = front[q - 1][0]
                while q > 0 and front[q - 1][0] == u: q -= 1
                if q == 0:
                    g = 0
                    i = 1
                    while i < len(front) and front[i][0] == u:
                        if entry_better(front[i], front[g]): g = i
                        i += 1
                    best = front.pop(g); front.insert(0, best); special = g
                    q = 1
            if q <= 0: break
            batch = front[:q]
            cnt = []
            for f in batch:
                cnt.append(sum(1 for y in range(len(rec)) if rec[y]['U'] > f[0] or (rec[y]['U'] == f[0] and rec_better(rec[y]['par'], f[1]))))
            perm = list(range(q))
            # insertion sort by total order
            for i in range(1, q):
                v = perm[i]; jj = i
                while jj > 0 and entry_better(batch[v], batch[perm[jj - 1]]):
                    perm[jj] = perm[jj - 1]; jj -= 1
                perm[jj] = v
            acc = [0] * q
            out = False; st = False; A = 0
            for jj in range(q):
                j = perm[jj]; f = batch[j]
                if cnt[j] + jj >= N + 1:
                    tau = f[0] if tau is None or f[0] > tau else tau
                    out = True; break
                if f[5] < D:
                    if len(ex) == p: st = True; break
                rec.append(dict(U=f[0], par=f[1], path=f[3], score=f[4], depth=f[5], m=f[2]))
                if f[5] < D: ex.append(len(rec) - 1)
                acc[j] = 1; A += 1
            if special is not False and A == 0 and not out:
                best = front.pop(0); front.insert(special, best)
            if out:
                front = []
            else:
                front = [batch[j] for j in range(q) if not acc[j]] + front[q:]
            stop = out or st or len(ex) == p
        if not ex:
            break
    # final ranking
    nx = len(rec)
    rank = [sum(1 for y in range(nx) if rec[y]['U'] > rec[x]['U'] or (rec[y]['U'] == rec[x]['U'] and y != x and rec_better(rec[y]['par'], rec[x]['par']))) for x in range(nx)]
    res = [None] * min(nx, N + 1)
    for x in range(nx):
        if rank[x] <= N:
            r = rec[x]
            res[rank[x]] = (r['path'], r['score'], rank[r['par']] if r['par'] >= 0 else -1, r['depth'])
    return res, steps



def _children_fn(case, D, M, k, mode):
    cache = {}

    def children(path):
        if len(path) >= D:
            return []
        if path not in cache:
            rng = random.Random(hash((path, case)))
            if mode < 0.4:      # heavy exact ties
                lps = [-float(rng.randint(0, 2)) for _ in range(M)]
            elif mode < 0.7:    # all equal
                lps = [-1.0] * M
            else:
                lps = [-rng.random() * 3 for _ in range(M)]
            order = sorted(range(M), key=lambda m: (-lps[m], m))[:k]
            ch = [(m, lps[m]) for m in order]
            if mode > 0.9 and rng.random() < 0.3:
                ch = ch[:max(0, len(ch) - 1)]   # a child without a finite log-prob
            cache[path] = ch
        return cache[path]
    return children


@pytest.mark.parametrize("seed", range(4))
def test_schedule_matches_sequential_heap(seed):
    rnd = random.Random(1000 + seed)
    for case in range(150):
        D, M = rnd.randint(1, 6), rnd.randint(1, 6)
        k, N = rnd.randint(1, M), rnd.randint(1, 60)
        p, qmax = rnd.randint(1, 16), rnd.choice([1, 2, 4, 8, 32])
        children = _children_fn((seed, case), D, M, k, rnd.random())
        ref = seq_build(children, N)
        got, steps = model_build(children, N, p, qmax, D)
        assert [tuple(r) for r in ref] == [tuple(g) for g in got], (seed, case, D, M, k, N, p, qmax)
        assert steps <= N + 1
