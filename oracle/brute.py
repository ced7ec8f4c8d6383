"""Brute-force forms used to pin the oracle (test infrastructure).

Nothing here sorts. Selection enumerates every K-subset of the pool and keeps
the one whose members all beat all non-members; the permutation is an explicit
counting pass over the slots in token order. Both follow the plain statements
of [Review] section 3 ("threshold interpretation", "implementation") and are
only meant for tiny inputs.
"""
from itertools import combinations


def beats(a, b):
    """Strict total order on pool entries (value, is_null, id): larger value
    wins; at equal value the null copy wins over a real expert (a real must
    strictly exceed the null logit); then lower id wins."""
    va, na, ia = a
    vb, nb, ib = b
    if va != vb:
        return va > vb
    if na != nb:
        return na
    return ia < ib


def select_token(real_logits, null_logit, M, K):
    """Returns (chosen real ids in dominance order, number of null copies chosen)."""
    N = len(real_logits)
    pool = [(float(real_logits[j]), False, j) for j in range(N)]
    pool += [(float(null_logit), True, N + c) for c in range(M)]
    winners = []
    for S in combinations(range(len(pool)), K):
        inside = set(S)
        if all(beats(pool[i], pool[o]) for i in S for o in range(len(pool)) if o not in inside):
            winners.append(S)
    assert len(winners) == 1, "the order is total, so exactly one K-subset dominates"
    S = winners[0]
    reals = [pool[i] for i in S if not pool[i][1]]
    # position of a chosen real = number of chosen reals that beat it
    ranked = sorted(reals, key=lambda e: sum(beats(o, e) for o in reals))
    return [e[2] for e in ranked], sum(1 for i in S if pool[i][1])


def counting_permute(topk_idx, N):
    """Slots in token-major order are appended to their expert's bucket; the
    buckets are concatenated in expert order; null slots are never appended."""
    T = len(topk_idx)
    K = len(topk_idx[0]) if T else 0
    buckets = [[] for _ in range(N)]
    for t in range(T):
        for k in range(K):
            e = int(topk_idx[t][k])
            if 0 <= e < N:
                buckets[e].append((t, k))
    counts = [len(b) for b in buckets]
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    perm_token, slot_pos = [], [[-1] * K for _ in range(T)]
    for e in range(N):
        for (t, k) in buckets[e]:
            slot_pos[t][k] = len(perm_token)
            perm_token.append(t)
    return counts, offsets, perm_token, slot_pos
