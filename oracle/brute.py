"""Independent brute-force definitions of the integer part of dispatch
(test infrastructure only; pure Python, no shared code with oracle.c or the
HIP library).

Where oracle.c builds positions with running counters, this module defines
them by sorting: a sender's rows are its (expert, t, k) triples in sorted
order, so a bug in either formulation shows as a disagreement.  The receive
and expert layouts are defined the same way, from sorted lists of row keys:

  send rows of sender s      : sorted (e, t, k)                over s's pairs
  receive rows (pooled)      : sorted (d, s, e, t, k)           d = e // L
  expert rows (pooled)       : sorted (e, s, t, k)

Pages: [EFA] "Send and receive buffers", "Dispatch and combine" (counts,
cumulative sums, contiguous per-peer buffers); [EPMC] "Dispatch" (grouped-GEMM
input and the stored source rank / expert / token index).
"""
from __future__ import annotations


def brute_plan(idx, E):
    """idx: nested lists / array [N][T][K] of ints in [0,E).  Returns dict of
    python lists: cnt, pos, send_rows, recv_rows, expert_rows, G, eoff."""
    N = len(idx)
    T = len(idx[0]) if N else 0
    K = len(idx[0][0]) if T else 0
    L = E // N
    cnt = [[0] * E for _ in range(N)]
    for s in range(N):
        for t in range(T):
            for k in range(K):
                cnt[s][int(idx[s][t][k])] += 1
    pos = [[[None] * K for _ in range(T)] for _ in range(N)]
    send_rows = []        # global send row -> (s, t, k)
    for s in range(N):
        keys = sorted((int(idx[s][t][k]), t, k) for t in range(T) for k in range(K))
        for p, (e, t, k) in enumerate(keys):
            pos[s][t][k] = p
            send_rows.append((s, t, k))
    recv_keys = sorted((int(idx[s][t][k]) // L, s, int(idx[s][t][k]), t, k)
                       for s in range(N) for t in range(T) for k in range(K))
    recv_rows = [(s, t, k) for (_, s, _, t, k) in recv_keys]
    G = [0] * (N + 1)
    for d in range(N):
        G[d + 1] = G[d] + sum(1 for key in recv_keys if key[0] == d)
    expert_keys = sorted((int(idx[s][t][k]), s, t, k)
                         for s in range(N) for t in range(T) for k in range(K))
    expert_rows = [(s, t, k) for (_, s, t, k) in expert_keys]
    eoff = [0] * (E + 1)
    for e in range(E):
        eoff[e + 1] = eoff[e] + sum(cnt[s][e] for s in range(N))
    return {"cnt": cnt, "pos": pos, "send_rows": send_rows, "recv_rows": recv_rows,
            "expert_rows": expert_rows, "G": G, "eoff": eoff}
