"""CPU oracle of acceptance telemetry and the per-route choice of the draft length k.

TEST INFRASTRUCTURE ONLY (see the package header).  Plain Python / numpy.

Sources (cited by title and section):
  [P1] "Decodificação especulativa explicada: rascunhe barato, verifique numa passada"
       (gsantana.dev) -- "Quanto mais rápido: a matemática": with a per-token acceptance rate
       alpha a round yields (1 - alpha^(k+1)) / (1 - alpha) tokens on average and the speedup
       is that over (k c + 1); "A tabela de speedup": the best k per alpha and c;
       "Checagem de realidade em produção": record the acceptance rate per route (tokens per
       target pass is enough) and decide per kind of traffic.
  [P3] "Speculative decoding: el secretario que adelanta lo que va a decir el jefe"
       (blog.lo0.es) -- "La matemática que importa: techo y speedup" (same formulas);
       "Pitfalls operacionales": goodput-oriented work tunes the draft length dynamically.

Readings where the pages leave a step open:
  T1  counters per route, accumulated over calls: rounds, drafted tokens sum k_b, accepted
      sum A_b, emitted sum (A_b + 1), full rounds (A_b = k_b), rejections (A_b < k_b),
      invalid rows, and a histogram of A_b (64 bins).  Rows whose route id is outside
      [0, n_routes) are not counted; a row is invalid when accept_len < 0 or k_b is outside
      [0, K] or A_b > k_b.
  T2  alpha is estimated as accepted / (accepted + rejections): each round is A_b kept
      positions followed, unless A_b = k_b, by one rejected one, so with a constant per-token
      rate this is the maximum-likelihood estimate.  No observed position: undefined (NaN).
  T3  the chosen k maximises P1's speedup over k in [k_min, k_max] (ties: the smaller k); a
      route without observations gets k_default.
  T4  the plan is applied by clamping each sequence's draft count to its route's k
      (num_draft[b] = min(num_draft[b], k_table[route[b]]) for valid rows and routes).
"""
from __future__ import annotations

import math

import numpy as np

from .closed_forms import speedup

FIELDS = ("rounds", "drafted", "accepted", "emitted", "full", "rejections", "invalid", "reserved")
N_FIELDS = len(FIELDS)
N_BINS = 64
ROW = N_FIELDS + N_BINS


def telemetry_update(counters, accept_len, num_draft, route, K):
    """counters [n_routes, ROW] int64 -> updated copy (T1)."""
    c = np.array(counters, dtype=np.int64, copy=True)
    n_routes = c.shape[0]
    B = len(accept_len)
    for b in range(B):
        r = 0 if route is None else int(route[b])
        if not (0 <= r < n_routes):
            continue
        A = int(accept_len[b])
        k = K if num_draft is None else int(num_draft[b])
        if A < 0 or not (0 <= k <= K) or A > k:
            c[r, FIELDS.index("invalid")] += 1
            continue
        c[r, 0] += 1
        c[r, 1] += k
        c[r, 2] += A
        c[r, 3] += A + 1
        c[r, 4] += int(A == k)
        c[r, 5] += int(A < k)
        c[r, N_FIELDS + A] += 1
    return c


def alpha_estimate(row) -> float:
    """T2."""
    acc, rej = int(row[2]), int(row[5])
    return acc / (acc + rej) if acc + rej > 0 else math.nan


def choose_k(alpha: float, c: float, k_min: int, k_max: int) -> int:
    """T3: argmax of the page's speedup over k in [k_min, k_max], the smaller k on ties."""
    best_k, best = k_min, -math.inf
    for k in range(k_min, k_max + 1):
        s = speedup(alpha, k, c)
        if s > best:
            best_k, best = k, s
    return best_k


def plan_k(counters, c: float, k_min: int, k_max: int, k_default: int) -> np.ndarray:
    out = np.empty(len(counters), dtype=np.int32)
    for r, row in enumerate(counters):
        a = alpha_estimate(row)
        out[r] = k_default if math.isnan(a) else choose_k(a, c, k_min, k_max)
    return out


def apply_k(num_draft, route, k_table, K):
    """T4 (num_draft None means every sequence drafted K)."""
    B = len(route) if route is not None else len(num_draft)
    nd = np.full(B, K, dtype=np.int32) if num_draft is None else np.array(num_draft, np.int32)
    for b in range(B):
        r = 0 if route is None else int(route[b])
        if 0 <= r < len(k_table) and nd[b] >= 0:
            nd[b] = min(int(nd[b]), int(k_table[r]))
    return nd
