"""Spark-Reblock reordering (oracle, float64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "深度解读|Spark-H3：从注意力几何到稀疏内核代码" -- section 04 (a
permutation of Q with the same permutation bound to K and V, followed by the
inverse permutation of the output, leaves dense attention unchanged), section
05 (the cross second-moment metric: with M_K = K^T K / N the inner product of
two queries' score profiles is N q_i^T M_K q_j, so their cosine can be taken
between q_i^T L and q_j^T L for any factor L L^T = M_K; keys are grouped with
the query-side moment M_Q = Q^T Q / N), section 06 (an equal-capacity
hierarchical split into 64-token leaves, split directions estimated from
midpoint landmarks) and its note that the default layout mode builds only the
key layout and lets the queries reuse it.

The production tree (fanout 16, 32 midpoint landmarks, a power-of-two fanout
schedule) is described but not specified; the reading implemented here is
the page's own equal-capacity binary grouping with landmark-estimated
principal directions:

* features: u_j = z_j / |z_j| with z_j = k_j^T L, L the lower Cholesky factor
  of M_Q + lam * I, lam = ridge * tr(M_Q) / D (ridge * 1 when the trace is 0;
  the page mentions a ridge in the source without its value, 1e-4 here keeps
  the factor well defined in fp32); a zero key has no score direction and
  gets the zero feature; the features are exact (float64): the section
  defines them as the normalised rows z_j / |z_j| and nothing rounds them;
* tree: a node holding n tokens spans c = ceil(n / M) leaves; its first child
  takes floor(c / 2) leaves (floor(c / 2) * M tokens), the second the rest; a
  node with c <= 1 is a leaf.  The ranges depend on N and M only;
* split of a node (its tokens in their current order): landmarks are the
  tokens at ranks floor((2s + 1) n / 64), s = 0..31; X = their features minus
  the landmark mean; a = 16 power iterations of G = X X^T from the ramp
  a_s = s - 15.5 (normalised each time; the all-ones vector would be useless,
  centring puts it in G's null space); direction v = X^T a / |X^T a|, signed so
  that its largest-magnitude entry (lowest index on ties) is positive; the
  node's tokens are stably sorted by u . v, the first floor(c / 2) * M go to
  the first child, the rest to the second;
* the root order is the token order; leaves in left-to-right order are the
  blocks (all full but the last).
"""

import numpy as np

N_LANDMARKS = 32
POWER_ITERS = 16
DEFAULT_RIDGE = 1e-4


def second_moment(X):
    """Uncentred second moment X^T X / N per (batch, head): [B, h, D, D]."""
    X = np.asarray(X, dtype=np.float64)
    B, N, h, D = X.shape
    Xt = np.transpose(X, (0, 2, 1, 3))  # [B, h, N, D]
    return np.matmul(np.swapaxes(Xt, -1, -2), Xt) / N


def metric_factor(M, ridge=DEFAULT_RIDGE):
    """Lower Cholesky factor of M + lam * I, lam = ridge * tr(M) / D (ridge when
    the trace is 0), over the last two axes."""
    M = np.asarray(M, dtype=np.float64)
    D = M.shape[-1]
    tr = np.trace(M, axis1=-2, axis2=-1)[..., None, None]
    lam = ridge * np.where(tr > 0, tr / D, 1.0)
    return np.linalg.cholesky(M + lam * np.eye(D))


def key_features(K, Q, ridge=DEFAULT_RIDGE):
    """Unit features of the keys under the query-side metric: [B, h, N, D]."""
    L = metric_factor(second_moment(Q), ridge)
    Kt = np.transpose(np.asarray(K, dtype=np.float64), (0, 2, 1, 3))
    z = np.matmul(Kt, L)
    nrm = np.linalg.norm(z, axis=-1, keepdims=True)
    return np.where(nrm > 0, z / np.where(nrm > 0, nrm, 1.0), 0.0)


def tree_slots(N, M):
    """Static node ranges: a list over levels of lists of (start, end, leaves)
    for the 2^level slots (empty slots have start == end).  Level 0 is the
    root; the last level holds only leaves."""
    c_root = -(-N // M)
    levels = [[(0, N, c_root)]]
    while any(c > 1 for (_, _, c) in levels[-1]):
        nxt = []
        for (s, e, c) in levels[-1]:
            if c <= 1:
                nxt += [(s, s, 0), (s, e, c)]
            else:
                cl = c // 2
                nxt += [(s, s + cl * M, cl), (s + cl * M, e, c - cl)]
        levels.append(nxt)
    return levels


def split_direction(U):
    """Direction of a node from its features in the node's current order."""
    n = U.shape[0]
    ranks = [(2 * s + 1) * n // (2 * N_LANDMARKS) for s in range(N_LANDMARKS)]
    X = U[ranks]
    X = X - X.mean(axis=0)
    G = X @ X.T
    a = np.arange(N_LANDMARKS) - (N_LANDMARKS - 1) / 2.0
    a = a / np.linalg.norm(a)
    for _ in range(POWER_ITERS):
        a = G @ a
        nrm = np.linalg.norm(a)
        if nrm == 0.0:
            break
        a = a / nrm
    v = X.T @ a
    nrm = np.linalg.norm(v)
    if nrm > 0.0:
        v = v / nrm
    if v[int(np.argmax(np.abs(v)))] < 0:
        v = -v
    return v


def reblock_orders(U, M):
    """Token order after every level for features U [N, D] of one head.
    Returns a list of int64 [N] arrays: level 0 = token order, then one per
    split level."""
    N = U.shape[0]
    slots = tree_slots(N, M)
    order = np.arange(N)
    orders = [order.copy()]
    for lvl in slots[:-1]:
        new = order.copy()
        for (s, e, c) in lvl:
            if c <= 1:
                continue
            members = order[s:e]
            v = split_direction(U[members])
            p = U[members] @ v
            new[s:e] = members[np.argsort(p, kind="stable")]
        order = new
        orders.append(order.copy())
    return orders


def reblock_tables(order, M):
    """perm [J*M] (tokens of leaf j at j*M.., -1 padding) and block_len [J]."""
    N = len(order)
    J = -(-N // M)
    perm = np.full(J * M, -1, dtype=np.int64)
    perm[:N] = order
    block_len = np.full(J, M, dtype=np.int64)
    block_len[-1] = N - (J - 1) * M
    return perm, block_len


def check_orders(U, orders, M, eps):
    """Check a device's per-level orders against the split rule, node by node,
    on the device's own node contents: at every split the node's tokens must
    appear sorted by the float64 projection up to eps (a pair out of order by
    more than eps is a violation), and the children are the cut of that order.
    A node whose order is the reverse one (the direction's sign taken the other
    way at a near-tie of the largest entry) counts as a flip.
    Returns (splits, violations, flips, worst): worst is the largest amount by
    which a consecutive pair of an accepted split is out of order."""
    N = U.shape[0]
    slots = tree_slots(N, M)
    if len(orders) != len(slots):
        raise ValueError("expected %d levels" % len(slots))
    if not np.array_equal(orders[0], np.arange(N)):
        raise ValueError("level 0 must be the token order")
    splits = violations = flips = 0
    worst = 0.0
    for li, lvl in enumerate(slots[:-1]):
        cur, nxt = orders[li], orders[li + 1]
        for (s, e, c) in lvl:
            if c <= 1:
                violations += int(not np.array_equal(cur[s:e], nxt[s:e]))
                continue
            splits += 1
            members = cur[s:e]
            if not np.array_equal(np.sort(members), np.sort(nxt[s:e])):
                violations += 1
                continue
            v = split_direction(U[members])
            p = U[nxt[s:e]] @ v
            dp = np.diff(p)
            if np.all(dp >= -eps):
                worst = max(worst, float(-dp.min()) if len(dp) else 0.0)
                continue
            if np.all(dp <= eps):
                flips += 1
                worst = max(worst, float(dp.max()) if len(dp) else 0.0)
                continue
            violations += 1
    return splits, violations, flips, worst


def check_splits(U, orders, dirs, M, eps, tau):
    """Validity of a device's tree given its own split directions.

    The top principal direction of 32 nearly isotropic landmarks is ill
    conditioned (close leading eigenvalues), so fp32 and float64 runs of the
    same 16 power iterations may end on different, equally principal axes.
    What is unique is the quality of the axis; the rest must be valid.  At every
    split, with the node's tokens in the device's current order and the
    oracle's features U: the device's direction v (dirs[level][slot]) must
    (a) have unit length and lie in the span of the centred landmarks (relative
    residual <= 1e-3), (b) have its largest-magnitude entry positive, (c) be as
    principal as the oracle's own direction v_o: |X v|^2 >= (1 - tau) |X v_o|^2,
    and (d) order the node's tokens: the device's next order sorted by U . v up
    to eps.  Unsplit nodes must keep their order.
    Returns (splits, violations, worst inversion, worst quotient shortfall)."""
    N = U.shape[0]
    slots = tree_slots(N, M)
    if len(orders) != len(slots) or not np.array_equal(orders[0], np.arange(N)):
        raise ValueError("expected %d levels starting from the token order" % len(slots))
    splits = violations = 0
    worst_inv = worst_short = 0.0
    for li, lvl in enumerate(slots[:-1]):
        cur, nxt = orders[li], orders[li + 1]
        for si, (s, e, c) in enumerate(lvl):
            if c <= 1:
                violations += int(not np.array_equal(cur[s:e], nxt[s:e]))
                continue
            splits += 1
            members = cur[s:e]
            if not np.array_equal(np.sort(members), np.sort(nxt[s:e])):
                violations += 1
                continue
            n = e - s
            ranks = [(2 * t + 1) * n // (2 * N_LANDMARKS) for t in range(N_LANDMARKS)]
            X = U[members[ranks]]
            X = X - X.mean(axis=0)
            v = np.asarray(dirs[li][si], dtype=np.float64)
            coef, *_ = np.linalg.lstsq(X.T, v, rcond=None)
            resid = np.linalg.norm(X.T @ coef - v)
            vo = split_direction(U[members])
            qo = float(np.sum((X @ vo) ** 2))
            qg = float(np.sum((X @ v) ** 2))
            short = (qo - qg) / qo if qo > 0 else 0.0
            worst_short = max(worst_short, short)
            ok = abs(np.linalg.norm(v) - 1.0) <= 1e-5 and resid <= 1e-3 and v[int(np.argmax(np.abs(v)))] > 0
            ok = ok and short <= tau
            dp = np.diff(U[nxt[s:e]] @ v)
            inv = float(-dp.min()) if len(dp) else 0.0
            worst_inv = max(worst_inv, inv)
            ok = ok and inv <= eps
            violations += int(not ok)
    return splits, violations, worst_inv, worst_short
