"""SVG2 mode of the oracle: semantic-aware permutation with centroid-based
top-p selection ("Sparse VideoGen2 ..." explainer, 2. Methodology, A and B).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py); shares no code with the
GPU library.  Plain numpy in float64; the steps follow the pages' order.

Readings (the pages give the steps, not these details):
  - k-means (Lloyd) on the Q rows and, independently, on the K rows of a
    head: C_q resp. C_k clusters, squared Euclidean distance, `iters`
    iterations of (assign every token to its nearest centroid, ties to the
    lower cluster index; move every centroid to the mean of its tokens, an
    empty cluster keeps its centroid).  Initial centroids: the caller's, or
    the tokens at indices floor(c * L / C) (the pages' centroid cache that
    seeds one step from the previous one is out of scope).  The returned
    labels are the last assignment, the centroids the means of it.
  - permutation: tokens in cluster order, stable (ascending token index
    inside a cluster); start[c] = first position of cluster c.
  - centroid scores: z_ab = scale * (mu_q[a] . mu_k[b]); the estimated share
    of query cluster a's attention on key cluster b counts its n_b tokens:
    P_ab = n_b exp(z_ab) / sum_b' n_b' exp(z_ab').
  - top-p: per query cluster, key clusters in descending P_ab (ties to the
    lower index), taken while the running sum before them is below p (so
    the cluster that reaches p is included); empty clusters are never taken.
  - attention: query token x of cluster a attends to key token y of cluster
    b exactly when b is selected for a; softmax over those keys.
"""
import numpy as np


def strided_init(x, C):
    L = x.shape[0]
    return np.asarray(x, dtype=np.float64)[(np.arange(C) * L) // C].copy()


def kmeans(x, C, iters, init=None):
    """Returns (labels int64 [L], centroids float64 [C, d], counts int64 [C])."""
    x = np.asarray(x, dtype=np.float64)
    mu = strided_init(x, C) if init is None else np.asarray(init, dtype=np.float64).copy()
    labels = None
    xx = (x * x).sum(axis=1)
    for _ in range(iters):
        labels = np.empty(x.shape[0], dtype=np.int64)
        mm = (mu * mu).sum(axis=1)
        for c0 in range(0, x.shape[0], 8192):  # squared distances |x|^2 - 2 x.mu + |mu|^2, in chunks of rows
            dist = xx[c0:c0 + 8192, None] - 2.0 * (x[c0:c0 + 8192] @ mu.T) + mm[None, :]
            labels[c0:c0 + 8192] = np.argmin(dist, axis=1)  # first minimum: ties to the lower index
        for c in range(C):
            members = x[labels == c]
            if members.shape[0]:
                mu[c] = members.mean(axis=0)
    counts = np.bincount(labels, minlength=C) if labels is not None else np.zeros(C, dtype=np.int64)
    return labels, mu, counts


def permutation(labels, C):
    """(perm [L]: token at each position of the cluster order, start [C+1])."""
    labels = np.asarray(labels)
    perm = np.argsort(labels, kind="stable")
    counts = np.bincount(labels, minlength=C)
    start = np.concatenate([[0], np.cumsum(counts)])
    return perm, start


def cluster_scores(mu_q, mu_k, counts_k, scale):
    """P [C_q, C_k]: size-weighted softmax of the centroid scores."""
    z = scale * (np.asarray(mu_q, dtype=np.float64) @ np.asarray(mu_k, dtype=np.float64).T)
    w = np.asarray(counts_k, dtype=np.float64)[None, :]
    z = np.where(w > 0, z, -np.inf)
    m = z.max(axis=1, keepdims=True)
    e = w * np.exp(z - m)
    return e / e.sum(axis=1, keepdims=True)


def top_p(P, counts_k, p):
    """sel [C_q, C_k] bool."""
    Cq, Ck = P.shape
    sel = np.zeros((Cq, Ck), dtype=bool)
    for a in range(Cq):
        order = sorted(range(Ck), key=lambda b: (-P[a, b], b))
        acc = 0.0
        for b in order:
            if acc >= p or counts_k[b] == 0:
                break
            sel[a, b] = True
            acc += P[a, b]
    return sel


def attention_rows(q, k, v, labels_q, labels_k, sel, scale, rows):
    """O [len(rows), d] float64 for the listed query tokens."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros((len(rows), q.shape[1]))
    for i, x in enumerate(rows):
        keys = np.flatnonzero(sel[labels_q[x]][labels_k])
        if keys.size == 0:
            continue
        s = scale * (k[keys] @ q[x])
        w = np.exp(s - s.max())
        out[i] = (w @ v[keys]) / w.sum()
    return out


def head(q, k, v, Cq, Ck, iters, p, scale, init_q=None, init_k=None):
    """The whole SVG2 step of one head (clustering, permutation, selection);
    returns a dict with every intermediate."""
    lq, mq, nq = kmeans(q, Cq, iters, init_q)
    lk, mk, nk = kmeans(k, Ck, iters, init_k)
    pq, sq = permutation(lq, Cq)
    pk, sk = permutation(lk, Ck)
    P = cluster_scores(mq, mk, nk, scale)
    sel = top_p(P, nk, p)
    return dict(labels_q=lq, mu_q=mq, n_q=nq, labels_k=lk, mu_k=mk, n_k=nk, perm_q=pq, start_q=sq, perm_k=pk,
                start_k=sk, P=P, sel=sel)
