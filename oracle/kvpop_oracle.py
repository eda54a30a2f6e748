"""CPU oracle for KVpop's per-KV-head fixed-budget sparse KV cache.

TEST INFRASTRUCTURE ONLY.  This is the plain, slow, obviously-correct
reference that the GPU path is checked against.  Only the test suite, the
package's smoke check and the benchmark's CPU-baseline leg may import it; the
product path never does.  It shares no code with the GPU path: it imports
NumPy and nothing else.

What it computes, and where that is stated:

* The cache of each KV head is bounded: some initial sink tokens, a protected
  window of the most recent tokens, and a scored top-k of older tokens
  ("Qwen3-8B-KVpop-4x" model card, intro: "a bounded sink + scored top-k +
  recent-window cache", 4 sink + 3,772 scored + 256 recent = 4,032 entries;
  aiweekly French article, second paragraph: each head keeps initial sink
  tokens, a protected recent window, and a learned top-k over older tokens).
* Delayed scoring: a token gets its long-range score only when it leaves the
  protected recent window (model card, "Paper highlights / Delayed scoring";
  KVpop abstract on the HF papers page: the scorer defers scoring by a fixed
  number of steps).  The score itself comes from a learned scorer; here it is
  an input.
* The eviction policy makes an online keep-or-drop decision under a fixed
  budget (KVpop abstract: "fixed-budget KV eviction policy", "keep-or-drop
  decision"); an evicted token is gone for good.
* Decode attention is ordinary softmax attention of each query head over the
  rows its KV head keeps (grouped-query attention).

Readings taken where the pages say nothing (each also listed in the design
notes of the repository):

1. The window holds the W newest positions including the token being
   decoded, so token t leaves the window when token t + W arrives.
2. Sinks are positions 0 .. s-1; they are never scored and never in the window.
3. Order of importance is the key (score, position), compared
   lexicographically: on an equal score the newer token counts as more
   important, so the lower score, then the older token, is evicted first.
4. While fewer than k tokens hold scored slots, a leaving token is admitted
   without a comparison.
5. Softmax scale defaults to 1/sqrt(D).
6. Query head h reads KV head floor(h * Hkv / Hq) (contiguous groups).
7. A NaN score is a caller error (the oracle raises).
8. At prefill the scores of positions [s, P - W) are used; the scores of
   window positions arrive later, one per decode step.
9. The prefix top-k thresholds the model card's cache-backends section names
   are read as: for every position n of a prompt, the key of the k-th most
   important member of Cand(n) (0 while there are fewer than k, KEY_NONE
   when k = 0), so that the kept set at n is the sinks, the window and the
   candidates whose key reaches it.
10. The future-attention target (the scorer's training target) sums, for
    each key, the causal softmax weight that every query of the KV head's
    group puts on it after the key has left the window; the pages do not say
    how query heads combine or whether it is normalised (summed here, not
    normalised).
11. The Dynamic backend the model card lists beside the Static one ("Cache
    backends": it grows, then prunes, under the same budget) is read as:
    every token leaving the window is held (the scored region grows without
    a comparison), and a prune cuts each head's scored region back to its
    top-k by key.  When it prunes is not on the pages; the prune is an
    explicit step here, and a cache that prunes after every step is the
    Static one.

All arithmetic is float64 on exactly decoded bfloat16 values.
"""
from __future__ import annotations

import math

import numpy as np


def bf16_to_f64(bits) -> np.ndarray:
    """Exact float64 value of bfloat16 bit patterns.

    A bfloat16 is the upper half of an IEEE binary32, so widening the pattern
    to 32 bits with sixteen zero bits below gives the same number.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def kv_head_of(h: int, n_q_heads: int, n_kv_heads: int) -> int:
    """KV head read by query head h (reading 6: contiguous query groups)."""
    return (h * n_kv_heads) // n_q_heads


def _check_score(x: float) -> float:
    x = float(x)
    if math.isnan(x):
        raise ValueError("NaN score: scores must be ordered numbers")
    return x


# ---------------------------------------------------------------------------
# The kept set by its definition (used to pin the streaming oracle)
# ---------------------------------------------------------------------------

def kept_by_definition(scores_g, n: int, n_sink: int, n_scored: int, n_recent: int):
    """Kept set of one KV head after position n, written from its definition.

    Kept(n) = Sink(n) | Win(n) | TopK(Cand(n)) where
      Sink(n) = {0 .. min(s, n+1) - 1}
      Win(n)  = {max(s, n - W + 1) .. n}      (reading 1)
      Cand(n) = {s .. n - W}                   (tokens that left the window)
      TopK    = the k members of Cand(n) with the largest (score, position).
    Scores only matter for positions in Cand(n).  Returns a sorted list.
    """
    s, k, W = n_sink, n_scored, n_recent
    if n < 0:
        return []
    sink = set(range(0, min(s, n + 1)))
    win = set(range(max(s, n - W + 1), n + 1))
    cand = range(s, n - W + 1)
    ranked = sorted(cand, key=lambda t: (_check_score(scores_g[t]), t), reverse=True)
    return sorted(sink | win | set(ranked[:k]))


def held_dynamic_by_definition(scores_g, n: int, n_pruned: int, n_sink: int, n_scored: int,
                               n_recent: int):
    """Rows a Dynamic-backend head holds after position n, when its scored
    region was last cut back at position n_pruned (-1: never; a prefill of P
    tokens counts as a cut at P - 1), written from the definition (reading
    11): the sinks and the window of n, the top-k of Cand(n_pruned), and
    every token that has left the window since, i.e. Cand(n) minus
    Cand(n_pruned).  Returns a sorted list.
    """
    s, k, W = n_sink, n_scored, n_recent
    if n < 0:
        return []
    sink = set(range(0, min(s, n + 1)))
    win = set(range(max(s, n - W + 1), n + 1))
    cand_pruned = range(s, n_pruned - W + 1)
    ranked = sorted(cand_pruned, key=lambda t: (_check_score(scores_g[t]), t), reverse=True)
    old = set(ranked[:k])                       # TopK(Cand(n_pruned))
    new = set(range(max(s, n_pruned - W + 1), n - W + 1))
    return sorted(sink | win | old | new)


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------

def softmax_attention(q, K, V, scale: float) -> np.ndarray:
    """out = sum_j softmax_j(scale * <q, K_j>) V_j, float64, rows in any order."""
    logits = scale * (K @ q)
    logits = logits - logits.max()
    w = np.exp(logits)
    w = w / w.sum()
    return w @ V


def masked_dense_attention(q, K_all, V_all, kept, scale: float) -> np.ndarray:
    """Attention of q over all positions 0..n, with -inf outside ``kept``.

    A second, independent route to the same number: the full logit row is
    formed and every position outside the kept set is masked out.
    """
    n1 = K_all.shape[0]
    mask = np.zeros(n1, dtype=bool)
    mask[np.asarray(list(kept), dtype=np.int64)] = True
    logits = np.full(n1, -np.inf)
    logits[mask] = scale * (K_all[mask] @ q)
    m = logits[mask].max()
    w = np.where(mask, np.exp(logits - m), 0.0)
    return (w / w.sum()) @ V_all


# ---------------------------------------------------------------------------
# Prefix top-k thresholds (every position of a prompt)
# ---------------------------------------------------------------------------

KEY_NONE = (1 << 64) - 1


def score_key(score, pos: int) -> int:
    """64-bit key of a scored token: order code of the float32 score in the
    high half, position in the low half.

    The code flips every bit of a negative float and sets the sign bit of a
    non-negative one, so unsigned order of codes is float order; -0 is taken
    as +0 first.  Comparing keys as integers is comparing (score, position)
    lexicographically (reading 3).
    """
    u = int(np.array([score], dtype=np.float32).view(np.uint32)[0])
    if u == 0x80000000:
        u = 0
    code = (~u & 0xFFFFFFFF) if (u & 0x80000000) else (u | 0x80000000)
    return (code << 32) | int(pos)


def prefix_thresholds(scores_g, n_tokens: int, n_sink: int, n_scored: int, n_recent: int):
    """Threshold key of every position n of a prompt, for one KV head.

    thr(n) is the key of the k-th most important member of Cand(n) =
    {s .. n - W}, so that Kept(n) = Sink(n) | Win(n) | {t in Cand(n) :
    key(t) >= thr(n)}; it is 0 (every candidate kept) while Cand(n) has fewer
    than k members, and KEY_NONE (no candidate kept) when k = 0.  The model
    card names a prefix top-k thresholds kernel among its cache backends; its
    exact contract is not on the pages, and this is the reading taken.

    Computed the plain way: Cand grows by one position per step, and the k-th
    largest key of a growing set is the root of a min-heap holding the k
    largest so far.  Returns a list of n_tokens Python ints.
    """
    import heapq
    s, k, W = n_sink, n_scored, n_recent
    out = []
    heap = []
    nxt = s                                    # next position to enter Cand
    for n in range(n_tokens):
        while nxt <= n - W:                     # positions that left the window
            key = score_key(_check_score(scores_g[nxt]), nxt)
            if len(heap) < k:
                heapq.heappush(heap, key)
            elif k > 0 and key > heap[0]:
                heapq.heapreplace(heap, key)
            nxt += 1
        if k == 0:
            out.append(KEY_NONE)
        elif len(heap) < k:
            out.append(0)
        else:
            out.append(heap[0])
    return out


# ---------------------------------------------------------------------------
# Future-attention target (the scorer's training target)
# ---------------------------------------------------------------------------

def future_attention_target(q_bits, k_bits, n_recent: int, scale: float) -> np.ndarray:
    """Attention mass each key receives from queries that come after it has
    left the recent window, per KV head.

    y[g][j] = sum over query heads h of group g, and over queries i >= j + W,
    of softmax_j'(scale * <q_h,i, k_g,j'>) over the causal keys j' <= i,
    taken at j' = j.  The English aiweekly article (its paragraph on how
    KVpop defines the right answer) and the French one (second paragraph)
    define the scorer's target as the attention mass a token will receive
    from queries that come after it has left the protected recent window,
    computed in training by a transposed-attention pass (KVpop abstract: no
    dense attention map is materialised).  How the query heads of a group
    combine and whether the sum is normalised is not on the pages (reading:
    summed over the group's query heads and over those queries, not
    normalised).

    q_bits [Hq][T][D], k_bits [Hkv][T][D] bfloat16 bit patterns; returns
    float64 [Hkv][T].
    """
    Q = bf16_to_f64(q_bits)
    K = bf16_to_f64(k_bits)
    Hq, T, _ = Q.shape
    Hkv = K.shape[0]
    W = n_recent
    y = np.zeros((Hkv, T))
    i_idx = np.arange(T)[:, None]
    j_idx = np.arange(T)[None, :]
    causal = j_idx <= i_idx
    future = i_idx >= j_idx + W
    for h in range(Hq):
        g = kv_head_of(h, Hq, Hkv)
        logits = scale * (Q[h] @ K[g].T)                  # [i][j]
        logits = np.where(causal, logits, -np.inf)
        logits = logits - logits.max(axis=1, keepdims=True)
        p = np.exp(logits)
        p = p / p.sum(axis=1, keepdims=True)
        y[g] += np.where(future, p, 0.0).sum(axis=0)
    return y


# ---------------------------------------------------------------------------
# Streaming oracle: one (layer, sequence) with all its KV heads
# ---------------------------------------------------------------------------

class KVpopOracle:
    """The cache of one (layer, sequence), followed step by step.

    prefill(k, v, scores)          fill from a P-token prompt
    decode(q, k_new, v_new, sl)    process one new token; returns the
                                   attention output of every query head
    prune()                        Dynamic backend: cut every head's scored
                                   region back to its top-k (reading 11)
    kept(g)                        sorted kept positions of KV head g

    dynamic=False is the Static backend (fixed buffers, online replacement);
    dynamic=True holds every leaving token until the next prune().
    """

    def __init__(self, n_q_heads: int, n_kv_heads: int, head_dim: int,
                 n_sink: int, n_scored: int, n_recent: int,
                 softmax_scale: float | None = None, dynamic: bool = False):
        if n_q_heads % n_kv_heads:
            raise ValueError("n_q_heads must be a multiple of n_kv_heads")
        if n_recent < 1 or n_sink < 0 or n_scored < 0:
            raise ValueError("bad cache geometry")
        self.Hq, self.Hkv, self.D = n_q_heads, n_kv_heads, head_dim
        self.s, self.k, self.W = n_sink, n_scored, n_recent
        self.scale = (1.0 / math.sqrt(head_dim)) if not softmax_scale or softmax_scale <= 0 \
            else float(softmax_scale)
        self.dynamic = bool(dynamic)
        self.n = -1                       # newest processed position
        self._cap = 0
        self._K = np.zeros((self.Hkv, 0, self.D))
        self._V = np.zeros((self.Hkv, 0, self.D))
        # Scored region per KV head: position -> score (reading 3 orders them).
        self.S = [dict() for _ in range(self.Hkv)]

    # -- storage of every row ever seen (the oracle never forgets a row) -----
    def _reserve(self, n_rows: int):
        if n_rows <= self._cap:
            return
        cap = max(n_rows, 2 * self._cap, 64)
        K = np.zeros((self.Hkv, cap, self.D))
        V = np.zeros((self.Hkv, cap, self.D))
        K[:, :self._cap] = self._K[:, :self._cap]
        V[:, :self._cap] = self._V[:, :self._cap]
        self._K, self._V, self._cap = K, V, cap

    # -- prefill -------------------------------------------------------------
    def prefill(self, k_bits, v_bits, scores):
        """Fill an empty cache from a P-token prompt.

        k_bits, v_bits: uint16 [Hkv][P][D]; scores: float32 [Hkv][P] (only
        positions s .. P-W-1 are read, reading 8).  After the call n = P-1 and
        each head's scored region is the top-k of Cand(P-1).
        """
        if self.n != -1:
            raise RuntimeError("prefill needs an empty cache")
        P = int(np.asarray(k_bits).shape[1])
        if P == 0:
            return
        self._reserve(P)
        self._K[:, :P] = bf16_to_f64(k_bits)
        self._V[:, :P] = bf16_to_f64(v_bits)
        self.n = P - 1
        cand = range(self.s, P - self.W)
        for g in range(self.Hkv):
            ranked = sorted(cand, key=lambda t: (_check_score(scores[g][t]), t), reverse=True)
            self.S[g] = {t: float(scores[g][t]) for t in ranked[:self.k]}

    # -- one decode step -----------------------------------------------------
    def _admit_leaving(self, g: int, t: int, score: float):
        """Token t has just left the window with ``score`` (delayed scoring)."""
        S = self.S[g]
        if self.dynamic:                          # reading 11: grow until the prune
            S[t] = score
            return
        if len(S) < self.k:                       # reading 4
            S[t] = score
            return
        if self.k == 0:
            return
        m = min(S, key=lambda p: (S[p], p))       # least important member
        if (score, t) > (S[m], m):                # keep-or-drop decision
            del S[m]                              # evicted for good
            S[t] = score
        # else: t is dropped for good

    def prune(self):
        """Dynamic backend: keep only the k most important members of every
        head's scored region (by (score, position), reading 3); the rest are
        evicted for good."""
        for g in range(self.Hkv):
            S = self.S[g]
            ranked = sorted(S, key=lambda p: (S[p], p), reverse=True)
            self.S[g] = {p: S[p] for p in ranked[:self.k]}

    def decode(self, q_bits, k_new_bits, v_new_bits, score_leaving, attend: bool = True):
        """Process token n = self.n + 1 and return out [Hq][D] (float64).

        q_bits: uint16 [Hq][D]; k_new_bits, v_new_bits: uint16 [Hkv][D];
        score_leaving: float [Hkv], the score of token n - W for each KV head
        (ignored when n - W < s).  With attend=False only the cache is
        updated and None is returned.
        """
        n = self.n + 1
        self._reserve(n + 1)
        self._K[:, n] = bf16_to_f64(k_new_bits)
        self._V[:, n] = bf16_to_f64(v_new_bits)
        t = n - self.W
        if t >= self.s:
            for g in range(self.Hkv):
                self._admit_leaving(g, t, _check_score(score_leaving[g]))
        self.n = n
        if not attend:
            return None
        return self.attend(q_bits)

    def attend(self, q_bits):
        """Attention output [Hq][D] (float64) of q over the current kept rows."""
        q = bf16_to_f64(q_bits)
        out = np.zeros((self.Hq, self.D))
        for g in range(self.Hkv):
            rows = np.asarray(self.kept(g), dtype=np.int64)
            Kg, Vg = self._K[g, rows], self._V[g, rows]
            for h in range(self.Hq):
                if kv_head_of(h, self.Hq, self.Hkv) == g:
                    out[h] = softmax_attention(q[h], Kg, Vg, self.scale)
        return out

    # -- state ---------------------------------------------------------------
    def kept(self, g: int):
        """Sorted kept positions of KV head g after position self.n."""
        n = self.n
        if n < 0:
            return []
        sink = set(range(0, min(self.s, n + 1)))
        win = set(range(max(self.s, n - self.W + 1), n + 1))
        return sorted(sink | win | set(self.S[g]))

    def rows(self, g: int):
        """All rows stored so far for KV head g (float64 K and V, [n+1][D])."""
        return self._K[g, :self.n + 1], self._V[g, :self.n + 1]
