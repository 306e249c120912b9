"""Paged decode attention, written out as its plain definition (float64).

Test infrastructure only (see the package docstring).

What the pages fix:
* [P1] §二 "具體運作方式" and [P2] "PagedAttention 的核心原理": a sequence's KV cache is
  logically contiguous but cut into fixed-size blocks placed anywhere; a per-sequence block
  table maps logical block j to a physical block.
* [P1] §三 步驟三: in decode, the new token's K/V is written first, then attention is computed
  over all of the sequence's KV found through the block table.

Paging changes only where K/V live, not what attention computes, so the oracle (1) gathers
each sequence's n = context_lens[i] tokens into contiguous float64 arrays by walking its block
table in logical order, then (2) runs dense scaled dot-product attention with a max-subtracted
softmax (the formula is the textbook one; the pages do not print any):

    s_t = scale * q . k_t,   out = sum_t exp(s_t - max s) v_t / sum_t exp(s_t - max s).

Grouped-query heads: q head h reads kv head h // (Hq // Hkv). A sequence with n = 0 gives a
zero row. The split-context pieces (``partition_partials`` / ``merge_partials``) restate the
same sums over token ranges and the standard log-sum-exp recombination.
"""

import numpy as np

from .layout import k_tile_tokens, to_f64, v_tile_tokens


def gather_sequence(k_cache, v_cache, table_row, n, *, num_blocks, hkv, hd, bs, dtype):
    """Logical K, V of one sequence as float64 arrays of shape [n, Hkv, hd].

    Token t is read from physical block table_row[t // bs] at offset t % bs ([P1] §二: the
    block table records which physical block holds each logical block).
    """
    K = np.empty((n, hkv, hd), dtype=np.float64)
    V = np.empty((n, hkv, hd), dtype=np.float64)
    for j in range((n + bs - 1) // bs):
        p = int(table_row[j])
        assert 0 <= p < num_blocks, f"table entry {j} = {p} outside the pool"
        cnt = min(bs, n - j * bs)
        K[j * bs:j * bs + cnt] = to_f64(k_tile_tokens(k_cache, p, hkv, hd, bs, dtype)[:cnt], dtype)
        V[j * bs:j * bs + cnt] = to_f64(v_tile_tokens(v_cache, p, hkv, hd, bs, dtype)[:cnt], dtype)
    return K, V


def _dense_attention_one(q_vec, K_g, V_g, scale):
    """Softmax attention of one query vector over n rows of K_g / V_g (float64)."""
    s = scale * (K_g @ q_vec)
    m = s.max()
    p = np.exp(s - m)
    return (p @ V_g) / p.sum()


def decode_attention(q, k_cache, v_cache, block_tables, context_lens, *, scale, hkv, hd, bs,
                     dtype, num_blocks=None):
    """out[i, h, :] for every sequence i and q head h, as float64 [B, Hq, hd]."""
    qf = to_f64(q, dtype)
    B, hq, _ = qf.shape
    assert hq % hkv == 0
    G = hq // hkv
    if num_blocks is None:
        num_blocks = np.asarray(k_cache).size // (hkv * hd * bs)
    out = np.zeros((B, hq, hd), dtype=np.float64)
    for i in range(B):
        n = int(context_lens[i])
        if n == 0:
            continue  # padding row: zeros
        K, V = gather_sequence(k_cache, v_cache, block_tables[i], n, num_blocks=num_blocks,
                               hkv=hkv, hd=hd, bs=bs, dtype=dtype)
        for h in range(hq):
            g = h // G
            out[i, h] = _dense_attention_one(qf[i, h], K[:, g, :], V[:, g, :], scale)
    return out


def decode_attention_rows(q, k_cache, v_cache, block_tables, context_lens, rows, *, scale, hkv,
                          hd, bs, dtype, num_blocks=None):
    """Same as ``decode_attention`` but only for the sequences listed in ``rows``.

    Returns float64 [len(rows), Hq, hd]. Used to check large batches one sampled sequence at a
    time.
    """
    rows = list(rows)
    sub = decode_attention(np.asarray(q)[rows], k_cache, v_cache,
                           np.asarray(block_tables)[rows], np.asarray(context_lens)[rows],
                           scale=scale, hkv=hkv, hd=hd, bs=bs, dtype=dtype,
                           num_blocks=num_blocks)
    return sub


def range_partials(q, k_cache, v_cache, block_tables, context_lens, *, seq, lo, hi, scale, hkv,
                   hd, bs, dtype, num_blocks=None):
    """Softmax pieces of one sequence over its token range [lo, min(hi, n)).

    For every q head h, over the range's tokens t (s_t = scale * q . k_t):
        m = max_t s_t,   l = sum_t exp(s_t - m),   o = sum_t exp(s_t - m) v_t.
    An empty range gives m = -inf, l = 0, o = 0. Returns (m [Hq], l [Hq], o [Hq, hd]) float64.
    """
    qf = to_f64(q, dtype)
    hq = qf.shape[1]
    G = hq // hkv
    if num_blocks is None:
        num_blocks = np.asarray(k_cache).size // (hkv * hd * bs)
    n = int(context_lens[seq])
    hi = min(int(hi), n)
    m = np.full(hq, -np.inf)
    l = np.zeros(hq)
    o = np.zeros((hq, hd))
    if hi <= lo:
        return m, l, o
    K, V = gather_sequence(k_cache, v_cache, block_tables[seq], n, num_blocks=num_blocks,
                           hkv=hkv, hd=hd, bs=bs, dtype=dtype)
    for h in range(hq):
        g = h // G
        s = scale * (K[lo:hi, g, :] @ qf[seq, h])
        m[h] = s.max()
        p = np.exp(s - m[h])
        l[h] = p.sum()
        o[h] = p @ V[lo:hi, g, :]
    return m, l, o


def partition_partials(q, k_cache, v_cache, block_tables, context_lens, *, scale, hkv, hd, bs,
                       dtype, part_tokens, num_blocks=None):
    """Per-partition softmax pieces for split-context decode.

    Sequence i is cut into ceil(n_i / P) consecutive token ranges of P = part_tokens tokens
    (the last one shorter); each range's (m, l, o) is ``range_partials`` of it.
    Returns a list over sequences of (m [np, Hq], l [np, Hq], o [np, Hq, hd]) float64 arrays.
    """
    res = []
    for i in range(len(context_lens)):
        n = int(context_lens[i])
        parts = [range_partials(q, k_cache, v_cache, block_tables, context_lens, seq=i,
                                lo=j * part_tokens, hi=(j + 1) * part_tokens, scale=scale,
                                hkv=hkv, hd=hd, bs=bs, dtype=dtype, num_blocks=num_blocks)
                 for j in range((n + part_tokens - 1) // part_tokens)]
        hq = np.asarray(q).shape[1]
        if parts:
            res.append(tuple(np.stack(x) for x in zip(*parts)))
        else:
            res.append((np.zeros((0, hq)), np.zeros((0, hq)), np.zeros((0, hq, hd))))
    return res


def merge_partials(m, l, o):
    """Log-sum-exp recombination of partition pieces of one (sequence, head).

    m, l: [np]; o: [np, hd]. With M = max_j m_j over pieces with m_j > -inf and
    w_j = exp(m_j - M):  out = sum_j w_j o_j / sum_j w_j l_j.  No pieces -> zeros.
    Real-arithmetic identity: exp(m_j - M) rescales each piece's sums to the common maximum,
    so the result equals the unsplit softmax average.
    """
    m = np.asarray(m, dtype=np.float64)
    l = np.asarray(l, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    keep = m > -np.inf
    if not keep.any():
        return np.zeros(o.shape[-1])
    M = m[keep].max()
    w = np.exp(m[keep] - M)
    return (w @ o[keep]) / (w @ l[keep])


def prefill_attention(q, k_cache, v_cache, block_tables, context_lens, query_start, *, scale,
                      hkv, hd, bs, dtype, num_blocks=None):
    """Causal attention of a batch's new prompt tokens over their paged K/V, float64
    [T, Hq, hd].

    [P1] §三 步驟二 (預填充): the input tokens' K/V are written into the sequence's blocks
    (a fresh block each time one fills) before attention. The pages do not write out the
    prefill attention itself; ours is the textbook causal form, found through the same block
    table as decode: sequence i holds context_lens[i] = n_i tokens in the cache, its new
    tokens are the last t_i = query_start[i+1] - query_start[i] of them (positions n_i - t_i
    .. n_i - 1; the earlier ones may have been cached before, e.g. a shared prefix or an
    earlier chunk of the prompt), and q row query_start[i] + k, the token at position
    p = n_i - t_i + k, attends over tokens 0..p of its sequence.
    """
    qf = to_f64(q, dtype)
    T, hq, _ = qf.shape
    assert hq % hkv == 0
    G = hq // hkv
    qs = [int(x) for x in query_start]
    assert qs[0] == 0 and qs[-1] == T and all(a <= b for a, b in zip(qs, qs[1:]))
    if num_blocks is None:
        num_blocks = np.asarray(k_cache).size // (hkv * hd * bs)
    out = np.zeros((T, hq, hd), dtype=np.float64)
    for i in range(len(qs) - 1):
        n, t = int(context_lens[i]), qs[i + 1] - qs[i]
        if t == 0:
            continue
        assert 0 < t <= n
        K, V = gather_sequence(k_cache, v_cache, block_tables[i], n, num_blocks=num_blocks,
                               hkv=hkv, hd=hd, bs=bs, dtype=dtype)
        for k in range(t):
            p = n - t + k
            for h in range(hq):
                g = h // G
                out[qs[i] + k, h] = _dense_attention_one(qf[qs[i] + k, h], K[:p + 1, g, :],
                                                         V[:p + 1, g, :], scale)
    return out
