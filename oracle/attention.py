"""CPU float64 oracle of unified paged, variable-length attention.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code,
table or constant with the GPU library, and the GPU library never calls it.

What it computes is the plain definition, assembled from the pages:

* Inputs (RocKE ``unified_attention`` README, opening list of the parity
  script): a paged K/V cache addressed through per-sequence block tables,
  queries batched by cumulative lengths, optional sliding window, softcap,
  sinks and ALiBi slopes.
* Cache layout: dimension 0 of each cache counts blocks and the block stride
  is block_size * num_kv_heads * head_size elements (README, section "Paged-cache
  size: 64-bit KV addressing"), so each cache is [num_blocks, block_size,
  num_kv_heads, head_size]; key j of sequence s lives in block
  ``block_table[s][j // block_size]`` at slot ``j % block_size``.
* Causal alignment: the q_len queries of a sequence are its last q_len
  positions, so query i sits at position ctx + i with ctx = kv_len - q_len
  (README, section "2D vs 2D", where biases are taken relative to
  ``context_len``; FA-RDNA2 PR #34, section "Change", chunks behind prefixes).
* Sliding window W: a query at position p sees keys p-W < j <= p, i.e. the last
  W positions including itself (AITER PR #3962, section "Changes": the split
  covers [seq_len - window, seq_len) for a decode query).
* ALiBi: slope_h * (j - ctx) added to the logit before the row maximum (README,
  section "2D vs 2D"; the pages give it in base 2 with a log2(e) factor, which is
  the same bias in natural units).
* QQ-bias: ``qq_bias[i, j - ctx]`` added to the logit of query i (its index
  inside the sequence's query chunk) for keys j >= ctx, i.e. a bias between the
  chunk's own tokens, applied with ALiBi before the row maximum (README, section
  "2D vs 2D", where the kernel adds it in base 2 with a 1/ln 2 factor).  The
  pages give only the indexing and a row stride ("stride=256", README section
  "Scenarios"); read here as one fp32 matrix with that row stride, shared by
  every head and sequence, read only where j >= ctx (keys of the prefix get no
  bias).
* Sinks: one logit per query head that joins the softmax normaliser but carries
  no value row (README, section "Prefill-2D trace cohort": the sink is the
  initial running maximum).
* Softcap c > 0: the scaled logit x becomes c * tanh(x / c) (the pages name the
  knob, README section "Scenarios", but never define it; this is the plainest
  reading and is applied before ALiBi).
* Grouped-query heads: q head h reads kv head h // (Hq / Hkv).
* fp8 KV: stored E4M3 codes (OCP e4m3fn or e4m3fnuz) times a per-tensor fp32
  scale, and, when given, times a per-token fp32 scale of the key's (block,
  slot, kv head) (AITER PR #3962, section "Testing": both dialects, per-tensor
  and per-token scales).  Both factors apply when both are given.
* Empty rows: a query that sees no key returns zeros (AITER PR #3962, review
  reply: rows with seq_len 0 return zeros).

Softmax is the two-pass definition per row: m = max logit, Z = sum exp(x - m),
o = sum exp(x - m) v / Z, in float64, over exactly the visible keys.  Nothing
here is blocked, partitioned or computed online.
"""

import numpy as np

from .formats import decode

_ROW_CHUNK = 256  # rows per matmul; only bounds memory, every row is independent


def gather_kv(cache_bits, kv_dtype, block_table_row, kv_len, block_size, dequant_scale,
              token_scales=None):
    """Key/value rows 0..kv_len-1 of one sequence as float64 [kv_len, Hkv, D].

    Row j comes from block ``block_table_row[j // block_size]``, slot
    ``j % block_size`` (block-table indirection of the paged cache), decoded and
    multiplied by the per-tensor dequantisation scale (1 unless fp8).
    ``token_scales``: optional per-token scales, float [num_blocks, block_size,
    Hkv] indexed like the cache; row j of kv head g is further multiplied by
    ``token_scales[page, slot, g]`` (AITER PR #3962, section "Testing" and the
    review reply: per-token K and V scales, each with its own strides).
    """
    j = np.arange(kv_len)
    pages = np.asarray(block_table_row)[j // block_size]
    slots = j % block_size
    raw = cache_bits[pages, slots]
    rows = float(dequant_scale) * decode(raw, kv_dtype)
    if token_scales is not None:
        ts = np.asarray(token_scales)[pages, slots].astype(np.float64)  # [kv_len, Hkv]
        rows = rows * ts[:, :, None]
    return rows


def visible_mask(pos, kv_len, window):
    """[n, kv_len] bool: key j visible to the query at position pos (causal + window)."""
    j = np.arange(kv_len)[None, :]
    p = np.asarray(pos)[:, None]
    vis = j <= p
    if window > 0:
        vis &= j > p - window
    return vis


def qq_terms(qq_bias, qi, rel):
    """[n, kv] QQ-bias terms: qq_bias[qi, rel] where rel = j - ctx >= 0, else 0.

    qi: [n] query indices inside the chunk; rel: [kv] key positions minus ctx.
    Entries past the matrix (rel beyond its row, reachable only by keys the
    causal mask hides) contribute 0 as well.
    """
    qq = np.asarray(qq_bias, dtype=np.float64)
    rel = np.asarray(rel)
    ok = (rel >= 0) & (rel < qq.shape[1])
    cols = np.where(ok, rel, 0)
    t = qq[np.asarray(qi)[:, None], cols[None, :]]
    return np.where(ok[None, :], t, 0.0)


def row_attention(x, vis, V, sink):
    """Two-pass softmax attention of a block of rows over one head.

    x: [n, kv] float64 logits (natural units), vis: [n, kv] bool,
    V: [kv, D] float64, sink: float or None.  Returns (o [n, D], lse [n]).
    The sink enters the normaliser only.  Rows with no visible key give o = 0.
    """
    n = x.shape[0]
    xm = np.where(vis, x, -np.inf)
    any_vis = vis.any(axis=1)
    m = xm.max(axis=1) if xm.shape[1] > 0 else np.full(n, -np.inf)
    if sink is not None:
        m = np.maximum(m, sink)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.where(vis, np.exp(np.where(vis, x, 0.0) - m_safe[:, None]), 0.0)
    Z = e.sum(axis=1)
    if sink is not None:
        Z = Z + np.exp(sink - m_safe)
    num = e @ V
    o = np.zeros_like(num)
    ok = any_vis & (Z > 0)
    o[ok] = num[ok] / Z[ok, None]
    with np.errstate(divide="ignore"):
        lse = np.where(Z > 0, m_safe + np.log(np.where(Z > 0, Z, 1.0)), -np.inf)
    return o, lse


def attention(q, k_cache, v_cache, block_table, cu_seqlens_q, seq_lens, *,
              q_dtype, kv_dtype, block_size, scale, num_q_heads, num_kv_heads,
              window=0, softcap=0.0, alibi_slopes=None, sinks=None,
              k_scale=1.0, v_scale=1.0, k_token_scales=None, v_token_scales=None,
              rows=None, qq_bias=None, **_unused):
    """Plain-definition attention in float64.

    q: stored bits [total_q, Hq, D]; k_cache/v_cache: stored bits
    [num_blocks, block_size, Hkv, D]; block_table int [num_seqs, max_blocks];
    cu_seqlens_q int [num_seqs + 1]; seq_lens int [num_seqs].
    rows: optional sorted array of query-token indices to compute (default all).
    qq_bias: optional float [rows >= max q_len, stride] matrix (natural units).
    k_token_scales / v_token_scales: optional float [num_blocks, block_size, Hkv].
    Returns (out [n_rows, Hq, D], lse [n_rows, Hq]) in float64, rows in the
    order of ``rows``.  lse includes the sink term; -inf where nothing is seen.
    """
    total_q = q.shape[0]
    D = q.shape[2]
    G = num_q_heads // num_kv_heads
    rows = np.arange(total_q) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(rows), num_q_heads, D))
    lse = np.full((len(rows), num_q_heads), -np.inf)
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    for s in range(len(seq_lens)):
        q0, q1 = int(cu[s]), int(cu[s + 1])
        sel = np.nonzero((rows >= q0) & (rows < q1))[0]
        if len(sel) == 0:
            continue
        kv_len = int(seq_lens[s])
        ctx = kv_len - (q1 - q0)
        K = gather_kv(k_cache, kv_dtype, block_table[s], kv_len, block_size, k_scale,
                      k_token_scales)
        V = gather_kv(v_cache, kv_dtype, block_table[s], kv_len, block_size, v_scale,
                      v_token_scales)
        rel = np.arange(kv_len) - ctx
        for c0 in range(0, len(sel), _ROW_CHUNK):
            idx = sel[c0:c0 + _ROW_CHUNK]
            tok = rows[idx]
            pos = ctx + (tok - q0)
            vis = visible_mask(pos, kv_len, window)
            Qd = decode(q[tok], q_dtype)  # [n, Hq, D]
            for h in range(num_q_heads):
                g = h // G
                x = scale * (Qd[:, h, :] @ K[:, g, :].T)
                if softcap > 0:
                    x = softcap * np.tanh(x / softcap)
                if alibi_slopes is not None:
                    x = x + float(alibi_slopes[h]) * rel[None, :]
                if qq_bias is not None:
                    x = x + qq_terms(qq_bias, tok - q0, rel)
                sink = None if sinks is None else float(sinks[h])
                o, l = row_attention(x, vis, V[:, g, :], sink)
                out[idx, h, :] = o
                lse[idx, h] = l
    return out, lse


def merge_partials_base2(m2, l, acc, sink=None, v_scale=1.0):
    """Merge per-partition softmax states, base-2 exponent domain.

    This is the reduce of split-KV / flash-decoding (AITER PR #3962, sections
    "Summary" and "Changes": partitions of the key range each keep their own
    softmax state and a second pass reduces them; review reply: partitions with
    l = 0 are skipped and rows without keys return zeros).  The base-2 domain
    (logits pre-multiplied by log2 e, exponentials as exp2) is the README's
    convention (section "2D vs 2D", RCP_LN2 factors).

    m2: [P, ...] partition maxima of log2-domain logits (-inf or anything when l == 0),
    l:  [P, ...] partition sums of 2^(x - m2),
    acc:[P, ..., D] partition sums of 2^(x - m2) * v (v without v_scale),
    sink: [...] natural-log sink logits or None.
    Returns (o [..., D], lse [...]) with lse in natural-log units.
    """
    m2 = np.asarray(m2, dtype=np.float64)
    l = np.asarray(l, dtype=np.float64)
    acc = np.asarray(acc, dtype=np.float64)
    live = l > 0
    mm = np.where(live, m2, -np.inf)
    M = mm.max(axis=0)
    if sink is not None:
        M = np.maximum(M, np.asarray(sink, dtype=np.float64) / np.log(2.0))
    Ms = np.where(np.isfinite(M), M, 0.0)
    w = np.where(live, np.exp2(np.where(live, m2, 0.0) - Ms), 0.0)
    L = (w * l).sum(axis=0)
    num = (w[..., None] * np.where(live[..., None], acc, 0.0)).sum(axis=0)
    any_live = live.any(axis=0)
    if sink is not None:
        L = L + np.exp2(np.asarray(sink, dtype=np.float64) / np.log(2.0) - Ms)
    o = np.zeros(num.shape)
    ok = any_live & (L > 0)
    o[ok] = v_scale * num[ok] / L[ok][..., None]
    with np.errstate(divide="ignore"):
        lse = np.where(L > 0, (Ms + np.log2(np.where(L > 0, L, 1.0))) * np.log(2.0), -np.inf)
    return o, lse


def partition_states_base2(x, vis, V, bounds):
    """Per-partition softmax states of one head's rows, base 2 (for the merge pin).

    x: [n, kv] natural-unit logits, vis: [n, kv], V: [kv, D] (without v_scale),
    bounds: list of (k0, k1) key ranges.  Returns m2, l [P, n] and acc [P, n, D];
    a partition with no visible key has l = 0 and m2 = -inf.
    """
    x2 = x / np.log(2.0)
    P = len(bounds)
    n, D = x.shape[0], V.shape[1]
    m2 = np.full((P, n), -np.inf)
    l = np.zeros((P, n))
    acc = np.zeros((P, n, D))
    for p, (k0, k1) in enumerate(bounds):
        sv = vis[:, k0:k1]
        if sv.shape[1] == 0:
            continue
        xs = np.where(sv, x2[:, k0:k1], -np.inf)
        mp = xs.max(axis=1)
        has = sv.any(axis=1)
        mps = np.where(has, mp, 0.0)
        e = np.where(sv, np.exp2(np.where(sv, x2[:, k0:k1], 0.0) - mps[:, None]), 0.0)
        m2[p] = np.where(has, mp, -np.inf)
        l[p] = e.sum(axis=1)
        acc[p] = e @ V[k0:k1]
    return m2, l, acc
