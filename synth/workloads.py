"""Seeded synthetic inputs for unified paged varlen attention.

This module only draws random numbers, rounds them to the storage types and
lays them out as a paged cache; it holds none of the attention arithmetic.  Both
the GPU tests/benchmark and the CPU oracle consume the bytes it produces.

Recipe (one ``numpy.random.Generator(PCG64(seed))`` per case, fixed draw order):

1. kv lengths that are drawn from a range (uniform integers, inclusive);
2. a permutation of the physical blocks;
3. Q, then K, then V as float32 N(0, 1) ("values N(0,1)" in every workload);
4. sink logits N(0, 1) when sinks are on;
5. the QQ-bias matrix N(0, 1) when it is on: float32 [max(max q_len, 1), stride]
   (one matrix for every head and sequence, row stride ``stride``).

The cache holds ``2 * N`` blocks where N = sum ceil(kv_len / block_size) blocks
are needed; the logical blocks of all sequences, in (sequence, block) order,
take the first N entries of the permutation ("block table = random permutation
of physical pages in a cache of 2x needed pages").  Block-table rows are padded
with the first unused physical block.  With ``poison=True`` every value the
attention must never read is NaN (fp8: the 0x7F NaN code): unused blocks, slots
past kv_len in a sequence's last block, and the padding block.

Storage rounding is round-to-nearest-even: float16 through numpy, bfloat16 and
both e4m3 dialects (OCP e4m3fn, e4m3fnuz) through torch's CPU casts, after
clamping to the dialect's largest finite magnitude (448, 240).  fp8 data is
quantised with a per-tensor scale amax / max_finite (so the largest magnitude
maps to the largest finite code), returned as ``k_scale`` / ``v_scale``; with
``token_scales=True`` each (block, slot, kv head) row of D values gets its own
scale amax(row) / max_finite instead (the per-tensor scales are then 1), returned
as ``k_token_scales`` / ``v_token_scales``: float32 arrays indexed [block, slot,
kv head] whose memory layouts differ on purpose (K: [block, kv head, slot]
underneath, V: [block, slot, kv head]), NaN wherever the cache is NaN.
"""

import math

import numpy as np

_FP8_MAX = {"e4m3fn": 448.0, "e4m3fnuz": 240.0}


def _round_storage(x32, dtype):
    """float32 array -> (stored bits, dtype tag). No attention arithmetic here."""
    if dtype == "f16":
        return x32.astype(np.float16).view(np.uint16)
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    if dtype == "bf16":
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if dtype in _FP8_MAX:
        t = torch.clamp(t, -_FP8_MAX[dtype], _FP8_MAX[dtype])
        tdt = torch.float8_e4m3fn if dtype == "e4m3fn" else torch.float8_e4m3fnuz
        return t.to(tdt).view(torch.uint8).numpy()
    raise ValueError(dtype)


def _nan_bits(dtype):
    return {"f16": 0x7E00, "bf16": 0x7FC0, "e4m3fn": 0x7F, "e4m3fnuz": 0x80}[dtype]


def _storage_np(dtype):
    return np.uint8 if dtype in _FP8_MAX else np.uint16


def alibi_slopes_pow2(num_heads):
    """Per-head slopes 2^(-8 i / H) for i = 1..H (the textbook ALiBi sequence)."""
    return np.array([2.0 ** (-8.0 * (h + 1) / num_heads) for h in range(num_heads)],
                    dtype=np.float32)


def make_case(*, seqs, head_dim, num_q_heads, num_kv_heads, block_size,
              q_dtype="f16", kv_dtype=None, o_dtype=None, seed=0,
              kv_range=None, num_seqs=None, q_len=None,
              window=0, softcap=0.0, alibi=False, sinks=False, qq_bias=False,
              token_scales=False, poison=True, scale=None, extra_pad_cols=1,
              cache_factor=2):
    """Build one seeded case.

    ``seqs``: list of (q_len, kv_len) pairs, or None to draw ``num_seqs`` kv
    lengths uniformly from ``kv_range`` (inclusive) with the given ``q_len``.
    ``alibi``: False, True (2^(-8i/H) slopes) or an explicit slope array.
    ``qq_bias``: False, True (row stride 256) or the row stride as an int.
    ``token_scales``: fp8 only; per-(block, slot, kv head) scales instead of
    per-tensor ones.
    Returns a dict whose keys match the oracle's and the binding's arguments.
    """
    kv_dtype = kv_dtype or q_dtype
    o_dtype = o_dtype or q_dtype
    rng = np.random.Generator(np.random.PCG64(seed))
    if seqs is None:
        lo, hi = kv_range
        kvs = rng.integers(lo, hi + 1, size=num_seqs)
        seqs = [(q_len, int(k)) for k in kvs]
    seqs = [(int(a), int(b)) for a, b in seqs]
    for ql, kl in seqs:
        if not 0 <= ql <= kl:
            raise ValueError("need 0 <= q_len <= kv_len")
    n_seqs = len(seqs)
    q_lens = np.array([s[0] for s in seqs], dtype=np.int64)
    kv_lens = np.array([s[1] for s in seqs], dtype=np.int64)
    nblk = [math.ceil(k / block_size) for k in kv_lens]
    N = int(sum(nblk))
    num_blocks = max(cache_factor * N, N + 1)
    perm = rng.permutation(num_blocks)
    pad_block = int(perm[N])
    max_blocks = max(max(nblk) if nblk else 0, 1) + extra_pad_cols
    block_table = np.full((n_seqs, max_blocks), pad_block, dtype=np.int32)
    off = 0
    for s, nb in enumerate(nblk):
        block_table[s, :nb] = perm[off:off + nb]
        off += nb
    total_q = int(q_lens.sum())
    H, Hk, D = num_q_heads, num_kv_heads, head_dim
    qf = rng.standard_normal((total_q, H, D), dtype=np.float32)
    kf = rng.standard_normal((N, block_size, Hk, D), dtype=np.float32)
    vf = rng.standard_normal((N, block_size, Hk, D), dtype=np.float32)
    sink_vals = rng.standard_normal(H, dtype=np.float32) if sinks else None
    qq = None
    if qq_bias is not False and qq_bias is not None:
        stride = 256 if qq_bias is True else int(qq_bias)
        rows = max(int(q_lens.max()) if n_seqs else 0, 1)
        if stride < rows:
            raise ValueError("qq_bias stride must cover the longest query chunk")
        qq = rng.standard_normal((rows, stride), dtype=np.float32)

    if token_scales and kv_dtype not in _FP8_MAX:
        raise ValueError("per-token scales need an fp8 cache")
    k_scale = v_scale = 1.0
    kts = vts = None
    if kv_dtype in _FP8_MAX:
        fmax = np.float32(_FP8_MAX[kv_dtype])
        if token_scales:
            def row_scales(x):
                a = np.abs(x).max(axis=-1) if x.size else np.zeros(x.shape[:-1], np.float32)
                return np.where(a > 0, a / fmax, np.float32(1.0)).astype(np.float32)
            kts, vts = row_scales(kf), row_scales(vf)  # [N, bs, Hk]
            kf = kf / kts[..., None]
            vf = vf / vts[..., None]
        else:
            k_scale = float(np.float32(np.abs(kf).max() / fmax)) if kf.size else 1.0
            v_scale = float(np.float32(np.abs(vf).max() / fmax)) if vf.size else 1.0
            kf = kf / np.float32(k_scale)
            vf = vf / np.float32(v_scale)

    sd = _storage_np(kv_dtype)
    fill = _nan_bits(kv_dtype) if poison else 0
    k_cache = np.full((num_blocks, block_size, Hk, D), fill, dtype=sd)
    v_cache = np.full((num_blocks, block_size, Hk, D), fill, dtype=sd)
    kb = _round_storage(kf, kv_dtype)
    vb = _round_storage(vf, kv_dtype)
    sfill = np.float32(np.nan) if poison else np.float32(1.0)
    if poison:
        # slots past kv_len in each sequence's last block stay NaN
        off = 0
        for s, nb in enumerate(nblk):
            tail = nb * block_size - int(kv_lens[s])
            if tail:
                kb[off + nb - 1, block_size - tail:] = fill
                vb[off + nb - 1, block_size - tail:] = fill
                if kts is not None:
                    kts[off + nb - 1, block_size - tail:] = sfill
                    vts[off + nb - 1, block_size - tail:] = sfill
            off += nb
    k_cache[perm[:N]] = kb
    v_cache[perm[:N]] = vb
    k_token_scales = v_token_scales = None
    if kts is not None:
        # K scales live as [block, kv head, slot], V scales as [block, slot, kv head];
        # both are handed out indexed [block, slot, kv head].
        k_phys = np.full((num_blocks, Hk, block_size), sfill, dtype=np.float32)
        k_phys[perm[:N]] = kts.transpose(0, 2, 1)
        k_token_scales = k_phys.transpose(0, 2, 1)
        v_token_scales = np.full((num_blocks, block_size, Hk), sfill, dtype=np.float32)
        v_token_scales[perm[:N]] = vts

    if alibi is True:
        slopes = alibi_slopes_pow2(H)
    elif alibi is False or alibi is None:
        slopes = None
    else:
        slopes = np.asarray(alibi, dtype=np.float32)

    cu = np.zeros(n_seqs + 1, dtype=np.int32)
    cu[1:] = np.cumsum(q_lens)
    return dict(
        q=_round_storage(qf, q_dtype), k_cache=k_cache, v_cache=v_cache,
        block_table=block_table, cu_seqlens_q=cu, seq_lens=kv_lens.astype(np.int32),
        alibi_slopes=slopes, sinks=sink_vals, qq_bias=qq,
        q_dtype=q_dtype, kv_dtype=kv_dtype, o_dtype=o_dtype,
        block_size=block_size, head_dim=D, num_q_heads=H, num_kv_heads=Hk,
        scale=float(scale if scale is not None else 1.0 / math.sqrt(D)),
        window=int(window), softcap=float(softcap),
        k_scale=k_scale, v_scale=v_scale, seed=seed,
        k_token_scales=k_token_scales, v_token_scales=v_token_scales,
        max_seqlen_q=int(q_lens.max()) if n_seqs else 0,
        max_seqlen_k=int(kv_lens.max()) if n_seqs else 0,
    )
