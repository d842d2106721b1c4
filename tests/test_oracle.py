"""Pins of the CPU oracle against facts that do not come from the oracle itself.

* format decoders: closed-form codes and library decoders (numpy float16, torch
  bfloat16 / float8_e4m3fn / float8_e4m3fnuz) over every code;
* the hand-worked examples in tests/golden/hand_example.json,
  tests/golden/qq_bias_example.json and tests/golden/token_scales_example.json;
* a brute-force loop implementation written independently below, on tiny
  random problems with every feature combination;
* torch's float64 scaled_dot_product_attention for the dense special case
  (also with a QQ-bias passed as its additive float mask);
* closed forms (all-zero keys, geometric ALiBi weights, two-key softcap) and
  invariants (window >= kv_len, window 1, block-table permutation, batching,
  partition merge for any partition count, per-token scales that are uniform
  or scaled by a constant).
"""

import json
import math
import os
import struct

import numpy as np
import pytest
import torch

import oracle
from oracle import attention, merge_partials_base2, partition_states_base2
from oracle.formats import decode, decode_bf16, decode_e4m3fn, decode_e4m3fnuz, decode_fp16
from synth import make_case

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_example.json")


# ----------------------------------------------------------------------------- formats

def test_fp16_closed_forms():
    codes = {0x3C00: 1.0, 0x7BFF: 65504.0, 0x0001: 2.0 ** -24, 0x0400: 2.0 ** -14,
             0xC000: -2.0, 0x3555: 0.333251953125, 0x8000: -0.0}
    for c, v in codes.items():
        assert decode_fp16(c) == v
    assert decode_fp16(0x7C00) == np.inf and decode_fp16(0xFC00) == -np.inf
    assert np.isnan(decode_fp16(0x7E00))


def test_fp16_all_codes_match_numpy():
    codes = np.arange(65536, dtype=np.uint16)
    ref = codes.view(np.float16).astype(np.float64)
    got = decode(codes, "f16")
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    m = ~np.isnan(ref)
    assert np.array_equal(ref[m], got[m])


def test_bf16_all_codes_match_bit_extension():
    codes = np.arange(65536, dtype=np.uint32)
    ref = np.array([struct.unpack("<f", struct.pack("<I", int(c) << 16))[0] for c in codes])
    got = decode(codes.astype(np.uint16), "bf16")
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    m = ~np.isnan(ref)
    assert np.array_equal(ref[m], got[m])
    assert decode_bf16(0x3F80) == 1.0 and decode_bf16(0x4049) == 3.140625


def test_e4m3fn_closed_forms_and_torch():
    assert decode_e4m3fn(0x38) == 1.0
    assert decode_e4m3fn(0x48) == 4.0
    assert decode_e4m3fn(0x50) == 8.0
    assert decode_e4m3fn(0x7E) == 448.0
    assert decode_e4m3fn(0xFE) == -448.0
    assert decode_e4m3fn(0x01) == 2.0 ** -9
    assert decode_e4m3fn(0x07) == 7 * 2.0 ** -9
    assert decode_e4m3fn(0x08) == 2.0 ** -6
    assert decode_e4m3fn(0x78) == 256.0  # all-ones exponent is a normal in E4M3FN
    assert np.isnan(decode_e4m3fn(0x7F)) and np.isnan(decode_e4m3fn(0xFF))
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = decode(codes.numpy(), "e4m3fn")
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    m = ~np.isnan(ref)
    assert np.array_equal(ref[m], got[m])


def test_e4m3fnuz_closed_forms_and_torch():
    assert decode_e4m3fnuz(0x40) == 1.0  # exponent 8 = bias
    assert decode_e4m3fnuz(0x38) == 0.5
    assert decode_e4m3fnuz(0x7F) == 240.0 and decode_e4m3fnuz(0xFF) == -240.0
    assert decode_e4m3fnuz(0x78) == 128.0  # all-ones exponent is a normal
    assert decode_e4m3fnuz(0x01) == 2.0 ** -10
    assert decode_e4m3fnuz(0x08) == 2.0 ** -7
    assert decode_e4m3fnuz(0x00) == 0.0
    assert np.isnan(decode_e4m3fnuz(0x80))
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fnuz).to(torch.float64).numpy()
    got = decode(codes.numpy(), "e4m3fnuz")
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    # same bits, half the value, wherever both dialects are finite
    fn = decode(codes.numpy(), "e4m3fn")
    both = fin & ~np.isnan(fn)
    assert np.array_equal(got[both], fn[both] / 2)


@pytest.mark.parametrize("dialect", ["e4m3fn", "e4m3fnuz"])
def test_e4m3_quantiser_roundtrip(dialect):
    """Every finite e4m3 value survives the generator's storage rounding unchanged."""
    from synth.workloads import _round_storage
    vals = decode(np.arange(256, dtype=np.uint8), dialect)
    fin = np.isfinite(vals)
    back = decode(_round_storage(vals[fin].astype(np.float32), dialect), dialect)
    assert np.array_equal(back, vals[fin])


# ----------------------------------------------------------------------------- helpers

def _bits(x, dtype):
    from synth.workloads import _round_storage
    return _round_storage(np.asarray(x, dtype=np.float32), dtype)


def paged_problem(seqs_kv, q_rows, *, block_size, dtype="f16", num_blocks=None,
                  rng=None, perm=None, extra=None):
    """Build a paged problem from dense per-sequence K/V.

    seqs_kv: list of (K [kv_len, Hkv, D], V [kv_len, Hkv, D]) float arrays,
    q_rows: list of Q [q_len, Hq, D] arrays.  Blocks are placed by ``perm`` (or
    a random permutation), unused blocks are NaN.
    """
    Hkv, D = seqs_kv[0][0].shape[1:]
    Hq = q_rows[0].shape[1]
    nblk = [math.ceil(k.shape[0] / block_size) for k, _ in seqs_kv]
    N = sum(nblk)
    nb = num_blocks or 2 * N + 1
    if perm is None:
        rng = rng or np.random.default_rng(0)
        perm = rng.permutation(nb)
    kc = np.full((nb, block_size, Hkv, D), np.nan, dtype=np.float32)
    vc = np.full((nb, block_size, Hkv, D), np.nan, dtype=np.float32)
    bt = np.full((len(seqs_kv), max(nblk) + 1), perm[N], dtype=np.int32)
    off = 0
    for s, (K, V) in enumerate(seqs_kv):
        for b in range(nblk[s]):
            phys = perm[off + b]
            bt[s, b] = phys
            rows = slice(b * block_size, min((b + 1) * block_size, K.shape[0]))
            n = rows.stop - rows.start
            kc[phys, :n] = K[rows]
            vc[phys, :n] = V[rows]
        off += nblk[s]
    q = np.concatenate(q_rows, axis=0)
    cu = np.zeros(len(q_rows) + 1, dtype=np.int32)
    cu[1:] = np.cumsum([r.shape[0] for r in q_rows])
    case = dict(q=_bits(q, dtype), k_cache=_bits(kc, dtype), v_cache=_bits(vc, dtype),
                block_table=bt, cu_seqlens_q=cu,
                seq_lens=np.array([k.shape[0] for k, _ in seqs_kv], dtype=np.int32),
                q_dtype=dtype, kv_dtype=dtype, block_size=block_size,
                num_q_heads=Hq, num_kv_heads=Hkv, scale=1.0)
    if extra:
        case.update(extra)
    return case


# ----------------------------------------------------------------------------- hand example

def _val(s):
    if isinstance(s, (int, float)):
        return float(s)
    return float(eval(s, {"ln2": math.log(2), "ln3": math.log(3), "ln4": math.log(4),
                          "ln5": math.log(5), "ln7": math.log(7), "ln8": math.log(8),
                          "ln11": math.log(11), "log2": math.log2}))


def _hand_case(case, inp):
    K = np.array(inp["keys"], dtype=np.float32)[:, None, :]
    V = np.array(inp["values"], dtype=np.float32)[:, None, :]
    gqa = case.get("gqa", False)
    q = np.array(inp["q_gqa"] if gqa else inp["q"], dtype=np.float32)[None, :, :]
    nb = inp["num_blocks"]
    kc = np.full((nb, 1, 1, 2), np.nan, dtype=np.float32)
    vc = np.full((nb, 1, 1, 2), np.nan, dtype=np.float32)
    for j, b in enumerate(inp["block_table"]):
        kc[b, 0] = K[j]
        vc[b, 0] = V[j]
    H = q.shape[1]
    return dict(q=_bits(q, "f16"), k_cache=_bits(kc, "f16"), v_cache=_bits(vc, "f16"),
                block_table=np.array([inp["block_table"]], dtype=np.int32),
                cu_seqlens_q=np.array([0, 1], dtype=np.int32),
                seq_lens=np.array([2], dtype=np.int32), q_dtype="f16", kv_dtype="f16",
                block_size=1, num_q_heads=H, num_kv_heads=1,
                scale=_val(case.get("scale", "ln3")), window=case.get("window", 0),
                softcap=_val(case["softcap"]) if "softcap" in case else 0.0,
                alibi_slopes=(np.array([_val(case["alibi"])] * H) if "alibi" in case else None),
                sinks=(np.array([_val(case["sink"])] * H) if "sink" in case else None))


@pytest.mark.parametrize("name", ["plain", "sink", "window1", "window2", "alibi", "softcap", "gqa"])
def test_hand_example(name):
    g = json.load(open(GOLDEN))
    case = next(c for c in g["cases"] if c["name"] == name)
    o, lse = attention(**_hand_case(case, g["inputs"]))
    exp = np.array(case["out"], dtype=np.float64).reshape(o.shape[1], 2)
    np.testing.assert_allclose(o[0], exp, rtol=0, atol=1e-12)
    if "lse" in case:
        assert abs(lse[0, 0] - _val(case["lse"])) < 1e-12


def test_hand_example_merge():
    g = json.load(open(GOLDEN))
    case = next(c for c in g["cases"] if c["name"] == "merge")
    m2 = np.array([[_val(p[0])] for p in case["partitions"]])
    l = np.array([[p[1]] for p in case["partitions"]])
    acc = np.array([[p[2]] for p in case["partitions"]])
    o, lse = merge_partials_base2(m2, l, acc)
    np.testing.assert_allclose(o[0], case["out"], atol=1e-12)
    assert abs(lse[0] - _val(case["lse"])) < 1e-12


def test_qq_bias_hand_example():
    g = json.load(open(os.path.join(os.path.dirname(GOLDEN), "qq_bias_example.json")))
    inp = g["inputs"]
    K = np.array(inp["keys"], dtype=np.float32)[:, None, :]
    V = np.array(inp["values"], dtype=np.float32)[:, None, :]
    Q = np.zeros((inp["q_len"], 1, 2), dtype=np.float32)
    qq = np.array([[_val(x) for x in row] for row in inp["qq_bias"]])
    c = paged_problem([(K, V)], [Q], block_size=2, extra=dict(scale=1.0, qq_bias=qq))
    o, lse = attention(**c)
    np.testing.assert_allclose(o[:, 0, :], np.array(g["out"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[:, 0], [_val(x) for x in g["lse"]], rtol=0, atol=1e-12)


@pytest.mark.parametrize("dialect", ["e4m3fn", "e4m3fnuz"])
def test_token_scales_hand_example(dialect):
    g = json.load(open(os.path.join(os.path.dirname(GOLDEN), "token_scales_example.json")))
    inp = g["inputs"]
    codes = inp["codes"][dialect]
    nb, bt = inp["num_blocks"], inp["block_table"]
    kc = np.full((nb, 1, 1, 2), codes["nan"], dtype=np.uint8)
    vc = np.full((nb, 1, 1, 2), codes["nan"], dtype=np.uint8)
    kts = np.full((nb, 1, 1), np.nan)
    vts = np.full((nb, 1, 1), np.nan)
    for j, b in enumerate(bt):
        kc[b, 0, 0] = codes["k"][j]
        vc[b, 0, 0] = codes["v"][j]
        kts[b, 0, 0] = inp["k_token_scales"][j]
        vts[b, 0, 0] = inp["v_token_scales"][j]
    q = _bits(np.array(inp["q"], dtype=np.float32)[None], "bf16")
    o, lse = attention(q, kc, vc, np.array([bt], dtype=np.int32), np.array([0, 1]),
                       np.array([2]), q_dtype="bf16", kv_dtype=dialect, block_size=1,
                       scale=_val(inp["scale"]), num_q_heads=1, num_kv_heads=1,
                       k_token_scales=kts, v_token_scales=vts)
    np.testing.assert_allclose(o[0, 0], g["out"], rtol=0, atol=1e-12)
    assert abs(lse[0, 0] - _val(g["lse"])) < 1e-12


def _token_case(dialect, seed, **kw):
    return make_case(seqs=[(3, 37), (1, 20), (5, 5)], head_dim=8, num_q_heads=4,
                     num_kv_heads=2, block_size=4, q_dtype="bf16", kv_dtype=dialect,
                     token_scales=True, seed=seed, **kw)


@pytest.mark.parametrize("dialect", ["e4m3fn", "e4m3fnuz"])
def test_uniform_token_scales_equal_a_tensor_scale(dialect):
    c = _token_case(dialect, 11)
    ks, vs = 0.375, 1.875  # exact in the float32 scale arrays
    ref = attention(**dict(c, k_token_scales=None, v_token_scales=None, k_scale=ks,
                           v_scale=vs))
    got = attention(**dict(c, k_token_scales=np.full_like(c["k_token_scales"], ks),
                           v_token_scales=np.full_like(c["v_token_scales"], vs)))
    np.testing.assert_allclose(got[0], ref[0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(got[1], ref[1], rtol=0, atol=1e-13)


@pytest.mark.parametrize("dialect", ["e4m3fn", "e4m3fnuz"])
def test_token_scale_identities(dialect):
    """Scaling every K token scale by c is scaling the softmax scale by c; scaling
    every V token scale by c scales the output by c; a per-tensor factor multiplies
    the per-token ones."""
    c = _token_case(dialect, 12, sinks=True, window=9)
    o, lse = attention(**c)
    k2 = attention(**dict(c, k_token_scales=c["k_token_scales"] * 2.0))
    s2 = attention(**dict(c, scale=c["scale"] * 2.0))
    np.testing.assert_allclose(k2[0], s2[0], rtol=1e-12, atol=1e-13)
    v2 = attention(**dict(c, v_token_scales=c["v_token_scales"] * 0.25))
    np.testing.assert_allclose(v2[0], o * 0.25, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(v2[1], lse, rtol=0, atol=1e-13)
    t2 = attention(**dict(c, k_scale=2.0, k_token_scales=c["k_token_scales"] / 2,
                          v_scale=4.0, v_token_scales=c["v_token_scales"] / 4))
    np.testing.assert_allclose(t2[0], o, rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------- brute force

def _dec_lib(bits, dtype):
    """Library decoders, independent of oracle.formats."""
    b = np.asarray(bits)
    if dtype == "f16":
        return b.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    fp8 = torch.float8_e4m3fn if dtype == "e4m3fn" else torch.float8_e4m3fnuz
    return torch.from_numpy(b.copy()).view(fp8).double().numpy()


def brute_force(c):
    """Loop-by-loop attention, written independently of oracle.attention."""
    qf = _dec_lib(c["q"], c["q_dtype"])
    kf = _dec_lib(c["k_cache"], c["kv_dtype"]) * c.get("k_scale", 1.0)
    vf = _dec_lib(c["v_cache"], c["kv_dtype"]) * c.get("v_scale", 1.0)
    kts = c.get("k_token_scales")
    vts = c.get("v_token_scales")
    H, Hk = c["num_q_heads"], c["num_kv_heads"]
    D = qf.shape[2]
    bs = c["block_size"]
    W = c.get("window", 0)
    cap = c.get("softcap", 0.0)
    slopes = c.get("alibi_slopes")
    sinks = c.get("sinks")
    qq = c.get("qq_bias")
    out = np.zeros(qf.shape)
    cu = c["cu_seqlens_q"]
    for s in range(len(c["seq_lens"])):
        kv = int(c["seq_lens"][s])
        ql = int(cu[s + 1] - cu[s])
        for i in range(ql):
            t = int(cu[s]) + i
            p = kv - ql + i
            for h in range(H):
                g = h * Hk // H
                logits = []
                vals = []
                for j in range(kv):
                    if j > p or (W > 0 and j <= p - W):
                        continue
                    blk = c["block_table"][s][j // bs]
                    krow = kf[blk, j % bs, g]
                    if kts is not None:
                        krow = krow * float(kts[blk][j % bs][g])
                    x = c["scale"] * sum(qf[t, h, d] * krow[d] for d in range(D))
                    if cap > 0:
                        x = cap * math.tanh(x / cap)
                    if slopes is not None:
                        x += float(slopes[h]) * (j - (kv - ql))
                    if qq is not None and j >= kv - ql:
                        x += float(qq[i][j - (kv - ql)])
                    logits.append(x)
                    vrow = vf[blk, j % bs, g]
                    if vts is not None:
                        vrow = vrow * float(vts[blk][j % bs][g])
                    vals.append(vrow)
                if not logits:
                    continue
                allx = logits + ([float(sinks[h])] if sinks is not None else [])
                mx = max(allx)
                z = sum(math.exp(x - mx) for x in allx)
                for x, v in zip(logits, vals):
                    out[t, h] += math.exp(x - mx) / z * v
    return out


FEATURES = [
    dict(),
    dict(window=3),
    dict(window=1),
    dict(softcap=0.7),
    dict(alibi=True),
    dict(sinks=True),
    dict(window=5, softcap=2.0, sinks=True),
    dict(window=4, alibi=True),
    dict(qq_bias=24),
    dict(qq_bias=20, alibi=True, softcap=1.5, window=6),
    dict(token_scales=True),
    dict(token_scales=True, window=4, sinks=True),
]


@pytest.mark.parametrize("fi", range(len(FEATURES)))
@pytest.mark.parametrize("dtype,kvd", [("f16", "f16"), ("bf16", "bf16"), ("bf16", "e4m3fn"),
                                       ("f16", "e4m3fnuz")])
def test_oracle_matches_brute_force(fi, dtype, kvd):
    if FEATURES[fi].get("token_scales") and not kvd.startswith("e4m3"):
        pytest.skip("per-token scales exist only for fp8 caches")
    rng = np.random.default_rng(fi * 7 + len(dtype) + len(kvd))
    for trial in range(3):
        D = int(rng.choice([2, 4, 8]))
        bs = int(rng.choice([1, 3, 16]))
        Hk = int(rng.choice([1, 2]))
        G = int(rng.choice([1, 2, 3]))
        n = int(rng.integers(1, 4))
        seqs = []
        for _ in range(n):
            kv = int(rng.integers(0, 20))
            ql = int(rng.integers(0, kv + 1))
            seqs.append((ql, kv))
        c = make_case(seqs=seqs, head_dim=D, num_q_heads=G * Hk, num_kv_heads=Hk,
                      block_size=bs, q_dtype=dtype, kv_dtype=kvd,
                      seed=int(rng.integers(1 << 30)), scale=0.9, **FEATURES[fi])
        o, _ = attention(**c)
        ref = brute_force(c)
        np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- library special case

@pytest.mark.parametrize("G", [1, 4])
def test_oracle_matches_torch_sdpa_fp64(G):
    rng = np.random.default_rng(5)
    Hk, D, L = 2, 16, 37
    K = rng.standard_normal((L, Hk, D)).astype(np.float16).astype(np.float32)
    V = rng.standard_normal((L, Hk, D)).astype(np.float16).astype(np.float32)
    Q = rng.standard_normal((L, G * Hk, D)).astype(np.float16).astype(np.float32)
    c = paged_problem([(K, V)], [Q], block_size=5, extra=dict(scale=0.3))
    o, _ = attention(**c)
    qt = torch.from_numpy(Q.astype(np.float64)).permute(1, 0, 2)[None]
    kt = torch.from_numpy(K.astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, 0)[None]
    vt = torch.from_numpy(V.astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, 0)[None]
    mask = torch.ones(L, L, dtype=torch.bool).tril()  # q_len == kv_len: bottom-right == top-left
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=0.3)
    np.testing.assert_allclose(o, ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("G", [1, 4])
def test_qq_bias_matches_torch_sdpa_float_mask(G):
    """q_len == kv_len (ctx = 0): the QQ-bias is SDPA's additive float mask on the
    causal triangle (qq[i][j] for j <= i, -inf above)."""
    rng = np.random.default_rng(6)
    Hk, D, L, stride = 2, 8, 29, 40
    K = rng.standard_normal((L, Hk, D)).astype(np.float16).astype(np.float32)
    V = rng.standard_normal((L, Hk, D)).astype(np.float16).astype(np.float32)
    Q = rng.standard_normal((L, G * Hk, D)).astype(np.float16).astype(np.float32)
    qq = rng.standard_normal((L, stride))
    c = paged_problem([(K, V)], [Q], block_size=3, extra=dict(scale=0.4, qq_bias=qq))
    o, _ = attention(**c)
    qt = torch.from_numpy(Q.astype(np.float64)).permute(1, 0, 2)[None]
    kt = torch.from_numpy(K.astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, 0)[None]
    vt = torch.from_numpy(V.astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, 0)[None]
    fm = torch.full((L, L), float("-inf"), dtype=torch.float64)
    tri = torch.ones(L, L, dtype=torch.bool).tril()
    fm[tri] = torch.from_numpy(qq[:, :L])[tri]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=fm, scale=0.4)
    np.testing.assert_allclose(o, ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_qq_bias_linear_rows_equal_alibi_without_prefix():
    """ctx = 0: qq[i][c] = slope * c for every row is ALiBi with that slope (one
    head), and a row-constant bias cancels in the softmax."""
    rng = np.random.default_rng(8)
    L, D, slope = 23, 4, 0.37
    K = rng.standard_normal((L, 1, D)).astype(np.float32)
    V = rng.standard_normal((L, 1, D)).astype(np.float32)
    Q = rng.standard_normal((L, 1, D)).astype(np.float32)
    qq = np.tile(slope * np.arange(32, dtype=np.float64), (L, 1))
    base = paged_problem([(K, V)], [Q], block_size=4, extra=dict(scale=0.5))
    o_qq, _ = attention(**dict(base, qq_bias=qq))
    o_al, _ = attention(**dict(base, alibi_slopes=np.array([slope])))
    np.testing.assert_allclose(o_qq, o_al, rtol=0, atol=1e-12)
    rowc = np.tile(rng.standard_normal((L, 1)), (1, 32))
    o_rc, _ = attention(**dict(base, qq_bias=rowc))
    o_0, _ = attention(**base)
    np.testing.assert_allclose(o_rc, o_0, rtol=0, atol=1e-12)
    # with a prefix the bias reaches only the chunk's keys: a row-constant bias
    # then shifts weight from the prefix to the chunk
    Qc = Q[-5:]
    pre = paged_problem([(K, V)], [Qc], block_size=4, extra=dict(scale=0.5))
    o_p0, _ = attention(**pre)
    o_p1, _ = attention(**dict(pre, qq_bias=np.full((5, 8), 3.0)))
    assert np.abs(o_p1 - o_p0).max() > 1e-3


# ----------------------------------------------------------------------------- closed forms

@pytest.mark.parametrize("bs", [1, 13, 16, 784])
@pytest.mark.parametrize("W", [0, 1, 17, 100])
def test_zero_keys_mean_of_window(bs, W):
    """K == 0: every logit is 0, so row i returns the mean of V over its visible range."""
    rng = np.random.default_rng(bs + W)
    Hk, G, D = 2, 3, 4
    lens = [(1, 200), (7, 50), (0, 9), (30, 30)]
    seqs, qs = [], []
    for ql, kv in lens:
        K = np.zeros((kv, Hk, D), dtype=np.float32)
        V = rng.integers(-8, 9, size=(kv, Hk, D)).astype(np.float32)
        seqs.append((K, V))
        qs.append(rng.standard_normal((ql, G * Hk, D)).astype(np.float32))
    c = paged_problem(seqs, qs, block_size=bs, rng=rng, extra=dict(window=W))
    o, _ = attention(**c)
    t = 0
    for (K, V), (ql, kv) in zip(seqs, lens):
        for i in range(ql):
            p = kv - ql + i
            lo = max(0, p - W + 1) if W > 0 else 0
            for h in range(G * Hk):
                np.testing.assert_allclose(o[t, h], V[lo:p + 1, h // G].mean(axis=0), atol=1e-12)
            t += 1


def test_zero_keys_with_sinks():
    rng = np.random.default_rng(3)
    kv, D = 25, 4
    V = rng.standard_normal((kv, 1, D)).astype(np.float16).astype(np.float32)
    K = np.zeros((kv, 1, D), dtype=np.float32)
    Q = rng.standard_normal((3, 2, D)).astype(np.float32)
    sinks = np.array([0.5, -1.25])
    c = paged_problem([(K, V)], [Q], block_size=4, extra=dict(sinks=sinks))
    o, lse = attention(**c)
    for i in range(3):
        p = kv - 3 + i
        for h in range(2):
            exp = V[:p + 1, 0].sum(axis=0) / (p + 1 + math.exp(sinks[h]))
            np.testing.assert_allclose(o[i, h], exp, atol=1e-12)
            assert abs(lse[i, h] - math.log(p + 1 + math.exp(sinks[h]))) < 1e-12


def test_alibi_geometric_weights():
    """K == 0 with slope a: weights proportional to exp(a * j)."""
    kv, D, a = 40, 3, 0.37
    rng = np.random.default_rng(9)
    V = rng.standard_normal((kv, 1, D)).astype(np.float16).astype(np.float32)
    K = np.zeros((kv, 1, D), dtype=np.float32)
    Q = np.ones((5, 1, D), dtype=np.float32)
    c = paged_problem([(K, V)], [Q], block_size=7, extra=dict(alibi_slopes=np.array([a])))
    o, _ = attention(**c)
    for i in range(5):
        p = kv - 5 + i
        w = np.exp(a * np.arange(p + 1))
        np.testing.assert_allclose(o[i, 0], (w[:, None] * V[:p + 1, 0]).sum(0) / w.sum(), atol=1e-12)


def test_softcap_two_keys_sigmoid():
    c_ = 1.5
    K = np.array([[[0.5, 0.0]], [[2.0, 1.0]]], dtype=np.float32)
    V = np.array([[[1.0, 0.0]], [[0.0, 1.0]]], dtype=np.float32)
    Q = np.array([[[1.0, 2.0]]], dtype=np.float32)
    c = paged_problem([(K, V)], [Q], block_size=1, extra=dict(softcap=c_, scale=0.8))
    o, _ = attention(**c)
    x0, x1 = 0.8 * 0.5, 0.8 * 4.0
    w1 = 1 / (1 + math.exp(-(c_ * math.tanh(x1 / c_) - c_ * math.tanh(x0 / c_))))
    np.testing.assert_allclose(o[0, 0], [1 - w1, w1], atol=1e-12)


# ----------------------------------------------------------------------------- invariants

def _case(**kw):
    base = dict(seqs=[(1, 300), (17, 90), (0, 12), (40, 40)], head_dim=8, num_q_heads=4,
                num_kv_heads=2, block_size=16, q_dtype="bf16", seed=77)
    base.update(kw)
    return make_case(**base)


def test_window_at_least_kv_len_is_no_window():
    o0, l0 = attention(**_case())
    o1, l1 = attention(**_case(window=300))
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_window_one_returns_own_value_row():
    c = _case(window=1)
    o, _ = attention(**c)
    from oracle.attention import gather_kv
    t = 0
    for s, (ql, kv) in enumerate([(1, 300), (17, 90), (0, 12), (40, 40)]):
        V = gather_kv(c["v_cache"], "bf16", c["block_table"][s], kv, 16, 1.0)
        for i in range(ql):
            p = kv - ql + i
            for h in range(4):
                np.testing.assert_allclose(o[t, h], V[p, h // 2], atol=1e-15)
            t += 1


def test_sink_minus_infinity_and_huge_softcap_are_off():
    c = _case(sinks=True, softcap=1e30)
    c_off = dict(c, sinks=np.full(4, -1e30), softcap=1e30)
    c_plain = dict(c, sinks=None, softcap=0.0)
    o_off, _ = attention(**c_off)
    o_plain, _ = attention(**c_plain)
    np.testing.assert_allclose(o_off, o_plain, atol=1e-14)


def test_block_table_permutation_and_block_size_invariance():
    rng = np.random.default_rng(11)
    K = rng.standard_normal((70, 2, 8)).astype(np.float32)
    V = rng.standard_normal((70, 2, 8)).astype(np.float32)
    Q = rng.standard_normal((9, 4, 8)).astype(np.float32)
    outs = []
    for bs, seed in [(1, 0), (13, 1), (16, 2), (70, 3), (128, 4)]:
        c = paged_problem([(K, V)], [Q], block_size=bs, dtype="bf16",
                          rng=np.random.default_rng(seed), extra=dict(scale=0.4))
        outs.append(attention(**c)[0])
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_batched_equals_per_sequence():
    seqs = [(1, 300), (17, 90), (0, 12), (40, 40)]
    c = _case(window=33, sinks=True, alibi=True)
    o, lse = attention(**c)
    from oracle.attention import gather_kv
    t = 0
    for s, (ql, kv) in enumerate(seqs):
        sub = dict(c, q=c["q"][t:t + ql], block_table=c["block_table"][s:s + 1],
                   cu_seqlens_q=np.array([0, ql], dtype=np.int32),
                   seq_lens=np.array([kv], dtype=np.int32))
        os_, ls_ = attention(**sub)
        assert np.array_equal(os_, o[t:t + ql]) and np.array_equal(ls_, lse[t:t + ql])
        t += ql


@pytest.mark.parametrize("n_part", [1, 2, 3, 4, 7, 16])
@pytest.mark.parametrize("with_sink", [False, True])
def test_partition_merge_equals_one_pass(n_part, with_sink):
    """Split-KV invariant: merging partition states (sink added once) equals the definition."""
    rng = np.random.default_rng(n_part)
    kv, n, D = 150, 6, 8
    x = rng.standard_normal((n, kv)) * 3
    pos = np.array([10, 60, 149, 149, 0, 149])
    from oracle.attention import row_attention, visible_mask
    vis = visible_mask(pos, kv, 40 if n_part % 2 else 0)
    vis[3] = False  # a row with no visible key
    V = rng.standard_normal((kv, D))
    sink = 0.7 if with_sink else None
    o_ref, lse_ref = row_attention(x, vis, V, sink)
    edges = np.linspace(0, kv, n_part + 1).astype(int)
    bounds = list(zip(edges[:-1], edges[1:]))
    m2, l, acc = partition_states_base2(x, vis, V, bounds)
    o, lse = merge_partials_base2(m2, l, acc, None if sink is None else np.full(n, sink))
    np.testing.assert_allclose(o, o_ref, atol=1e-12)
    fin = np.isfinite(lse_ref)
    np.testing.assert_allclose(lse[fin], lse_ref[fin], atol=1e-12)
    assert np.array_equal(np.isfinite(lse), fin)


def test_merge_adds_sink_once():
    """Adding the sink per partition instead of once would change the result."""
    m2 = np.array([[0.0], [1.0]])
    l = np.array([[1.0], [1.0]])
    acc = np.array([[[1.0]], [[2.0]]])
    o_once, _ = merge_partials_base2(m2, l, acc, np.array([0.0]))
    # sink once: L = 2^-1 + 1 + 2^-1 = 2, O = (0.5*1 + 2) / 2
    np.testing.assert_allclose(o_once[0], [1.25], atol=1e-15)


def test_empty_sequences_and_rows():
    c = make_case(seqs=[(0, 0), (0, 5), (3, 3)], head_dim=4, num_q_heads=2, num_kv_heads=1,
                  block_size=2, q_dtype="f16", seed=1, sinks=True)
    o, lse = attention(**c)
    assert o.shape == (3, 2, 4) and np.isfinite(o).all()
    c2 = make_case(seqs=[(2, 2)], head_dim=4, num_q_heads=2, num_kv_heads=1, block_size=2,
                   q_dtype="f16", seed=1)
    c2["seq_lens"] = np.array([0], dtype=np.int32)
    c2["cu_seqlens_q"] = np.array([0, 0], dtype=np.int32)
    o2, _ = attention(**dict(c2, q=c2["q"][:0]))
    assert o2.shape[0] == 0


def test_feature_sensitivity_at_test_settings():
    """Features used in GPU tests move the output by far more than the tolerances."""
    base = dict(seqs=[(1, 40), (9, 64)], head_dim=32, num_q_heads=8, num_kv_heads=2,
                block_size=16, q_dtype="bf16", seed=5)
    short = dict(base, seqs=[(1, 4), (3, 6), (2, 300)])
    for b, kw in [(base, dict(softcap=3.0)), (short, dict(sinks=True)),
                  (base, dict(window=17)), (base, dict(alibi=True))]:
        o0, _ = attention(**make_case(**b))
        o1, _ = attention(**make_case(**b, **kw))
        assert np.abs(o1 - o0).max() > 0.05, kw


def test_oracle_package_exports():
    assert callable(oracle.attention) and callable(oracle.merge_partials_base2)
