"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Every case is seeded; unused cache blocks, slots past kv_len, the block-table
padding block, the output buffer and the split-KV workspace are NaN-poisoned,
so any read of them or any unwritten output shows up as a failure.
"""

import ctypes
import math
import functools

import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS, make_case
from synth.configs import NEXT_DECODE_WORKLOADS, NEXT_PREFILL_WORKLOADS
from tests.gpu_common import (block_edge_rows, check_lse, compare, oracle_parallel, run,
                              sample_rows, to_device, tolerance, ulp)

pytestmark = pytest.mark.gpu

PATHS = [("auto", 0), ("2d", 0), ("splitkv", 1), ("splitkv", 4), ("splitkv", 7), ("splitkv", 16)]


@functools.lru_cache(maxsize=None)
def _workload(name):
    case = make_case(**WORKLOADS[name])
    ref, lse = oracle.attention(**case)
    return case, ref, lse


@functools.lru_cache(maxsize=None)
def _dev(name):
    return to_device(_workload(name)[0])


DECODE_AND_MIXED = [
    "decode_fp16_d128_16q2kv",
    "mixed_fp16_d128_16q2kv",
    "mixed_fp16_d128_16q2kv_alibi",
    "long_decode_bf16_d128_32q8kv_w4096",
    "long_decode_bf16_d128_32q8kv_w4096_softcap_sinks",
    "fp8kv_decode_b32_ctx590",
    "fp8kv_decode_b8_ctx6700_w4096",
]


@pytest.mark.parametrize("path,n_part", PATHS, ids=[f"{p}{n}" for p, n in PATHS])
@pytest.mark.parametrize("name", DECODE_AND_MIXED)
def test_workload_full_size(name, path, n_part):
    case, ref, ref_lse = _workload(name)
    print(f"[case] {name} path={path} n_part={n_part}", flush=True)
    got, lse, plan = run(case, _dev(name), path=path, n_part=n_part, lse=True)
    err = compare(case, got, ref, label=f"{name}/{path}{n_part}")
    check_lse(lse, ref_lse, case, label=name)
    print(f"[ok] {name} path={plan.path} n_part={plan.n_part} max_abs={err:.3e}", flush=True)


PREFILL = ["prefill_chunk1k_prefix8k_bf16", "prefill_chunk2k_prefix16k_bf16",
           "prefill_4x1k_bf16", "prefill_8k_d256_24q4kv_bs784_bf16", "prefill_8k_d128_bf16"]


@functools.lru_cache(maxsize=2)
def _workload_full(name):
    """Case and full float64 oracle output (row chunks over the host cores)."""
    case = make_case(**WORKLOADS[name])
    ref, lse = oracle_parallel(case)
    return case, ref, lse


@pytest.mark.parametrize("name", PREFILL)
def test_prefill_full_size(name):
    """Every output element of each chunked-prefill workload, on the planned
    path and on a forced three-partition split, against the oracle."""
    print(f"[case] {name} oracle (all rows)", flush=True)
    case, ref, ref_lse = _workload_full(name)
    dev = to_device(case)
    for path, n_part in (("auto", 0), ("splitkv", 3)):
        print(f"[case] {name} path={path} n_part={n_part}", flush=True)
        got, lse, plan = run(case, dev, path=path, n_part=n_part, lse=True)
        err = compare(case, got, ref, label=f"{name}/{path}{n_part}")
        check_lse(lse, ref_lse, case, label=name)
        print(f"[ok] {name} kernel={plan.kernel} path={plan.path} n_part={plan.n_part} "
              f"max_abs={err:.3e}", flush=True)
    del dev
    torch.cuda.empty_cache()


@pytest.mark.parametrize("extra", [1000, 2000, 3000])
@pytest.mark.parametrize("name", DECODE_AND_MIXED)
def test_workload_extra_seeds(name, extra):
    """Each decode / mixed workload on three more seeds (auto path)."""
    kw = dict(WORKLOADS[name])
    kw["seed"] = kw["seed"] + extra
    case = make_case(**kw)
    print(f"[case] {name} seed={kw['seed']}", flush=True)
    ref, ref_lse = oracle.attention(**case)
    got, lse, plan = run(case, lse=True)
    err = compare(case, got, ref, label=f"{name}/seed{kw['seed']}")
    check_lse(lse, ref_lse, case, label=name)
    print(f"[ok] {name} seed={kw['seed']} max_abs={err:.3e}", flush=True)


@pytest.mark.parametrize("extra", [1000, 2000, 3000])
@pytest.mark.parametrize("name", PREFILL)
def test_prefill_extra_seeds(name, extra):
    """Three more seeds per prefill workload: the first and last row of every
    query block the planned kernel cuts, plus random rows."""
    kw = dict(WORKLOADS[name])
    kw["seed"] = kw["seed"] + extra
    case = make_case(**kw)
    print(f"[case] {name} seed={kw['seed']}", flush=True)
    got, lse, plan = run(case, lse=True)
    rows = np.union1d(block_edge_rows(case, plan.block_q),
                      sample_rows(case["q"].shape[0], 24, seed=extra))
    ref, ref_lse = oracle_parallel(case, rows)
    assert np.isfinite(got).all(), "unwritten or NaN output rows"
    err = compare(case, got, ref, rows=rows, label=f"{name}/seed{kw['seed']}")
    check_lse(lse[rows], ref_lse, case, label=name)
    print(f"[ok] {name} seed={kw['seed']} rows={len(rows)} max_abs={err:.3e}", flush=True)


NEXT_DECODE = NEXT_DECODE_WORKLOADS
NEXT_PREFILL = NEXT_PREFILL_WORKLOADS


@pytest.mark.parametrize("path,n_part", [("auto", 0), ("2d", 0), ("splitkv", 4)])
@pytest.mark.parametrize("name", NEXT_DECODE)
def test_next_decode_workloads(name, path, n_part):
    """64K-context, MQA (G = 32, large-block kernel), d256 and block-size-64 decode."""
    case, ref, ref_lse = _workload(name)
    print(f"[case] {name} path={path} n_part={n_part}", flush=True)
    got, lse, plan = run(case, _dev(name), path=path, n_part=n_part, lse=True)
    err = compare(case, got, ref, label=f"{name}/{path}{n_part}")
    check_lse(lse, ref_lse, case, label=name)
    print(f"[ok] {name} kernel={plan.kernel} path={plan.path} n_part={plan.n_part} "
          f"max_abs={err:.3e}", flush=True)


@pytest.mark.parametrize("name", NEXT_PREFILL)
def test_next_prefill_workloads(name):
    """d64 / block 32 / GQA-8 chunked prefill with sinks and window 128, and the
    bf16-Q + fp8-KV variants: every output element, planned path and a
    two-partition split."""
    print(f"[case] {name} oracle (all rows)", flush=True)
    case, ref, ref_lse = _workload_full(name)
    dev = to_device(case)
    for path, n_part in (("auto", 0), ("splitkv", 2)):
        print(f"[case] {name} path={path} n_part={n_part}", flush=True)
        got, lse, plan = run(case, dev, path=path, n_part=n_part, lse=True)
        err = compare(case, got, ref, label=f"{name}/{path}{n_part}")
        check_lse(lse, ref_lse, case, label=name)
        print(f"[ok] {name} path={plan.path} max_abs={err:.3e}", flush=True)


# ----------------------------------------------------------------------------- edge cases

def _check(case, path="auto", n_part=0, lse=True, label=""):
    ref, ref_lse = oracle.attention(**case)
    got, l, plan = run(case, path=path, n_part=n_part, lse=lse)
    err = compare(case, got, ref, label=label)
    if lse:
        check_lse(l, ref_lse, case, label=label)
    return err, plan


BASE = dict(head_dim=128, num_q_heads=16, num_kv_heads=2, block_size=16, q_dtype="bf16")
MIXED_SEQS = [(1, 300), (17, 90), (0, 12), (40, 40), (1, 1), (33, 700)]


@pytest.mark.parametrize("path,n_part", [("2d", 0), ("splitkv", 5)])
def test_empty_sequences(path, n_part):
    case = make_case(seqs=[(0, 0), (3, 10), (0, 7), (1, 1), (0, 0), (2, 40)], seed=11, **BASE)
    _check(case, path, n_part, label="empty")


@pytest.mark.parametrize("window", [1, 17, 100])
@pytest.mark.parametrize("path,n_part", [("2d", 0), ("splitkv", 3)])
def test_windows(window, path, n_part):
    case = make_case(seqs=MIXED_SEQS, window=window, seed=12 + window, **BASE)
    _check(case, path, n_part, label=f"w{window}")


@pytest.mark.parametrize("bs", [1, 3, 13, 32, 784])
@pytest.mark.parametrize("path,n_part", [("2d", 0), ("splitkv", 4)])
def test_block_sizes(bs, path, n_part):
    case = make_case(seqs=MIXED_SEQS, seed=20 + bs, **dict(BASE, block_size=bs))
    _check(case, path, n_part, label=f"bs{bs}")


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("dt,kvd", [("f16", "f16"), ("bf16", "bf16"), ("bf16", "e4m3fn"),
                                     ("f16", "e4m3fn"), ("bf16", "e4m3fnuz"),
                                     ("f16", "e4m3fnuz")])
def test_head_dims_and_dtypes(D, dt, kvd):
    case = make_case(seqs=MIXED_SEQS, seed=30 + D, **dict(BASE, head_dim=D, q_dtype=dt,
                                                           kv_dtype=kvd))
    _check(case, "auto", 0, label=f"D{D}-{dt}-{kvd}")
    _check(case, "splitkv", 3, label=f"D{D}-{dt}-{kvd}-split")


# Decode-shaped batch (q_len * G <= 16: the small-block kernel).
DECODE_SEQS = [(1, 300), (2, 90), (0, 12), (1, 1), (1, 700), (2, 33), (1, 1500)]


@pytest.mark.parametrize("bs", [13, 16, 32])
@pytest.mark.parametrize("shape", ["decode", "mixed"])
@pytest.mark.parametrize("kvd", ["e4m3fn", "e4m3fnuz"])
def test_per_token_scales(kvd, shape, bs):
    """Per-token K/V scales (K and V arrays with different strides), both dialects,
    both kernels, paged (bs 16, 32) and unaligned (bs 13) block sizes; scales of
    unused slots are NaN."""
    seqs = DECODE_SEQS if shape == "decode" else MIXED_SEQS
    case = make_case(seqs=seqs, seed=60 + bs + len(kvd), token_scales=True,
                     **dict(BASE, block_size=bs, kv_dtype=kvd))
    assert case["k_token_scales"].strides != case["v_token_scales"].strides
    for path, n_part in [("2d", 0), ("splitkv", 3), ("auto", 0)]:
        _, plan = _check(case, path, n_part, label=f"{kvd}-{shape}-bs{bs}-{path}{n_part}")
        assert (plan.kernel == 0) == (shape == "decode")


@pytest.mark.parametrize("D", [64, 256])
@pytest.mark.parametrize("kvd", ["e4m3fn", "e4m3fnuz"])
def test_per_token_scales_head_dims(kvd, D):
    for seqs, name in [(DECODE_SEQS, "decode"), (MIXED_SEQS, "mixed")]:
        case = make_case(seqs=seqs, seed=70 + D, token_scales=True,
                         **dict(BASE, head_dim=D, kv_dtype=kvd, q_dtype="f16"))
        _check(case, "auto", 0, label=f"{kvd}-D{D}-{name}")
        _check(case, "splitkv", 2, label=f"{kvd}-D{D}-{name}-split")


@pytest.mark.parametrize("kvd", ["e4m3fn", "e4m3fnuz"])
def test_per_token_scales_with_features(kvd):
    """Window, sinks, softcap, ALiBi and QQ-bias together with per-token scales."""
    for seqs in (DECODE_SEQS, [(1, 4), (3, 6), (2, 300), (5, 60), (64, 200)]):
        for kw in [dict(window=17, sinks=True), dict(softcap=3.0, alibi=True),
                   dict(qq_bias=128, window=40)]:
            case = make_case(seqs=seqs, seed=80, token_scales=True,
                             **dict(BASE, kv_dtype=kvd), **kw)
            _check(case, "2d", 0, label=f"{kvd}-{kw}")
            _check(case, "splitkv", 4, label=f"{kvd}-{kw}-split")


def test_per_token_tile_ring_lengths():
    """Large-kernel scale ring (three slots, filled two tiles ahead) over partitions
    of 1 .. 6 tiles and a window that starts mid-tile."""
    for kv, w in [(64, 0), (128, 0), (192, 0), (380, 0), (700, 150)]:
        case = make_case(seqs=[(40, kv), (64, kv + 3)], seed=90 + kv, token_scales=True,
                         window=w, **dict(BASE, kv_dtype="e4m3fnuz"))
        for n_part in (1, 2, 3):
            path = "2d" if n_part == 1 else "splitkv"
            _check(case, path, n_part, label=f"kv{kv}-w{w}-p{n_part}")


def test_deep_copy_ring_tile_counts():
    """16-bit K/V copy ring (two deep for D = 256, four deep for 256-row
    blocks): key ranges and partitions of 1 .. 7 tiles (copies still in flight
    when a partition ends)."""
    for kv in (20, 40, 70, 100, 130, 200):  # D = 256: 32-key tiles
        case = make_case(seqs=[(17, kv), (5, kv + 9)], seed=100 + kv,
                         **dict(BASE, head_dim=256))
        _, plan = _check(case, "2d", 0, label=f"d256-kv{kv}")
        assert plan.kernel == 1
    case = make_case(seqs=[(300, 4400), (40, 4200)], seed=120, **BASE)
    for n_part in (1, 17, 33, 70):  # 256-row blocks, 64-key tiles
        path = "2d" if n_part == 1 else "splitkv"
        _, plan = _check(case, path, n_part, label=f"rows256-p{n_part}")
        assert plan.kernel == 2


def test_eight_wave_interval_schedule_tile_counts():
    """256-row blocks run their two wave halves half a tile apart (two barriers
    per tile, copies two tiles ahead): partitions of 1 .. 9 tiles, blocks whose
    last waves hold no rows, sinks, and a window that starts mid-tile."""
    case = make_case(seqs=[(300, 4400), (40, 4200), (0, 100), (257, 4097)], seed=130,
                     sinks=True, **BASE)
    for n_part in (1, 9, 13, 18, 23, 30, 45):
        path = "2d" if n_part == 1 else "splitkv"
        _, plan = _check(case, path, n_part, label=f"pp-p{n_part}")
        assert plan.kernel == 2
    case = make_case(seqs=[(300, 6000), (33, 5000)], seed=131, window=4100, **BASE)
    for n_part in (1, 3):
        path = "2d" if n_part == 1 else "splitkv"
        _, plan = _check(case, path, n_part, label=f"pp-w-p{n_part}")
        assert plan.kernel == 2


@pytest.mark.parametrize("D,dt", [(64, "bf16"), (128, "f16"), (64, "f16")])
def test_eight_wave_head_dims_and_dtypes(D, dt):
    """The 256-row (eight-wave) kernel for the other head dim and query dtype it
    is built for: one pass and split, with sinks and a short second sequence."""
    case = make_case(seqs=[(40, 4300), (3, 800)], seed=140 + D, sinks=True,
                     **dict(BASE, head_dim=D, q_dtype=dt))
    for path, n_part in (("2d", 0), ("splitkv", 3)):
        _, plan = _check(case, path, n_part, label=f"eight-d{D}-{dt}-{path}")
        assert plan.kernel == 2


@pytest.mark.parametrize("Hq,Hkv", [(24, 1), (32, 1), (64, 2)])
def test_wide_group_decode_head_groups(Hq, Hkv):
    """Decode with G > 16 runs as head groups of <= 16 rows on the small kernel;
    per-head sinks and ALiBi slopes catch a wrong head mapping."""
    seqs = [(1, 300), (1, 90), (0, 12), (1, 1), (1, 700), (1, 1500)]
    case = make_case(seqs=seqs, seed=130 + Hq, sinks=True, alibi=True, window=600,
                     **dict(BASE, num_q_heads=Hq, num_kv_heads=Hkv))
    for path, n_part in [("2d", 0), ("splitkv", 3), ("auto", 0)]:
        _, plan = _check(case, path, n_part, label=f"G{Hq // Hkv}-{path}{n_part}")
        assert plan.kernel == 0 and plan.grid_y > Hkv


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (6, 2), (24, 4), (32, 2), (8, 1)])
def test_group_sizes(Hq, Hkv):
    case = make_case(seqs=MIXED_SEQS, seed=40 + Hq, **dict(BASE, num_q_heads=Hq,
                                                            num_kv_heads=Hkv))
    _check(case, "2d", 0, label=f"G{Hq // Hkv}")
    _check(case, "splitkv", 4, label=f"G{Hq // Hkv}-split")


@pytest.mark.parametrize("path,n_part", [("2d", 0), ("splitkv", 3)])
def test_features_visible_at_tolerance(path, n_part):
    """Softcap 3, sinks on short sequences and ALiBi: each moves outputs >> tol."""
    seqs = [(1, 4), (3, 6), (2, 300), (5, 60)]
    for kw in [dict(softcap=3.0), dict(sinks=True), dict(alibi=True),
               dict(softcap=3.0, sinks=True, window=9)]:
        case = make_case(seqs=seqs, seed=50, **BASE, **kw)
        _check(case, path, n_part, label=str(kw))


@pytest.mark.parametrize("path,n_part", [("auto", 0), ("2d", 0), ("splitkv", 3)])
def test_qq_bias_scenario(path, n_part):
    """The README's QQ-bias prefill scenario (row stride 256) through both kernels."""
    case, ref, ref_lse = _workload("qq_bias_prefill_fp16_d128_16q2kv")
    print(f"[case] qq_bias path={path} n_part={n_part}", flush=True)
    got, lse, plan = run(case, _dev("qq_bias_prefill_fp16_d128_16q2kv"), path=path,
                         n_part=n_part, lse=True)
    compare(case, got, ref, label=f"qq/{path}{n_part}")
    check_lse(lse, ref_lse, case, label="qq")


@pytest.mark.parametrize("path,n_part", [("2d", 0), ("splitkv", 3)])
def test_qq_bias_with_other_features(path, n_part):
    """QQ-bias on decode rows (small kernel), mixed chunks and prefixes (large
    kernel), combined with ALiBi, softcap, sinks and a window, bf16 and fp8 KV."""
    seqs = [(1, 40), (3, 6), (70, 300), (5, 60), (0, 9), (129, 129)]
    for kw in [dict(), dict(alibi=True, softcap=2.5), dict(sinks=True, window=50),
               dict(kv_dtype="e4m3fn", o_dtype="bf16", q_dtype="bf16")]:
        base = dict(BASE)
        base.update({k: v for k, v in kw.items() if k in ("q_dtype",)})
        rest = {k: v for k, v in kw.items() if k not in ("q_dtype",)}
        case = make_case(seqs=seqs, seed=51, qq_bias=160, **base, **rest)
        _check(case, path, n_part, label=f"qq+{kw}")
    dec = make_case(seqs=[(1, 700), (1, 33), (2, 90)], seed=52, qq_bias=8, **BASE)
    _check(dec, path, n_part, label="qq-decode")


@pytest.mark.parametrize("name", ["long_decode_bf16_d128_32q8kv_w4096_softcap_sinks",
                                  "decode_fp16_d128_16q2kv", "fp8kv_decode_b8_ctx6700_w4096"])
def test_split_partition_counts_agree(name):
    """Decode (small-block kernel): split-KV with any partition count equals one
    pass, each within tolerance of the oracle, and every pair of results within
    one output ULP (taken at max(|a|, |b|, 1e-3): the fp32 accumulation error is
    absolute at the scale of a row's partial sums, so near-zero outputs are held
    to the ULP at 1e-3, 7.6e-6 for bf16).  The kernel keeps running maxima
    integral, so the 16-bit rounding of p and every rescale are the same for
    any partitioning."""
    case, ref, _ = _workload(name)
    outs = {}
    for n in (1, 2, 4, 16, 31, 64):
        got, _, plan = run(case, _dev(name), path="splitkv", n_part=n)
        assert plan.kernel == 0
        compare(case, got, ref, label=f"{name}/split{n}")
        outs[f"split{n}"] = got
    outs["2d"], _, _ = run(case, _dev(name), path="2d")
    keys = list(outs)
    for i, a in enumerate(keys):
        for b in keys[i + 1:]:
            x, y = outs[a], outs[b]
            diff = np.abs(x - y)
            one = ulp(np.maximum(np.maximum(np.abs(x), np.abs(y)), 1e-3), case["o_dtype"])
            assert (diff <= one).all(), f"{a} vs {b}: {int((diff > one).sum())} elements " \
                                        f"differ by more than one ULP (max {diff.max():.3e})"


# Decode shapes with a multiple of four row blocks (kv heads x head groups),
# where the planner gives each wave its own row block: head dims 64 and 256,
# four-token query blocks (with a window; with a QQ-bias), fp8 with per-token
# scales and a softcap, 64 query heads over 2 kv heads (two head groups of 32
# each -> 4 row blocks), and a batch whose row blocks fill the device four
# times over (planned one-pass).
WAVE_ROW_CASES = {
    "d64_bf16_32q8kv_bs32_sinks": dict(
        seqs=None, num_seqs=6, q_len=1, kv_range=(2500, 3100), head_dim=64, num_q_heads=32,
        num_kv_heads=8, block_size=32, q_dtype="bf16", sinks=True, seed=301),
    "d256_fp16_16q4kv_alibi": dict(
        seqs=None, num_seqs=4, q_len=1, kv_range=(1800, 2200), head_dim=256, num_q_heads=16,
        num_kv_heads=4, block_size=16, q_dtype="f16", alibi=True, seed=302),
    "q4_bf16_32q8kv_window2000": dict(
        seqs=None, num_seqs=8, q_len=4, kv_range=(3000, 3500), head_dim=128, num_q_heads=32,
        num_kv_heads=8, block_size=16, q_dtype="bf16", window=2000, seed=303),
    "fnuz_pertoken_softcap": dict(
        seqs=None, num_seqs=4, q_len=1, kv_range=(2000, 2600), head_dim=128, num_q_heads=32,
        num_kv_heads=8, block_size=32, q_dtype="bf16", kv_dtype="e4m3fnuz", o_dtype="bf16",
        token_scales=True, softcap=30.0, seed=304),
    "e4m3fn_64q2kv": dict(
        seqs=None, num_seqs=8, q_len=1, kv_range=(1400, 1700), head_dim=128, num_q_heads=64,
        num_kv_heads=2, block_size=16, q_dtype="bf16", kv_dtype="e4m3fn", o_dtype="bf16",
        seed=305),
    "q4_qqbias_bf16_32q8kv": dict(
        seqs=None, num_seqs=8, q_len=4, kv_range=(2000, 2600), head_dim=128, num_q_heads=32,
        num_kv_heads=8, block_size=16, q_dtype="bf16", qq_bias=True, seed=306),
    # 160 sequences x 8 kv heads = 1280 row blocks, over four per CU: one pass
    "b160_onepass_bf16_32q8kv": dict(
        seqs=None, num_seqs=160, q_len=1, kv_range=(300, 500), head_dim=128, num_q_heads=32,
        num_kv_heads=8, block_size=16, q_dtype="bf16", seed=307),
}


@functools.lru_cache(maxsize=2)
def _wave_row_case(name):
    case = make_case(**WAVE_ROW_CASES[name])
    ref, lse = oracle.attention(**case)
    return case, ref, lse, to_device(case)


def _set_flag4(plan):
    plan.flags |= 4


def _clear_flag4(plan):
    plan.flags &= ~4


@pytest.mark.parametrize("name", list(WAVE_ROW_CASES))
def test_wave_per_row_block_matches_shared_row_block(name):
    """A wave per row block (plan flag bit 2) and four waves per row block give
    results within tolerance of the oracle and within one output ULP of each
    other, one-pass and split; the planner picks the former for these shapes."""
    case, ref, ref_lse, dev = _wave_row_case(name)
    outs = {}
    got, lse, plan = run(case, dev, lse=True)
    assert plan.kernel == 0 and plan.flags & 4
    compare(case, got, ref, label=f"{name}/auto-wave")
    check_lse(lse, ref_lse, case=case, label=f"{name}/auto-wave")
    outs["auto-wave"] = got
    for label, path, n, edit in (("auto-shared", "auto", 0, _clear_flag4),
                                 ("split5-wave", "splitkv", 5, _set_flag4),
                                 ("split5-shared", "splitkv", 5, _clear_flag4),
                                 ("2d-wave", "2d", 0, _set_flag4),
                                 ("2d-shared", "2d", 0, _clear_flag4)):
        got, lse, plan = run(case, dev, path=path, n_part=n, lse=True, plan_edit=edit)
        assert bool(plan.flags & 4) == (edit is _set_flag4)
        compare(case, got, ref, label=f"{name}/{label}")
        check_lse(lse, ref_lse, case=case, label=f"{name}/{label}")
        outs[label] = got
    keys = list(outs)
    for i, a in enumerate(keys):
        for b in keys[i + 1:]:
            x, y = outs[a], outs[b]
            diff = np.abs(x - y)
            one = ulp(np.maximum(np.maximum(np.abs(x), np.abs(y)), 1e-3), case["o_dtype"])
            assert (diff <= one).all(), f"{a} vs {b}: {int((diff > one).sum())} elements " \
                                        f"differ by more than one ULP (max {diff.max():.3e})"


@pytest.mark.parametrize("factor", [8.0, 1.5])
@pytest.mark.parametrize("q_dtype", ["bf16", "f16"])
def test_d256_held_maximum_second_pass(q_dtype, factor):
    """Head dim 256 (four-wave groups hold each row's running maximum instead
    of rescaling O, and run the tiles again when a later tile exceeds it by
    more than 64 in base 2 for bf16, 15 for fp16).  One key is made `factor`
    x a query row: 8x scores ~128 natural units (~185 in base 2) above the
    row's first tile, past both spans, so its workgroup runs a second pass;
    1.5x scores ~24 (~35 in base 2), which bf16 carries in one pass (p up to
    2^35) and fp16 cannot (65504 < 2^16), so only fp16 runs the second pass.
    Every row, that one included, matches the oracle, one-pass and split."""
    case = make_case(seqs=[(200, 600)], head_dim=256, num_q_heads=8, num_kv_heads=2,
                     block_size=16, q_dtype=q_dtype, seed=401)
    q_bits = case["q"]
    k_bits = case["k_cache"]
    if q_dtype == "bf16":  # bf16 bits -> float32 and back (truncating; the
        # oracle reads the stored bits either way)
        qf = (q_bits[150, 0].astype(np.uint32) << 16).view(np.float32)
        kf = (np.float32(factor) * qf).astype(np.float32)
        kb = (kf.view(np.uint32) >> 16).astype(np.uint16)
    else:
        qf = q_bits[150, 0].view(np.float16).astype(np.float32)
        kb = (np.float32(factor) * qf).astype(np.float16).view(np.uint16)
    key = 500  # visible to query tokens 100.. (context 400)
    blk = int(case["block_table"][0][key // 16])
    k_bits[blk, key % 16, 0] = kb
    ref, ref_lse = oracle.attention(**case)
    dev = to_device(case)
    for path, n in (("auto", 0), ("2d", 0), ("splitkv", 3)):
        got, lse, plan = run(case, dev, path=path, n_part=n, lse=True)
        assert plan.kernel == 1
        label = f"d256-hold{factor:g}/{path}{n}"
        compare(case, got, ref, label=label)
        check_lse(lse, ref_lse, case=case, label=label)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("kvd", ["bf16", "e4m3fn"])
def test_four_wave_logit_forms(D, kvd):
    """The four-wave prefill kernel runs one tile loop per logit form (plain;
    ALiBi or QQ-bias without softcap; softcap): each form at head dims 64 and
    128, 16-bit and per-tensor fp8 caches, one pass and split."""
    seqs = [(150, 600), (37, 37), (70, 300)]
    forms = [dict(), dict(alibi=True), dict(qq_bias=256, window=90), dict(softcap=15.0),
             dict(softcap=15.0, alibi=True, sinks=True)]
    for i, kw in enumerate(forms):
        case = make_case(seqs=seqs, seed=170 + i,
                         **dict(BASE, head_dim=D, kv_dtype=kvd, q_dtype="bf16"), **kw)
        for path, n_part in (("2d", 0), ("splitkv", 2)):
            _, plan = _check(case, path, n_part, label=f"fw-D{D}-{kvd}-{i}-{path}{n_part}")
            assert plan.kernel == 1


@pytest.mark.parametrize("q_dtype,kvd", [("bf16", "bf16"), ("f16", "f16"), ("bf16", "e4m3fn")])
def test_d256_prefill_features(q_dtype, kvd):
    """Head dim 256 prefill (four-wave groups: held running maximum, key ranges
    walked backwards from the diagonal) with a window that starts mid-tile,
    softcap with sinks, ALiBi (alone and with window and sinks) and QQ-bias,
    16-bit and per-tensor fp8 caches, one pass and split."""
    seqs = [(200, 700), (37, 37), (90, 400)]
    for i, kw in enumerate([dict(window=100), dict(softcap=20.0, sinks=True), dict(alibi=True),
                            dict(alibi=True, window=70, sinks=True), dict(qq_bias=256)]):
        case = make_case(seqs=seqs, seed=160 + i,
                         **dict(BASE, head_dim=256, num_q_heads=8, q_dtype=q_dtype,
                                kv_dtype=kvd), **kw)
        for path, n_part in (("2d", 0), ("splitkv", 3)):
            _, plan = _check(case, path, n_part, label=f"d256-{q_dtype}-{kvd}-{i}-{path}{n_part}")
            assert plan.kernel == 1


@pytest.mark.parametrize("token_scale_mult", [None, 1.0, 4.0])
def test_d256_held_maximum_fp8_cache(token_scale_mult):
    """The held maximum of the head-dim-256 prefill kernel with fp8 caches
    (staged through registers; per-token scales multiply S and P).  Key 500
    of kv head 0 is planted as the largest e4m3 code with the sign of each
    element of query row 150, head 0.  Per-tensor scale (None): it scores ~86
    in base 2 against the row's first tile (the one holding its diagonal,
    ~3), past the 64 a bf16 P holds,
    so the workgroup runs a second pass.  Per-token scales: with the key's own
    scale (1.0) it scores ~51, held in one pass with p up to ~2^48; with that
    scale x4 it scores ~205 and forces the second pass.  Outputs and LSE
    match the oracle on auto, one-pass and split-3 paths."""
    tok = token_scale_mult is not None
    case = make_case(seqs=[(200, 600)], head_dim=256, num_q_heads=8, num_kv_heads=2,
                     block_size=16, q_dtype="bf16", kv_dtype="e4m3fn", token_scales=tok,
                     seed=403 if tok else 402)
    q = oracle.decode(case["q"][150, 0], "bf16")
    key = 500  # visible to query tokens 100.. (context 400)
    blk = int(case["block_table"][0][key // 16])
    case["k_cache"][blk, key % 16, 0] = np.where(q >= 0, 0x7E, 0xFE).astype(np.uint8)
    if tok:
        case["k_token_scales"][blk, key % 16, 0] *= np.float32(token_scale_mult)

    def k_row(k):
        b = int(case["block_table"][0][k // 16])
        s = case["k_token_scales"][b, k % 16, 0] if tok else case["k_scale"]
        return oracle.decode(case["k_cache"][b, k % 16, 0], "e4m3fn") * np.float64(s)

    # The kernel walks each range backwards from the tile holding the diagonal:
    # row 150 (position 550) first sees keys 544..550 of the 32-key tile 544.
    c2 = case["scale"] / math.log(2.0)
    pos = 400 + 150
    first = max(float(q @ k_row(k)) * c2 for k in range(pos - pos % 32, pos + 1))
    excess = float(q @ k_row(key)) * c2 - first
    assert (excess > 64.0) == (token_scale_mult != 1.0), excess
    ref, ref_lse = oracle.attention(**case)
    dev = to_device(case)
    for path, n in (("auto", 0), ("2d", 0), ("splitkv", 3)):
        got, lse, plan = run(case, dev, path=path, n_part=n, lse=True)
        assert plan.kernel == 1
        label = f"d256-hold-fp8-{token_scale_mult}/{path}{n}"
        compare(case, got, ref, label=label)
        check_lse(lse, ref_lse, case=case, label=label)


@pytest.mark.parametrize("num_short", [40, 100, 4200])
def test_large_block_sequence_search(num_short):
    """Large-block launches that locate each workgroup's sequence by a search
    over the query offsets (neither one block per sequence nor rank order: one
    200-token chunk among 40, 100 or 4200 chunks of 1-3 tokens); every
    sequence's rows match the oracle."""
    rng = np.random.default_rng(7000 + num_short)
    seqs = [(int(q), int(q + rng.integers(0, 48))) for q in rng.integers(1, 4, num_short)]
    seqs.insert(num_short // 2, (200, 300))
    case = make_case(seqs=seqs, head_dim=64, num_q_heads=8, num_kv_heads=1, block_size=16,
                     q_dtype="f16", seed=7100 + num_short)
    ref, _ = oracle.attention(**case)
    got, _, plan = run(case, path="2d")
    assert plan.kernel in (1, 2) and (plan.flags & 3) == 0, (plan.kernel, plan.flags)
    compare(case, got, ref, label=f"seq-search-{num_short}")


def test_nan_workspace_not_read():
    case, ref, _ = _workload("fp8kv_decode_b8_ctx6700_w4096")
    dev = _dev("fp8kv_decode_b8_ctx6700_w4096")
    ws = torch.full((64 << 20,), 0xFF, dtype=torch.uint8, device="cuda")  # NaN bytes
    got, _, _ = run(case, dev, path="splitkv", n_part=16, ws=ws)
    compare(case, got, ref, label="nan-ws")


def test_repeat_is_bit_identical():
    case, _, _ = _workload("mixed_fp16_d128_16q2kv")
    dev = _dev("mixed_fp16_d128_16q2kv")
    a, _, _ = run(case, dev, path="splitkv", n_part=5)
    b, _, _ = run(case, dev, path="splitkv", n_part=5)
    assert np.array_equal(a, b)
    c, _, _ = run(case, dev, path="2d")
    d, _, _ = run(case, dev, path="2d")
    assert np.array_equal(c, d)


@pytest.mark.parametrize("path,n_part", [("2d", 0), ("splitkv", 4)])
def test_graph_capture_replays(path, n_part):
    """One forward (split: partition kernel + reduce) captured in a HIP graph and
    replayed several times, with eager work and an input change in between:
    every replay equals an eager run on the same inputs, bit for bit."""
    import paged_varlen_attention_ua_amd.attention as A
    case, ref, _ = _workload("long_decode_bf16_d128_32q8kv_w4096_softcap_sinks")
    d = {k: (v.clone() if v is not None else None)
         for k, v in _dev("long_decode_bf16_d128_32q8kv_w4096_softcap_sinks").items()}
    kw = dict(max_seqlen_q=case["max_seqlen_q"], max_seqlen_k=case["max_seqlen_k"],
              scale=case["scale"], softcap=case["softcap"], window=case["window"],
              sinks=d["sinks"], path=path, n_part=n_part)
    args = (d["q"], d["k_cache"], d["v_cache"], d["block_table"], d["cu_seqlens_q"],
            d["seq_lens"])
    out = torch.full_like(d["q"], float("nan"))
    ws = torch.empty(64 << 20, dtype=torch.uint8, device=d["q"].device)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        A.forward(*args, out=out, ws=ws, **kw)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        A.forward(*args, out=out, ws=ws, **kw)
    q0 = d["q"].clone()
    for rep in range(3):
        if rep == 2:
            d["q"].copy_(torch.flip(q0, dims=[0]))  # new inputs, same buffers
        out.fill_(float("nan"))
        junk = torch.randn(1 << 20, device=d["q"].device).sum()  # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        eager = torch.full_like(out, float("nan"))
        A.forward(*args, out=eager, **kw)
        torch.cuda.synchronize()
        assert torch.equal(got, eager), f"replay {rep} differs from eager"
        if rep < 2:
            compare(case, got.float().cpu().numpy().astype(np.float64), ref,
                    label=f"graph replay {rep}")
        assert torch.isfinite(junk)


def test_check_inputs_reports_each_violation():
    """ua_check_inputs: valid inputs give no bits; each broken precondition sets
    its bit (the forward is never run on the broken inputs)."""
    import paged_varlen_attention_ua_amd.attention as A
    base = make_case(seqs=MIXED_SEQS, seed=140, **BASE)

    def check(case, **over):
        d = to_device(case)
        kw = dict(max_seqlen_q=case["max_seqlen_q"], max_seqlen_k=case["max_seqlen_k"])
        kw.update(over)
        return A.check_inputs(d["q"], d["k_cache"], d["v_cache"], d["block_table"],
                              d["cu_seqlens_q"], d["seq_lens"], **kw)

    assert check(base) == set()
    c = dict(base, cu_seqlens_q=base["cu_seqlens_q"].copy())
    c["cu_seqlens_q"][2] = c["cu_seqlens_q"][1] - 1
    assert "cu_seqlens_q" in check(c)
    assert check(base, max_seqlen_q=base["max_seqlen_q"] - 1) == {"q_len"}
    c = dict(base, seq_lens=base["seq_lens"].copy())
    c["seq_lens"][1] = 16  # sequence 1 has 17 queries
    assert check(c) == {"kv_len"}
    assert check(base, max_seqlen_k=base["max_seqlen_k"] - 1) == {"kv_len"}
    for bad in (base["k_cache"].shape[0], -1):
        c = dict(base, block_table=base["block_table"].copy())
        c["block_table"][5, 2] = bad  # a block sequence 5 (700 keys) uses
        assert check(c) == {"block_table"}
    c = dict(base, block_table=base["block_table"].copy())
    c["block_table"][0, -1] = -7  # padding column: not used by any sequence
    assert check(c) == set()


def test_two_streams_separate_workspaces():
    import paged_varlen_attention_ua_amd.attention as A
    c1, r1, _ = _workload("long_decode_bf16_d128_32q8kv_w4096")
    c2, r2, _ = _workload("long_decode_bf16_d128_32q8kv_w4096_softcap_sinks")
    d1, d2 = _dev("long_decode_bf16_d128_32q8kv_w4096"), \
        _dev("long_decode_bf16_d128_32q8kv_w4096_softcap_sinks")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for c, d, s in ((c1, d1, s1), (c2, d2, s2)):
        with torch.cuda.stream(s):
            o = torch.full_like(d["q"], float("nan"))
            A.forward(d["q"], d["k_cache"], d["v_cache"], d["block_table"], d["cu_seqlens_q"],
                      d["seq_lens"], max_seqlen_q=c["max_seqlen_q"],
                      max_seqlen_k=c["max_seqlen_k"], scale=c["scale"], softcap=c["softcap"],
                      window=c["window"], sinks=d["sinks"], out=o, path="splitkv", n_part=16)
            outs.append(o)
    torch.cuda.synchronize()
    compare(c1, outs[0].float().cpu().numpy().astype(np.float64), r1, label="stream1")
    compare(c2, outs[1].float().cpu().numpy().astype(np.float64), r2, label="stream2")


def test_reduce_alone_matches_oracle_merge():
    """ua_reduce on random partition states equals the oracle's base-2 merge."""
    import paged_varlen_attention_ua_amd as U
    import paged_varlen_attention_ua_amd.attention as A
    case = make_case(seqs=[(3, 50), (1, 20), (2, 9)], seed=60, sinks=True, **BASE)
    dev = to_device(case)
    P = 6
    prob = A.make_problem(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_table"],
                          num_seqs=3, max_seqlen_q=3, max_seqlen_k=50, scale=case["scale"],
                          sinks=dev["sinks"])
    plan = U.ua_plan(prob, 256, U.UA_PATH_SPLITKV, P)
    R = case["q"].shape[0] * 16
    rng = np.random.default_rng(0)
    m2 = rng.standard_normal((P, R)).astype(np.float32) * 4
    l = rng.uniform(0.5, 30, (P, R)).astype(np.float32)
    l[rng.random((P, R)) < 0.3] = 0.0
    l[:, 5] = 0.0  # a row no partition saw
    acc = rng.standard_normal((P, R, 128)).astype(np.float32) * 5
    ws = torch.full((plan.workspace_bytes,), 0xFF, dtype=torch.uint8, device="cuda")
    wf = ws.view(torch.float32)
    wf[:P * R] = torch.from_numpy(m2.ravel()).cuda()
    wf[P * R:2 * P * R] = torch.from_numpy(l.ravel()).cuda()
    off = U.ua_workspace_acc_offset(prob, plan) // 4
    acc_dev = torch.from_numpy(np.where(l[..., None] > 0, acc, np.nan).astype(np.float32).ravel())
    wf[off:off + P * R * 128] = acc_dev.cuda()
    out = torch.full_like(dev["q"], float("nan"))
    lse = torch.full((R,), float("nan"), dtype=torch.float32, device="cuda")
    args = A.make_args(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_table"],
                       dev["cu_seqlens_q"], dev["seq_lens"], out, lse=lse, sinks=dev["sinks"])
    U.ua_reduce(prob, plan, args, ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    sinks = np.tile(case["sinks"].astype(np.float64), R // 16)
    o_ref, lse_ref = oracle.merge_partials_base2(m2, l, acc, sinks)
    got = out.float().cpu().numpy().reshape(R, 128).astype(np.float64)
    compare(case, got, o_ref, label="reduce")
    check_lse(lse.cpu().numpy().astype(np.float64), lse_ref, case, label="reduce-lse")


def test_cache_offsets_beyond_2gib():
    """Blocks placed past 2 GiB of cache: 64-bit block offsets (README 64-bit addressing)."""
    case = make_case(seqs=[(1, 700), (5, 64), (1, 33)], seed=70, **dict(BASE, num_kv_heads=2))
    ref, _ = oracle.attention(**case)
    dev = to_device(case)
    nb_small, bs, hk, d = case["k_cache"].shape
    block_bytes = bs * hk * d * 2
    shift = (3 << 30) // block_bytes  # 3 GiB into the cache
    big_nb = shift + nb_small
    kc = torch.full((big_nb, bs, hk, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    kc[shift:] = dev["k_cache"]
    vc[shift:] = dev["v_cache"]
    bt = dev["block_table"] + shift
    big = dict(dev, k_cache=kc, v_cache=vc, block_table=bt)
    for path, n in (("2d", 0), ("splitkv", 4)):
        got, _, _ = run(case, big, path=path, n_part=n)
        compare(case, got, ref, label=f"big-{path}")
    del kc, vc
    torch.cuda.empty_cache()


def test_strided_query_output_and_cache():
    """Q/O as views into wider buffers and a cache with padded head stride."""
    import paged_varlen_attention_ua_amd.attention as A
    case = make_case(seqs=MIXED_SEQS, seed=80, **BASE)
    ref, _ = oracle.attention(**case)
    dev = to_device(case)
    T, H, D = dev["q"].shape
    qbig = torch.zeros((T, H + 3, D + 8), dtype=dev["q"].dtype, device="cuda")
    qbig[:, :H, :D] = dev["q"]
    q = qbig[:, :H, :D]
    nb, bs, hk, _ = dev["k_cache"].shape
    kbig = torch.full((nb, bs, hk, D + 16), float("nan"), dtype=dev["q"].dtype, device="cuda")
    vbig = torch.full_like(kbig, float("nan"))
    kbig[..., :D] = dev["k_cache"]
    vbig[..., :D] = dev["v_cache"]
    obig = torch.full((T, H, D + 24), float("nan"), dtype=dev["q"].dtype, device="cuda")
    o = obig[:, :, :D]
    A.forward(q, kbig[..., :D], vbig[..., :D], dev["block_table"], dev["cu_seqlens_q"],
              dev["seq_lens"], max_seqlen_q=case["max_seqlen_q"],
              max_seqlen_k=case["max_seqlen_k"], scale=case["scale"], out=o, path="splitkv",
              n_part=3)
    torch.cuda.synchronize()
    compare(case, o.float().cpu().numpy().astype(np.float64), ref, label="strided")
    assert torch.isnan(obig[:, :, D:]).all(), "wrote outside the output view"


def test_large_kernel_block_table_beyond_staged_entries():
    """Large-block key ranges spanning more than the 2048 block-table entries a
    workgroup stages in LDS (block size 1): the rest are read from the table
    in memory.  Four-wave (128-row) and eight-wave (256-row) groups."""
    c4 = make_case(seqs=[(64, 3000), (5, 2100)], seed=150, **dict(BASE, block_size=1))
    c8 = make_case(seqs=[(300, 4400), (16, 2500)], seed=151, **dict(BASE, block_size=1))
    for case, kernel in ((c4, 1), (c8, 2)):
        for path, n_part in (("2d", 0), ("splitkv", 3)):
            _, plan = _check(case, path, n_part, label=f"bt-beyond-k{kernel}-{path}{n_part}")
            assert plan.kernel == kernel


def _hand_gpu_case(hc, inp, q_dtype, kv_dtype, D=64):
    """The hand-worked example of tests/golden/hand_example.json, head dim
    zero-padded to D (the padding adds nothing to any dot product or output
    column), paged through block table [2, 0] of four blocks whose blocks 1
    and 3 hold NaN."""
    import json
    import math
    import os

    from synth.workloads import _round_storage

    def val(x):
        if isinstance(x, (int, float)):
            return float(x)
        return float(eval(x, {"ln2": math.log(2), "ln3": math.log(3), "ln4": math.log(4),
                              "log2": math.log2}))

    gqa = hc.get("gqa", False)
    q2 = np.array(inp["q_gqa"] if gqa else inp["q"], dtype=np.float32)
    H = q2.shape[0]
    q = np.zeros((1, H, D), np.float32)
    q[0, :, :2] = q2
    nb = inp["num_blocks"]
    kc = np.full((nb, 1, 1, D), np.nan, np.float32)
    vc = np.full((nb, 1, 1, D), np.nan, np.float32)
    for j, b in enumerate(inp["block_table"]):
        kc[b, 0, 0] = 0.0
        vc[b, 0, 0] = 0.0
        kc[b, 0, 0, :2] = inp["keys"][j]
        vc[b, 0, 0, :2] = inp["values"][j]
    nan = {"f16": 0x7E00, "bf16": 0x7FC0, "e4m3fn": 0x7F, "e4m3fnuz": 0x80}[kv_dtype]
    kb, vb = _round_storage(kc, kv_dtype), _round_storage(vc, kv_dtype)
    for b in inp["nan_blocks"]:
        kb[b] = nan
        vb[b] = nan
    case = dict(q=_round_storage(q, q_dtype), k_cache=kb, v_cache=vb,
                block_table=np.array([inp["block_table"] + [1]], dtype=np.int32),
                cu_seqlens_q=np.array([0, 1], dtype=np.int32),
                seq_lens=np.array([2], dtype=np.int32), q_dtype=q_dtype, kv_dtype=kv_dtype,
                o_dtype=q_dtype, block_size=1, head_dim=D, num_q_heads=H, num_kv_heads=1,
                scale=val(hc.get("scale", "ln3")), window=int(hc.get("window", 0)),
                softcap=val(hc["softcap"]) if "softcap" in hc else 0.0,
                alibi_slopes=(np.full(H, val(hc["alibi"]), np.float32) if "alibi" in hc
                              else None),
                sinks=np.full(H, val(hc["sink"]), np.float32) if "sink" in hc else None,
                qq_bias=None, k_scale=1.0, v_scale=1.0, k_token_scales=None,
                v_token_scales=None, max_seqlen_q=1, max_seqlen_k=2)
    exp = np.zeros((1, H, D))
    exp[0, :, :2] = np.array(hc["out"], dtype=np.float64).reshape(H, 2)
    lse = math.log(val(hc["lse"].replace("ln", ""))) if "lse" in hc else None
    return case, exp, lse


@pytest.mark.parametrize("dts", [("f16", "f16"), ("bf16", "bf16"), ("bf16", "e4m3fn"),
                                 ("f16", "e4m3fnuz")])
@pytest.mark.parametrize("name", ["plain", "sink", "window1", "window2", "alibi", "softcap",
                                  "gqa"])
def test_hand_example_on_gpu(name, dts):
    """The hand-worked example (exact in every storage type) through the one-pass
    and the split path (two partitions: keys 0 and 1 in the first, the second
    empty, so the reduce also merges an empty partition), against the values
    derived by hand, not the oracle."""
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_example.json")))
    hc = next(c for c in g["cases"] if c["name"] == name)
    case, exp, lse_exp = _hand_gpu_case(hc, g["inputs"], *dts)
    for path, n_part in (("2d", 0), ("splitkv", 2)):
        got, lse, _ = run(case, path=path, n_part=n_part, lse=True)
        compare(case, got, exp, label=f"hand-{name}-{dts[0]}-{dts[1]}/{path}")
        if lse_exp is not None:
            check_lse(lse[:, :1], np.array([[lse_exp]]), case, label=f"hand-{name}-lse")


@pytest.mark.parametrize("seqs,kw", [
    ([(100, 100), (32, 32)], {}),
    ([(33, 40), (64, 64), (5, 9), (31, 31)], {}),
    ([(300, 300), (129, 200)], dict(window=64)),
    ([(100, 100), (100, 150), (32, 32), (64, 64), (31, 31), (100, 100)], dict(sinks=True)),
    ([(120, 130), (97, 97)], dict(head_dim=256)),
    ([(300, 4400), (300, 4300)], {}),  # 256-row (eight-wave) blocks
])
def test_rank_order_batches(seqs, kw):
    """Large blocks dispatched in rank order (heaviest block of every sequence
    first; forced here by planning for a one-CU device): one pass and split."""
    case = make_case(seqs=seqs, seed=160 + len(seqs), **dict(BASE, **kw))
    ref, ref_lse = oracle.attention(**case)
    for path, n_part in (("2d", 0), ("splitkv", 3)):
        got, lse, plan = run(case, path=path, n_part=n_part, lse=True, num_cus=1)
        assert plan.kernel != 0 and plan.flags & 2, (plan.kernel, plan.flags)
        compare(case, got, ref, label=f"rank-{len(seqs)}-{path}")
        check_lse(lse, ref_lse, case, label="rank")
