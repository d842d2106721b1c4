"""Helpers shared by the GPU parity tests and smoke(): upload a seeded case,
run it through the C ABI, compare with the oracle.

Parity gate (max-abs against the float64 oracle; fp8 KV against the oracle on
the dequantised cache, either e4m3 dialect): fp16 2e-3, bf16 1e-2, fp8 KV 2e-2,
element by element.  One allowance: an element whose output type is bf16 and
whose oracle value has |o| >= 2 may additionally differ by half a bf16 unit in
the last place at that value (7.8e-3 on [2, 4), 1.56e-2 on [4, 8)).  That is the
error of rounding the exact value once to bf16, which no kernel can avoid, and
at |o| >= 4 it exceeds the 1e-2 gate on its own.  Every element that needed the
allowance is counted; fp16 outputs (half-ULP <= 1.95e-3 below 8) and bf16
outputs below 2 get no allowance.

Every comparison is recorded in RECORDS (label, max-abs, elements, elements
that needed the allowance); tests/conftest.py prints a per-workload summary at
the end of the pytest run.
"""

import math
import os

import numpy as np
import torch

TOL = {"f16": 2e-3, "bf16": 1e-2, "e4m3fn": 2e-2, "e4m3fnuz": 2e-2}
_MANT = {"f16": 10, "bf16": 7}


def tolerance(case):
    kvd = case["kv_dtype"]
    return TOL[kvd] if kvd.startswith("e4m3") else TOL[case["q_dtype"]]


def half_ulp(ref, o_dtype):
    a = np.abs(ref)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -14 if o_dtype == "f16" else -126)
    return np.where(a > 0, 2.0 ** (e - _MANT[o_dtype] - 1), 0.0)


def _torch_bits(arr, dtype, device):
    t = torch.from_numpy(np.ascontiguousarray(arr))
    if dtype == "f16":
        return t.view(torch.int16).view(torch.float16).to(device)
    if dtype == "bf16":
        return t.view(torch.int16).view(torch.bfloat16).to(device)
    fp8 = torch.float8_e4m3fn if dtype == "e4m3fn" else torch.float8_e4m3fnuz
    return t.view(torch.uint8).view(fp8).to(device)


def _scales(arr, device):
    """Per-token scales with their numpy strides kept (a transposed view stays one)."""
    if arr is None:
        return None
    t = torch.from_numpy(arr).to(device)
    assert t.stride() == tuple(s // 4 for s in arr.strides)
    return t


def to_device(case, device="cuda"):
    d = dict(
        q=_torch_bits(case["q"], case["q_dtype"], device),
        k_cache=_torch_bits(case["k_cache"], case["kv_dtype"], device),
        v_cache=_torch_bits(case["v_cache"], case["kv_dtype"], device),
        block_table=torch.from_numpy(case["block_table"]).to(device),
        cu_seqlens_q=torch.from_numpy(case["cu_seqlens_q"]).to(device),
        seq_lens=torch.from_numpy(case["seq_lens"]).to(device),
        alibi_slopes=(None if case["alibi_slopes"] is None
                      else torch.from_numpy(np.asarray(case["alibi_slopes"], np.float32)).to(device)),
        sinks=(None if case["sinks"] is None
               else torch.from_numpy(np.asarray(case["sinks"], np.float32)).to(device)),
        qq_bias=(None if case.get("qq_bias") is None
                 else torch.from_numpy(np.asarray(case["qq_bias"], np.float32)).to(device)),
        k_token_scales=_scales(case.get("k_token_scales"), device),
        v_token_scales=_scales(case.get("v_token_scales"), device),
    )
    return d


def run(case, dev=None, path="auto", n_part=0, lse=False, poison_out=True, ws=None,
        out=None, num_cus=None, plan_edit=None):
    """Run one case on the GPU through the C ABI; returns (out fp64 numpy, lse, plan).
    plan_edit: optional function applied to the plan before the launches (the
    calls of attention.forward, made here so that a test can change the plan)."""
    import paged_varlen_attention_ua_amd.attention as A
    dev = dev or to_device(case)
    q = dev["q"]
    if out is None:
        out = torch.empty_like(q)
        if poison_out:
            out.fill_(float("nan"))
    lse_t = None
    if lse:
        lse_t = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device=q.device)
    if plan_edit is not None:
        o, plan = _forward_edited(case, dev, out, lse_t, path, n_part, ws, num_cus, plan_edit)
        torch.cuda.synchronize()
        res = o.float().cpu().numpy().astype(np.float64)
        l = lse_t.cpu().numpy().astype(np.float64) if lse_t is not None else None
        return res, l, plan
    o, plan = A.forward(q, dev["k_cache"], dev["v_cache"], dev["block_table"],
                        dev["cu_seqlens_q"], dev["seq_lens"],
                        max_seqlen_q=case["max_seqlen_q"], max_seqlen_k=case["max_seqlen_k"],
                        scale=case["scale"], softcap=case["softcap"], window=case["window"],
                        k_scale=case["k_scale"], v_scale=case["v_scale"],
                        alibi_slopes=dev["alibi_slopes"], sinks=dev["sinks"], out=out,
                        lse=lse_t, path=path, n_part=n_part, ws=ws, qq_bias=dev.get("qq_bias"),
                        k_token_scales=dev.get("k_token_scales"),
                        v_token_scales=dev.get("v_token_scales"), num_cus=num_cus)
    torch.cuda.synchronize()
    res = o.float().cpu().numpy().astype(np.float64)
    l = lse_t.cpu().numpy().astype(np.float64) if lse_t is not None else None
    return res, l, plan


RECORDS = []
BAND_MIN = 2.0  # |oracle| from which bf16 outputs get the half-ULP allowance


def _forward_edited(case, dev, out, lse_t, path, n_part, ws, num_cus, plan_edit):
    import ctypes
    import paged_varlen_attention_ua_amd.attention as A
    from paged_varlen_attention_ua_amd import binding as B
    q = dev["q"]
    prob = A.make_problem(q, dev["k_cache"], dev["v_cache"], dev["block_table"],
                          num_seqs=len(case["seq_lens"]), max_seqlen_q=case["max_seqlen_q"],
                          max_seqlen_k=case["max_seqlen_k"], scale=case["scale"],
                          softcap=case["softcap"], window=case["window"],
                          k_scale=case["k_scale"], v_scale=case["v_scale"],
                          alibi_slopes=dev["alibi_slopes"], sinks=dev["sinks"], out=out,
                          qq_bias=dev.get("qq_bias"), k_token_scales=dev.get("k_token_scales"),
                          v_token_scales=dev.get("v_token_scales"))
    path_code = {"auto": B.UA_PATH_AUTO, "2d": B.UA_PATH_2D, "splitkv": B.UA_PATH_SPLITKV}[path]
    plan = B.ua_plan(prob, num_cus if num_cus is not None else A.device_cus(q.device),
                     path_code, n_part)
    plan_edit(plan)
    args = A.make_args(q, dev["k_cache"], dev["v_cache"], dev["block_table"],
                       dev["cu_seqlens_q"], dev["seq_lens"], out, lse_t, dev["alibi_slopes"],
                       dev["sinks"], dev.get("qq_bias"), dev.get("k_token_scales"),
                       dev.get("v_token_scales"))
    sp = ctypes.c_void_p(torch.cuda.current_stream(q.device).cuda_stream)
    if plan.path == B.UA_PATH_2D:
        B.ua_forward_2d(prob, plan, args, sp)
    else:
        if ws is None:
            ws = torch.empty(max(int(plan.workspace_bytes), 256), dtype=torch.uint8,
                             device=q.device)
        B.ua_forward_splitkv(prob, plan, args, ctypes.c_void_p(ws.data_ptr()), ws.numel(), sp)
        B.ua_reduce(prob, plan, args, ctypes.c_void_p(ws.data_ptr()), ws.numel(), sp)
    return out, plan


def allowed_error(case, ref):
    """Per-element bound: the dtype's tolerance, plus half a bf16 ULP where the
    output is bf16 and |ref| >= 2 (the unavoidable rounding of the exact value)."""
    tol = tolerance(case)
    allowed = np.full(np.shape(ref), tol)
    if case["o_dtype"] == "bf16":
        band = np.abs(ref) >= BAND_MIN
        allowed = np.where(band, tol + half_ulp(ref, "bf16"), allowed)
    return allowed


def compare(case, got, ref, rows=None, label=""):
    """Assert |got - ref| <= allowed_error elementwise; record and return max-abs."""
    if rows is not None:
        got = got[rows]
    tol = tolerance(case)
    err = np.abs(got - ref)
    allowed = allowed_error(case, ref)
    bad = ~(err <= allowed)  # NaN counts as bad
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(
            f"{label}: {int(bad.sum())} elements outside tolerance {tol}; max err "
            f"{np.nanmax(err) if np.isfinite(err).any() else float('nan')}; first "
            f"{[(tuple(i), float(got[tuple(i)]), float(ref[tuple(i)])) for i in idx]}")
    max_abs = float(err.max()) if err.size else 0.0
    n_band = int(np.count_nonzero(err > tol))
    RECORDS.append(dict(label=label, max_abs=max_abs, n=int(err.size), n_band=n_band,
                        tol=tol, o_dtype=case["o_dtype"]))
    return max_abs


def ulp(x, o_dtype):
    """One unit in the last place of the output type at |x| (subnormal floor)."""
    return 2.0 * half_ulp(np.where(np.asarray(x) == 0, 1e-30, x), o_dtype)


def oracle_parallel(case, rows=None, chunk=256, workers=None):
    """The oracle on `rows` (default: all query rows), row chunks spread over
    host threads (every row is independent; numpy's elementwise work and BLAS
    release the GIL).  BLAS runs one thread per worker meanwhile."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    total_q = case["q"].shape[0]
    rows = np.arange(total_q) if rows is None else np.asarray(rows, dtype=np.int64)
    parts = [rows[i:i + chunk] for i in range(0, len(rows), chunk)]
    workers = workers or min(16, os.cpu_count() or 1, max(1, len(parts)))
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(1)
    except Exception:  # threadpoolctl missing: BLAS keeps its own threads
        limit = None
    try:
        with ThreadPoolExecutor(workers) as ex:
            res = list(ex.map(lambda r: oracle.attention(**case, rows=r), parts))
    finally:
        if limit is not None:
            limit.restore_original_limits()
    if not res:
        Hq, D = case["q"].shape[1:]
        return np.zeros((0, Hq, D)), np.zeros((0, Hq))
    return np.concatenate([o for o, _ in res]), np.concatenate([l for _, l in res])


def block_edge_rows(case, block_q):
    """First and last query row of every query block (blocks of block_q tokens
    inside each sequence, as the kernels cut them)."""
    cu = case["cu_seqlens_q"]
    out = []
    for s in range(len(cu) - 1):
        for t0 in range(int(cu[s]), int(cu[s + 1]), block_q):
            out += [t0, min(t0 + block_q, int(cu[s + 1])) - 1]
    return np.array(sorted(set(out)), dtype=np.int64)


def sample_rows(total_q, n, seed):
    """First, last and random query rows (sorted, unique) for full-size sampled parity."""
    rng = np.random.default_rng(seed)
    k = min(total_q, n)
    base = set(range(min(8, total_q))) | set(range(max(0, total_q - 8), total_q))
    base |= set(rng.choice(total_q, size=k, replace=False).tolist())
    return np.array(sorted(base), dtype=np.int64)


def lse_tolerance(case):
    """The kernels' log-sum-exp is that of the softmax weights as rounded to the
    query dtype for the P*V product (the normaliser the output is divided by):
    each weight carries at most half an ULP of relative error, 2^-8 for bf16 and
    2^-11 for fp16, so the log of their sum is within ln(1 + 2^-8) (resp.
    ln(1 + 2^-11)) of the exact value, plus 1e-4 for fp32 arithmetic."""
    return math.log1p(2.0 ** (-8 if case["q_dtype"] == "bf16" else -11)) + 1e-4


def check_lse(got, ref, case=None, label="", atol=None):
    """LSE (natural log, fp32 on the GPU): same -inf pattern, finite values within
    atol (default: lse_tolerance(case))."""
    if atol is None:
        atol = lse_tolerance(case)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isneginf(got), ~fin), f"{label}: -inf pattern of lse differs"
    err = np.abs(got[fin] - ref[fin]).max() if fin.any() else 0.0
    assert err <= atol, f"{label}: lse max err {err}"
    return float(err)
