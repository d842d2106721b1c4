"""ua_forward_noalloc (the split-KV workspace in the library's static device
array) against ua_forward with a caller workspace: two calls in a row, the
second on a smaller problem, each bit-identical to the workspace form (same
kernels, same inputs) and within tolerance of the float64 oracle; the
one-pass path; a plan too large for the array is refused before any launch.
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS, make_case
from tests.gpu_common import compare, to_device

pytestmark = pytest.mark.gpu


def _call(case, dev, path, n_part, noalloc):
    import paged_varlen_attention_ua_amd as U
    import paged_varlen_attention_ua_amd.attention as A
    out = torch.full_like(dev["q"], float("nan"))
    prob = A.make_problem(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_table"],
                          num_seqs=len(case["seq_lens"]), max_seqlen_q=case["max_seqlen_q"],
                          max_seqlen_k=case["max_seqlen_k"], scale=case["scale"],
                          softcap=case["softcap"], window=case["window"],
                          k_scale=case["k_scale"], v_scale=case["v_scale"],
                          alibi_slopes=dev["alibi_slopes"], sinks=dev["sinks"], out=out)
    force = {"auto": U.UA_PATH_AUTO, "2d": U.UA_PATH_2D, "splitkv": U.UA_PATH_SPLITKV}[path]
    plan = U.ua_plan(prob, A.num_cus(dev["q"].device), force, n_part)
    args = A.make_args(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_table"],
                       dev["cu_seqlens_q"], dev["seq_lens"], out,
                       alibi_slopes=dev["alibi_slopes"], sinks=dev["sinks"])
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    lib = U.lib()
    if noalloc:
        st = lib.ua_forward_noalloc(ctypes.byref(prob), ctypes.byref(plan), ctypes.byref(args),
                                    sp)
    else:
        ws = torch.full((max(int(plan.workspace_bytes), 256),), 0xFF, dtype=torch.uint8,
                        device=dev["q"].device)
        st = lib.ua_forward(ctypes.byref(prob), ctypes.byref(plan), ctypes.byref(args),
                            ctypes.c_void_p(ws.data_ptr()), ws.numel(), sp)
    torch.cuda.synchronize()
    return st, plan, out.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("path,n_part", [("auto", 0), ("splitkv", 7)])
def test_noalloc_matches_workspace_form(path, n_part):
    big = make_case(**WORKLOADS["long_decode_bf16_d128_32q8kv_w4096_softcap_sinks"])
    small = make_case(**WORKLOADS["decode_fp16_d128_16q2kv"])
    for name, case in (("long decode", big), ("decode", small)):  # second call: smaller
        print(f"[case] noalloc {name} path={path} n_part={n_part}", flush=True)
        dev = to_device(case)
        ref, _ = oracle.attention(**case)
        st_n, plan, got_n = _call(case, dev, path, n_part, True)
        st_w, _, got_w = _call(case, dev, path, n_part, False)
        assert st_n == 0 and st_w == 0, (st_n, st_w)
        assert plan.path == 2, "these cases must take the split path"
        assert np.array_equal(got_n, got_w), "noalloc differs from the workspace form"
        compare(case, got_n, ref, label=f"noalloc-{name}/{path}{n_part}")


def test_noalloc_one_pass_and_oversized_plan():
    import paged_varlen_attention_ua_amd as U
    case = make_case(**WORKLOADS["mixed_fp16_d128_16q2kv"])
    dev = to_device(case)
    ref, _ = oracle.attention(**case)
    st, plan, got = _call(case, dev, "2d", 0, True)
    assert st == 0 and plan.path == 1
    compare(case, got, ref, label="noalloc-2d")
    # A split plan whose workspace exceeds the static array: refused, nothing written.
    pre = make_case(**WORKLOADS["prefill_chunk2k_prefix16k_bf16"])
    pdev = to_device(pre)
    st, plan, got = _call(pre, pdev, "splitkv", 4, True)
    assert plan.workspace_bytes > U.binding.UA_NOALLOC_SCRATCH_BYTES
    assert st == U.binding.UA_ESCRATCH
    assert np.isnan(got).all()
