"""CPU tests of the C-ABI library: exported symbols and the pure-host planner.

No kernel is launched: ua_plan is a host function, and the forward entry
points are only called on inputs they must reject before any launch.
"""

import ctypes
import os
import re

import pytest

import paged_varlen_attention_ua_amd as U
from paged_varlen_attention_ua_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "ua.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(ua_[a-z_0-9]+)\s*\(",
                                 src, flags=re.M)))


def test_header_declares_the_four_entry_points():
    names = _declared_functions()
    for fn in ("ua_plan", "ua_forward_2d", "ua_forward_splitkv", "ua_reduce"):
        assert fn in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(B.LIB_PATH)
    for fn in _declared_functions():
        assert hasattr(lib, fn), fn
    assert U.ua_abi_version() == 5


def test_struct_sizes_match_header_layout():
    # ua_problem: 6 int32, int64, 3 int32, 3 int32, 2 float, int32, 2 float, 2 int32, pad,
    # 7 int64, 2 int32 (QQ-bias), 2 int32 + 6 int64 (per-token scales)
    assert ctypes.sizeof(B.UaProblem) == 208
    assert B.UaProblem.ks_stride_block.offset == 160
    assert ctypes.sizeof(B.UaPlan) == 48
    assert ctypes.sizeof(B.UaArgs) == 104


def problem(**kw):
    p = B.UaProblem()
    d = dict(num_seqs=8, total_q=8, num_q_heads=32, num_kv_heads=8, head_dim=128,
             block_size=16, num_blocks=1000, max_blocks_per_seq=500, max_seqlen_q=1,
             max_seqlen_k=6900, q_dtype=B.UA_BF16, kv_dtype=B.UA_BF16, o_dtype=B.UA_BF16,
             scale=0.088, softcap=0.0, window=4096, k_scale=1.0, v_scale=1.0, has_alibi=0,
             has_sinks=0)
    d.update(kw)
    D, H, Hk = d["head_dim"], d["num_q_heads"], d["num_kv_heads"]
    d.setdefault("q_stride_tok", H * D)
    d.setdefault("q_stride_head", D)
    d.setdefault("o_stride_tok", H * D)
    d.setdefault("o_stride_head", D)
    d.setdefault("kv_stride_block", d["block_size"] * Hk * D)
    d.setdefault("kv_stride_slot", Hk * D)
    d.setdefault("kv_stride_head", D)
    for k, v in d.items():
        setattr(p, k, v)
    return p


def status_of(p, force_path=0, n_part=0):
    plan = B.UaPlan()
    return B.lib().ua_plan(ctypes.byref(p), 256, force_path, n_part, ctypes.byref(plan)), plan


def test_long_decode_splits_to_fill_the_device():
    # 8 seqs x 8 kv heads = 64 row blocks, a wave each (flag bit 2): 16
    # workgroups of four per partition, 16 partitions = one workgroup per CU.
    st, plan = status_of(problem())
    assert st == 0 and plan.path == B.UA_PATH_SPLITKV and plan.flags & 4
    assert plan.n_part == 16
    assert plan.grid_y == 8 and plan.grid_z == 16 and plan.grid_x == 8  # one block per sequence
    R = 8 * 32
    assert plan.workspace_bytes == ((2 * 16 * R * 4 + 255) & ~255) + 16 * R * 128 * 4
    st, plan = status_of(problem(kv_dtype=B.UA_FP8_E4M3FN, kv_stride_block=16 * 8 * 128))
    assert st == 0 and plan.n_part == 16 and plan.flags & 4


def test_wave_per_row_block_needs_four_row_blocks_and_16_slot_halves():
    # 2 kv heads (2 row blocks): one row block per workgroup, 4 x as many
    # workgroups per partition, a quarter of the partitions.
    st, plan = status_of(problem(num_q_heads=16, num_kv_heads=2))
    assert st == 0 and not plan.flags & 4 and plan.n_part == 16
    # block size 8: no 16-slot halves
    st, plan = status_of(problem(block_size=8, kv_stride_block=8 * 8 * 128, num_blocks=8192,
                                 max_blocks_per_seq=1024))
    assert st == 0 and not plan.flags & 4 and plan.n_part == 4
    # MQA decode, 32 query heads over 1 kv head: 2 head groups, 2 row blocks
    st, plan = status_of(problem(num_kv_heads=1, kv_stride_block=16 * 128,
                                 kv_stride_slot=128))
    assert st == 0 and not plan.flags & 4 and plan.grid_y == 2
    # a full grid (32 sequences of 630 keys) stays one-pass without the flag;
    # 512 sequences (4096 row blocks = 4 x 4 per CU) take it one-pass
    st, plan = status_of(problem(num_seqs=32, total_q=32, max_seqlen_k=630))
    assert st == 0 and plan.n_part == 1 and not plan.flags & 4
    st, plan = status_of(problem(num_seqs=512, total_q=512, max_seqlen_k=630, num_blocks=1 << 15,
                                 max_blocks_per_seq=40))
    assert st == 0 and plan.n_part == 1 and plan.flags & 4


def test_wave_per_row_block_flag_is_checked_at_launch():
    # A plan whose flag bit 2 does not fit the problem is refused before any launch.
    p = problem(num_q_heads=16, num_kv_heads=2)
    st, plan = status_of(p)
    assert st == 0 and not plan.flags & 4
    plan.flags |= 4
    args = B.UaArgs()
    for f in ("q", "k_cache", "v_cache", "block_table", "cu_seqlens_q", "seq_lens", "out"):
        setattr(args, f, 1 << 20)
    assert B.lib().ua_forward_splitkv(ctypes.byref(p), ctypes.byref(plan), ctypes.byref(args),
                                      ctypes.c_void_p(1 << 20), plan.workspace_bytes,
                                      None) == B.UA_EPLAN


def test_few_sequence_decode_splits_to_two_tile_partitions():
    # 4 sequences x 2 kv heads (fp16 decode, longest 4096 keys): 256 / 8 = 32
    # partitions of 128 keys; 2 sequences of d256 (longest 2048): 2048 / 64 = 32.
    f16 = dict(q_dtype=B.UA_F16, kv_dtype=B.UA_F16, o_dtype=B.UA_F16, window=0,
               num_q_heads=16, num_kv_heads=2)
    st, plan = status_of(problem(num_seqs=4, total_q=4, max_seqlen_k=4096, **f16))
    assert st == 0 and plan.path == B.UA_PATH_SPLITKV and plan.n_part == 32
    st, plan = status_of(problem(num_seqs=2, total_q=2, max_seqlen_k=2048, head_dim=256, **f16))
    assert st == 0 and plan.path == B.UA_PATH_SPLITKV and plan.n_part == 32


def test_mixed_batch_splits_to_four_tile_partitions():
    # (q, kv) = (1, 1328), (5, 18), (129, 463), (64, 64), (128, 256), 16q/2kv
    # fp16: 128-row blocks (16 tokens x G = 8) leave CUs idle; the longest key
    # range (1328) in partitions of at least 256 keys gives 5.
    st, plan = status_of(problem(num_seqs=5, total_q=327, max_seqlen_q=129, max_seqlen_k=1328,
                                 num_q_heads=16, num_kv_heads=2, window=0, q_dtype=B.UA_F16,
                                 kv_dtype=B.UA_F16, o_dtype=B.UA_F16))
    assert st == 0 and plan.kernel == 1 and plan.path == B.UA_PATH_SPLITKV and plan.n_part == 5


def test_eight_wave_blocks_only_for_plain_logits():
    # A long chunked prefill (2048 queries behind 16384 keys, 32q/8kv, bf16)
    # takes 256-row blocks; with softcap, ALiBi or a QQ-bias it must take the
    # 128-row kernel, the one with those paths.
    long_prefill = dict(num_seqs=1, total_q=2048, max_seqlen_q=2048, max_seqlen_k=18432,
                        window=0, num_blocks=2400, max_blocks_per_seq=1200)
    st, plan = status_of(problem(**long_prefill))
    assert st == 0 and plan.kernel == 2
    for extra in (dict(softcap=30.0), dict(has_alibi=1),
                  dict(has_qq_bias=1, qq_bias_stride=2048)):
        st, plan = status_of(problem(**long_prefill, **extra))
        assert st == 0 and plan.kernel == 1, extra


def test_short_context_full_grid_stays_one_pass():
    st, plan = status_of(problem(num_seqs=32, total_q=32, max_seqlen_k=630))
    assert st == 0 and plan.path == B.UA_PATH_2D and plan.n_part == 1
    assert plan.workspace_bytes == 0


def test_wide_group_decode_splits_heads_into_small_blocks():
    # MQA-style decode, 32 query heads on one kv head: two groups of 16 rows
    st, plan = status_of(problem(num_q_heads=32, num_kv_heads=1, kv_stride_block=16 * 128,
                                 kv_stride_slot=128))
    assert st == 0 and plan.kernel == 0 and plan.grid_y == 2 and plan.block_q == 1
    # 24 heads: two groups of 12
    st, plan = status_of(problem(num_q_heads=24, num_kv_heads=1, kv_stride_block=16 * 128,
                                 kv_stride_slot=128))
    assert st == 0 and plan.kernel == 0 and plan.grid_y == 2 and plan.block_q == 1
    # more than one query per sequence: large kernel, one block per kv head
    st, plan = status_of(problem(num_q_heads=32, num_kv_heads=1, kv_stride_block=16 * 128,
                                 kv_stride_slot=128, max_seqlen_q=2, total_q=16))
    assert st == 0 and plan.kernel == 1 and plan.grid_y == 1


def test_forced_paths():
    st, plan = status_of(problem(), force_path=B.UA_PATH_2D)
    assert st == 0 and plan.path == B.UA_PATH_2D and plan.n_part == 1
    st, plan = status_of(problem(num_seqs=32, total_q=32, max_seqlen_k=630),
                         force_path=B.UA_PATH_SPLITKV, n_part=7)
    assert st == 0 and plan.path == B.UA_PATH_SPLITKV and plan.n_part == 7
    st, _ = status_of(problem(), force_path=B.UA_PATH_2D, n_part=4)
    assert st == -1


def test_grid_covers_every_query_block():
    # slots = total_q / block_q + num_seqs >= sum ceil(q_len / block_q)
    st, plan = status_of(problem(num_seqs=5, total_q=327, max_seqlen_q=129, max_seqlen_k=1328,
                                 num_q_heads=16, num_kv_heads=2, window=0))
    assert st == 0
    bq = plan.block_q
    lens = [1, 5, 129, 64, 128]
    assert sum(-(-q // bq) for q in lens) <= plan.grid_x == 327 // bq + 5


@pytest.mark.parametrize("kw,code", [
    (dict(num_q_heads=30, num_kv_heads=8), -1),
    (dict(head_dim=96), -2),
    (dict(block_size=0), -1),
    (dict(max_seqlen_q=7000), -1),
    (dict(max_blocks_per_seq=10), -1),
    (dict(q_dtype=B.UA_FP8_E4M3FN), -2),
    (dict(kv_dtype=B.UA_F16), -2),
    (dict(o_dtype=B.UA_F16), -2),
    (dict(scale=float("nan")), -1),
    (dict(softcap=float("inf")), -1),
    (dict(kv_dtype=B.UA_FP8_E4M3FN, k_scale=0.0), -1),
    (dict(kv_stride_slot=1028), -2),
    (dict(q_stride_head=0), -1),
    (dict(total_q=9), -1),
    (dict(has_qq_bias=1, qq_bias_stride=0), -1),
    (dict(max_seqlen_q=300, total_q=8, has_qq_bias=1, qq_bias_stride=256), -1),
    (dict(has_kv_token_scales=1), -2),  # bf16 cache: per-token scales need fp8
    (dict(kv_dtype=B.UA_FP8_E4M3FNUZ, kv_stride_block=16 * 8 * 128, has_kv_token_scales=1,
          ks_stride_slot=-1), -1),
    (dict(kv_dtype=B.UA_FP8_E4M3FNUZ, kv_stride_block=16 * 8 * 128, has_kv_token_scales=1,
          vs_stride_block=1 << 22), -2),  # block offsets past 32 bits
    (dict(reserved0=1), -1),
    (dict(kv_dtype=B.UA_FP8_E4M3FNUZ, k_scale=float("nan")), -1),
])
def test_invalid_problems_are_rejected(kw, code):
    st, _ = status_of(problem(**kw))
    assert st == code


def test_fp8_dialects_and_per_token_scales_plan():
    for kvd in (B.UA_FP8_E4M3FN, B.UA_FP8_E4M3FNUZ):
        st, plan = status_of(problem(kv_dtype=kvd, kv_stride_block=16 * 8 * 128))
        assert st == 0 and plan.n_part == 16
        p = problem(kv_dtype=kvd, kv_stride_block=16 * 8 * 128, has_kv_token_scales=1,
                    ks_stride_block=8 * 16, ks_stride_slot=1, ks_stride_head=16,
                    vs_stride_block=16 * 8, vs_stride_slot=8, vs_stride_head=1)
        st, plan2 = status_of(p)
        assert st == 0 and plan2.n_part == 16
        assert plan2.problem_hash != plan.problem_hash
        # per-token arrays missing from the call
        args = B.UaArgs()
        for f in ("q", "k_cache", "v_cache", "block_table", "cu_seqlens_q", "seq_lens", "out"):
            setattr(args, f, 1 << 20)
        assert B.lib().ua_forward_splitkv(ctypes.byref(p), ctypes.byref(plan2),
                                          ctypes.byref(args), ctypes.c_void_p(1 << 21),
                                          1 << 30, None) == -1


def test_forward_rejects_mismatched_plan_and_missing_workspace():
    p = problem()
    st, plan = status_of(p)
    args = B.UaArgs()
    # plan made for another problem
    p2 = problem(window=100)
    assert B.lib().ua_forward_2d(ctypes.byref(p2), ctypes.byref(plan), ctypes.byref(args),
                                 None) == -5
    # split plan passed to the 2D entry point
    assert B.lib().ua_forward_2d(ctypes.byref(p), ctypes.byref(plan), ctypes.byref(args),
                                 None) == -5
    # missing device pointers
    assert B.lib().ua_forward_splitkv(ctypes.byref(p), ctypes.byref(plan), ctypes.byref(args),
                                      None, 0, None) == -1
    # workspace too small (pointers set to fake aligned non-null values; nothing launches)
    for f in ("q", "k_cache", "v_cache", "block_table", "cu_seqlens_q", "seq_lens", "out"):
        setattr(args, f, 1 << 20)
    assert B.lib().ua_forward_splitkv(ctypes.byref(p), ctypes.byref(plan), ctypes.byref(args),
                                      ctypes.c_void_p(1 << 21), 16, None) == -3
    assert B.lib().ua_reduce(ctypes.byref(p), ctypes.byref(plan), ctypes.byref(args),
                             None, 0, None) == -3


def test_check_inputs_rejects_missing_pointers():
    p = problem()
    args = B.UaArgs()
    assert B.lib().ua_check_inputs(ctypes.byref(p), ctypes.byref(args), None, None) == -1
    assert B.lib().ua_check_inputs(ctypes.byref(p), ctypes.byref(args),
                                   ctypes.c_void_p(1 << 20), None) == -1
    assert B.lib().ua_check_inputs(ctypes.byref(problem(head_dim=96)), ctypes.byref(args),
                                   ctypes.c_void_p(1 << 20), None) == -2


def test_empty_batch_is_a_no_op():
    p = problem(num_seqs=0, total_q=0, max_seqlen_q=0, max_seqlen_k=0)
    st, plan = status_of(p)
    assert st == 0 and plan.grid_x == 0
    args = B.UaArgs()
    assert B.lib().ua_forward(ctypes.byref(p), ctypes.byref(plan), ctypes.byref(args), None, 0,
                              None) == 0


def test_status_strings():
    assert B.lib().ua_status_string(0) == b"ok"
    assert B.lib().ua_status_string(-3).startswith(b"workspace")


def test_noalloc_refuses_before_touching_the_device():
    """ua_forward_noalloc checks the call on the host first: a missing plan or
    pointers, a plan of another problem, and a split plan whose workspace
    exceeds the static scratch (UA_ESCRATCH) all return before any HIP call."""
    L = B.lib()
    p = problem()
    args = B.UaArgs()
    assert L.ua_forward_noalloc(ctypes.byref(p), None, ctypes.byref(args), None) == -1
    st, plan = status_of(p, force_path=B.UA_PATH_SPLITKV, n_part=4)
    assert st == 0 and plan.workspace_bytes <= B.UA_NOALLOC_SCRATCH_BYTES
    assert L.ua_forward_noalloc(ctypes.byref(p), ctypes.byref(plan), ctypes.byref(args),
                                None) == -1  # null device pointers
    assert L.ua_forward_noalloc(ctypes.byref(problem(window=100)), ctypes.byref(plan),
                                ctypes.byref(args), None) == -5
    for f in ("q", "k_cache", "v_cache", "block_table", "cu_seqlens_q", "seq_lens", "out"):
        setattr(args, f, 1 << 20)  # fake aligned pointers: nothing may launch
    big = problem(num_seqs=1, total_q=8192, max_seqlen_q=8192, max_seqlen_k=8192, window=0,
                  num_blocks=1200, max_blocks_per_seq=600)
    st, plan = status_of(big, force_path=B.UA_PATH_SPLITKV, n_part=4)
    assert st == 0 and plan.workspace_bytes > B.UA_NOALLOC_SCRATCH_BYTES
    assert L.ua_forward_noalloc(ctypes.byref(big), ctypes.byref(plan), ctypes.byref(args),
                                None) == B.UA_ESCRATCH
    assert L.ua_status_string(B.UA_ESCRATCH).startswith(b"split-KV workspace")


def _rank_order_blocks(grid_x, q_lens, bq):
    """The large kernel's rank-order mapping, restated: slot x is block
    n_s - 1 - x // S of sequence x % S (none when x // S >= n_s)."""
    S = len(q_lens)
    got = []
    for x in range(grid_x):
        s, r = x % S, x // S
        nb = -(-q_lens[s] // bq)
        if r < nb:
            got.append((s, nb - 1 - r))
    return got


def test_rank_order_for_multi_round_prompt_batches():
    """4 x 1k causal prompts (1024 four-wave blocks on 256 CUs): slots in rank
    order, heaviest block of every sequence first, every block exactly once."""
    p = problem(num_seqs=4, total_q=4096, max_seqlen_q=1024, max_seqlen_k=1024, window=0,
                max_blocks_per_seq=64)
    st, plan = status_of(p)
    assert st == 0 and plan.kernel == 1 and plan.flags & 2
    bq = plan.block_q
    assert plan.grid_x == 4 * (1024 // bq)
    blocks = _rank_order_blocks(plan.grid_x, [1024] * 4, bq)
    assert sorted(blocks) == [(s, b) for s in range(4) for b in range(1024 // bq)]
    assert blocks[:4] == [(s, 1024 // bq - 1) for s in range(4)]
    # one round of workgroups (the 2k chunk behind 16k: 256 eight-wave blocks): packed order
    st, plan = status_of(problem(num_seqs=1, total_q=2048, max_seqlen_q=2048,
                                 max_seqlen_k=18432, window=0, max_blocks_per_seq=1200,
                                 num_blocks=2400))
    assert st == 0 and plan.kernel == 2 and not plan.flags & 2


@pytest.mark.parametrize("seed", range(20))
def test_rank_order_covers_every_block_of_varlen_batches(seed):
    import random
    rng = random.Random(seed)
    S = rng.randint(1, 9)
    q_lens = [rng.choice([0, 1, 5, 31, 32, 33, 64, 100, 129, 300]) for _ in range(S)]
    if max(q_lens) == 0:
        q_lens[0] = 40
    p = problem(num_seqs=S, total_q=sum(q_lens), max_seqlen_q=max(q_lens),
                max_seqlen_k=max(q_lens) + 50, window=0, max_blocks_per_seq=64)
    st, plan = status_of(p, force_path=B.UA_PATH_2D)
    assert st == 0
    if plan.kernel == 0:
        return
    # force the rank order through a small device, when the planner allows it
    st, plan = B.lib().ua_plan(ctypes.byref(p), 1, B.UA_PATH_2D, 0, ctypes.byref(plan)), plan
    bq = plan.block_q
    if plan.flags & 2:
        blocks = _rank_order_blocks(plan.grid_x, q_lens, bq)
        want = [(s, b) for s in range(S) for b in range(-(-q_lens[s] // bq))]
        assert sorted(blocks) == sorted(want)
