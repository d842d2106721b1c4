"""torch-facing wrapper over the C ABI: builds ua_problem / ua_args from tensors.

torch is used only for device memory (outputs, the split-KV workspace) and the
current HIP stream; the computation is entirely the library's kernels.
"""

import ctypes
import threading

import torch

from . import binding as B

_DT = {torch.float16: B.UA_F16, torch.bfloat16: B.UA_BF16}
_KV_DT = {torch.float16: B.UA_F16, torch.bfloat16: B.UA_BF16,
          torch.float8_e4m3fn: B.UA_FP8_E4M3FN, torch.float8_e4m3fnuz: B.UA_FP8_E4M3FNUZ,
          torch.uint8: B.UA_FP8_E4M3FN}
_PATH = {"auto": B.UA_PATH_AUTO, "2d": B.UA_PATH_2D, "splitkv": B.UA_PATH_SPLITKV}

_NUM_CUS = {}
_WS = {}
_WS_LOCK = threading.Lock()


def device_cus(device):
    idx = device.index if device.index is not None else torch.cuda.current_device()
    if idx not in _NUM_CUS:
        _NUM_CUS[idx] = torch.cuda.get_device_properties(idx).multi_processor_count
    return _NUM_CUS[idx]


num_cus = device_cus


def make_problem(q, k_cache, v_cache, block_table, *, num_seqs, max_seqlen_q, max_seqlen_k,
                 scale, softcap=0.0, window=0, k_scale=1.0, v_scale=1.0, alibi_slopes=None,
                 sinks=None, out=None, qq_bias=None, k_token_scales=None,
                 v_token_scales=None):
    """ua_problem for Q [total_q, Hq, D], caches [num_blocks, block_size, Hkv, D].

    qq_bias: optional [rows, stride] fp32 matrix (row-contiguous).
    k_token_scales / v_token_scales: optional fp32 [num_blocks, block_size, Hkv]
    per-token scales of an fp8 cache, any strides (passed through)."""
    total_q, Hq, D = q.shape
    nb, bs, Hkv, Dk = k_cache.shape
    if Dk != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("cache shapes must be [num_blocks, block_size, Hkv, D] and match")
    if q.stride(2) != 1 or k_cache.stride(3) != 1 or v_cache.stride(3) != 1:
        raise ValueError("head_dim must be contiguous")
    if tuple(k_cache.stride()) != tuple(v_cache.stride()):
        raise ValueError("K and V caches must share strides")
    o = out if out is not None else q
    p = B.UaProblem()
    p.num_seqs = num_seqs
    p.total_q = total_q
    p.num_q_heads = Hq
    p.num_kv_heads = Hkv
    p.head_dim = D
    p.block_size = bs
    p.num_blocks = nb
    p.max_blocks_per_seq = block_table.shape[1] if block_table.dim() == 2 else 0
    p.max_seqlen_q = max_seqlen_q
    p.max_seqlen_k = max_seqlen_k
    p.q_dtype = _DT[q.dtype]
    p.kv_dtype = _KV_DT[k_cache.dtype]
    p.o_dtype = _DT[o.dtype]
    p.scale = scale
    p.softcap = softcap
    p.window = window
    p.k_scale = k_scale
    p.v_scale = v_scale
    p.has_alibi = 1 if alibi_slopes is not None else 0
    p.has_sinks = 1 if sinks is not None else 0
    if qq_bias is not None:
        if qq_bias.dim() != 2 or qq_bias.stride(1) != 1:
            raise ValueError("qq_bias must be a 2-D matrix with contiguous rows")
        if qq_bias.shape[0] < max(max_seqlen_q, 1):
            raise ValueError("qq_bias needs at least max_seqlen_q rows")
        p.has_qq_bias = 1
        p.qq_bias_stride = qq_bias.stride(0)
    if (k_token_scales is None) != (v_token_scales is None):
        raise ValueError("give both per-token scale arrays or neither")
    if k_token_scales is not None:
        for t in (k_token_scales, v_token_scales):
            if t.dtype != torch.float32 or tuple(t.shape) != (nb, bs, Hkv):
                raise ValueError("per-token scales must be float32 [num_blocks, block_size, Hkv]")
        p.has_kv_token_scales = 1
        p.ks_stride_block, p.ks_stride_slot, p.ks_stride_head = k_token_scales.stride()
        p.vs_stride_block, p.vs_stride_slot, p.vs_stride_head = v_token_scales.stride()
    p.q_stride_tok, p.q_stride_head = q.stride(0), q.stride(1)
    p.o_stride_tok, p.o_stride_head = o.stride(0), o.stride(1)
    p.kv_stride_block, p.kv_stride_slot, p.kv_stride_head = k_cache.stride()[:3]
    return p


def make_args(q, k_cache, v_cache, block_table, cu_seqlens_q, seq_lens, out, lse=None,
              alibi_slopes=None, sinks=None, qq_bias=None, k_token_scales=None,
              v_token_scales=None):
    for name, t, dt in (("block_table", block_table, torch.int32),
                        ("cu_seqlens_q", cu_seqlens_q, torch.int32),
                        ("seq_lens", seq_lens, torch.int32)):
        if t.dtype != dt or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous int32")
    for name, t in (("alibi_slopes", alibi_slopes), ("sinks", sinks), ("lse", lse)):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError(f"{name} must be contiguous float32")
    if qq_bias is not None and qq_bias.dtype != torch.float32:
        raise ValueError("qq_bias must be float32")
    a = B.UaArgs()
    a.q, a.k_cache, a.v_cache = q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr()
    a.block_table, a.cu_seqlens_q = block_table.data_ptr(), cu_seqlens_q.data_ptr()
    a.seq_lens = seq_lens.data_ptr()
    a.alibi_slopes = alibi_slopes.data_ptr() if alibi_slopes is not None else None
    a.sinks = sinks.data_ptr() if sinks is not None else None
    a.out = out.data_ptr()
    a.lse = lse.data_ptr() if lse is not None else None
    a.qq_bias = qq_bias.data_ptr() if qq_bias is not None else None
    a.k_token_scales = k_token_scales.data_ptr() if k_token_scales is not None else None
    a.v_token_scales = v_token_scales.data_ptr() if v_token_scales is not None else None
    return a


def workspace(nbytes, device, stream):
    """Grow-only workspace per (device, stream).  Sizes are rounded up to a power
    of two, so a slowly growing demand reallocates O(log) times; replaced buffers
    stay alive (a captured graph may still point at one), and since sizes at
    least double, all of them together are smaller than the current buffer."""
    key = (device.index, int(stream.cuda_stream))
    with _WS_LOCK:
        buf = _WS.get(key)
        if buf is None or buf.numel() < nbytes:
            size = 1 << max(8, (max(int(nbytes), 1) - 1).bit_length())
            old = _WS.get(key)
            if old is not None:
                _WS.setdefault(("retired",) + key, []).append(old)
            buf = torch.empty(size, dtype=torch.uint8, device=device)
            _WS[key] = buf
    return buf


def forward(q, k_cache, v_cache, block_table, cu_seqlens_q, seq_lens, *, max_seqlen_q,
            max_seqlen_k, scale, softcap=0.0, window=0, k_scale=1.0, v_scale=1.0,
            alibi_slopes=None, sinks=None, out=None, lse=None, path="auto", n_part=0,
            ws=None, qq_bias=None, k_token_scales=None, v_token_scales=None, num_cus=None):
    """Unified paged varlen attention; returns (out, plan).

    path: "auto" (dispatcher), "2d" (one pass) or "splitkv" (partitions + reduce).
    n_part: forced partition count for the split path (0 = automatic).
    num_cus: compute units the planner assumes (default: the device's).
    """
    if not q.is_cuda:
        raise ValueError("q must be a GPU tensor")
    if out is None:
        out = torch.empty_like(q)
    num_seqs = seq_lens.shape[0]
    prob = make_problem(q, k_cache, v_cache, block_table, num_seqs=num_seqs,
                        max_seqlen_q=max_seqlen_q, max_seqlen_k=max_seqlen_k, scale=scale,
                        softcap=softcap, window=window, k_scale=k_scale, v_scale=v_scale,
                        alibi_slopes=alibi_slopes, sinks=sinks, out=out, qq_bias=qq_bias,
                        k_token_scales=k_token_scales, v_token_scales=v_token_scales)
    plan = B.ua_plan(prob, num_cus if num_cus is not None else device_cus(q.device),
                     _PATH[path], n_part)
    args = make_args(q, k_cache, v_cache, block_table, cu_seqlens_q, seq_lens, out, lse,
                     alibi_slopes, sinks, qq_bias, k_token_scales, v_token_scales)
    stream = torch.cuda.current_stream(q.device)
    sp = ctypes.c_void_p(stream.cuda_stream)
    if plan.path == B.UA_PATH_2D:
        B.ua_forward_2d(prob, plan, args, sp)
    else:
        if ws is None:
            ws = workspace(plan.workspace_bytes, q.device, stream)
        B.ua_forward_splitkv(prob, plan, args, ctypes.c_void_p(ws.data_ptr()), ws.numel(), sp)
        B.ua_reduce(prob, plan, args, ctypes.c_void_p(ws.data_ptr()), ws.numel(), sp)
    return out, plan


def check_inputs(q, k_cache, v_cache, block_table, cu_seqlens_q, seq_lens, *, max_seqlen_q,
                 max_seqlen_k, scale=1.0, k_scale=1.0, v_scale=1.0):
    """Run ua_check_inputs on the device; returns the set of violated preconditions
    (names from binding.UA_CHECK_BITS), empty when the inputs are valid."""
    out = torch.empty_like(q)
    prob = make_problem(q, k_cache, v_cache, block_table, num_seqs=seq_lens.shape[0],
                        max_seqlen_q=max_seqlen_q, max_seqlen_k=max_seqlen_k, scale=scale,
                        k_scale=k_scale, v_scale=v_scale, out=out)
    args = make_args(q, k_cache, v_cache, block_table, cu_seqlens_q, seq_lens, out)
    flags = torch.full((1,), -1, dtype=torch.int32, device=q.device)
    stream = torch.cuda.current_stream(q.device)
    B.ua_check_inputs(prob, args, ctypes.c_void_p(flags.data_ptr()),
                      ctypes.c_void_p(stream.cuda_stream))
    bits = int(flags.item())
    return {name for bit, name in B.UA_CHECK_BITS.items() if bits & bit}
