"""The five workload shapes, as keyword sets for ``make_case``.

Each entry is (name, kwargs).  Seeds: decode fp16 101, mixed 102, long decode
103, fp8 decode 104, chunked prefill 105; variant k of a workload uses seed +
10 k.  Shapes follow the pages' own scenarios: the RocKE README's
``decode_d128_b16`` and ``mixed_d128_b16`` / ``prefill_d128_b16`` scenarios
(section "Scenarios"), AITER PR #3962's sliding-window fp8 decode (section
"Performance": batch 8 at ctx ~6700 with window 4096, batch 32 at ctx ~590) and
FA-RDNA2 PR #34's prefill benchmark (section "Change": 4 x 1k prompts, chunks
of 1k behind 8k and 2k behind 16k, d256 with 24/4 heads and block size 784).
"""

from .workloads import alibi_slopes_pow2

C1 = dict(seqs=[(1, 1024), (1, 2048), (1, 4096), (1, 512)], head_dim=128,
          num_q_heads=16, num_kv_heads=2, block_size=16, q_dtype="f16", seed=101)

C2 = dict(seqs=[(1, 1328), (5, 18), (129, 463), (64, 64), (128, 256)], head_dim=128,
          num_q_heads=16, num_kv_heads=2, block_size=16, q_dtype="f16", seed=102)
C2_ALIBI = dict(C2, alibi=alibi_slopes_pow2(16), seed=112)

C3 = dict(seqs=None, num_seqs=8, q_len=1, kv_range=(6500, 6900), head_dim=128,
          num_q_heads=32, num_kv_heads=8, block_size=16, q_dtype="bf16",
          window=4096, seed=103)
C3_SOFTCAP_SINKS = dict(C3, softcap=50.0, sinks=True, seed=113)

C4A = dict(seqs=None, num_seqs=32, q_len=1, kv_range=(550, 630), head_dim=128,
           num_q_heads=32, num_kv_heads=8, block_size=32, q_dtype="bf16",
           kv_dtype="e4m3fn", o_dtype="bf16", window=4096, seed=104)
C4B = dict(C4A, num_seqs=8, kv_range=(6500, 6900), seed=114)

C5A = dict(seqs=[(1024, 9216)], head_dim=128, num_q_heads=32, num_kv_heads=8,
           block_size=16, q_dtype="bf16", seed=105)
C5B = dict(C5A, seqs=[(2048, 18432)], seed=115)
C5C = dict(C5A, seqs=[(1024, 1024)] * 4, seed=125)
C5D = dict(seqs=[(8192, 8192)], head_dim=256, num_q_heads=24, num_kv_heads=4,
           block_size=784, q_dtype="bf16", seed=135)
C5E = dict(C5A, seqs=[(8192, 8192)], seed=145)  # optional (e): the 8k prompt at D = 128

# QQ-bias scenario of the RocKE README ("qq_bias_prefill_d128_b16": the
# prefill_d128_b16 sequences with a QQ-bias of row stride 256).
QQ = dict(seqs=[(64, 64), (128, 256), (32, 256)], head_dim=128, num_q_heads=16,
          num_kv_heads=2, block_size=16, q_dtype="f16", qq_bias=256, seed=106)

# Second workload family (RocKE README, "Prefill-2D trace cohort"): head size
# 64, block size 32, 64 query / 8 kv heads, attention sinks, sliding window
# (127, 0) -- 127 keys to the left plus the query's own, W = 128 here -- or full,
# bf16 or bf16 Q with fp8 KV, chunked prefill over many sequences.  The serving
# traces themselves are not available; these are synthetic shapes of that kind.
D64_SW = dict(seqs=[(256, 2048)] * 16, head_dim=64, num_q_heads=64, num_kv_heads=8,
              block_size=32, q_dtype="bf16", window=128, sinks=True, seed=201)
D64_FP8 = dict(seqs=[(1024, 5120)] * 4, head_dim=64, num_q_heads=64, num_kv_heads=8,
               block_size=32, q_dtype="bf16", kv_dtype="e4m3fn", o_dtype="bf16",
               sinks=True, seed=202)

# Decode variants the README's scenario sets name (section "Scenarios":
# decode_d256_b16, decode_d128_b64, and the long-context / MQA decode of the
# "creative" set).
DEC_64K = dict(seqs=[(1, 65536)] * 4, head_dim=128, num_q_heads=32, num_kv_heads=8,
               block_size=16, q_dtype="bf16", seed=203)
DEC_MQA = dict(seqs=None, num_seqs=8, q_len=1, kv_range=(6500, 6900), head_dim=128,
               num_q_heads=32, num_kv_heads=1, block_size=16, q_dtype="bf16", seed=204)
DEC_D256 = dict(seqs=[(1, 1024), (1, 2048)], head_dim=256, num_q_heads=16, num_kv_heads=2,
                block_size=16, q_dtype="f16", seed=205)
DEC_B64 = dict(C1, block_size=64, seed=206)

# fp8 variants AITER PR #3962 tests (section "Testing": both e4m3 dialects,
# per-tensor and per-token scales): the sliding-window fp8 decode shapes with
# per-token K/V scales (K and V scale arrays laid out differently), in e4m3fn
# and e4m3fnuz, and the d64 fp8 prefill with per-token e4m3fnuz scales.
C4B_TOK = dict(C4B, token_scales=True, seed=124)
C4B_FNUZ_TOK = dict(C4B, kv_dtype="e4m3fnuz", token_scales=True, seed=134)
C4A_FNUZ = dict(C4A, kv_dtype="e4m3fnuz", seed=144)
D64_FNUZ_TOK = dict(D64_FP8, kv_dtype="e4m3fnuz", token_scales=True, seed=212)

WORKLOADS = {
    "decode_fp16_d128_16q2kv": C1,
    "mixed_fp16_d128_16q2kv": C2,
    "mixed_fp16_d128_16q2kv_alibi": C2_ALIBI,
    "long_decode_bf16_d128_32q8kv_w4096": C3,
    "long_decode_bf16_d128_32q8kv_w4096_softcap_sinks": C3_SOFTCAP_SINKS,
    "fp8kv_decode_b32_ctx590": C4A,
    "fp8kv_decode_b8_ctx6700_w4096": C4B,
    "prefill_chunk1k_prefix8k_bf16": C5A,
    "prefill_chunk2k_prefix16k_bf16": C5B,
    "prefill_4x1k_bf16": C5C,
    "prefill_8k_d256_24q4kv_bs784_bf16": C5D,
    "prefill_8k_d128_bf16": C5E,
    "qq_bias_prefill_fp16_d128_16q2kv": QQ,
    "d64_chunked_prefill_bf16_64q8kv_bs32_sinks_w128": D64_SW,
    "d64_prefill_bf16q_fp8kv_64q8kv_bs32_sinks": D64_FP8,
    "decode_64k_bf16_d128_32q8kv": DEC_64K,
    "decode_mqa_bf16_d128_32q1kv": DEC_MQA,
    "decode_d256_fp16_16q2kv": DEC_D256,
    "decode_fp16_d128_16q2kv_bs64": DEC_B64,
    "fp8kv_pertoken_decode_b8_ctx6700_w4096": C4B_TOK,
    "fp8kv_fnuz_pertoken_decode_b8_ctx6700_w4096": C4B_FNUZ_TOK,
    "fp8kv_fnuz_decode_b32_ctx590": C4A_FNUZ,
    "d64_prefill_bf16q_fnuz_pertoken_64q8kv_bs32_sinks": D64_FNUZ_TOK,
}

NEXT_DECODE_WORKLOADS = [
    "decode_64k_bf16_d128_32q8kv",
    "decode_mqa_bf16_d128_32q1kv",
    "decode_d256_fp16_16q2kv",
    "decode_fp16_d128_16q2kv_bs64",
    "fp8kv_pertoken_decode_b8_ctx6700_w4096",
    "fp8kv_fnuz_pertoken_decode_b8_ctx6700_w4096",
    "fp8kv_fnuz_decode_b32_ctx590",
]
NEXT_PREFILL_WORKLOADS = [
    "d64_chunked_prefill_bf16_64q8kv_bs32_sinks_w128",
    "d64_prefill_bf16q_fp8kv_64q8kv_bs32_sinks",
    "d64_prefill_bf16q_fnuz_pertoken_64q8kv_bs32_sinks",
]

DECODE_WORKLOADS = [
    "decode_fp16_d128_16q2kv",
    "long_decode_bf16_d128_32q8kv_w4096",
    "long_decode_bf16_d128_32q8kv_w4096_softcap_sinks",
    "fp8kv_decode_b32_ctx590",
    "fp8kv_decode_b8_ctx6700_w4096",
]
PREFILL_WORKLOADS = [
    "prefill_chunk1k_prefix8k_bf16",
    "prefill_chunk2k_prefix16k_bf16",
    "prefill_4x1k_bf16",
    "prefill_8k_d256_24q4kv_bs784_bf16",
    "prefill_8k_d128_bf16",
]
