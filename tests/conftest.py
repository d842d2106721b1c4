import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(ROOT)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


# Workloads named in the summary, in order, with a short tag (decode, mixed,
# long decode, fp8 decode, chunked prefill).
_SUMMARY = [
    ("C1", "decode_fp16_d128_16q2kv"),
    ("C2", "mixed_fp16_d128_16q2kv"),
    ("C2+alibi", "mixed_fp16_d128_16q2kv_alibi"),
    ("C3", "long_decode_bf16_d128_32q8kv_w4096"),
    ("C3+cap+sinks", "long_decode_bf16_d128_32q8kv_w4096_softcap_sinks"),
    ("C4a", "fp8kv_decode_b32_ctx590"),
    ("C4b", "fp8kv_decode_b8_ctx6700_w4096"),
    ("C5a", "prefill_chunk1k_prefix8k_bf16"),
    ("C5b", "prefill_chunk2k_prefix16k_bf16"),
    ("C5c", "prefill_4x1k_bf16"),
    ("C5d", "prefill_8k_d256_24q4kv_bs784_bf16"),
    ("C5e", "prefill_8k_d128_bf16"),
]


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Max-abs error against the oracle per workload (all paths and seeds),
    elements compared, and how many bf16 elements (|o| >= 2) needed the
    half-ULP allowance; then one line for every other comparison."""
    try:
        from tests.gpu_common import RECORDS
    except Exception:
        return
    if not RECORDS:
        return
    w = terminalreporter.write_line
    w("parity vs float64 oracle: max-abs (gate) / elements / bf16 |o|>=2 beyond the gate")
    used = set()
    for tag, name in _SUMMARY:
        recs = [i for i, r in enumerate(RECORDS) if r["label"].split("/")[0] == name]
        if not recs:
            continue
        used.update(recs)
        rs = [RECORDS[i] for i in recs]
        w(f"  {tag:13s} max_abs {max(r['max_abs'] for r in rs):.3e} (tol {rs[0]['tol']:g}) "
          f"n={sum(r['n'] for r in rs)} band={sum(r['n_band'] for r in rs)} "
          f"compares={len(rs)}")
    rest = [r for i, r in enumerate(RECORDS) if i not in used]
    for tol in sorted({r["tol"] for r in rest}):
        rs = [r for r in rest if r["tol"] == tol]
        worst = max(rs, key=lambda r: r["max_abs"] / r["tol"])
        w(f"  other (tol {tol:g}): {len(rs)} compares, max_abs {worst['max_abs']:.3e} "
          f"[{worst['label'][:40]}], n={sum(r['n'] for r in rs)} "
          f"band={sum(r['n_band'] for r in rs)}")
