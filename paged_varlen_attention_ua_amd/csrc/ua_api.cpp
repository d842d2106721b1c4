// Host side of the C ABI: validation, the 2D / split-KV dispatcher and launches.
//
// The dispatcher follows the pages' rule (AITER PR #3962, section "Changes";
// RocKE README, "Why three tables"): stay one-pass when the one-pass grid
// already fills the device or the visible key range is short; otherwise split
// each query block's (window-bounded) key range into partitions so the grid
// fills the device.  Partitions are sized per query block on the device so
// that n_part of them always cover the block's whole visible range (the
// capped-partition defect of AITER PR #3962's review cannot occur), and it uses
// host integers only (max_seqlen_q / max_seqlen_k), never a device sync.

#include <cmath>
#include <algorithm>
#include <cstring>

#include "ua_internal.h"

using namespace ua;

namespace {

struct Hasher {
  uint64_t h = 1469598103934665603ull;  // FNV-1a 64
  template <typename T>
  void add(const T& v) {
    const unsigned char* b = reinterpret_cast<const unsigned char*>(&v);
    for (size_t i = 0; i < sizeof(T); ++i) {
      h ^= b[i];
      h *= 1099511628211ull;
    }
  }
};

uint64_t problem_hash(const ua_problem* p) {
  Hasher hs;
  hs.add(p->num_seqs); hs.add(p->total_q); hs.add(p->num_q_heads); hs.add(p->num_kv_heads);
  hs.add(p->head_dim); hs.add(p->block_size); hs.add(p->num_blocks);
  hs.add(p->max_blocks_per_seq); hs.add(p->max_seqlen_q); hs.add(p->max_seqlen_k);
  hs.add(p->q_dtype); hs.add(p->kv_dtype); hs.add(p->o_dtype); hs.add(p->scale);
  hs.add(p->softcap); hs.add(p->window); hs.add(p->k_scale); hs.add(p->v_scale);
  hs.add(p->has_alibi); hs.add(p->has_sinks); hs.add(p->q_stride_tok); hs.add(p->q_stride_head);
  hs.add(p->o_stride_tok); hs.add(p->o_stride_head); hs.add(p->kv_stride_block);
  hs.add(p->kv_stride_slot); hs.add(p->kv_stride_head); hs.add(p->has_qq_bias);
  hs.add(p->qq_bias_stride); hs.add(p->has_kv_token_scales);
  hs.add(p->ks_stride_block); hs.add(p->ks_stride_slot); hs.add(p->ks_stride_head);
  hs.add(p->vs_stride_block); hs.add(p->vs_stride_slot); hs.add(p->vs_stride_head);
  return hs.h;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool is_16bit(int32_t t) { return t == UA_F16 || t == UA_BF16; }
bool is_fp8(int32_t t) { return t == UA_FP8_E4M3FN || t == UA_FP8_E4M3FNUZ; }

ua_status validate(const ua_problem* p) {
  if (!p) return UA_EINVAL;
  if (p->num_seqs < 0 || p->total_q < 0) return UA_EINVAL;
  if (p->num_q_heads <= 0 || p->num_kv_heads <= 0) return UA_EINVAL;
  if (p->num_q_heads % p->num_kv_heads != 0) return UA_EINVAL;
  if (p->block_size <= 0 || p->num_blocks < 0) return UA_EINVAL;
  if (p->max_seqlen_q < 0 || p->max_seqlen_k < 0 || p->max_seqlen_q > p->max_seqlen_k)
    return UA_EINVAL;
  if (p->max_seqlen_k > 0 && p->num_blocks == 0) return UA_EINVAL;
  if (p->max_blocks_per_seq < 0 || p->max_blocks_per_seq < ceil_div(p->max_seqlen_k, p->block_size))
    return UA_EINVAL;
  if (p->num_seqs > 0 && p->total_q > (int64_t)p->num_seqs * p->max_seqlen_q) return UA_EINVAL;
  if (!std::isfinite(p->scale) || !std::isfinite(p->softcap)) return UA_EINVAL;
  if (!is_16bit(p->q_dtype)) return UA_EUNSUPPORTED;
  if (p->kv_dtype != p->q_dtype && !is_fp8(p->kv_dtype)) return UA_EUNSUPPORTED;
  if (p->o_dtype != p->q_dtype) return UA_EUNSUPPORTED;
  if (is_fp8(p->kv_dtype)) {
    if (!std::isfinite(p->k_scale) || !std::isfinite(p->v_scale) || p->k_scale <= 0.f ||
        p->v_scale <= 0.f)
      return UA_EINVAL;
  }
  if (p->reserved0 != 0) return UA_EINVAL;
  if (p->has_kv_token_scales) {
    if (!is_fp8(p->kv_dtype)) return UA_EUNSUPPORTED;
    if (p->ks_stride_block < 0 || p->ks_stride_slot < 0 || p->ks_stride_head < 0 ||
        p->vs_stride_block < 0 || p->vs_stride_slot < 0 || p->vs_stride_head < 0)
      return UA_EINVAL;
    // The kernels form (block, slot) offsets of the scale arrays in 32 bits.
    const int64_t lim = (int64_t)1 << 31;
    auto fits = [&](int64_t sb, int64_t ss) {
      return sb < lim && ss < lim &&
             std::max<int64_t>(p->num_blocks - 1, 0) * sb + (int64_t)(p->block_size - 1) * ss < lim;
    };
    if (!fits(p->ks_stride_block, p->ks_stride_slot) || !fits(p->vs_stride_block, p->vs_stride_slot))
      return UA_EUNSUPPORTED;
  }
  if (p->head_dim != 64 && p->head_dim != 128 && p->head_dim != 256) return UA_EUNSUPPORTED;
  if ((int64_t)p->total_q * p->num_q_heads >= (int64_t)1 << 31) return UA_EUNSUPPORTED;
  if (p->q_stride_tok <= 0 || p->q_stride_head <= 0 || p->o_stride_tok <= 0 ||
      p->o_stride_head <= 0 || p->kv_stride_block <= 0 || p->kv_stride_slot <= 0 ||
      p->kv_stride_head <= 0)
    return UA_EINVAL;
  // 16-byte vector access: strides in whole 16-byte units.
  const int64_t kv_vec = is_fp8(p->kv_dtype) ? 16 : 8;
  if (p->q_stride_tok % 8 || p->q_stride_head % 8 || p->o_stride_tok % 8 || p->o_stride_head % 8)
    return UA_EUNSUPPORTED;
  if (p->kv_stride_block % kv_vec || p->kv_stride_slot % kv_vec || p->kv_stride_head % kv_vec)
    return UA_EUNSUPPORTED;
  if (p->has_qq_bias && p->qq_bias_stride < std::max(p->max_seqlen_q, 1)) return UA_EINVAL;
  const int G = p->num_q_heads / p->num_kv_heads;
  if (G > kLargeRows) return UA_EUNSUPPORTED;
  if (!(p->scale > 0.f)) return UA_EUNSUPPORTED;
  return UA_OK;
}

ua_status check_args(const ua_problem* p, const ua_args* a) {
  if (!a) return UA_EINVAL;
  if (p->total_q == 0 || p->num_seqs == 0) return UA_OK;
  if (!a->q || !a->k_cache || !a->v_cache || !a->block_table || !a->cu_seqlens_q ||
      !a->seq_lens || !a->out)
    return UA_EINVAL;
  if ((p->has_alibi != 0) != (a->alibi_slopes != nullptr)) return UA_EINVAL;
  if ((p->has_sinks != 0) != (a->sinks != nullptr)) return UA_EINVAL;
  if ((p->has_qq_bias != 0) != (a->qq_bias != nullptr)) return UA_EINVAL;
  if ((p->has_kv_token_scales != 0) != (a->k_token_scales != nullptr) ||
      (p->has_kv_token_scales != 0) != (a->v_token_scales != nullptr))
    return UA_EINVAL;
  auto aligned = [](const void* ptr, uintptr_t n) { return ((uintptr_t)ptr % n) == 0; };
  if (!aligned(a->q, 16) || !aligned(a->out, 16) || !aligned(a->k_cache, 16) ||
      !aligned(a->v_cache, 16))
    return UA_EUNSUPPORTED;
  return UA_OK;
}

uint64_t ml_bytes(const ua_problem* p, int n_part) {
  return 2ull * n_part * (uint64_t)p->total_q * p->num_q_heads * 4ull;
}

uint64_t acc_offset(const ua_problem* p, int n_part) {
  return (ml_bytes(p, n_part) + 255ull) & ~255ull;
}

Params make_params(const ua_problem* p, const ua_plan_t* plan, const ua_args* a, void* ws) {
  Params q;
  std::memset(&q, 0, sizeof(q));
  q.q = a->q;
  q.k = a->k_cache;
  q.v = a->v_cache;
  q.block_table = a->block_table;
  q.cu_seqlens_q = a->cu_seqlens_q;
  q.seq_lens = a->seq_lens;
  q.alibi = a->alibi_slopes;
  q.sinks = a->sinks;
  q.out = a->out;
  q.lse = a->lse;
  q.qq_bias = p->has_qq_bias ? a->qq_bias : nullptr;
  q.qq_stride = p->has_qq_bias ? p->qq_bias_stride : 0;
  if (p->has_kv_token_scales) {
    q.k_tscale = a->k_token_scales;
    q.v_tscale = a->v_token_scales;
    q.ks_stride_block = p->ks_stride_block;
    q.ks_stride_slot = p->ks_stride_slot;
    q.ks_stride_head = p->ks_stride_head;
    q.vs_stride_block = p->vs_stride_block;
    q.vs_stride_slot = p->vs_stride_slot;
    q.vs_stride_head = p->vs_stride_head;
  }
  if (ws) {
    const int64_t R = (int64_t)p->total_q * p->num_q_heads;
    char* base = reinterpret_cast<char*>(ws);
    q.ws_m = reinterpret_cast<float*>(base);
    q.ws_l = reinterpret_cast<float*>(base + (uint64_t)plan->n_part * R * 4);
    q.ws_acc = reinterpret_cast<float*>(base + acc_offset(p, plan->n_part));
  }
  q.q_stride_tok = p->q_stride_tok;
  q.q_stride_head = p->q_stride_head;
  q.o_stride_tok = p->o_stride_tok;
  q.o_stride_head = p->o_stride_head;
  q.kv_stride_block = p->kv_stride_block;
  q.kv_stride_slot = p->kv_stride_slot;
  q.kv_stride_head = p->kv_stride_head;
  q.num_seqs = p->num_seqs;
  q.total_q = p->total_q;
  q.num_q_heads = p->num_q_heads;
  q.num_kv_heads = p->num_kv_heads;
  q.group = p->num_q_heads / p->num_kv_heads;
  q.head_groups = plan->grid_y / p->num_kv_heads;
  q.group_rows = q.group / q.head_groups;
  q.block_size = p->block_size;
  q.max_blocks_per_seq = p->max_blocks_per_seq;
  q.bs_div = make_fastdiv((uint32_t)p->block_size);
  q.block_q = plan->block_q;
  q.n_part = plan->n_part;
  q.window = p->window > 0 ? p->window : 0;
  const bool fp8 = is_fp8(p->kv_dtype);
  // e4m3fnuz codes are decoded to twice their value: halve both factors.
  const double half = p->kv_dtype == UA_FP8_E4M3FNUZ ? 0.5 : 1.0;
  const double ks = fp8 ? (double)p->k_scale * half : 1.0;
  const double log2e = 1.4426950408889634;
  q.qk_scale2 = (float)((double)p->scale * ks * log2e);
  q.softcap_on = p->softcap > 0.f ? 1 : 0;
  if (q.softcap_on) {
    q.cap_in = (float)((double)p->scale * ks / p->softcap);
    q.cap_out2 = (float)((double)p->softcap * log2e);
  }
  q.v_scale = fp8 ? (float)((double)p->v_scale * half) : 1.0f;
  q.seq_blocks = plan->flags & 1;
  q.rank_order = (plan->flags >> 1) & 1;
  q.head_waves = (plan->flags >> 2) & 1;
  return q;
}

}  // namespace

extern "C" {

int32_t ua_abi_version(void) { return UA_ABI_VERSION; }

const char* ua_status_string(int32_t s) {
  switch (s) {
    case UA_OK: return "ok";
    case UA_EINVAL: return "invalid argument";
    case UA_EUNSUPPORTED: return "unsupported configuration";
    case UA_EWORKSPACE: return "workspace missing or too small";
    case UA_EHIP: return "HIP launch error";
    case UA_EPLAN: return "plan does not match the problem or the call";
    case UA_ESCRATCH:
      return "split-KV workspace of the plan exceeds UA_NOALLOC_SCRATCH_BYTES (use ua_forward "
             "with a caller workspace)";
    default: return "unknown status";
  }
}

ua_status ua_plan(const ua_problem* prob, int32_t num_cus, int32_t force_path,
                  int32_t force_n_part, ua_plan_t* plan) {
  if (!plan) return UA_EINVAL;
  ua_status st = validate(prob);
  if (st != UA_OK) return st;
  if (force_path != UA_PATH_AUTO && force_path != UA_PATH_2D && force_path != UA_PATH_SPLITKV)
    return UA_EINVAL;
  if (force_n_part < 0 || force_n_part > 65535) return UA_EINVAL;
  if (force_path == UA_PATH_2D && force_n_part > 1) return UA_EINVAL;
  if (num_cus <= 0) num_cus = 256;
  std::memset(plan, 0, sizeof(*plan));
  const int G = prob->num_q_heads / prob->num_kv_heads;
  // Small blocks (<= 16 rows, bandwidth-shaped) when every sequence's query
  // run fits one of them; large MFMA blocks otherwise: 256 rows (eight waves,
  // half the K/V reads per flop, a four-deep copy ring) for 16-bit caches with
  // D <= 128 when some sequence fills one and blocks walk >= 4096 keys
  // (measured on MI355X: a few % faster there; slower on shorter ranges and
  // for fp8 caches, where two independent four-wave groups per CU overlap
  // better), else 128 rows.
  // Decode (one query per sequence) with G > 16: split each kv head's query
  // heads into HG groups of at most 16, one small block each (they read the
  // same K/V rows), instead of a large block with most MFMA rows idle.
  int HG = 1;
  if (G > kSmallRows && prob->max_seqlen_q <= 1) {
    for (int h = 2; h <= G; ++h) {
      if (G % h == 0 && G / h <= kSmallRows) {
        HG = h;
        break;
      }
    }
  }
  const int Gs = G / HG;  // query heads per block and token
  const bool small = Gs <= kSmallRows && (int64_t)prob->max_seqlen_q * Gs <= kSmallRows;
  if (!small) HG = 1;
  int64_t eff_k = prob->max_seqlen_k;
  if (prob->window > 0)
    eff_k = std::min<int64_t>(eff_k, (int64_t)prob->window + prob->max_seqlen_q - 1);
  // The eight-wave kernel has no softcap / ALiBi / QQ-bias path.
  const bool plain_logits = !(prob->softcap > 0.f) && !prob->has_alibi && !prob->has_qq_bias;
  const bool eight = !small && prob->head_dim <= 128 && is_16bit(prob->kv_dtype) &&
                     plain_logits && (int64_t)prob->max_seqlen_q * G >= kLarge8Rows &&
                     eff_k >= 4096;
  plan->kernel = small ? 0 : (eight ? 2 : 1);
  plan->block_q = small ? kSmallRows / Gs : (eight ? kLarge8Rows : kLargeRows) / G;
  const int bq = plan->block_q;
  const int64_t slots = prob->num_seqs > 0 ? (int64_t)prob->total_q / bq + prob->num_seqs : 0;
  const int64_t est_blocks =
      std::min<int64_t>(slots, (int64_t)prob->num_seqs * ceil_div(prob->max_seqlen_q, bq));
  if (prob->window > 0) eff_k = std::min<int64_t>(eff_k, (int64_t)prob->window + bq - 1);
  const int64_t wgs_rb = est_blocks * prob->num_kv_heads * HG;  // one per row block
  // Small blocks split when the row blocks do not fill the device and the
  // range is long; stay one-pass for short ranges.
  const bool small_split = small && wgs_rb > 0 && wgs_rb < num_cus && eff_k > 1024;
  // Wave per row block (a multiple of four row blocks, i.e. kv heads x head
  // groups, and 16-slot-aligned cache blocks): each wave owns one row block and
  // walks the whole partition, the four waves of a workgroup reading adjacent
  // kv heads' rows of the same cache slots.  Used where the small blocks split
  // anyway (the partition count then grows four-fold to keep the wave count)
  // or where even a quarter of the workgroups fills the device four times.
  const bool head_waves = small && (prob->num_kv_heads * HG) % kSmallWaves == 0 &&
                          prob->block_size % 16 == 0 &&
                          (small_split || wgs_rb >= (int64_t)kSmallWaves * num_cus);
  const int64_t wgs = head_waves ? wgs_rb / kSmallWaves : wgs_rb;

  // Automatic partition count: fill the device with small workgroups, keep at
  // least two tiles per partition, and stay one-pass for short ranges.
  int auto_parts = 1;
  if (small_split) {
    // Measured on MI355X: about one small workgroup per CU for 16-bit KV and two
    // for fp8 KV (half the bytes per key); one for both with a wave per row
    // block (long decode, 8 x 8 row blocks: 16 partitions 33.1 us per step
    // against 35.2 at 32; fp8 cache 24.4 against 24.7; partition counts that
    // leave 1.5 workgroups per CU ran 10-13% slower).  At least 64 keys per
    // partition: decode of a few sequences is latency-bound, and 32 partitions
    // of its 4096-key or 2048-key (d256) ranges ran 7% and 24% faster than the
    // 16 and 8 that a 256-key minimum gave.
    const int64_t per_cu = (is_fp8(prob->kv_dtype) && !head_waves) ? 2 : 1;
    const int64_t want = ceil_div(per_cu * num_cus, wgs);
    const int64_t by_len = std::max<int64_t>(1, eff_k / 64);
    auto_parts = (int)std::max<int64_t>(1, std::min<int64_t>(std::min(want, by_len), 64));
  } else if (!small && wgs > 0 && wgs < (eight ? 1ll : 2ll) * num_cus && eff_k >= 1024) {
    // Four-wave large blocks run two per CU, eight-wave ones one: split a grid
    // that does not fill that, keeping at least 256 keys (four tiles) per
    // partition, up to 16 partitions (64 when at most half of a block's rows
    // are live, e.g. decode with G > 16: there the key walk is bandwidth-shaped
    // like the small blocks').  Measured on MI355X: the mixed decode + prefill
    // batch (longest range 1328 keys) ran 20-25% faster at the 5 partitions of
    // a 256-key minimum than at the 2 of a 512-key one.
    const bool sparse_rows = (int64_t)std::min(prob->max_seqlen_q, bq) * G * 2 <= kLargeRows;
    const int64_t want = ceil_div((eight ? 1ll : 2ll) * num_cus, wgs);
    const int64_t by_len = std::max<int64_t>(1, eff_k / 256);
    auto_parts = (int)std::max<int64_t>(
        1, std::min<int64_t>(std::min(want, by_len), sparse_rows ? 64 : 16));
  }
  int n_part;
  if (force_path == UA_PATH_2D) {
    n_part = 1;
    plan->path = UA_PATH_2D;
  } else if (force_path == UA_PATH_SPLITKV) {
    n_part = force_n_part > 0 ? force_n_part : auto_parts;
    plan->path = UA_PATH_SPLITKV;
  } else {
    n_part = force_n_part > 0 ? force_n_part : auto_parts;
    plan->path = n_part > 1 ? UA_PATH_SPLITKV : UA_PATH_2D;
  }
  plan->n_part = n_part;
  if (slots > 0x7fffffff) return UA_EUNSUPPORTED;
  plan->grid_x = (int32_t)slots;
  // Every sequence's query run fits one block: block x is the sequence index.
  if (prob->max_seqlen_q <= bq) {
    plan->flags |= 1;
    plan->grid_x = prob->num_seqs;
  }
  // Rank order for large blocks when the grid takes more than one round of
  // the device's workgroup slots: slot x is block n_s - 1 - x / num_seqs of
  // sequence x % num_seqs, so workgroups start heaviest-first across all
  // sequences (under a causal mask a sequence's later blocks walk more keys),
  // the order that lets later, lighter blocks fill the gaps.  It needs
  // num_seqs * max_blocks slots (slots past a sequence's block count exit at
  // once), so it is used only when that is at most 1.5 x the packed count.
  // Measured on MI355X: 4 x 1k causal prompts 498 -> 521 TFLOP/s (the packed
  // order ran each sequence's blocks heaviest-first, but sequence by sequence,
  // so the first sequence's heavy blocks started last); other prefills
  // unchanged.
  {
    const int64_t per_cu = eight ? 1 : (prob->head_dim > 128 ? 1 : 2);
    const int64_t max_nb = ceil_div(prob->max_seqlen_q, bq);
    const int64_t ranked = (int64_t)prob->num_seqs * max_nb;
    if (!small && !(plan->flags & 1) && ranked * prob->num_kv_heads * n_part > per_cu * num_cus &&
        2 * ranked <= 3 * slots && ranked <= 0x7fffffff) {
      plan->flags |= 2;
      plan->grid_x = (int32_t)ranked;
    }
  }
  if (head_waves) plan->flags |= 4;
  plan->grid_y = prob->num_kv_heads * HG;
  plan->grid_z = n_part;
  plan->workspace_bytes =
      plan->path == UA_PATH_SPLITKV
          ? acc_offset(prob, n_part) +
                (uint64_t)n_part * prob->total_q * prob->num_q_heads * prob->head_dim * 4ull
          : 0;
  plan->problem_hash = problem_hash(prob);
  return UA_OK;
}

uint64_t ua_workspace_acc_offset(const ua_problem* prob, const ua_plan_t* plan) {
  if (!prob || !plan) return 0;
  return acc_offset(prob, plan->n_part);
}

static ua_status check_plan(const ua_problem* prob, const ua_plan_t* plan, int32_t path) {
  if (!prob || !plan) return UA_EINVAL;
  ua_status st = validate(prob);
  if (st != UA_OK) return st;
  if (plan->problem_hash != problem_hash(prob) || plan->path != path) return UA_EPLAN;
  if (plan->n_part < 1 || plan->block_q < 1 || plan->kernel < 0 || plan->kernel > 2)
    return UA_EPLAN;
  if (plan->grid_y < prob->num_kv_heads || plan->grid_y % prob->num_kv_heads != 0 ||
      (prob->num_q_heads / prob->num_kv_heads) % (plan->grid_y / prob->num_kv_heads) != 0 ||
      (plan->kernel != 0 && plan->grid_y != prob->num_kv_heads))
    return UA_EPLAN;
  // Wave per row block: small kernel, whole workgroups of row blocks, cache
  // blocks of whole 16-slot halves.
  if ((plan->flags & 4) &&
      (plan->kernel != 0 || plan->grid_y % kSmallWaves != 0 || prob->block_size % 16 != 0))
    return UA_EPLAN;
  return UA_OK;
}

static ua_status launch_main(const ua_problem* prob, const ua_plan_t* plan, const Params& q,
                             bool split, void* stream) {
  dim3 grid((unsigned)plan->grid_x, (unsigned)plan->grid_y, (unsigned)plan->grid_z);
  const int fmt = prob->kv_dtype == UA_FP8_E4M3FN     ? kKvE4m3fn
                  : prob->kv_dtype == UA_FP8_E4M3FNUZ ? kKvE4m3fnuz
                                                      : kKv16;
  hipError_t e = plan->kernel == 0
                     ? launch_small(q, prob->q_dtype, fmt, prob->head_dim, split, grid,
                                    (hipStream_t)stream)
                     : launch_large(q, prob->q_dtype, fmt, prob->head_dim, split,
                                    plan->kernel == 2, grid, (hipStream_t)stream);
  return e == hipSuccess ? UA_OK : UA_EHIP;
}

ua_status ua_forward_2d(const ua_problem* prob, const ua_plan_t* plan, const ua_args* args,
                        void* stream) {
  ua_status st = check_plan(prob, plan, UA_PATH_2D);
  if (st != UA_OK) return st;
  if ((st = check_args(prob, args)) != UA_OK) return st;
  if (prob->total_q == 0 || prob->num_seqs == 0) return UA_OK;
  Params q = make_params(prob, plan, args, nullptr);
  return launch_main(prob, plan, q, false, stream);
}

ua_status ua_forward_splitkv(const ua_problem* prob, const ua_plan_t* plan, const ua_args* args,
                             void* workspace, size_t workspace_bytes, void* stream) {
  ua_status st = check_plan(prob, plan, UA_PATH_SPLITKV);
  if (st != UA_OK) return st;
  if ((st = check_args(prob, args)) != UA_OK) return st;
  if (prob->total_q == 0 || prob->num_seqs == 0) return UA_OK;
  if (!workspace || workspace_bytes < plan->workspace_bytes || ((uintptr_t)workspace % 256))
    return UA_EWORKSPACE;
  Params q = make_params(prob, plan, args, workspace);
  return launch_main(prob, plan, q, true, stream);
}

ua_status ua_reduce(const ua_problem* prob, const ua_plan_t* plan, const ua_args* args,
                    const void* workspace, size_t workspace_bytes, void* stream) {
  ua_status st = check_plan(prob, plan, UA_PATH_SPLITKV);
  if (st != UA_OK) return st;
  if (!args) return UA_EINVAL;
  if (prob->total_q == 0 || prob->num_seqs == 0) return UA_OK;
  if (!args->out) return UA_EINVAL;
  if ((prob->has_sinks != 0) != (args->sinks != nullptr)) return UA_EINVAL;
  if (((uintptr_t)args->out % 16)) return UA_EUNSUPPORTED;
  if (!workspace || workspace_bytes < plan->workspace_bytes || ((uintptr_t)workspace % 256))
    return UA_EWORKSPACE;
  Params q = make_params(prob, plan, args, const_cast<void*>(workspace));
  hipError_t e = launch_reduce(q, prob->o_dtype, prob->head_dim, (hipStream_t)stream);
  return e == hipSuccess ? UA_OK : UA_EHIP;
}

ua_status ua_check_inputs(const ua_problem* prob, const ua_args* args, int32_t* flags,
                          void* stream) {
  ua_status st = validate(prob);
  if (st != UA_OK) return st;
  if (!args || !flags) return UA_EINVAL;
  if (prob->num_seqs > 0 && (!args->cu_seqlens_q || !args->seq_lens || !args->block_table))
    return UA_EINVAL;
  if (prob->num_seqs == 0 && !args->cu_seqlens_q) return UA_EINVAL;
  hipError_t e = launch_check(prob, args, flags, (hipStream_t)stream);
  return e == hipSuccess ? UA_OK : UA_EHIP;
}

ua_status ua_forward(const ua_problem* prob, const ua_plan_t* plan, const ua_args* args,
                     void* workspace, size_t workspace_bytes, void* stream) {
  if (!plan) return UA_EINVAL;
  if (plan->path == UA_PATH_2D) return ua_forward_2d(prob, plan, args, stream);
  ua_status st = ua_forward_splitkv(prob, plan, args, workspace, workspace_bytes, stream);
  if (st != UA_OK) return st;
  return ua_reduce(prob, plan, args, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace ua {
// Host checks of a split-KV call (plan, problem and argument pointers), as
// ua_forward_splitkv makes them before it needs the workspace.
ua_status check_split_call(const ua_problem* prob, const ua_plan_t* plan, const ua_args* args) {
  ua_status st = check_plan(prob, plan, UA_PATH_SPLITKV);
  if (st != UA_OK) return st;
  return check_args(prob, args);
}
}  // namespace ua
