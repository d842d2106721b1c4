/*
 * ua.h — C ABI of unified paged, variable-length attention for MI355X (gfx950).
 *
 * The operation (RocKE unified_attention README, opening list of the parity
 * script and sections "Why three tables" / "3D vs 3D"; AITER PR #3962,
 * sections "Summary" and "Changes"): for every sequence s of a batch, its
 * q_len query tokens (rows cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1 of Q) are
 * the last q_len positions of a sequence of kv_len = seq_lens[s] keys held in
 * a paged K/V cache.  Query i of the sequence sits at position
 * ctx + i, ctx = kv_len - q_len, and attends causally to keys j <= ctx + i
 * (and, with a sliding window W > 0, only to keys j > ctx + i - W).  Each
 * query head h reads kv head h / (Hq / Hkv) (grouped-query attention).  Key j
 * is row (j % block_size) of cache block block_table[s][j / block_size].
 * The logit of key j is
 *     x = scale * <q, k_j>                    (k_j dequantised for fp8 KV, below)
 *     x = softcap * tanh(x / softcap)         if softcap > 0
 *     x = x + alibi_slopes[h] * (j - ctx)     if alibi_slopes != NULL
 * and the output row is sum_j softmax(x)_j * v_j (v_j dequantised for fp8),
 * where an optional per-head sink logit sinks[h] joins the softmax
 * normaliser but has no value row (README section "Prefill-2D trace cohort").
 * A row that sees no key is written as zeros (AITER PR #3962 review reply).
 * fp8 K/V (AITER PR #3962, section "Testing": both e4m3 dialects, per-tensor
 * and per-token scales, K and V scales with their own strides): the stored
 * code's value times k_scale (v_scale), times, when has_kv_token_scales, the
 * fp32 per-token scale of the key's (block, slot, kv head).
 *
 * Two equivalent forms are offered (README "Why three tables"):
 *   ua_forward_2d      one pass: one workgroup per (query block, kv head);
 *   ua_forward_splitkv + ua_reduce
 *                      split-KV / flash-decoding: each query block's visible
 *                      key range is cut into n_part partitions whose partial
 *                      softmax states go to a caller-owned fp32 workspace and
 *                      are merged by ua_reduce (AITER PR #3962 "Summary").
 * ua_plan chooses between them from host integers only (no device sync).
 *
 * Threading / ownership: every pointer in ua_args and the workspace are
 * device memory owned by the caller; the library allocates no device memory,
 * keeps no state between calls and never synchronises the device.  Calls are
 * asynchronous on the given stream (a hipStream_t passed as void*, NULL = the
 * default stream).  Two calls in flight at once on different streams need
 * different workspaces.
 *
 * Errors: every entry point returns a ua_status.  Violations detectable on
 * the host are reported synchronously and nothing is launched.  Device-side
 * data preconditions are NOT checked: 0 <= q_len <= kv_len <= max_seqlen_k,
 * q_len <= max_seqlen_q, non-decreasing cu_seqlens_q with cu_seqlens_q[0] = 0
 * and cu_seqlens_q[num_seqs] = total_q, block-table entries in [0, num_blocks)
 * for every block a sequence uses.  Violating them is undefined behaviour;
 * ua_check_inputs checks them on the device without faulting (debugging aid).
 */
#ifndef UA_H
#define UA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define UA_ABI_VERSION 5

/* UA_FP8_E4M3FN: OCP E4M3 (bias 7, max 448, no inf, NaN = S.1111.111).
 * UA_FP8_E4M3FNUZ: E4M3 with bias 8 (max 240, no inf, no -0, NaN = 0x80). */
typedef enum { UA_F16 = 0, UA_BF16 = 1, UA_FP8_E4M3FN = 2, UA_FP8_E4M3FNUZ = 3 } ua_dtype;

typedef enum {
  UA_OK = 0,
  UA_EINVAL = -1,       /* malformed problem or argument */
  UA_EUNSUPPORTED = -2, /* well-formed but not implemented (head size, dtype mix, alignment) */
  UA_EWORKSPACE = -3,   /* workspace missing or smaller than plan->workspace_bytes */
  UA_EHIP = -4,         /* a HIP launch reported an error */
  UA_EPLAN = -5,        /* plan does not belong to this problem, or wrong path for this call */
  UA_ESCRATCH = -6      /* ua_forward_noalloc: plan needs more than UA_NOALLOC_SCRATCH_BYTES */
} ua_status;

typedef enum { UA_PATH_AUTO = 0, UA_PATH_2D = 1, UA_PATH_SPLITKV = 2 } ua_path;

/* Host-side description of one call.  Every field is a host value. */
typedef struct {
  int32_t num_seqs;            /* sequences in the batch, >= 0 */
  int32_t total_q;             /* query tokens = cu_seqlens_q[num_seqs] */
  int32_t num_q_heads;         /* Hq */
  int32_t num_kv_heads;        /* Hkv; Hq % Hkv == 0 */
  int32_t head_dim;            /* D in {64, 128, 256} */
  int32_t block_size;          /* slots per cache block, >= 1 */
  int64_t num_blocks;          /* blocks in each cache (dimension 0) */
  int32_t max_blocks_per_seq;  /* block_table row stride (entries) */
  int32_t max_seqlen_q;        /* upper bound of q_len over the batch */
  int32_t max_seqlen_k;        /* upper bound of kv_len over the batch */
  int32_t q_dtype;             /* ua_dtype: UA_F16 or UA_BF16 */
  int32_t kv_dtype;            /* q_dtype, UA_FP8_E4M3FN or UA_FP8_E4M3FNUZ */
  int32_t o_dtype;             /* must equal q_dtype */
  float scale;                 /* logit scale, finite */
  float softcap;               /* <= 0: off */
  int32_t window;              /* <= 0: off; else keys p-window < j <= p */
  float k_scale, v_scale;      /* fp8 per-tensor dequantisation scales (ignored otherwise) */
  int32_t has_alibi;           /* args->alibi_slopes is [Hq] fp32 */
  int32_t has_sinks;           /* args->sinks is [Hq] fp32, natural-log units */
  /* Strides in elements.  The head_dim axis is contiguous.  Q and O are
   * [total_q, Hq, D]; each cache is [num_blocks, block_size, Hkv, D]. */
  int64_t q_stride_tok, q_stride_head;
  int64_t o_stride_tok, o_stride_head;
  int64_t kv_stride_block, kv_stride_slot, kv_stride_head;
  /* QQ-bias (RocKE unified_attention README, sections "Scenarios" and "2D vs
   * 2D"): when has_qq_bias, args->qq_bias is one fp32 matrix shared by every
   * head and sequence, row stride qq_bias_stride elements, at least
   * max_seqlen_q rows; qq_bias[i * stride + (j - ctx)] (natural-log units) is
   * added to the logit of query i of a sequence's chunk for keys j >= ctx
   * (ctx = kv_len - q_len), after softcap and with ALiBi.  Requires
   * qq_bias_stride >= max_seqlen_q. */
  int32_t has_qq_bias;
  int32_t qq_bias_stride;
  /* Per-token fp8 scales (AITER PR #3962, section "Testing" and review reply):
   * when has_kv_token_scales (fp8 kv_dtype only), args->k_token_scales and
   * args->v_token_scales are fp32 arrays; the key in slot t of block b, kv head
   * g, is dequantised with k_token_scales[b * ks_stride_block + t *
   * ks_stride_slot + g * ks_stride_head] (V likewise with the vs_ strides),
   * multiplied with k_scale / v_scale.  Strides in elements, >= 0 (0
   * broadcasts).  Entries of slots no sequence uses are never read. */
  int32_t has_kv_token_scales;
  int32_t reserved0;           /* must be 0 */
  int64_t ks_stride_block, ks_stride_slot, ks_stride_head;
  int64_t vs_stride_block, vs_stride_slot, vs_stride_head;
} ua_problem;

/* Output of ua_plan; treat as opaque except path, n_part and workspace_bytes. */
typedef struct {
  int32_t path;             /* UA_PATH_2D or UA_PATH_SPLITKV, never AUTO */
  int32_t kernel;           /* 0: small query blocks (<= 16 rows), 1: large (128 rows,
                               MFMA prefill), 2: large with 256 rows (head_dim <= 128) */
  int32_t block_q;          /* query tokens per query block */
  int32_t n_part;           /* key-range partitions per query block (1 for 2D) */
  int32_t grid_x, grid_y, grid_z; /* grid_y = kv heads x head groups (small kernel: decode
                                     with G > 16 splits a kv head's query heads) */
  int32_t flags;            /* bit 0: one query block per sequence (block x = sequence);
                               bit 1: rank order (block x = block n_s - 1 - x / num_seqs
                               of sequence x % num_seqs: heaviest blocks first);
                               bit 2: wave per row block (small kernel: each wave of
                               a workgroup owns one of grid_y's row blocks and walks
                               the whole partition; needs grid_y % 4 == 0 and
                               block_size % 16 == 0, else calls return UA_EPLAN) */
  uint64_t workspace_bytes; /* bytes ua_forward_splitkv needs; 0 for 2D */
  uint64_t problem_hash;    /* ties the plan to the ua_problem it was made for */
} ua_plan_t;

/* Device pointers of one call (all caller-owned). */
typedef struct {
  const void* q;               /* [total_q, Hq, D] q_dtype, 16-byte aligned rows */
  const void* k_cache;         /* [num_blocks, block_size, Hkv, D] kv_dtype */
  const void* v_cache;         /* same layout as k_cache */
  const int32_t* block_table;  /* [num_seqs, max_blocks_per_seq] */
  const int32_t* cu_seqlens_q; /* [num_seqs + 1] */
  const int32_t* seq_lens;     /* [num_seqs] kv_len per sequence */
  const float* alibi_slopes;   /* [Hq] or NULL (must match has_alibi) */
  const float* sinks;          /* [Hq] or NULL (must match has_sinks) */
  void* out;                   /* [total_q, Hq, D] o_dtype */
  float* lse;                  /* optional [total_q, Hq] fp32 log-sum-exp (natural log,
                                  sink included; -inf for a row that sees nothing
                                  and has no sink), or NULL.  It is the log of the
                                  normaliser the output was divided by; the weights
                                  enter the P*V product rounded to q_dtype (small
                                  query blocks sum them as rounded), so it is within
                                  ln(1 + 2^-8) (bf16) or ln(1 + 2^-11) (fp16) of
                                  the exact value. */
  const float* qq_bias;        /* [>= max_seqlen_q, qq_bias_stride] fp32 or NULL
                                  (must match has_qq_bias) */
  const float* k_token_scales; /* per-token K scales or NULL (must match
                                  has_kv_token_scales) */
  const float* v_token_scales; /* per-token V scales or NULL (likewise) */
} ua_args;

/*
 * ua_plan: validate the problem and choose the path.
 *   num_cus       compute units of the device (hipDeviceProp_t::multiProcessorCount);
 *                 <= 0 means 256 (MI355X).
 *   force_path    UA_PATH_AUTO lets the dispatcher choose (2D when its grid fills
 *                 the device or the visible key range is short; split-KV when the
 *                 grid underfills and the key walk is long — AITER PR #3962
 *                 "Changes", README "Why three tables"); 2D or SPLITKV forces it.
 *   force_n_part  0 = automatic; >= 1 sets the partition count of the split path
 *                 (partitions always cover each query block's whole visible range).
 * Pure host function: touches no device and may be called without a GPU.
 */
ua_status ua_plan(const ua_problem* prob, int32_t num_cus, int32_t force_path,
                  int32_t force_n_part, ua_plan_t* plan);

/* One-pass form; requires plan->path == UA_PATH_2D. */
ua_status ua_forward_2d(const ua_problem* prob, const ua_plan_t* plan, const ua_args* args,
                        void* stream);

/*
 * Split-KV partition pass; requires plan->path == UA_PATH_SPLITKV and a
 * workspace of at least plan->workspace_bytes (256-byte aligned).  Writes,
 * for every query row r (token, head) and partition p, fp32 values
 *   m[p][r]   the base-2 reference the partition's weights are taken against:
 *             within 8 of the largest base-2 logit (x * log2 e) over the
 *             partition's visible keys (small query blocks, plan->kernel 0:
 *             that largest logit rounded up to an integer; large query blocks
 *             at head dim 256: at most 64 below it for bf16 queries, 15 for
 *             fp16, never above it),
 *   l[p][r]   sum of the weights w = 2^(x*log2e - m) over those keys (0: the
 *             partition saw nothing),
 *   acc[p][r][D]  sum of w * v (v without v_scale),
 * at workspace offsets 0, P*R*4 and ua_workspace_acc_offset(), P = n_part,
 * R = total_q*Hq.  Entries with l == 0 leave m and acc unspecified.  Does not
 * write args->out.
 */
ua_status ua_forward_splitkv(const ua_problem* prob, const ua_plan_t* plan, const ua_args* args,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Merge the partition states of ua_forward_splitkv into args->out (and
 * args->lse): M = max over partitions with l > 0 (and the sink), L = sum
 * l_p 2^(m_p - M) (+ 2^(sink*log2e - M)), out = v_scale * sum acc_p 2^(m_p - M) / L,
 * lse = (M + log2 L) ln 2, zeros when no partition saw a key (AITER PR #3962
 * review reply).
 */
ua_status ua_reduce(const ua_problem* prob, const ua_plan_t* plan, const ua_args* args,
                    const void* workspace, size_t workspace_bytes, void* stream);

/* Convenience: run the planned path (2D, or split-KV then reduce). */
ua_status ua_forward(const ua_problem* prob, const ua_plan_t* plan, const ua_args* args,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Byte offset of the acc array inside the split-KV workspace. */
uint64_t ua_workspace_acc_offset(const ua_problem* prob, const ua_plan_t* plan);

/* Static string for a status code. */
const char* ua_status_string(int32_t status);

/* Violation bits written by ua_check_inputs. */
#define UA_CHECK_CU 1     /* cu_seqlens_q[0] != 0, decreasing, or last != total_q */
#define UA_CHECK_QLEN 2   /* some q_len > max_seqlen_q */
#define UA_CHECK_KVLEN 4  /* some kv_len < 0, < q_len or > max_seqlen_k */
#define UA_CHECK_BLOCK 8  /* a block-table entry a sequence uses is outside [0, num_blocks) */

/*
 * ua_check_inputs: debugging aid for the device-side data preconditions the
 * forward entry points do not check (see "Errors" above).  Launches one small
 * workgroup on `stream` that reads cu_seqlens_q, seq_lens and, per sequence,
 * the first ceil(kv_len / block_size) block-table entries (kv_len clamped to
 * the row), and stores the OR of the UA_CHECK_* bits that apply (0: all
 * preconditions hold) to flags[0], a caller-owned device int32.  Reads stay
 * inside the arrays the problem sizes, whatever their contents; nothing is
 * trapped.  The result is valid once the stream reaches the launch.  Returns
 * UA_EINVAL for an invalid problem or missing pointers, UA_EHIP on a launch
 * error.
 */
ua_status ua_check_inputs(const ua_problem* prob, const ua_args* args, int32_t* flags,
                          void* stream);

/*
 * ua_forward_noalloc: ua_forward without a caller workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same problem, plan and arguments
 * as ua_forward; the one-pass path runs as ua_forward_2d; the split-KV path
 * keeps its partition states in a static device array of the library,
 * UA_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends (looked up
 * once per device on the first call there).  Allocates nothing.
 *   Returns UA_ESCRATCH (nothing launched) when plan->workspace_bytes exceeds
 *   UA_NOALLOC_SCRATCH_BYTES: use ua_forward with a workspace, or a plan with
 *   fewer partitions.  UA_EINVAL when `stream` is not on the current device.
 *   Other statuses as ua_forward.
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (two streams, two threads) race and give undefined results.
 * The array keeps the last call's contents; nothing in it needs clearing.
 */
#define UA_NOALLOC_SCRATCH_BYTES (64ull << 20)
ua_status ua_forward_noalloc(const ua_problem* prob, const ua_plan_t* plan, const ua_args* args,
                             void* stream);

/* UA_ABI_VERSION of the built library. */
int32_t ua_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* UA_H */
