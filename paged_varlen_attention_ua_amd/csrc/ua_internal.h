// Internal definitions shared by the host planner and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ua.h"

namespace ua {

// Largest query group a small-block kernel packs into its 16 MFMA rows.
constexpr int kSmallRows = 16;
// Rows of a large (prefill) query block: 32 per wave, four or eight waves.
constexpr int kLargeRows = 128;
constexpr int kLarge8Rows = 256;
// Keys per inner tile of the small-block kernel (two 16-key MFMA blocks).
constexpr int kSmallTile = 32;
// Waves per small-block workgroup; they split the key range of one block.
constexpr int kSmallWaves = 4;

// Division by a run-time invariant divisor with one multiply-high
// (Granlund & Montgomery, "Division by Invariant Integers using
// Multiplication", PLDI 1994, section 4): for d >= 1, l = ceil(log2 d),
// m = floor(2^32 (2^l - d) / d) + 1; then n / d = (umulhi(n, m) + n) >> l
// for every 32-bit n.
struct FastDiv {
  uint32_t d, m, l;
};

inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  f.l = l;
  f.m = (uint32_t)((((1ull << l) - d) << 32) / d + 1);
  return f;
}

// Everything a kernel launch needs, passed by value.
struct Params {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* block_table;
  const int32_t* cu_seqlens_q;
  const int32_t* seq_lens;
  const float* alibi;  // [Hq] or null
  const float* sinks;  // [Hq] or null
  void* out;
  float* lse;  // [total_q, Hq] or null
  const float* qq_bias;  // [>= max q_len, qq_stride] or null
  // Per-token fp8 scales (or null): key in (block b, slot t) of kv head g is
  // scaled by k_tscale[b * ks_stride_block + t * ks_stride_slot + g * ks_stride_head]
  // (and likewise v_tscale), on top of the per-tensor factors below.
  const float* k_tscale;
  const float* v_tscale;
  float* ws_m;
  float* ws_l;
  float* ws_acc;
  int64_t q_stride_tok, q_stride_head;
  int64_t o_stride_tok, o_stride_head;
  int64_t kv_stride_block, kv_stride_slot, kv_stride_head;
  int64_t ks_stride_block, ks_stride_slot, ks_stride_head;
  int64_t vs_stride_block, vs_stride_slot, vs_stride_head;
  int32_t num_seqs, total_q, num_q_heads, num_kv_heads, group;
  int32_t block_size, max_blocks_per_seq;
  FastDiv bs_div;
  int32_t block_q;      // query tokens per query block
  int32_t n_part;       // partitions (1 = one pass)
  int32_t window;       // <= 0: off
  float qk_scale2;      // scale * kf * log2(e): raw dot -> base-2 logit
  float cap_in;         // scale * kf / softcap (softcap on)
  float cap_out2;       // softcap * log2(e)
  float v_scale;        // vf
  // kf, vf: the per-tensor k_scale / v_scale for fp8 caches (1 otherwise),
  // halved for e4m3fnuz, whose codes the kernels decode to twice their value.
  int32_t softcap_on;
  int32_t seq_blocks;   // 1: block x is the sequence index (every query run fits one block)
  int32_t qq_stride;    // QQ-bias row stride (elements)
  int32_t head_groups;  // blocks per kv head along y (small kernel; 1 otherwise)
  int32_t group_rows;   // query heads per block and token: group / head_groups
  int32_t rank_order;   // 1: block x is block n_s - 1 - x / num_seqs of sequence x % num_seqs
  int32_t head_waves;   // 1: small kernel, the waves of a workgroup take consecutive row blocks
};

// Storage format of the K/V cache as the kernels see it.
enum KvFmt { kKv16 = 0, kKvE4m3fn = 1, kKvE4m3fnuz = 2 };

// Launchers (defined next to their kernels, one per query dtype).  Return
// hipError_t of the launch.
hipError_t launch_small_f16(const Params& p, int kv_fmt, int head_dim, bool split, dim3 grid,
                            hipStream_t stream);
hipError_t launch_small_bf16(const Params& p, int kv_fmt, int head_dim, bool split, dim3 grid,
                             hipStream_t stream);
hipError_t launch_large_f16(const Params& p, int kv_fmt, int head_dim, bool split,
                            bool eight_waves, dim3 grid, hipStream_t stream);
hipError_t launch_large_bf16(const Params& p, int kv_fmt, int head_dim, bool split,
                             bool eight_waves, dim3 grid, hipStream_t stream);

inline hipError_t launch_small(const Params& p, int q_dtype, int kv_fmt, int head_dim,
                               bool split, dim3 grid, hipStream_t stream) {
  return q_dtype == UA_F16 ? launch_small_f16(p, kv_fmt, head_dim, split, grid, stream)
                           : launch_small_bf16(p, kv_fmt, head_dim, split, grid, stream);
}
inline hipError_t launch_large(const Params& p, int q_dtype, int kv_fmt, int head_dim,
                               bool split, bool eight_waves, dim3 grid, hipStream_t stream) {
  return q_dtype == UA_F16
             ? launch_large_f16(p, kv_fmt, head_dim, split, eight_waves, grid, stream)
             : launch_large_bf16(p, kv_fmt, head_dim, split, eight_waves, grid, stream);
}
ua_status check_split_call(const ua_problem* prob, const ua_plan_t* plan, const ua_args* args);
hipError_t launch_reduce(const Params& p, int o_dtype, int head_dim, hipStream_t stream);
hipError_t launch_check(const ua_problem* p, const ua_args* a, int32_t* flags,
                        hipStream_t stream);

}  // namespace ua
