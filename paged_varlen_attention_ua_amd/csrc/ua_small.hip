// Small-query-block attention kernel for gfx950: decode and split-KV partitions.
//
// A row block is block_q consecutive query tokens of one sequence times the
// G = Hq / Hkv query heads that share a kv head (grouped-query packing: every
// row of the block reads the same K/V rows), at most 16 rows: the N side of a
// 16x16x32 MFMA.  Decode with G > 16 (e.g. multi-query attention) splits the G
// heads into groups of at most 16, one row block each, which read the same K/V
// rows.  A workgroup of four waves owns (query block, key partition) and
// either one row block, whose interleaved 32-key tiles the four waves share
// (each keeping its own online-softmax state: running max m, sum l and output
// accumulator, AITER PR #3962 review diff, merged through LDS at the end), or
// four consecutive row blocks, one per wave, each walking every tile of the
// partition (wave per row block, see small_kernel).  With one partition the
// block writes the final rows (the one-pass form of the RocKE README, "Why
// three tables"); otherwise it writes the partition's (m, l, acc) for ua_reduce.
//
// Data flow per 32-key tile and wave (K/V data never pass through LDS):
//   * K rows go straight from HBM into registers already in the MFMA A-operand
//     layout (lane l: key key_of_row(l % 16)), and S^T = K Q^T comes out with
//     one query row per lane (row = l % 16).
//   * Because P^T then sits in the B-operand layout of O^T = V^T P^T, P stays
//     in registers; the eight keys a lane contributes are the ones its S^T
//     accumulator holds.
//   * V is loaded as whole 16-byte row pieces (four full rows per load
//     instruction) and the per-lane transposition the A operand needs is done
//     with byte permutes in registers.
//   * When block_size is a multiple of 16 each 16-key half tile lies in one
//     cache block; the block-table entries of all of a wave's tiles are fetched
//     in one lane-parallel load up front, so a tile's K/V loads never wait on a
//     block-table load of their own.  Interior tiles then need no per-lane
//     address arithmetic (a uniform half base plus fixed lane offsets) and run
//     two deep: the next tile's loads are in flight while a tile is computed.
//   * Logits are kept in the base-2 domain (pre-multiplied by log2 e, exp2 for
//     the exponentials), the README's convention (section "2D vs 2D").
//   * fp8 caches with per-token scales: each lane loads one scale per tile (K
//     or V, of a key whose score its own 16-lane row holds) and ds_bpermute
//     hands the scales to the lanes that need them; the K scale multiplies the
//     raw dot product, the V scale the probability fed to the PV MFMA (the
//     softmax sum keeps the unscaled probability).

#include <type_traits>

#include "ua_device.h"

namespace ua {
namespace {

// Running maxima of the online softmax (base-2 logit units) are kept at whole
// numbers: the maximum m a row's p = 2^(x - m) are formed against is rounded
// up to an integer.  p <= 1 still holds at the row maximum, but the mantissa
// of p is then that of 2^(x - rint(x)) whatever m is (p is formed as that
// value times an exact power of two), so the 16-bit rounding of p before
// the PV MFMA is the same in every partition, wave or tile order, and every
// rescale factor 2^(m_old - m_new) (and each partition's weight in the merge)
// is an exact power of two: split and one-pass results differ only by the
// order of fp32 additions.  -inf stays -inf.
// The row sum l that normalises O (and gives the log-sum-exp) is the sum of p
// exactly as rounded for the PV MFMA, so O / l is a convex combination of V
// rows (exact for a row that sees one key) and O and the log-sum-exp agree
// with each other; the log-sum-exp then carries the 16-bit rounding of p, at
// most ln(1 + 2^-8) for bf16 and ln(1 + 2^-11) for fp16.
__device__ __forceinline__ float integral_max(float m) { return __builtin_ceilf(m); }

// Load N dwords (N in {1, 2, 4, 8}) from a 4*N-byte aligned address.
template <int N>
__device__ __forceinline__ void load_dw(const char* ptr, uint32_t* dst) {
  if constexpr (N == 1) {
    dst[0] = *reinterpret_cast<const uint32_t*>(ptr);
  } else if constexpr (N == 2) {
    u32x2 v = *reinterpret_cast<const u32x2*>(ptr);
    dst[0] = v[0];
    dst[1] = v[1];
  } else {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      u32x4 v = *reinterpret_cast<const u32x4*>(ptr + 16 * i);
      dst[4 * i + 0] = v[0];
      dst[4 * i + 1] = v[1];
      dst[4 * i + 2] = v[2];
      dst[4 * i + 3] = v[3];
    }
  }
}

template <int QT, bool FP8, int D>
struct SmallCfg {
  static constexpr int E = D / 16;         // head-dim values per lane per V row = PV MFMAs per tile
  static constexpr int QC = D / 32;        // QK MFMAs per 16 keys
  static constexpr int DQ = D / 4;         // head-dim values per lane per K/Q row
  static constexpr int EB = FP8 ? 1 : 2;   // bytes per stored K/V element
  static constexpr int KW = DQ * EB / 4;   // dwords per lane per K row
  static constexpr int VW = E * EB / 4 > 0 ? E * EB / 4 : 1;  // dwords per lane per V row
};

// Head-dim index of element 0 of the c-th QK operand held by lane group g
// (K and Q use the same map, so the contraction covers every index once).
// 16-bit K: each load instruction covers 64 contiguous bytes of a row
// (d = 32c + 8g + j); fp8 K: each lane owns one contiguous quarter of the
// row (d = D/4 * g + 8c + j).
template <bool FP8, int D>
__device__ __forceinline__ int kq_index(int c, int g) {
  return FP8 ? (D / 4) * g + 8 * c : 32 * c + 8 * g;
}

// Key order inside a 16-key half.  S^T row i of the QK MFMA (A-operand row
// i, loaded by lanes with l % 16 == i) is key key_of_row(i) = 4 (i % 4) + i / 4,
// so the four keys a lane group g holds in its S^T accumulator (rows 4g..4g+3)
// are g, 4 + g, 8 + g, 12 + g, and the V rows a load instruction jj fetches for
// lane groups 0..3 (keys 4 jj + g) are four adjacent cache slots.
__device__ __forceinline__ int key_of_row(int i) { return 4 * (i & 3) + (i >> 2); }

template <int QT, bool FP8, int D>
struct Tile {
  using C = SmallCfg<QT, FP8, D>;
  uint32_t k[2][C::KW];
  uint32_t v[8][C::VW];
  float sc;  // per-token scale loaded by this lane (fp8 with per-token scales)
};

// K row piece of one lane (`row` = byte address of the key's head row).
template <int QT, bool FP8, int D>
__device__ __forceinline__ void load_k_row(const char* row, int g, uint32_t* dst) {
  using C = SmallCfg<QT, FP8, D>;
  if constexpr (FP8) {
    load_dw<C::KW>(row + kq_index<FP8, D>(0, g), dst);
  } else {
#pragma unroll
    for (int c = 0; c < C::QC; ++c) load_dw<4>(row + 2 * kq_index<FP8, D>(c, g), dst + 4 * c);
  }
}

// Tile loader for block_size % 16 == 0: `page[hb]` is the cache block of half
// hb (wave-uniform; -1 when the half has no loadable key).  Loads are
// unconditional: a lane whose key lies outside the tile's loadable range
// [max(kl, kt), min(k1, kt + 32)) reads the nearest loadable key instead (a
// real row of the same sequence, so finite), and the logit mask, which uses
// the true key index, gives it zero weight.  Every issued tile has at least
// one loadable key.
template <int QT, bool FP8, int D>
__device__ __forceinline__ void load_tile_paged16(Tile<QT, FP8, D>& t, const Params& p,
                                                  const char* kbase, const char* vbase, int kt,
                                                  const int32_t* page, int kl, int k1, int g,
                                                  int r16) {
  using C = SmallCfg<QT, FP8, D>;
  const int64_t slot_b = p.kv_stride_slot * C::EB;
  const int64_t blk_b = p.kv_stride_block * C::EB;
  const int klo = max(kl, kt), khi = min(k1, kt + 32) - 1;
  // Byte offset of the (page, slot) holding loadable key k of this tile.
  int64_t hoff[2];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int kb0 = kt + 16 * hb;
    const uint32_t bi = fastdiv((uint32_t)kb0, p.bs_div);
    const int slot0 = kb0 - (int)bi * p.block_size;
    hoff[hb] = (int64_t)page[hb] * blk_b + (int64_t)(slot0 - kb0) * slot_b;
  }
  auto key_off = [&](int key) -> int64_t {
    const int kc = min(max(key, klo), khi);
    return (kc - kt < 16 ? hoff[0] : hoff[1]) + (int64_t)kc * slot_b;
  };
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    load_k_row<QT, FP8, D>(kbase + key_off(kt + 16 * hb + key_of_row(r16)), g, t.k[hb]);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      load_dw<C::VW>(vbase + key_off(kt + 16 * hb + 4 * jj + g) + C::E * r16 * C::EB,
                     t.v[4 * hb + jj]);
  }
}

// Tile loader for an interior tile (block_size % 16 == 0 and all 32 keys
// loadable): half hb is slots slot0 .. slot0 + 15 of cache block page[hb], so
// every address is a wave-uniform half base plus a fixed per-lane offset
// (k_lane: key r16 and this lane's K pieces; v_lane[jj]: key 4g + jj and this
// lane's 16-byte V piece).
template <int QT, bool FP8, int D>
__device__ __forceinline__ void load_tile_fast(Tile<QT, FP8, D>& t, const Params& p,
                                               const char* kbase, const char* vbase, int kt,
                                               const int32_t* page, uint32_t k_lane,
                                               const uint32_t* v_lane) {
  using C = SmallCfg<QT, FP8, D>;
  const int64_t slot_b = p.kv_stride_slot * C::EB;
  const int64_t blk_b = p.kv_stride_block * C::EB;
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int kb0 = kt + 16 * hb;
    const uint32_t bi = fastdiv((uint32_t)kb0, p.bs_div);
    const int slot0 = kb0 - (int)bi * p.block_size;
    const int64_t half = (int64_t)page[hb] * blk_b + (int64_t)slot0 * slot_b;
    load_k_row<QT, FP8, D>(kbase + half + k_lane, 0, t.k[hb]);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) load_dw<C::VW>(vbase + half + v_lane[jj], t.v[4 * hb + jj]);
  }
}

// Tile loader for any block size: one block-table lookup per key and lane.
template <int QT, bool FP8, int D>
__device__ __forceinline__ void load_tile_any(Tile<QT, FP8, D>& t, const Params& p,
                                              const int32_t* __restrict__ bt_row,
                                              const char* kbase, const char* vbase, int kt,
                                              int kl, int k1, int g, int r16) {
  using C = SmallCfg<QT, FP8, D>;
  const int64_t slot_b = p.kv_stride_slot * C::EB;
  const int64_t blk_b = p.kv_stride_block * C::EB;
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int kb0 = kt + 16 * hb;
    {
      const int key = kb0 + key_of_row(r16);
      if (key >= kl && key < k1) {
        const uint32_t bi = fastdiv((uint32_t)key, p.bs_div);
        const int slot = key - (int)bi * p.block_size;
        const int64_t off = (int64_t)bt_row[bi] * blk_b + (int64_t)slot * slot_b;
        load_k_row<QT, FP8, D>(kbase + off, g, t.k[hb]);
      } else {
#pragma unroll
        for (int i = 0; i < C::KW; ++i) t.k[hb][i] = 0;
      }
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int key = kb0 + 4 * jj + g;
      if (key >= kl && key < k1) {
        const uint32_t bi = fastdiv((uint32_t)key, p.bs_div);
        const int slot = key - (int)bi * p.block_size;
        const int64_t off = (int64_t)bt_row[bi] * blk_b + (int64_t)slot * slot_b;
        load_dw<C::VW>(vbase + off + C::E * r16 * C::EB, t.v[4 * hb + jj]);
      } else {
#pragma unroll
        for (int i = 0; i < C::VW; ++i) t.v[4 * hb + jj][i] = 0;
      }
    }
  }
}

// A operand of the c-th QK MFMA for key half hb.
template <int QT, bool FP8, int D, bool FNUZ>
__device__ __forceinline__ u32x4 k_operand(const Tile<QT, FP8, D>& t, int hb, int c) {
  if constexpr (FP8) {
    u32x2 raw = {t.k[hb][2 * c], t.k[hb][2 * c + 1]};
    return fp8x8_to<QT, FNUZ>(raw);
  } else {
    u32x4 r = {t.k[hb][4 * c], t.k[hb][4 * c + 1], t.k[hb][4 * c + 2], t.k[hb][4 * c + 3]};
    return r;
  }
}

// A operand of the c-th PV MFMA (O^T = V^T P^T).  Lane l supplies
// V[key_j][E*(l%16) + c] for its eight keys j (j < 4: 4j + g, else
// 16 + 4(j - 4) + g: the keys its S^T accumulator holds), two keys per dword.
template <int QT, bool FP8, int D, bool FNUZ>
__device__ __forceinline__ u32x4 v_operand(const Tile<QT, FP8, D>& t, int c) {
  u32x4 op;
  if constexpr (!FP8) {
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int q = 0; q < 4; ++q) op[q] = perm_b32(t.v[2 * q + 1][c >> 1], t.v[2 * q][c >> 1], sel);
  } else {
    // Gather byte c of keys 2q and 2q+1 into the low half, then convert the pair.
    const uint32_t bc = c & 3;
    const uint32_t sel = bc | ((bc + 4) << 8) | 0x0c0c0000u;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      op[q] = fp8x2_to<QT, FNUZ>(perm_b32(t.v[2 * q + 1][c >> 2], t.v[2 * q][c >> 2], sel),
                                 false);
  }
  return op;
}

// fp8 caches: the A operands of PV MFMAs c and c + 1 (c even) together.  One
// byte permute gathers byte c of keys 2q and 2q+1 into the low half and byte
// c + 1 into the high half; the two halves convert to the two operands.
template <int QT, int D, bool FNUZ>
__device__ __forceinline__ void v_operand_pair(const Tile<QT, true, D>& t, int c, u32x4& op0,
                                               u32x4& op1) {
  const uint32_t bc = c & 3;
  const uint32_t sel = bc | ((bc + 4) << 8) | ((bc + 1) << 16) | ((bc + 5) << 24);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t w = perm_b32(t.v[2 * q + 1][c >> 2], t.v[2 * q][c >> 2], sel);
    op0[q] = fp8x2_to<QT, FNUZ>(w, false);
    op1[q] = fp8x2_to<QT, FNUZ>(w, true);
  }
}

// Float handed from lane src to this lane (ds_bpermute; byte address 4 src).
__device__ __forceinline__ float lane_get(float v, int src) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * src, __builtin_bit_cast(int, v)));
}

// HW (wave per row block): the four waves of a workgroup own four consecutive
// row blocks (unit u = kv head x head groups + group, u = 4 blockIdx.y + wave),
// each walking every tile of the partition, so at any time they read the same
// cache slots of adjacent kv heads: with the usual [block][slot][head][dim]
// cache layout that is one contiguous run of 4 head rows per slot instead of
// one head row (measured on MI355X with a load-only kernel over that layout:
// fp8 rows 4.0-4.3 -> 4.5-5.0 TB/s, 16-bit rows 4.9 -> 5.1 TB/s).  The waves
// share the staged block-table entries and need no merge.  Otherwise the four
// waves of a workgroup share one row block and interleave its tiles.
template <int QT, bool FP8, int D, bool SPLIT, bool PAGE16, bool FNUZ, bool TS, bool HW>
__global__ __launch_bounds__(64 * kSmallWaves, 2) void small_kernel(Params p) {
  using C = SmallCfg<QT, FP8, D>;
  constexpr int E = C::E;
  constexpr int QC = C::QC;
  constexpr int DQ = C::DQ;
  static_assert(!HW || PAGE16, "wave-per-row-block mode stages the block table");
  constexpr int kStride = HW ? kSmallTile : kSmallTile * kSmallWaves;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int qb = blockIdx.x, part = blockIdx.z;
  // Row block: kv head x head groups + group; decode with G > 16 splits a kv
  // head's query heads into head_groups groups of group_rows heads.
  const int unit = HW ? (int)blockIdx.y * kSmallWaves + wave : (int)blockIdx.y;
  const int HG = p.head_groups;
  const int kvh = HG == 1 ? unit : unit / HG;
  const int hg = unit - kvh * HG;

  int s, tok0;
  if (p.seq_blocks) {
    s = qb;
    tok0 = p.cu_seqlens_q[s];
  } else {
    s = find_seq(p.cu_seqlens_q, p.num_seqs, qb, p.block_q);
    const int qs = p.cu_seqlens_q[s];
    tok0 = qs + (qb - (qs / p.block_q + s)) * p.block_q;
  }
  const int q_start = p.cu_seqlens_q[s], q_end = p.cu_seqlens_q[s + 1];
  if (tok0 >= q_end) return;
  const int ntok = min(p.block_q, q_end - tok0);
  const int kv_len = p.seq_lens[s];
  const int ctx = kv_len - (q_end - q_start);
  const int p0 = ctx + (tok0 - q_start);  // position of the block's first query
  const int hi = p0 + ntok;               // keys >= hi are invisible to every row
  const int lo = p.window > 0 ? max(0, p0 - p.window + 1) : 0;
  const int lo_a = lo & ~31;
  const int plen = ((hi - lo_a + p.n_part - 1) / p.n_part + 31) & ~31;
  const int k0 = lo_a + part * plen;
  const int k1 = min(k0 + plen, hi);
  const int kl = max(k0, lo);
  const int G = p.group_rows;                    // query heads of this block per token
  const int hbase = kvh * p.group + hg * G;      // head of block row 0
  const int R = p.total_q * p.num_q_heads;

  __shared__ float sm_m[kSmallWaves][16];
  __shared__ float sm_l[kSmallWaves][16];
  __shared__ float sm_o[kSmallWaves][16][D + 4];

  if (k0 >= k1) {
    // Empty partition: l = 0 tells the reduce to skip it.
    if constexpr (SPLIT) {
      const int t16 = HW ? lane : tid;  // HW: every wave writes its own rows
      if (t16 < 16) {
        const int rt = t16 / G, rh = t16 - (t16 / G) * G;
        if (t16 < p.block_q * G && rt < ntok) {
          const int64_t row = (int64_t)(tok0 + rt) * p.num_q_heads + hbase + rh;
          p.ws_l[(int64_t)part * R + row] = 0.0f;
          p.ws_m[(int64_t)part * R + row] = -INFINITY;
        }
      }
    }
    return;
  }

  // This wave's tiles: kt = wk0 + kStride * i, i < nt.
  const int wk0 = HW ? k0 : k0 + kSmallTile * wave;
  const int nt = wk0 < k1 ? (k1 - wk0 + kStride - 1) / kStride : 0;
  const int32_t* bt_row = p.block_table + (int64_t)s * p.max_blocks_per_seq;

  // Block-table entries of this wave's first kPreTiles tiles, staged in LDS
  // (the wave's own slice; HW: one copy for the whole workgroup, whose waves
  // walk the same tiles): entry 2i + hb is the block of tile i, half hb (-1 when
  // the half has no loadable key).  Reading them later waits only on LDS, never
  // on the tile loads in flight.
  constexpr int kPreTiles = HW ? 256 * kSmallWaves : 256;
  __shared__ int32_t sm_pg_all[kSmallWaves * 2 * 256];
  int32_t* sm_pg = HW ? sm_pg_all : sm_pg_all + wave * 2 * kPreTiles;
  auto entry = [&](int j) -> int32_t {
    const int i = j >> 1;
    const int kb0 = wk0 + kStride * i + 16 * (j & 1);
    return (kb0 < k1 && kb0 + 16 > kl) ? bt_row[fastdiv((uint32_t)kb0, p.bs_div)] : -1;
  };
  if constexpr (HW) {
    const int ne = 2 * min(nt, kPreTiles);
    for (int j = tid; j < ne; j += 64 * kSmallWaves) sm_pg[j] = entry(j);
    __syncthreads();
  } else if constexpr (PAGE16) {
    const int ne = 2 * min(nt, kPreTiles);
    for (int j = lane; j < ne; j += 64) sm_pg[j] = entry(j);
  }

  // This lane's query row.
  const int rt = r16 / G, rh = r16 - rt * G;
  const bool row_ok = (r16 < p.block_q * G) && (rt < ntok);
  const int h = hbase + rh;
  const int pos = p0 + rt;
  const int row_lo = p.window > 0 ? max(kl, pos - p.window + 1) : kl;
  const int row_hi = min(k1, pos + 1);
  // Keys every row of the block sees, [vis_lo, vis_hi): the window start of
  // its last token and the causal end of its first.  Tiles inside it need no
  // per-key mask.
  const int vis_lo = p.window > 0 ? max(kl, p0 + ntok - p.window) : kl;
  const int vis_hi = min(k1, p0 + 1);
  const float slope2 = (p.alibi != nullptr && row_ok) ? p.alibi[h] * kLog2e : 0.0f;

  // Q as the B operand of S^T = K Q^T (same head-dim map as K).
  u32x4 qop[QC];
  if (row_ok) {
    const char* qp = reinterpret_cast<const char*>(p.q) +
                     ((int64_t)(tok0 + rt) * p.q_stride_tok + (int64_t)h * p.q_stride_head) * 2;
#pragma unroll
    for (int c = 0; c < QC; ++c)
      qop[c] = *reinterpret_cast<const u32x4*>(qp + 2 * kq_index<FP8, D>(c, g));
  } else {
#pragma unroll
    for (int c = 0; c < QC; ++c) qop[c] = u32x4{0, 0, 0, 0};
  }

  const char* kbase = reinterpret_cast<const char*>(p.k) + kvh * p.kv_stride_head * C::EB;
  const char* vbase = reinterpret_cast<const char*>(p.v) + kvh * p.kv_stride_head * C::EB;

  // Per-lane byte offsets inside a 16-key half (interior tiles).
  const uint32_t slot_b32 = (uint32_t)(p.kv_stride_slot * C::EB);
  const uint32_t k_lane = key_of_row(r16) * slot_b32 + kq_index<FP8, D>(0, g) * C::EB;
  uint32_t v_lane[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) v_lane[jj] = (4 * jj + g) * slot_b32 + C::E * r16 * C::EB;

  // Per-token scales (fp8 only): lane (g, r16) loads the scale of tile key
  // 16 hb + 4 r + g, hb = (r16 / 4) % 2, r = r16 % 4, from the K scales
  // (r16 < 8) or the V scales (r16 >= 8).  Offsets fit 32 bits (host check).
  constexpr bool tsc = FP8 && TS;
  const int sc_key = 16 * ((r16 >> 2) & 1) + 4 * (r16 & 3) + g;
  const float* sc_base = nullptr;
  int32_t sc_sb = 0, sc_ss = 0;
  if constexpr (tsc) {
    const bool kside = r16 < 8;
    sc_base = kside ? p.k_tscale + kvh * p.ks_stride_head : p.v_tscale + kvh * p.vs_stride_head;
    sc_sb = (int32_t)(kside ? p.ks_stride_block : p.vs_stride_block);
    sc_ss = (int32_t)(kside ? p.ks_stride_slot : p.vs_stride_slot);
  }
  // Scale of tile key kt + sc_key, clamped into the loadable range [kl, k1) of
  // the partition (a clamped key is masked; its scale is a real, finite one).
  // page2: the tile's two half-tile blocks (block_size % 16 == 0), else null.
  auto load_scale = [&](Tile<QT, FP8, D>& t, int kt, const int32_t* page2)
      __attribute__((always_inline)) {
    if constexpr (tsc) {
      {
        const int key = min(max(kt + sc_key, kl), k1 - 1);
        const uint32_t bi = fastdiv((uint32_t)key, p.bs_div);
        const int slot = key - (int)bi * p.block_size;
        const int32_t pg = page2 != nullptr ? (key - kt < 16 ? page2[0] : page2[1]) : bt_row[bi];
        t.sc = sc_base[pg * sc_sb + slot * sc_ss];
      }
    }
  };

  auto tile_pages = [&](int i, int32_t* page) __attribute__((always_inline)) {
    if (i < kPreTiles) {
      page[0] = __builtin_amdgcn_readfirstlane(sm_pg[2 * i]);
      page[1] = __builtin_amdgcn_readfirstlane(sm_pg[2 * i + 1]);
    } else {
      page[0] = entry(2 * i);
      page[1] = entry(2 * i + 1);
    }
  };
  // Any tile (clamped loads; the first and last tile of a partition).
  auto load = [&](Tile<QT, FP8, D>& t, int i) __attribute__((always_inline)) {
    const int kt = wk0 + kStride * i;
    if constexpr (PAGE16) {
      int32_t page[2];
      tile_pages(i, page);
      load_tile_paged16<QT, FP8, D>(t, p, kbase, vbase, kt, page, kl, k1, g, r16);
      load_scale(t, kt, page);
    } else {
      load_tile_any<QT, FP8, D>(t, p, bt_row, kbase, vbase, kt, kl, k1, g, r16);
      load_scale(t, kt, nullptr);
    }
  };
  // Interior tile (PAGE16 only): all 32 keys loadable.
  auto load_fast = [&](Tile<QT, FP8, D>& t, int i) __attribute__((always_inline)) {
    int32_t page[2];
    tile_pages(i, page);
    load_tile_fast<QT, FP8, D>(t, p, kbase, vbase, wk0 + kStride * i, page, k_lane, v_lane);
    load_scale(t, wk0 + kStride * i, page);
  };

  f32x4 oacc[E];
#pragma unroll
  for (int c = 0; c < E; ++c) oacc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  // l: sum of the p as rounded for the PV MFMA (with per-token V scales,
  // whose PV weights carry the scales: of the unscaled p as computed).
  float m_run = -INFINITY, l_run = 0.0f;

  auto compute = [&](const Tile<QT, FP8, D>& t, int i) {
    const int kt = wk0 + kStride * i;
    f32x4 sacc[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      sacc[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < QC; ++c)
        sacc[hb] = mfma16<QT>(k_operand<QT, FP8, D, FNUZ>(t, hb, c), qop[c], sacc[hb]);
    }
    // Per-token K scales of this lane's eight keys (from lanes 16 g + 4 hb + r).
    float ksc[8];
    if constexpr (tsc) {
#pragma unroll
      for (int j = 0; j < 8; ++j) ksc[j] = lane_get(t.sc, 16 * g + j);
    }
    // Logits in base-2 units; the feature tests are uniform, one branch each.
    float x[8];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float raw = sacc[hb][r];
        if constexpr (tsc) raw *= ksc[4 * hb + r];
        x[4 * hb + r] = raw;
      }
    }
    if (p.softcap_on) {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = p.cap_out2 * tanh_fast(x[j] * p.cap_in);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] *= p.qk_scale2;
    }
    if (p.alibi != nullptr) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = kt + 16 * hb + 4 * r + g;
          x[4 * hb + r] = x[4 * hb + r] + slope2 * (float)(key - ctx);
        }
      }
    }
    // QQ-bias qq[i][key - ctx] (i = this row's index in its chunk) on the
    // chunk's own keys; tiles wholly inside the prefix skip it.
    if (p.qq_bias != nullptr && kt + kSmallTile > ctx) {
      const float* qrow = p.qq_bias + (int64_t)(row_ok ? pos - ctx : 0) * p.qq_stride;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int rel = kt + 16 * hb + 4 * r + g - ctx;
          const float b = (row_ok && (uint32_t)rel < (uint32_t)p.qq_stride) ? qrow[rel] : 0.0f;
          x[4 * hb + r] = __builtin_fmaf(b, kLog2e, x[4 * hb + r]);
        }
    }
    const bool full = kt >= vis_lo && kt + kSmallTile <= vis_hi;  // uniform
    float mt = -INFINITY;
    if (full) {
#pragma unroll
      for (int j = 0; j < 8; ++j) mt = fmaxf(mt, x[j]);
    } else {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = kt + 16 * hb + 4 * r + g;
          const bool vis = key >= row_lo && key < row_hi;
          x[4 * hb + r] = vis ? x[4 * hb + r] : -INFINITY;
          mt = fmaxf(mt, x[4 * hb + r]);
        }
      }
    }
    mt = wave_max_xor(mt, 16);
    mt = wave_max_xor(mt, 32);
    const float m_new = integral_max(fmaxf(m_run, mt));
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    // p = 2^(x - m) as 2^(x - rint(x)) scaled by 2^(rint(x) - m) (ldexp, exact):
    // x - rint(x) is exact for every float while x - m is not (|x| < 1 < m), so
    // p's mantissa depends on x alone, never on the running maximum.  Keys more
    // than 200 below m give 0, and so do masked keys (-inf), clamped to that
    // floor first (tiles without masked keys skip the clamp).
    const float x_lo = m_use - 200.0f;
    u32x4 pb;
    float pr = 0.0f;
    auto form_p = [&](auto clamp) __attribute__((always_inline)) {
      auto pexp = [&](float xv) __attribute__((always_inline)) {
        const float xc = decltype(clamp)::value ? fmaxf(xv, x_lo) : xv;
        const float kx = __builtin_rintf(xc);
        return __builtin_amdgcn_ldexpf(fast_exp2(xc - kx), (int)(kx - m_use));
      };
      if constexpr (tsc) {
        // The PV weights carry the V scales (from lanes 16 g + 8 + 4 hb + r);
        // the softmax sum does not.
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float e0 = pexp(x[2 * q]), e1 = pexp(x[2 * q + 1]);
          pb[q] = pack2<QT>(e0 * lane_get(t.sc, 16 * g + 8 + 2 * q),
                            e1 * lane_get(t.sc, 16 * g + 9 + 2 * q));
          pr += e0 + e1;
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float e0 = pexp(x[2 * q]), e1 = pexp(x[2 * q + 1]);
          const uint32_t pk = pack2<QT>(e0, e1);
          pb[q] = pk;
          pr = add_pair<QT>(pk, pr);
        }
      }
    };
    if (full)
      form_p(std::false_type{});
    else
      form_p(std::true_type{});
    l_run = l_run * alpha + pr;
    // The integral maximum rarely moves once a row has seen its largest keys:
    // rescale the accumulators only when it moved in some lane of the wave.
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
      for (int c = 0; c < E; ++c) oacc[c] *= alpha;
    }
    if constexpr (FP8 && E % 2 == 0) {
#pragma unroll
      for (int c = 0; c < E; c += 2) {
        u32x4 op0, op1;
        v_operand_pair<QT, D, FNUZ>(t, c, op0, op1);
        oacc[c] = mfma16<QT>(op0, pb, oacc[c]);
        oacc[c + 1] = mfma16<QT>(op1, pb, oacc[c + 1]);
      }
    } else {
#pragma unroll
      for (int c = 0; c < E; ++c)
        oacc[c] = mfma16<QT>(v_operand<QT, FP8, D, FNUZ>(t, c), pb, oacc[c]);
    }
  };

  // Tile loop.  Paged caches with D <= 128 keep two tiles in flight per wave
  // (the partial first and last tiles are peeled off so that the interior
  // loop carries no clamping); otherwise one tile at a time.
  if constexpr (PAGE16 && D <= 128) {
    // Only a wave's first tile (partition or window start) and last tile
    // (partition end) can be partial; the interior tiles run two deep: the
    // next tile's loads are issued before the current tile is computed, and
    // every load of a tile is issued before the first wait on any of them.
    int i = 0;
    if (nt > 0 && wk0 < kl) {
      Tile<QT, FP8, D> t1;
      load(t1, 0);
      __builtin_amdgcn_sched_barrier(0);
      compute(t1, 0);
      i = 1;
    }
    const int ie = (nt > i && wk0 + kStride * (nt - 1) + kSmallTile > k1) ? nt - 1 : nt;
    if (i < ie) {
      Tile<QT, FP8, D> ta, tb;
      load_fast(ta, i);
      for (; i < ie; i += 2) {
        if (i + 1 < ie) load_fast(tb, i + 1);
        __builtin_amdgcn_sched_barrier(0);
        compute(ta, i);
        if (i + 1 >= ie) {
          i += 1;
          break;
        }
        if (i + 2 < ie) load_fast(ta, i + 2);
        __builtin_amdgcn_sched_barrier(0);
        compute(tb, i + 1);
      }
      i = ie;
    }
    if (i < nt) {
      Tile<QT, FP8, D> t1;
      load(t1, i);
      __builtin_amdgcn_sched_barrier(0);
      compute(t1, i);
    }
  } else {
    // One tile in flight (D = 256: a second tile does not fit beside the
    // accumulators; any block size: per-key block-table lookups).
    for (int i = 0; i < nt; ++i) {
      Tile<QT, FP8, D> t1;
      load(t1, i);
      compute(t1, i);
    }
  }

  // Row state of this wave: m_run is already the row maximum across the four
  // lanes holding a row; l needs their sum.
  float l_row = wave_sum_xor(l_run, 16);
  l_row = wave_sum_xor(l_row, 32);

  // Merge the waves' states through LDS.
  if (g == 0) {
    sm_m[wave][r16] = m_run;
    sm_l[wave][r16] = l_row;
  }
  // O^T accumulator: register (c, r) holds O[row l%16][D/4*g + E*r + c].
#pragma unroll
  for (int c = 0; c < E; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) sm_o[wave][r16][DQ * g + E * r + c] = oacc[c][r];
  __syncthreads();

  // Rows x 16 chunks of E values: each thread merges the waves' states of one
  // (row, chunk) (HW: each wave emits its own rows, four items per lane).
  constexpr int NW = HW ? 1 : kSmallWaves;
  const int w0 = HW ? wave : 0;
  for (int idx = HW ? lane : tid; idx < 256; idx += HW ? 64 : 64 * kSmallWaves) {
    const int row = idx >> 4, chunk = idx & 15;
    const int mrt = row / G, mrh = row - (row / G) * G;
    if (!(row < p.block_q * G && mrt < ntok)) continue;
    const int tok = tok0 + mrt, hh = hbase + mrh;
    float mw[NW];
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      mw[w] = sm_m[w0 + w][row];
      M = fmaxf(M, mw[w]);
    }
    const float sink2 = (!SPLIT && p.sinks != nullptr) ? p.sinks[hh] * kLog2e : -INFINITY;
    const float Mt = fmaxf(M, sink2);
    const float Ms = (Mt == -INFINITY) ? 0.0f : Mt;
    float L = 0.0f;
    float f[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      f[w] = fast_exp2(mw[w] - Ms);
      L += f[w] * sm_l[w0 + w][row];
    }
    const bool any_key = L > 0.0f;
    float o[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float a = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) a += f[w] * sm_o[w0 + w][row][E * chunk + e];
      o[e] = a;
    }
    const int64_t rrow = (int64_t)tok * p.num_q_heads + hh;
    if constexpr (SPLIT) {
      if (chunk == 0) {
        p.ws_m[(int64_t)part * R + rrow] = M;
        p.ws_l[(int64_t)part * R + rrow] = L;
      }
      float* dst = p.ws_acc + ((int64_t)part * R + rrow) * D + E * chunk;
#pragma unroll
      for (int e = 0; e < E; e += 4)
        *reinterpret_cast<f32x4*>(dst + e) = f32x4{o[e], o[e + 1], o[e + 2], o[e + 3]};
    } else {
      if (sink2 != -INFINITY) L += fast_exp2(sink2 - Ms);
      const float inv = any_key ? p.v_scale / L : 0.0f;
      uint32_t packed[E / 2];
#pragma unroll
      for (int e = 0; e < E; e += 2) packed[e / 2] = pack2<QT>(o[e] * inv, o[e + 1] * inv);
      char* dst = reinterpret_cast<char*>(p.out) +
                  ((int64_t)tok * p.o_stride_tok + (int64_t)hh * p.o_stride_head + E * chunk) * 2;
      if constexpr (E == 8) {
        *reinterpret_cast<u32x4*>(dst) = u32x4{packed[0], packed[1], packed[2], packed[3]};
      } else if constexpr (E == 16) {
        *reinterpret_cast<u32x4*>(dst) = u32x4{packed[0], packed[1], packed[2], packed[3]};
        *reinterpret_cast<u32x4*>(dst + 16) = u32x4{packed[4], packed[5], packed[6], packed[7]};
      } else {
        *reinterpret_cast<u32x2*>(dst) = u32x2{packed[0], packed[1]};
      }
      if (p.lse != nullptr && chunk == 0)
        p.lse[rrow] = (L > 0.0f) ? (Ms + fast_log2(L)) * kLn2 : -INFINITY;
    }
  }
}

template <int QT, bool FP8, int D, bool FNUZ, bool TS>
hipError_t launch_small_t(const Params& p, bool split, dim3 grid, hipStream_t stream) {
  const bool page16 = (p.block_size % 16) == 0;
  const dim3 block(64 * kSmallWaves);
  if (p.head_waves) {
    // grid.y counts row blocks; a workgroup takes kSmallWaves of them.
    if (!page16 || grid.y % kSmallWaves != 0) return hipErrorInvalidValue;
    const dim3 g4(grid.x, grid.y / kSmallWaves, grid.z);
    if (split)
      hipLaunchKernelGGL((small_kernel<QT, FP8, D, true, true, FNUZ, TS, true>), g4, block, 0, stream, p);
    else
      hipLaunchKernelGGL((small_kernel<QT, FP8, D, false, true, FNUZ, TS, true>), g4, block, 0, stream, p);
  } else if (split) {
    if (page16)
      hipLaunchKernelGGL((small_kernel<QT, FP8, D, true, true, FNUZ, TS, false>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((small_kernel<QT, FP8, D, true, false, FNUZ, TS, false>), grid, block, 0, stream, p);
  } else {
    if (page16)
      hipLaunchKernelGGL((small_kernel<QT, FP8, D, false, true, FNUZ, TS, false>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((small_kernel<QT, FP8, D, false, false, FNUZ, TS, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

template <int QT, bool FP8, bool FNUZ, bool TS>
hipError_t launch_small_d(const Params& p, int head_dim, bool split, dim3 grid,
                          hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_small_t<QT, FP8, 64, FNUZ, TS>(p, split, grid, stream);
    case 128: return launch_small_t<QT, FP8, 128, FNUZ, TS>(p, split, grid, stream);
    case 256: return launch_small_t<QT, FP8, 256, FNUZ, TS>(p, split, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

// Per-token scales are a template switch: kernels without them are unchanged.
template <int QT>
hipError_t launch_small_q(const Params& p, int kv_fmt, int head_dim, bool split, dim3 grid,
                          hipStream_t stream) {
  const bool ts = p.k_tscale != nullptr;
  switch (kv_fmt) {
    case kKv16: return launch_small_d<QT, false, false, false>(p, head_dim, split, grid, stream);
    case kKvE4m3fn:
      return ts ? launch_small_d<QT, true, false, true>(p, head_dim, split, grid, stream)
                : launch_small_d<QT, true, false, false>(p, head_dim, split, grid, stream);
    case kKvE4m3fnuz:
      return ts ? launch_small_d<QT, true, true, true>(p, head_dim, split, grid, stream)
                : launch_small_d<QT, true, true, false>(p, head_dim, split, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// One entry per query dtype; the build compiles this file once per dtype
// (UA_QT = 0: fp16, 1: bf16) so the two halves of the instantiations compile in
// parallel.  Without UA_QT both are defined.
#if !defined(UA_QT) || UA_QT == 0
hipError_t launch_small_f16(const Params& p, int kv_fmt, int head_dim, bool split, dim3 grid,
                            hipStream_t stream) {
  return launch_small_q<UA_F16>(p, kv_fmt, head_dim, split, grid, stream);
}
#endif
#if !defined(UA_QT) || UA_QT == 1
hipError_t launch_small_bf16(const Params& p, int kv_fmt, int head_dim, bool split, dim3 grid,
                             hipStream_t stream) {
  return launch_small_q<UA_BF16>(p, kv_fmt, head_dim, split, grid, stream);
}
#endif

}  // namespace ua
