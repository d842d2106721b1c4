// Large-query-block attention kernel for gfx950: prefill and chunked prefill.
//
// One workgroup owns (query block, kv head, key partition); a query block is
// block_q = 32 NW / G tokens times the G query heads of the kv head (grouped
// rows share every K/V tile).  NW = 4 or 8 waves own 32 rows each; every K/V
// tile staged in LDS serves all of them, so 8 waves halve the K/V reads per
// flop (they come from L2 and bound long chunks); their two halves of four
// waves run half a tile apart, one half's MFMAs between two barriers while the
// other half runs its softmax.  Per 64-key tile (32 keys for head dim 256):
//   * the byte offsets of the tile's K/V rows are looked up through the block
//     table one tile ahead (its entries for the workgroup's key range are
//     staged in LDS once) by one wave, into a small LDS table;
//   * the rows are copied HBM -> LDS with global_load_lds_dwordx4 (16-bit
//     caches; no register staging) or through registers with the fp8 -> 16-bit
//     conversion (fp8 caches), into double-buffered 256-byte-aligned rows whose
//     16-byte slots are XOR-swizzled so that both read patterns below are
//     free of LDS bank conflicts;
//   * S^T = K Q^T on 32x32x16 MFMA (A = K from LDS, B = Q held in registers),
//     so each lane owns one query row and 16 keys of each 32-key block;
//   * online softmax in the base-2 domain (README section "2D vs 2D") on the
//     raw dot products (the logit scale is applied inside the one FMA that
//     feeds exp2), with the running maximum only moved when a tile's maximum
//     exceeds it by more than 8 (exact up to rounding: every key of a row is
//     scaled by the same maximum between moves, and p <= 2^8 stays
//     representable); eight-wave groups form p against the running maximum
//     first and take the tile maximum only when a lane's sum of p exceeds
//     2^8; head dim 256 instead holds each row's first maximum and runs the
//     tiles again from the largest one in the rare case a later tile exceeds
//     it by more than the P type can carry;
//   * causal, window and range masks are applied only on tiles that need them
//     (the mask-phase split of the README's "BLOCK_M=128" section);
//   * O^T = V^T P^T on 32x32x16 MFMA: P^T is already the B operand in the
//     registers the S^T accumulator left it in, and V^T comes from
//     ds_read_b64_tr_b16 transposed LDS reads (README "3D vs 3D");
//   * fp8 caches with per-token scales: the wave that looks up a tile's rows
//     also loads the tile's K and V scales into a three-deep LDS ring; the K
//     scale multiplies the raw dot product and the V scale the probability
//     fed to the PV MFMA (the softmax sum keeps the unscaled probability).
// Output: the final rows (one pass) or the partition's (m, l, acc) (split).

#include <type_traits>

#include "ua_device.h"

namespace ua {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Transposed LDS read: within each 16-lane group, lane s gives the address of
// 4 consecutive 16-bit values of row s/4 (columns 4(s%4)..+3) of a 4 x 16
// block; lane i receives column i of the 4 rows.
__device__ __forceinline__ u32x2 lds_read_tr16(const char* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)((__attribute__((address_space(3))) char*)(p)));
  return __builtin_bit_cast(u32x2, v);
#else
  (void)p;
  return u32x2{0, 0};
#endif
}

// The same read at a 32-bit LDS byte address.
__device__ __forceinline__ u32x2 lds_read_tr16_at(uint32_t a) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)a);
  return __builtin_bit_cast(u32x2, v);
#else
  (void)a;
  return u32x2{0, 0};
#endif
}

// LDS byte address of buffer p plus off, formed by one VALU add where it is
// written (so the compiler neither keeps a copy per buffer live across the
// loop nor splits it into one add per immediate offset).
__device__ __forceinline__ uint32_t lds_offset_add(const char* p, int off) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t base =
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)(p);
  uint32_t r;
  asm volatile("v_add_u32 %0, %1, %2" : "=v"(r) : "s"(base), "v"(off));
  return r;
#else
  (void)p;
  return (uint32_t)off;
#endif
}

// Asynchronous 16-byte copy global -> LDS: lane i's 16 bytes land at
// lds_uniform + 16 i (the LDS address is wave-uniform, passed in M0).
// Completion is tracked by vmcnt.  Issued as inline assembly so that the
// compiler does not track it: its wait insertion cannot tell the ring buffer
// being copied into from the one being read and would drain every copy in
// flight before each LDS read.  The kernel waits for each tile explicitly
// (wait_vmem_n, then a barrier); vmcnt completes in issue order, so waits the
// compiler computes for its own loads can only wait longer, never shorter.
// M0 has no other use in this kernel.
__device__ __forceinline__ void load_lds16(const char* src, char* lds_uniform) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds_uniform);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0v), "v"(src)
               : "memory");
#else
  (void)src;
  (void)lds_uniform;
#endif
}

// Wait until every global load of this wave (including LDS copies) is done.
__device__ __forceinline__ void wait_vmem() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt and lgkmcnt not waited on
}

// Workgroup barrier that orders LDS only: this wave's LDS reads and writes
// have completed (lgkmcnt(0)) before it arrives.  DMA copies into LDS are not
// drained (__syncthreads() would wait for every outstanding global load,
// including copies of tiles needed only several steps later); the ring waits
// for exactly the tile it needs with wait_vmem_n before arriving.  The empty
// asm statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt not waited on
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait until at most N of this wave's global loads are outstanding (gfx9
// s_waitcnt: vmcnt bits 3:0 and 15:14; expcnt and lgkmcnt not waited on).
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

template <int D, int NW>
struct LargeCfg {
  static constexpr int TK = D > 128 ? 32 : 64;  // keys per tile
  static constexpr int NC = D / 8;               // 16-byte slots per K/V row (16-bit values)
  static constexpr int ROWB = 2 * D;             // LDS bytes per row
  static constexpr int TILEB = TK * ROWB;        // LDS bytes per K (or V) tile buffer
  static constexpr int NT = 64 * NW;             // threads per workgroup
  static constexpr int BPW = TILEB / 1024 / NW;  // 1 KiB copy blocks per wave per buffer
  static constexpr int KB = TK / 32;             // 32-key blocks per tile
  static constexpr int QC = D / 16;              // QK MFMAs per 32-key block
  static constexpr int DB = D / 32;              // PV output blocks of 32 head-dim rows
  static constexpr int CPT = TK * NC / NT;       // slots per thread per tile (fp8 staging)
  static constexpr int MAXPG = 2048;             // block-table entries staged in LDS
  static_assert(BPW >= 1 && CPT >= 1, "tile too small for the workgroup");
};

// Physical 16-byte slot of logical slot c in LDS row r is c ^ swz<D>(r).
// gfx950 LDS serves 256 bytes (64 banks) per cycle: 16 lanes of a 16-byte
// read, 32 lanes of an 8-byte read.  The K reads (16 consecutive rows, one
// slot) need swz to be one-to-one on those rows' bank groups; the transposed
// V reads (4 consecutive rows x 4 consecutive slots starting at a multiple of
// 4) need the 16 (row, slot) pairs to land on 16 different bank groups.
// D >= 128 (rows of >= 16 slots): swz(r) = 4 (r mod 4) + (r / 4) mod 4.
// D = 64 (rows of 8 slots, two rows per 256 bytes): swz(r) = 4 ((r / 2) mod 2)
// + (r / 4) mod 4.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D >= 128)
    return ((r & 3) << 2) | ((r >> 2) & 3);
  else
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

template <bool FP8, int D, int NW>
struct Stage {
  // fp8 staging only: 8 codes (2 dwords) per slot.
  uint32_t k[FP8 ? LargeCfg<D, NW>::CPT : 1][2];
  uint32_t v[FP8 ? LargeCfg<D, NW>::CPT : 1][2];
};

// Ring slots of the per-token scale buffer (one dummy slot without scales).
template <bool ON>
constexpr int tsc_lds() {
  return ON ? 3 : 1;  // per-token scales exist for fp8 only, whose ring is two deep
}

// Workgroups per CU the register budget is sized for: two waves per SIMD
// (four-wave groups, D <= 128; eight-wave groups), one for D = 256.  D = 64
// with per-token fp8 scales, whose scale loads and conversions leave the most
// latency to hide, runs three four-wave groups per CU (measured on MI355X:
// 13% faster on a 64q/8kv 4 x 1k-behind-4k prefill, at the cost of 8-24 bytes
// per lane of spills).  The other four-wave D = 64 variants (<= 168 VGPRs)
// already fit three groups per CU.
template <int D, int NW, bool TSC>
constexpr int large_min_groups() {
  return NW == 8 ? 1 : (D > 128 ? 1 : (D == 64 && TSC ? 3 : 2));
}

template <int QT, bool FP8, int D, bool SPLIT, bool FNUZ, bool TS, int NW>
__global__ __launch_bounds__(64 * NW, (large_min_groups<D, NW, FP8 && TS>())) void large_kernel(Params p) {
  using C = LargeCfg<D, NW>;
  constexpr int TK = C::TK;
  constexpr int ROWB = C::ROWB;
  // Eight-wave groups exist for 16-bit caches only (their launcher) and run
  // the two-half interval schedule.
  constexpr bool kPingPong = NW == 8;
  static_assert(NW == 4 || !FP8, "eight-wave groups read 16-bit caches");
  // K/V tile ring: NBUF buffers each.  Eight-wave groups (one per CU, LDS to
  // spare) run four deep, with each tile's copy issued two tiles (four
  // intervals) before it is first read; four-wave groups two deep, the copy of
  // tile t + 1 in flight while tile t is computed (measured on MI355X: a
  // four-deep ring was 7% slower for D = 256).
  constexpr int NBUF = NW == 8 ? 4 : 2;
  // Ring buffers: K of slot b at sRing + b * TILEB, V at sRing + (NBUF + b) * TILEB.
  __shared__ __attribute__((aligned(1024))) char sRing[2 * NBUF * C::TILEB];
  // Row-offset table of tile t in slot t % NBUF.
  __shared__ int64_t sTab[NBUF][TK];
  __shared__ int32_t sm_pg[C::MAXPG];
  // Per-token scales of tile t in ring slot t % (NBUF + 1): [slot][0: K, 1: V][key].
  __shared__ __attribute__((aligned(16))) float sSc[tsc_lds<FP8 && TS>()][2][TK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g2 = lane >> 5;

  // XCD-aware order: consecutive logical blocks (the query blocks of one kv
  // head and partition, which read the same K/V) stay on one XCD; heavier
  // (later) query blocks go first (p.rank_order: logical block x is block
  // n_s - 1 - x / num_seqs of sequence x % num_seqs, so the last, heaviest
  // block of every sequence is dispatched before any sequence's second-last).
  const int gx = gridDim.x, gy = gridDim.y;
  const int nwg = gx * gy * gridDim.z;
  int lin = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
  if ((nwg & 7) == 0) lin = (lin & 7) * (nwg >> 3) + (lin >> 3);
  const int qb = gx - 1 - (lin % gx);
  const int kvh = (lin / gx) % gy;
  const int part = lin / (gx * gy);

  int s, tok0;
  if (p.rank_order) {
    const int r = lin % gx;  // rank from the end of the sequence: 0 first
    s = r % p.num_seqs;
    const int qs = p.cu_seqlens_q[s];
    const int nb = (p.cu_seqlens_q[s + 1] - qs + p.block_q - 1) / p.block_q;
    tok0 = qs + (nb - 1 - r / p.num_seqs) * p.block_q;  // r / num_seqs >= nb: no block
    if (r / p.num_seqs >= nb) return;
  } else if (p.seq_blocks) {
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
  const int p0 = ctx + (tok0 - q_start);
  const int hi = p0 + ntok;
  const int lo = p.window > 0 ? max(0, p0 - p.window + 1) : 0;
  const int lo_a = (lo / TK) * TK;
  const int plen = ((hi - lo_a + p.n_part - 1) / p.n_part + TK - 1) / TK * TK;
  const int k0 = lo_a + part * plen;
  const int k1 = min(k0 + plen, hi);
  const int kl = max(k0, lo);
  const int G = p.group;
  const int R = p.total_q * p.num_q_heads;
  const int nrows = p.block_q * G;

  // This lane's row (wave owns rows 32*wave .. 32*wave + 31).
  const int row = 32 * wave + l32;
  const int rt = row / G, rh = row - rt * G;
  const bool row_ok = row < nrows && rt < ntok;
  const int h = kvh * G + rh;
  const int pos = p0 + rt;

  if (k0 >= k1) {
    if constexpr (SPLIT) {
      if (g2 == 0 && row_ok) {
        const int64_t rr = (int64_t)(tok0 + rt) * p.num_q_heads + h;
        p.ws_l[(int64_t)part * R + rr] = 0.0f;
        p.ws_m[(int64_t)part * R + rr] = -INFINITY;
      }
    }
    return;
  }

  // Wave-uniform position range of this wave's rows, for the mask-free test.
  const int w_row0 = 32 * wave;
  const int w_rowl = min(32 * wave + 31, nrows - 1);
  const int wave_pmin = p0 + min(w_row0 / G, ntok - 1);
  const int wave_pmax = p0 + min(w_rowl / G, ntok - 1);
  const bool wave_live = w_row0 < nrows && w_row0 / G < ntok;

  const int row_lo = p.window > 0 ? max(kl, pos - p.window + 1) : kl;
  const int row_hi = min(k1, pos + 1);
  const float slope2 = (p.alibi != nullptr && row_ok) ? p.alibi[h] * kLog2e : 0.0f;
  // Softcap, ALiBi and QQ-bias (not in eight-wave groups, whose launcher
  // refuses them).
  const bool general = NW == 4 && (p.softcap_on || p.alibi != nullptr || p.qq_bias != nullptr);

  // Q as the B operand of S^T = K Q^T: lane holds Q[row][16c + 8*g2 .. + 8].
  u32x4 qop[C::QC];
  if (row_ok) {
    const char* qp = reinterpret_cast<const char*>(p.q) +
                     ((int64_t)(tok0 + rt) * p.q_stride_tok + (int64_t)h * p.q_stride_head) * 2;
#pragma unroll
    for (int c = 0; c < C::QC; ++c)
      qop[c] = *reinterpret_cast<const u32x4*>(qp + (16 * c + 8 * g2) * 2);
  } else {
#pragma unroll
    for (int c = 0; c < C::QC; ++c) qop[c] = u32x4{0, 0, 0, 0};
  }

  const int32_t* bt_row = p.block_table + (int64_t)s * p.max_blocks_per_seq;
  constexpr int EB = FP8 ? 1 : 2;
  const char* kbase = reinterpret_cast<const char*>(p.k) + kvh * p.kv_stride_head * EB;
  const char* vbase = reinterpret_cast<const char*>(p.v) + kvh * p.kv_stride_head * EB;
  const int64_t slot_b = p.kv_stride_slot * EB;
  const int64_t blk_b = p.kv_stride_block * EB;

  f32x16 oacc[C::DB];
#pragma unroll
  for (int d = 0; d < C::DB; ++d) oacc[d] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;
  // Head dim 256 in four-wave groups keeps O in AGPRs, where any rescale of it
  // inside the tile loop (however written) made the compiler copy all 128
  // accumulators to VGPRs on every tile (measured on MI355X: the 8k prompt at
  // D = 256 ran at 670 TFLOP/s with the copies, 800 without).  So the running
  // maximum is held: a row's first visible tile sets it (O and l are still
  // zero then) and p = 2^(x - m) stays at or below 2^kHoldSpan unless a later
  // tile's maximum exceeds it by more than that; then the workgroup runs its
  // tiles a second time from each row's largest maximum (m_seen), which no tile
  // can exceed.  l is then the sum of p as rounded for the PV MFMA (see below).
  // The span keeps p finite in the P type: 2^15 < 65504, the largest finite
  // fp16 value; bf16 has the exponent range of fp32.
  constexpr bool kHold = D > 128 && NW == 4;
  constexpr float kHoldSpan = QT == UA_F16 ? 15.0f : 64.0f;
  float m_seen = -INFINITY;
  bool redo = false;
  const float c2 = p.qk_scale2;

  // Stage the block-table entries of the workgroup's key range [kl, k1).
  const int pg_first = (int)fastdiv((uint32_t)kl, p.bs_div);
  {
    const int npg = min((int)fastdiv((uint32_t)(k1 - 1), p.bs_div) - pg_first + 1, C::MAXPG);
    for (int j = tid; j < npg; j += C::NT) sm_pg[j] = bt_row[pg_first + j];
  }
  // Every load issued so far (Q operands, slopes, block-table entries) has
  // landed: from here on outstanding vector loads are the tile copies, and no
  // compiler-placed wait for these registers can fall inside the copy ring.
  wait_vmem();
  __syncthreads();

  // Row byte offsets (page * block stride + slot * slot stride) of keys
  // kt .. kt + TK - 1, each clamped into [kl, k1 - 1]: a key outside the range
  // reads a real row of the sequence (finite values) whose score is masked.
  // With per-token scales the lane also loads its key's K and V scales into
  // sc_k / sc_v (offsets fit 32 bits: host check); store_sc puts them in the
  // ring once they have arrived.
  constexpr bool tsc = FP8 && TS;
  float sc_k = 0.0f, sc_v = 0.0f;
  auto fill_tab = [&](int64_t* tab, int kt) __attribute__((always_inline)) {
    if (lane < TK) {
      const int key = min(max(kt + lane, kl), k1 - 1);
      const uint32_t bi = fastdiv((uint32_t)key, p.bs_div);
      const int slot = key - (int)bi * p.block_size;
      const int j = (int)bi - pg_first;
      int32_t page;
      if (j < C::MAXPG) {
        page = sm_pg[j];
      } else {
        // Rare (ranges beyond the staged entries): settle this load here so
        // that the common path waits on LDS only, not on the copies in flight.
        page = bt_row[bi];
        wait_vmem();
      }
      tab[lane] = (int64_t)page * blk_b + (int64_t)slot * slot_b;
      if constexpr (tsc) {
        sc_k = p.k_tscale[(int64_t)kvh * p.ks_stride_head +
                          (page * (int32_t)p.ks_stride_block + slot * (int32_t)p.ks_stride_slot)];
        sc_v = p.v_tscale[(int64_t)kvh * p.vs_stride_head +
                          (page * (int32_t)p.vs_stride_block + slot * (int32_t)p.vs_stride_slot)];
      }
    }
  };
  auto store_sc = [&](int tile) __attribute__((always_inline)) {
    if constexpr (tsc) {
      if (lane < TK) {
        float* dst = &sSc[tile % tsc_lds<tsc>()][0][0];
        dst[lane] = sc_k;
        dst[TK + lane] = sc_v;
      }
    }
  };

  // 16-bit caches: copy block b = NW u + wave (1 KiB = 64 slots) of a tile;
  // lane i fills physical slot n = 64 b + i, i.e. row n / NC, logical slot
  // (n % NC) ^ swz(row).  swz reads bits 0..3 of the row, which depend on u
  // only for 32-slot rows with four waves (through u % 2): NSRC distinct
  // per-lane sources.
  constexpr int NSRC = (C::NC == 32 && NW == 4 && C::BPW > 1) ? 2 : 1;
  const char* ksrc[NSRC];
  const char* vsrc[NSRC];
#pragma unroll
  for (int u = 0; u < NSRC; ++u) {
    const int n = 64 * (NW * u + wave) + lane;
    const int r = n / C::NC;
    const int c = (n % C::NC) ^ swz<D>(r);
    ksrc[u] = kbase + 16 * c;
    vsrc[u] = vbase + 16 * c;
  }
  auto issue_copy = [&](char* dk, char* dv, const int64_t* tab) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < C::BPW; ++u) {
      const int b = NW * u + wave;
      const int64_t off = tab[(64 * b + lane) / C::NC];
      load_lds16(ksrc[u % NSRC] + off, dk + 1024 * b);
      load_lds16(vsrc[u % NSRC] + off, dv + 1024 * b);
    }
  };

  // fp8 caches: thread slot i = tid + NT u is row i / NC, logical slot i % NC.
  Stage<FP8, D, NW> st;
  auto stage_load = [&](const int64_t* tab) __attribute__((always_inline)) {
    if constexpr (FP8) {
#pragma unroll
      for (int u = 0; u < C::CPT; ++u) {
        const int i = tid + C::NT * u;
        const int64_t off = tab[i / C::NC] + 8 * (i % C::NC);
        const u32x2 a = *reinterpret_cast<const u32x2*>(kbase + off);
        const u32x2 b = *reinterpret_cast<const u32x2*>(vbase + off);
        st.k[u][0] = a[0]; st.k[u][1] = a[1];
        st.v[u][0] = b[0]; st.v[u][1] = b[1];
      }
    }
  };
  auto stage_store = [&](char* dk, char* dv) __attribute__((always_inline)) {
    if constexpr (FP8) {
#pragma unroll
      for (int u = 0; u < C::CPT; ++u) {
        const int i = tid + C::NT * u;
        const int r = i / C::NC;
        const int at = r * ROWB + 16 * ((i % C::NC) ^ swz<D>(r));
        *reinterpret_cast<u32x4*>(dk + at) = fp8x8_to<QT, FNUZ>(u32x2{st.k[u][0], st.k[u][1]});
        *reinterpret_cast<u32x4*>(dv + at) = fp8x8_to<QT, FNUZ>(u32x2{st.v[u][0], st.v[u][1]});
      }
    }
  };

  // LDS read addresses (bytes within a tile buffer).
  // K operand of MFMA c of key block kb: row 32 kb + l32, logical slot 2c + g2.
  int kaddr[C::QC];
  {
    const int f = swz<D>(l32);
#pragma unroll
    for (int c = 0; c < C::QC; ++c) kaddr[c] = l32 * ROWB + 16 * ((2 * c + g2) ^ f);
  }
  // V^T operand of output block d, keys 16 kk + {0..7} (hh = 0) / {8..15}
  // (hh = 1): lane reads row 16 kk + 4 g2 + s16 / 4 + 8 hh, bytes
  // 64 d + 32 (q16 & 1) + 8 (s16 & 3) of the logical row.
  const int s16 = lane & 15, q16 = lane >> 4;
  int vaddr[2][C::DB];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int r = 4 * g2 + (s16 >> 2) + 8 * hh;
    const int f = swz<D>(r);
#pragma unroll
    for (int d = 0; d < C::DB; ++d) {
      const int lc = 4 * d + 2 * (q16 & 1) + ((s16 & 3) >> 1);
      vaddr[hh][d] = r * ROWB + 16 * (lc ^ f) + 8 * (s16 & 1);
    }
  }

  const int ntiles = (k1 - k0 + TK - 1) / TK;
  // First key of the t-th tile a workgroup walks.  With the held maximum
  // (head dim 256) the range is walked backwards, from the tile holding the
  // diagonal: each row's maximum then comes from its nearest keys, which
  // ALiBi (or any bias growing toward the query) scores highest, so later
  // tiles rarely exceed it.  Walked forwards, an ALiBi row's first (farthest)
  // tile sat hundreds of base-2 units below its last and sent nearly every
  // workgroup through the second pass (measured on MI355X, 8k prompt with
  // ALiBi: 2.48 ms against 1.87 for the rescaling kernel; 1.25 backwards).
  auto tile_key = [&](int t) __attribute__((always_inline)) -> int {
    return kHold ? k0 + (ntiles - 1 - t) * TK : k0 + t * TK;
  };

  // Eight-wave groups (16-bit caches, plain logits: no softcap, ALiBi,
  // QQ-bias or per-token scales) run the tile in three parts that the two wave
  // halves interleave (see the interval schedule below): qk, smax, pv.
  // ---- S^T = K Q^T of the tile in LDS buffer sk.  The scheduling-group hint
  // used by four-wave groups is not honoured here (the reads landed right
  // before their MFMAs), so the order is pinned: K reads run four MFMAs ahead.
  auto qk = [&](const char* sk, f32x16* sacc) __attribute__((always_inline)) {
    constexpr int NQ = C::KB * C::QC;
    constexpr int LEAD = 4;
    u32x4 kr[NQ];
#pragma unroll
    for (int i = 0; i < LEAD; ++i)
      kr[i] = *reinterpret_cast<const u32x4*>(sk + 32 * (i / C::QC) * ROWB + kaddr[i % C::QC]);
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      if (i + LEAD < NQ) {
        const int j = i + LEAD;
        kr[j] = *reinterpret_cast<const u32x4*>(sk + 32 * (j / C::QC) * ROWB + kaddr[j % C::QC]);
      }
      const int kb = i / C::QC, c = i % C::QC;
      sacc[kb] = mfma32<QT>(kr[i], qop[c], c == 0 ? f32x16{} : sacc[kb]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // ---- Masks and P of the tile starting at key kt (raw S^T in sacc): moves
  // the running maximum and sum (rescaling O when the maximum moves) and leaves
  // P^T in pop as the B operands of the PV MFMAs.  P = 2^(s * c2 - m) is formed
  // against the running maximum m first; the tile's own maximum is only needed
  // when m must move, i.e. when some p of the tile exceeds 2^8 (then the sum of
  // the lane's p exceeds 2^8 too) or the row has no maximum yet and sees keys
  // of this tile (its p were formed against 0 and may all have underflowed);
  // when no lane of the wave sees either, the rule "move m when the tile's
  // maximum exceeds it by more than 8" would not move it (up to the rounding
  // of exp2), so the tile maximum is skipped.
  auto smax = [&](f32x16* sacc, int kt, u32x4* pop) __attribute__((always_inline)) {
    const bool full = kt >= kl && kt + TK <= k1 && kt + TK - 1 <= wave_pmin &&
                      (p.window <= 0 || kt > wave_pmax - p.window);
    // key of register r of block kb: kt + 32 kb + 8 (r / 4) + 4 g2 + r % 4;
    // visible iff row_lo <= key < row_hi, tested as one unsigned compare.
    if (!full) {
      const uint32_t span = (uint32_t)max(row_hi - row_lo, 0);
      const int kd0 = kt + 4 * g2 - row_lo;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int o = 32 * kb + 8 * (r >> 2) + (r & 3);
          sacc[kb][r] = (uint32_t)(kd0 + o) < span ? sacc[kb][r] : -INFINITY;
        }
    }
    float psum;
    auto make_p = [&]() __attribute__((always_inline)) {
      const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;
      float ps = 0.0f;
#pragma unroll
      for (int kk = 0; kk < TK / 16; ++kk) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float a =
              fast_exp2(__builtin_fmaf(sacc[kk >> 1][8 * (kk & 1) + 2 * q], c2, -m_use));
          const float b =
              fast_exp2(__builtin_fmaf(sacc[kk >> 1][8 * (kk & 1) + 2 * q + 1], c2, -m_use));
          ps += a + b;  // the row sum is of the fp32 p
          pop[kk][q] = pack2<QT>(a, b);
        }
      }
      psum = ps;
    };
    // Tile maximum (across the lane pair (l, l ^ 32) holding the same row, in
    // base-2 logit units: c2 > 0, and -inf stays -inf); m moves to it when it
    // exceeds m by more than 8.  Returns whether any row of the wave moved.
    auto move_max = [&]() __attribute__((always_inline)) -> bool {
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[kb][r]);
      mt = wave_max_xor(mt, 32) * c2;
      const bool need = mt > m_run + 8.0f;
      if (!__builtin_amdgcn_ballot_w64(need)) return false;
      const float m_new = need ? mt : m_run;
      const float alpha = need ? fast_exp2(m_run - m_new) : 1.0f;  // m_run = -inf -> 0
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < C::DB; ++d) oacc[d] *= alpha;
      m_run = m_new;
      return true;
    };
    make_p();
    const bool first = m_run == -INFINITY && max(kt, row_lo) < min(kt + TK, row_hi);
    if (__builtin_amdgcn_ballot_w64(!(psum <= 256.0f) || first))
      if (move_max()) make_p();
    l_run += psum;
  };
  // ---- O^T += V^T P^T (V tile in LDS buffer sv).
  auto pv = [&](const char* sv, const u32x4* pop) __attribute__((always_inline)) {
    // With a ring of more than 64 KB the V buffers lie beyond the reads'
    // 16-bit immediate offset: then the buffer base goes into the address
    // register with one add per read address and tile (the compiler's own
    // form took one per read), and only 16 kk rows stay immediate.
    constexpr bool kVHigh = 2 * NBUF * C::TILEB > 65536;
    uint32_t vb[2][C::DB];
    if constexpr (kVHigh) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int d = 0; d < C::DB; ++d) vb[hh][d] = lds_offset_add(sv, vaddr[hh][d]);
    }
#pragma unroll
    for (int d = 0; d < C::DB; ++d) {
#pragma unroll
      for (int kk = 0; kk < TK / 16; ++kk) {
        u32x2 lo2, hi2;
        if constexpr (kVHigh) {
          lo2 = lds_read_tr16_at(vb[0][d] + 16 * kk * ROWB);
          hi2 = lds_read_tr16_at(vb[1][d] + 16 * kk * ROWB);
        } else {
          lo2 = lds_read_tr16(sv + 16 * kk * ROWB + vaddr[0][d]);
          hi2 = lds_read_tr16(sv + 16 * kk * ROWB + vaddr[1][d]);
        }
        oacc[d] = mfma32<QT>(u32x4{lo2[0], lo2[1], hi2[0], hi2[1]}, pop[kk], oacc[d]);
      }
    }
    // Schedule: eight transposed V reads (four MFMAs' operands) in flight ahead
    // of the PV MFMAs (measured: a further 4% for D = 256).
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int k = 0; k < C::DB * (TK / 16) - 4; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  };
  auto compute = [&](const char* sk, const char* sv, int kt, const float* sc)
      __attribute__((always_inline)) {
    // ---- S^T = K Q^T
    f32x16 sacc[C::KB];
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) {
      sacc[kb] = f32x16{};
#pragma unroll
      for (int c = 0; c < C::QC; ++c) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(sk + 32 * kb * ROWB + kaddr[c]);
        sacc[kb] = mfma32<QT>(a, qop[c], sacc[kb]);
      }
    }
    // Schedule: keep four K reads in flight ahead of the QK MFMAs (the
    // default schedule issued them two MFMAs ahead, exposing LDS latency;
    // measured on MI355X: 9% faster for D = 256).
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // DS reads
#pragma unroll
    for (int k = 0; k < C::KB * C::QC - 4; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    // Per-token K scales: registers 4j .. 4j + 3 of block kb are keys
    // 32 kb + 8 j + 4 g2 + 0..3 of the tile.
    if constexpr (tsc) {
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 k4 = *reinterpret_cast<const f32x4*>(sc + 32 * kb + 8 * j + 4 * g2);
#pragma unroll
          for (int i = 0; i < 4; ++i) sacc[kb][4 * j + i] *= k4[i];
        }
    }
    // ---- logits and masks.  Without softcap/ALiBi the raw dot products are
    // kept (cs = scale * log2 e is applied in the FMA feeding exp2); with them
    // the base-2 logits are formed here (cs = 1).
    const bool full = kt >= kl && kt + TK <= k1 && kt + TK - 1 <= wave_pmin &&
                      (p.window <= 0 || kt > wave_pmax - p.window);
    float cs = c2;
    // key of register r of block kb: kt + 32 kb + 8 (r / 4) + 4 g2 + r % 4;
    // visible iff row_lo <= key < row_hi, tested as one unsigned compare.
    const uint32_t span = (uint32_t)max(row_hi - row_lo, 0);
    const int kd0 = kt + 4 * g2 - row_lo;
    if (general) {
      // Base-2 logits (softcap or plain scale), then the ALiBi bias and the
      // mask in one shared pass.
      cs = 1.0f;
      if (p.softcap_on) {
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            sacc[kb][r] = p.cap_out2 * tanh_fast(sacc[kb][r] * p.cap_in);
            // Keep the scheduler from interleaving all 16 tanh chains.
            if ((r & 3) == 3) __builtin_amdgcn_sched_barrier(0);
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[kb][r] *= c2;
      }
      const float al0 = slope2 * (float)(kt + 4 * g2 - ctx);
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int o = 32 * kb + 8 * (r >> 2) + (r & 3);
          const float v = sacc[kb][r] + __builtin_fmaf(slope2, (float)o, al0);
          sacc[kb][r] = (uint32_t)(kd0 + o) < span ? v : -INFINITY;
        }
      // QQ-bias qq[i][key - ctx] (i = this row's index in its chunk) on the
      // chunk's own keys; tiles wholly inside the prefix skip it.
      if (p.qq_bias != nullptr && kt + TK > ctx && row_ok) {
        const float* qrow = p.qq_bias + (int64_t)(pos - ctx) * p.qq_stride;
        const int rel0 = kt + 4 * g2 - ctx;
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rel = rel0 + 32 * kb + 8 * (r >> 2) + (r & 3);
            const float b = (uint32_t)rel < (uint32_t)p.qq_stride ? qrow[rel] : 0.0f;
            sacc[kb][r] = __builtin_fmaf(b, kLog2e, sacc[kb][r]);
          }
      }
    } else if (!full) {
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int o = 32 * kb + 8 * (r >> 2) + (r & 3);
          sacc[kb][r] = (uint32_t)(kd0 + o) < span ? sacc[kb][r] : -INFINITY;
        }
    }
    // ---- P = 2^(s * cs - m), packed as the B operands of the PV MFMAs; the
    // running maximum moves first when the tile's maximum exceeds it by more
    // than 8.
    u32x4 pop[TK / 16];
    float psum;
    {
      // Four-wave groups keep QK, softmax and PV in one body: head dim 256
      // runs at the register limit, where composing it from the eight-wave
      // parts (or from lambdas) cost the K reads their lead over the QK MFMAs
      // (measured on MI355X: 17% slower).
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[kb][r]);
      mt = wave_max_xor(mt, 32) * cs;
      if constexpr (kHold) {
        // Branch-free: a branch here splits the scheduling region of the PV
        // loop below, which then loses its V-read lead.
        m_seen = fmaxf(m_seen, mt);
        const bool first = m_run == -INFINITY;  // O and l are still zero
        redo = redo || (!first && mt > m_run + kHoldSpan);
        m_run = first ? mt : m_run;
      } else {
        const bool need = mt > m_run + 8.0f;
        if (__builtin_amdgcn_ballot_w64(need)) {
          const float m_new = need ? mt : m_run;
          const float alpha = need ? fast_exp2(m_run - m_new) : 1.0f;  // m_run = -inf -> 0
          l_run *= alpha;
#pragma unroll
          for (int d = 0; d < C::DB; ++d) oacc[d] *= alpha;
          m_run = m_new;
        }
      }
      const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;
      psum = 0.0f;
#pragma unroll
      for (int kk = 0; kk < TK / 16; ++kk) {
        f32x4 v4[2] = {f32x4{1.f, 1.f, 1.f, 1.f}, f32x4{1.f, 1.f, 1.f, 1.f}};
        if constexpr (tsc) {
          v4[0] = *reinterpret_cast<const f32x4*>(sc + TK + 16 * kk + 4 * g2);
          v4[1] = *reinterpret_cast<const f32x4*>(sc + TK + 16 * kk + 4 * g2 + 8);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float a =
              fast_exp2(__builtin_fmaf(sacc[kk >> 1][8 * (kk & 1) + 2 * q], cs, -m_use));
          const float b =
              fast_exp2(__builtin_fmaf(sacc[kk >> 1][8 * (kk & 1) + 2 * q + 1], cs, -m_use));
          if constexpr (tsc) {
            psum += a + b;
            pop[kk][q] = pack2<QT>(a * v4[q >> 1][2 * (q & 1)], b * v4[q >> 1][2 * (q & 1) + 1]);
          } else {
            // Normalise by the sum of p as rounded for the PV MFMA: O is then a
            // weighted mean of V rows, so a row whose weight sits on a few keys
            // loses nothing to the rounding of their p (dividing their rounded
            // weights by an unrounded sum would cost up to 2^-9 of max |V|).
            pop[kk][q] = pack2<QT>(a, b);
            psum = add_pair<QT>(pop[kk][q], psum);
          }
        }
      }
    }
    l_run += psum;
    // ---- O^T += V^T P^T
    // With a ring of more than 64 KB the V buffers lie beyond the reads'
    // 16-bit immediate offset: then the buffer base goes into the address
    // register with one add per read address and tile (the compiler's own
    // form took one per read), and only 16 kk rows stay immediate.
    constexpr bool kVHigh = 2 * NBUF * C::TILEB > 65536;
    uint32_t vb[2][C::DB];
    if constexpr (kVHigh) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int d = 0; d < C::DB; ++d) vb[hh][d] = lds_offset_add(sv, vaddr[hh][d]);
    }
#pragma unroll
    for (int d = 0; d < C::DB; ++d) {
#pragma unroll
      for (int kk = 0; kk < TK / 16; ++kk) {
        u32x2 lo2, hi2;
        if constexpr (kVHigh) {
          lo2 = lds_read_tr16_at(vb[0][d] + 16 * kk * ROWB);
          hi2 = lds_read_tr16_at(vb[1][d] + 16 * kk * ROWB);
        } else {
          lo2 = lds_read_tr16(sv + 16 * kk * ROWB + vaddr[0][d]);
          hi2 = lds_read_tr16(sv + 16 * kk * ROWB + vaddr[1][d]);
        }
        oacc[d] = mfma32<QT>(u32x4{lo2[0], lo2[1], hi2[0], hi2[1]}, pop[kk], oacc[d]);
      }
    }
    // Schedule: eight transposed V reads (four MFMAs' operands) in flight ahead
    // of the PV MFMAs (measured: a further 4% for D = 256).
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int k = 0; k < C::DB * (TK / 16) - 4; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  };

  // Buffer B of the ring (compile-time B).
  auto kbuf = [&](auto bc) __attribute__((always_inline)) -> char* {
    constexpr int B = decltype(bc)::value % NBUF;
    return sRing + B * C::TILEB;
  };
  auto vbuf = [&](auto bc) __attribute__((always_inline)) -> char* {
    constexpr int B = decltype(bc)::value % NBUF;
    return sRing + (NBUF + B) * C::TILEB;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  // Copy instructions one wave issues per tile (K and V).
  constexpr int CPW = 2 * C::BPW;

  __shared__ int sRedo[NW];
  for (int pass = 0; pass < (kHold ? 2 : 1); ++pass) {
  // Prologue: tables (and scales) of tiles 0 .. NBUF - 1, one wave each; then
  // tiles 0 .. NBUF - 2 are copied (fp8: tile 0 staged) and tile 0 waited for.
  if (wave < NBUF && wave < ntiles) {
    fill_tab(sTab[wave], tile_key(wave));
    store_sc(wave);
  }
  __syncthreads();
  if constexpr (FP8) {
    stage_load(sTab[0]);
    stage_store(kbuf(I0{}), vbuf(I0{}));
  } else {
    issue_copy(kbuf(I0{}), vbuf(I0{}), sTab[0]);
    if constexpr (NBUF > 2) {
      if (ntiles > 1) issue_copy(kbuf(I1{}), vbuf(I1{}), sTab[1]);
      if (ntiles > 2) issue_copy(kbuf(I2{}), vbuf(I2{}), sTab[2]);
      if (ntiles > 2)
        wait_vmem_n<2 * CPW>();
      else
        wait_vmem();
    } else {
      wait_vmem();
    }
  }
  barrier_lds();

  // Step t (tile t in buffer t % NBUF): issue the copy of tile t + NBUF - 1
  // (fp8: stage tile t + 1 in registers), let one wave fill the table of tile
  // t + NBUF (the slot tile t was copied with), compute tile t, then wait until
  // tile t + 1 has landed while later tiles' copies stay in flight.
  auto step = [&](auto bufc, int t) __attribute__((always_inline)) {
    constexpr int B = decltype(bufc)::value;
    using NB = std::integral_constant<int, (B + NBUF - 1) % NBUF>;
    const int kt = tile_key(t);
    const bool copy = t + NBUF - 1 < ntiles;
    if constexpr (FP8) {
      if (copy) stage_load(sTab[NB::value]);
    } else {
      if (copy) issue_copy(kbuf(NB{}), vbuf(NB{}), sTab[NB::value]);
    }
    const bool filler = t + NBUF < ntiles && wave == (t & (NW - 1));
    if (filler) fill_tab(sTab[B], kHold ? tile_key(t + NBUF) : kt + NBUF * TK);
    if (wave_live) compute(kbuf(bufc), vbuf(bufc), kt, &sSc[tsc ? t % tsc_lds<tsc>() : 0][0][0]);
    if constexpr (FP8) {
      if (copy) stage_store(kbuf(NB{}), vbuf(NB{}));
    } else if (t + 1 < ntiles) {
      if (copy)
        wait_vmem_n<(NBUF - 2) * CPW>();
      else
        wait_vmem();
    }
    if (filler) store_sc(t + NBUF);
    barrier_lds();
  };
  static_assert(NBUF == 2 || NBUF == 4, "ring depth");
  if constexpr (kPingPong) {
    // Eight-wave groups on 16-bit caches run as two halves, waves 0-3 (A) and
    // 4-7 (B), one of each on every SIMD, half a tile apart: between two
    // barriers one half runs MFMAs (PV of tile t, then QK of tile t + 1)
    // while the other runs the softmax VALU work of its tile, and the next
    // interval they swap, so one wave's MFMAs run beside the other wave's VALU
    // work (the MFMA half at raised wave priority).  Measured on MI355X: 0-3%
    // faster than both halves in step; one wave alone issues VALU work at half
    // the SIMD's rate, and MFMAs slow the other wave's VALU stream, which
    // bound the gain.
    //   interval 0:        A: QK(0), softmax(0)       B: QK(0)
    //   interval 2t + 1:   A: PV(t), QK(t + 1)        B: softmax(t)
    //   interval 2t + 2:   A: softmax(t + 1)          B: PV(t), QK(t + 1)
    // Every wave passes the same barriers (none inside the group branches).
    // Ring (four deep): the copy of tile t + 3 is issued at interval 2t + 1
    // into the slot of tile t - 1, whose K was last read at interval 2t - 2
    // and V at 2t; tile j is waited for at the end of interval 2j - 2, before
    // its K is first read at 2j - 1 (tile j + 1 stays in flight).  The table
    // of tile t + 4 is filled at interval 2t + 1 into the slot tile t was
    // copied with; the copy that reads it is issued at interval 2t + 3.
    const int grp = wave >> 2;
    auto kslot = [&](int t) __attribute__((always_inline)) -> char* {
      return sRing + (t & 3) * C::TILEB;
    };
    auto vslot = [&](int t) __attribute__((always_inline)) -> char* {
      return sRing + (4 + (t & 3)) * C::TILEB;
    };
    // Interval i starts with the copy of tile (i + 5) / 2 and the table of
    // tile (i + 7) / 2 (odd i) and ends, before its barrier, with the wait for
    // tile i / 2 + 1 (even i).
    auto start_interval = [&](int i) __attribute__((always_inline)) {
      if (i & 1) {
        const int t = (i - 1) >> 1;
        if (t + 3 < ntiles) issue_copy(kslot(t + 3), vslot(t + 3), sTab[(t + 3) & 3]);
        if (t + 4 < ntiles && wave == (t & (NW - 1))) fill_tab(sTab[t & 3], k0 + (t + 4) * TK);
      }
    };
    auto end_interval = [&](int i) __attribute__((always_inline)) {
      if (!(i & 1)) {
        const int j = (i >> 1) + 1;
        if (j < ntiles) {
          if (j + 1 < ntiles)
            wait_vmem_n<CPW>();
          else
            wait_vmem();
        }
      }
      barrier_lds();
    };
    f32x16 st[C::KB];
    u32x4 pp[TK / 16];
    if (wave_live) qk(kslot(0), st);
    if (grp == 0) {
      if (wave_live) smax(st, k0, pp);
      end_interval(0);
      for (int t = 0; t < ntiles; ++t) {
        start_interval(2 * t + 1);
        if (wave_live) {
          __builtin_amdgcn_s_setprio(1);
          pv(vslot(t), pp);
          if (t + 1 < ntiles) {
            __builtin_amdgcn_sched_barrier(0);
            qk(kslot(t + 1), st);
          }
          __builtin_amdgcn_s_setprio(0);
        }
        end_interval(2 * t + 1);
        if (t + 1 < ntiles) {
          start_interval(2 * t + 2);
          if (wave_live) smax(st, k0 + (t + 1) * TK, pp);
          end_interval(2 * t + 2);
        }
      }
    } else {
      end_interval(0);
      for (int t = 0; t < ntiles; ++t) {
        start_interval(2 * t + 1);
        if (wave_live) smax(st, k0 + t * TK, pp);
        end_interval(2 * t + 1);
        start_interval(2 * t + 2);
        if (wave_live) {
          __builtin_amdgcn_s_setprio(1);
          pv(vslot(t), pp);
          if (t + 1 < ntiles) {
            __builtin_amdgcn_sched_barrier(0);
            qk(kslot(t + 1), st);
          }
          __builtin_amdgcn_s_setprio(0);
        }
        if (t + 1 < ntiles) end_interval(2 * t + 2);
      }
    }
  } else if constexpr (!(FP8 && TS)) {
    auto run = [&]() __attribute__((always_inline)) {
      for (int t = 0; t < ntiles; t += NBUF) {
        step(I0{}, t);
        if (t + 1 < ntiles) step(I1{}, t + 1);
        if constexpr (NBUF > 2) {
          if (t + 2 < ntiles) step(I2{}, t + 2);
          if (t + 3 < ntiles) step(I3{}, t + 3);
        }
      }
    };
    // One copy of the loop per value of the uniform flag; in each the
    // compiler drops the other branch of the logit code, which otherwise
    // splits the tile's scheduling regions.  (fp8 kernels with per-token
    // scales, whose staging holds more registers, spilled with two copies.)
    // Head dims <= 128 split the featured copy once more, by softcap (ALiBi
    // or QQ-bias alone then skip the tanh branch: mixed fp16 batch with ALiBi
    // 15.4 -> 14.6 µs); at head dim 256 that third copy cost the plain one 1%.
    if (general) {
      if (D <= 128 && p.softcap_on)
        run();
      else
        run();
    } else {
      run();
    }
  } else {
    for (int t = 0; t < ntiles; t += NBUF) {
      step(I0{}, t);
      if (t + 1 < ntiles) step(I1{}, t + 1);
      if constexpr (NBUF > 2) {
        if (t + 2 < ntiles) step(I2{}, t + 2);
        if (t + 3 < ntiles) step(I3{}, t + 3);
      }
    }
  }
  if constexpr (kHold) {
    // Second pass when any row of the workgroup exceeded its held maximum.
    const bool wr = __builtin_amdgcn_ballot_w64(redo) != 0;
    if (lane == 0) sRedo[wave] = wr ? 1 : 0;
    __syncthreads();
    bool any = false;
#pragma unroll
    for (int w = 0; w < NW; ++w) any = any || sRedo[w] != 0;
    __syncthreads();
    if (!any || pass > 0) break;
#pragma unroll
    for (int d = 0; d < C::DB; ++d) oacc[d] = f32x16{};
    l_run = 0.0f;
    m_run = m_seen;
    redo = false;
  }
  }  // pass

  if (!row_ok) return;
  // Lanes l and l ^ 32 hold the same row: total l.
  l_run = wave_sum_xor(l_run, 32);
  const int tok = tok0 + rt;
  const int64_t rrow = (int64_t)tok * p.num_q_heads + h;
  // O^T accumulator: register r of block d holds O[row][32d + 8(r/4) + 4*g2 + r%4].
  if constexpr (SPLIT) {
    if (g2 == 0) {
      p.ws_m[(int64_t)part * R + rrow] = (l_run > 0.0f) ? m_run : -INFINITY;
      p.ws_l[(int64_t)part * R + rrow] = l_run;
    }
    float* dst = p.ws_acc + ((int64_t)part * R + rrow) * D;
#pragma unroll
    for (int d = 0; d < C::DB; ++d)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<f32x4*>(dst + 32 * d + 8 * r4 + 4 * g2) =
            f32x4{oacc[d][4 * r4], oacc[d][4 * r4 + 1], oacc[d][4 * r4 + 2], oacc[d][4 * r4 + 3]};
  } else {
    const float sink2 = p.sinks != nullptr ? p.sinks[h] * kLog2e : -INFINITY;
    const float Mt = fmaxf(m_run, sink2);
    const float Ms = (Mt == -INFINITY) ? 0.0f : Mt;
    const float f = fast_exp2(m_run - Ms);
    float L = l_run * f;
    const bool any_key = L > 0.0f;
    if (sink2 != -INFINITY) L += fast_exp2(sink2 - Ms);
    const float inv = any_key ? p.v_scale * f / L : 0.0f;
    char* dst = reinterpret_cast<char*>(p.out) +
                ((int64_t)tok * p.o_stride_tok + (int64_t)h * p.o_stride_head) * 2;
#pragma unroll
    for (int d = 0; d < C::DB; ++d)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<u32x2*>(dst + (32 * d + 8 * r4 + 4 * g2) * 2) =
            u32x2{pack2<QT>(oacc[d][4 * r4] * inv, oacc[d][4 * r4 + 1] * inv),
                  pack2<QT>(oacc[d][4 * r4 + 2] * inv, oacc[d][4 * r4 + 3] * inv)};
    if (p.lse != nullptr && g2 == 0)
      p.lse[rrow] = (L > 0.0f) ? (Ms + fast_log2(L)) * kLn2 : -INFINITY;
  }
}

template <int QT, bool FP8, int D, bool FNUZ, bool TS>
hipError_t launch_large_t(const Params& p, bool split, bool eight, dim3 grid, hipStream_t stream) {
  if constexpr (D <= 128 && !FP8) {
    if (eight) {
      if (p.softcap_on || p.alibi != nullptr || p.qq_bias != nullptr) return hipErrorInvalidValue;
      if (split)
        hipLaunchKernelGGL((large_kernel<QT, FP8, D, true, FNUZ, TS, 8>), grid, dim3(512), 0,
                           stream, p);
      else
        hipLaunchKernelGGL((large_kernel<QT, FP8, D, false, FNUZ, TS, 8>), grid, dim3(512), 0,
                           stream, p);
      return hipGetLastError();
    }
  } else {
    if (eight) return hipErrorInvalidValue;
  }
  if (split)
    hipLaunchKernelGGL((large_kernel<QT, FP8, D, true, FNUZ, TS, 4>), grid, dim3(256), 0, stream,
                       p);
  else
    hipLaunchKernelGGL((large_kernel<QT, FP8, D, false, FNUZ, TS, 4>), grid, dim3(256), 0, stream,
                       p);
  return hipGetLastError();
}

template <int QT, bool FP8, bool FNUZ, bool TS>
hipError_t launch_large_d(const Params& p, int head_dim, bool split, bool eight, dim3 grid,
                          hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_large_t<QT, FP8, 64, FNUZ, TS>(p, split, eight, grid, stream);
    case 128: return launch_large_t<QT, FP8, 128, FNUZ, TS>(p, split, eight, grid, stream);
    case 256: return launch_large_t<QT, FP8, 256, FNUZ, TS>(p, split, eight, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

// Per-token scales are a template switch: kernels without them are unchanged.
template <int QT>
hipError_t launch_large_q(const Params& p, int kv_fmt, int head_dim, bool split, bool eight,
                          dim3 grid, hipStream_t stream) {
  const bool ts = p.k_tscale != nullptr;
  switch (kv_fmt) {
    case kKv16:
      return launch_large_d<QT, false, false, false>(p, head_dim, split, eight, grid, stream);
    case kKvE4m3fn:
      return ts ? launch_large_d<QT, true, false, true>(p, head_dim, split, eight, grid, stream)
                : launch_large_d<QT, true, false, false>(p, head_dim, split, eight, grid, stream);
    case kKvE4m3fnuz:
      return ts ? launch_large_d<QT, true, true, true>(p, head_dim, split, eight, grid, stream)
                : launch_large_d<QT, true, true, false>(p, head_dim, split, eight, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// One entry per query dtype (see launch_small_f16 for the UA_QT split).
#if !defined(UA_QT) || UA_QT == 0
hipError_t launch_large_f16(const Params& p, int kv_fmt, int head_dim, bool split,
                            bool eight_waves, dim3 grid, hipStream_t stream) {
  return launch_large_q<UA_F16>(p, kv_fmt, head_dim, split, eight_waves, grid, stream);
}
#endif
#if !defined(UA_QT) || UA_QT == 1
hipError_t launch_large_bf16(const Params& p, int kv_fmt, int head_dim, bool split,
                             bool eight_waves, dim3 grid, hipStream_t stream) {
  return launch_large_q<UA_BF16>(p, kv_fmt, head_dim, split, eight_waves, grid, stream);
}
#endif

}  // namespace ua
