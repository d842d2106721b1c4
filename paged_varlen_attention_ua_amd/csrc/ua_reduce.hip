// Split-KV reduce for gfx950: merges the per-partition softmax states.
//
// For each query row (token, head): M = max over partitions with l > 0 (and
// the sink, in base 2), L = sum l_p 2^(m_p - M) + 2^(sink - M),
// out = v_scale * sum acc_p 2^(m_p - M) / L; a row no partition saw is written
// as zeros (AITER PR #3962, sections "Summary" and review reply: partitions
// with l = 0 are skipped, their acc is never read, rows without keys return
// zeros).  HBM-bound: each partition's acc row is read once with 16-byte loads.

#include "ua_device.h"

namespace ua {
namespace {

// 256-thread workgroups.  A row is owned by SP groups of TPR threads; a thread
// owns 8 head-dim values, and group g merges partitions g, g + SP, g + 2 SP, ...
// (SP > 1 when a row has many partitions, so that few rows still spread over
// many threads).  Within a group, partition states are fetched U at a time
// with every load of a batch issued before any is used, and merged online
// (running maximum); the SP group states of a row are then merged through LDS.
template <int OT, int D, int SP>
__global__ __launch_bounds__(256) void reduce_kernel(Params p) {
  constexpr int VPT = 8;              // values per thread
  constexpr int TPR = D / VPT;        // threads per row and group
  constexpr int RPB = 256 / (TPR * SP);  // rows per workgroup
  constexpr int U = 8;                // partitions fetched per batch
  __shared__ float sm_m[SP > 1 ? RPB * SP : 1];
  __shared__ float sm_l[SP > 1 ? RPB * SP : 1];
  __shared__ __attribute__((aligned(16))) float sm_acc[SP > 1 ? RPB * SP * D : 1];
  const int R = p.total_q * p.num_q_heads;
  const int tid = threadIdx.x;
  const int rl = tid / (TPR * SP);
  const int grp = (tid / TPR) % SP;
  const int row = blockIdx.x * RPB + rl;
  const int d0 = (tid % TPR) * VPT;
  const bool valid = row < R;
  const int P = p.n_part;

  float M = -INFINITY, L = 0.0f;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  for (int q0 = grp; valid && q0 < P; q0 += U * SP) {
    float mv[U], lv[U];
    f32x4 a0[U], a1[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int q = q0 + u * SP;
      const bool in = q < P;
      const int64_t qr = (int64_t)q * R + row;
      mv[u] = in ? p.ws_m[qr] : -INFINITY;
      lv[u] = in ? p.ws_l[qr] : 0.0f;
      const float* src = p.ws_acc + qr * D + d0;
      a0[u] = in ? *reinterpret_cast<const f32x4*>(src) : f32x4{0.f, 0.f, 0.f, 0.f};
      a1[u] = in ? *reinterpret_cast<const f32x4*>(src + 4) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float mb = M;
#pragma unroll
    for (int u = 0; u < U; ++u) mb = lv[u] > 0.0f ? fmaxf(mb, mv[u]) : mb;
    if (mb == -INFINITY) continue;  // nothing live yet
    const float f = fast_exp2(M - mb);  // M = -inf -> 0 (L and acc are 0 then)
    L *= f;
    acc0 *= f;
    acc1 *= f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool live = lv[u] > 0.0f;  // l == 0: acc and m are unspecified, never used
      const float w = live ? fast_exp2(mv[u] - mb) : 0.0f;
      L += w * lv[u];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc0[e] += live ? w * a0[u][e] : 0.0f;
        acc1[e] += live ? w * a1[u][e] : 0.0f;
      }
    }
    M = mb;
  }
  if constexpr (SP > 1) {
    // Group states of each row -> LDS; group 0 folds the other groups in.
    const int slot = rl * SP + grp;
    if ((tid % TPR) == 0) {
      sm_m[slot] = M;
      sm_l[slot] = L;
    }
    *reinterpret_cast<f32x4*>(sm_acc + slot * D + d0) = acc0;
    *reinterpret_cast<f32x4*>(sm_acc + slot * D + d0 + 4) = acc1;
    __syncthreads();
    if (grp != 0) return;
    float Mg = -INFINITY;
#pragma unroll
    for (int g = 0; g < SP; ++g)
      Mg = sm_l[rl * SP + g] > 0.0f ? fmaxf(Mg, sm_m[rl * SP + g]) : Mg;
    L = 0.0f;
    acc0 = f32x4{0.f, 0.f, 0.f, 0.f};
    acc1 = f32x4{0.f, 0.f, 0.f, 0.f};
    if (Mg != -INFINITY) {
#pragma unroll
      for (int g = 0; g < SP; ++g) {
        const int sl = rl * SP + g;
        const float lg = sm_l[sl];
        const float w = lg > 0.0f ? fast_exp2(sm_m[sl] - Mg) : 0.0f;
        L += w * lg;
        const f32x4 b0 = *reinterpret_cast<const f32x4*>(sm_acc + sl * D + d0);
        const f32x4 b1 = *reinterpret_cast<const f32x4*>(sm_acc + sl * D + d0 + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc0[e] += lg > 0.0f ? w * b0[e] : 0.0f;
          acc1[e] += lg > 0.0f ? w * b1[e] : 0.0f;
        }
      }
    }
    M = Mg;
  }
  if (!valid) return;
  const int tok = row / p.num_q_heads;
  const int h = row - tok * p.num_q_heads;
  const bool any_key = L > 0.0f;
  const float sink2 = (p.sinks != nullptr) ? p.sinks[h] * kLog2e : -INFINITY;
  const float Mt = fmaxf(M, sink2);
  const float Ms = (Mt == -INFINITY) ? 0.0f : Mt;
  const float f = any_key ? fast_exp2(M - Ms) : 0.0f;
  L *= f;
  if (sink2 != -INFINITY) L += fast_exp2(sink2 - Ms);
  const float inv = any_key ? p.v_scale * f / L : 0.0f;
  char* dst = reinterpret_cast<char*>(p.out) +
              ((int64_t)tok * p.o_stride_tok + (int64_t)h * p.o_stride_head + d0) * 2;
  *reinterpret_cast<u32x4*>(dst) =
      u32x4{pack2<OT>(acc0[0] * inv, acc0[1] * inv), pack2<OT>(acc0[2] * inv, acc0[3] * inv),
            pack2<OT>(acc1[0] * inv, acc1[1] * inv), pack2<OT>(acc1[2] * inv, acc1[3] * inv)};
  if (p.lse != nullptr && d0 == 0) p.lse[row] = (L > 0.0f) ? (Ms + fast_log2(L)) * kLn2 : -INFINITY;
}

template <int OT, int D, int SP>
void launch_reduce_sp(const Params& p, int64_t R, hipStream_t stream) {
  constexpr int RPB = 256 / ((D / 8) * SP);
  hipLaunchKernelGGL((reduce_kernel<OT, D, SP>), dim3((unsigned)((R + RPB - 1) / RPB)), dim3(256),
                     0, stream, p);
}

// Groups per row: one batch of 8 partitions per group where possible.
template <int OT, int D>
void launch_reduce_d(const Params& p, int64_t R, hipStream_t stream) {
  if (p.n_part <= 8)
    launch_reduce_sp<OT, D, 1>(p, R, stream);
  else if (p.n_part <= 16)
    launch_reduce_sp<OT, D, 2>(p, R, stream);
  else if (p.n_part <= 32)
    launch_reduce_sp<OT, D, 4>(p, R, stream);
  else
    launch_reduce_sp<OT, D, 8>(p, R, stream);
}

template <int OT>
hipError_t launch_reduce_t(const Params& p, int head_dim, hipStream_t stream) {
  const int64_t R = (int64_t)p.total_q * p.num_q_heads;
  if (R == 0) return hipSuccess;
  switch (head_dim) {
    case 64: launch_reduce_d<OT, 64>(p, R, stream); break;
    case 128: launch_reduce_d<OT, 128>(p, R, stream); break;
    case 256: launch_reduce_d<OT, 256>(p, R, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_reduce(const Params& p, int o_dtype, int head_dim, hipStream_t stream) {
  return o_dtype == UA_F16 ? launch_reduce_t<UA_F16>(p, head_dim, stream)
                           : launch_reduce_t<UA_BF16>(p, head_dim, stream);
}

}  // namespace ua
