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

// One 64-thread workgroup per row group: TPR threads own 4 head-dim values of
// a row each.  Partition states are fetched U at a time with every load of a
// batch issued before any is used, and merged online (running maximum), so
// up to U partitions cost one memory round trip.
template <int OT, int D>
__global__ __launch_bounds__(64) void reduce_kernel(Params p) {
  constexpr int TPR = D / 4;          // threads per row, 4 values each
  constexpr int RPB = 64 / TPR;       // rows per workgroup
  constexpr int U = 16;               // partitions fetched per batch
  const int R = p.total_q * p.num_q_heads;
  const int tid = threadIdx.x;
  const int64_t row = (int64_t)blockIdx.x * RPB + tid / TPR;
  const int d0 = (tid % TPR) * 4;
  if (row >= R) return;
  const int h = (int)(row % p.num_q_heads);
  const int P = p.n_part;

  float M = -INFINITY, L = 0.0f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int q0 = 0; q0 < P; q0 += U) {
    float mv[U], lv[U];
    f32x4 av[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int q = q0 + u;
      const bool in = q < P;
      mv[u] = in ? p.ws_m[(int64_t)q * R + row] : -INFINITY;
      lv[u] = in ? p.ws_l[(int64_t)q * R + row] : 0.0f;
      av[u] = in ? *reinterpret_cast<const f32x4*>(p.ws_acc + ((int64_t)q * R + row) * D + d0)
                 : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float mb = M;
#pragma unroll
    for (int u = 0; u < U; ++u) mb = lv[u] > 0.0f ? fmaxf(mb, mv[u]) : mb;
    if (mb == -INFINITY) continue;  // nothing live yet
    const float f = fast_exp2(M - mb);  // M = -inf -> 0 (L and acc are 0 then)
    L *= f;
    acc *= f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool live = lv[u] > 0.0f;  // l == 0: acc and m are unspecified, never used
      const float w = live ? fast_exp2(mv[u] - mb) : 0.0f;
      L += w * lv[u];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += live ? w * av[u][e] : 0.0f;
    }
    M = mb;
  }
  const bool any_key = L > 0.0f;
  const float sink2 = (p.sinks != nullptr) ? p.sinks[h] * kLog2e : -INFINITY;
  const float Mt = fmaxf(M, sink2);
  const float Ms = (Mt == -INFINITY) ? 0.0f : Mt;
  const float f = any_key ? fast_exp2(M - Ms) : 0.0f;
  L *= f;
  if (sink2 != -INFINITY) L += fast_exp2(sink2 - Ms);
  const float inv = any_key ? p.v_scale * f / L : 0.0f;
  const int64_t tok = row / p.num_q_heads;
  char* dst = reinterpret_cast<char*>(p.out) +
              (tok * p.o_stride_tok + (int64_t)h * p.o_stride_head + d0) * 2;
  *reinterpret_cast<u32x2*>(dst) =
      u32x2{pack2<OT>(acc[0] * inv, acc[1] * inv), pack2<OT>(acc[2] * inv, acc[3] * inv)};
  if (p.lse != nullptr && d0 == 0) p.lse[row] = (L > 0.0f) ? (Ms + fast_log2(L)) * kLn2 : -INFINITY;
}

template <int OT>
hipError_t launch_reduce_t(const Params& p, int head_dim, hipStream_t stream) {
  const int64_t R = (int64_t)p.total_q * p.num_q_heads;
  if (R == 0) return hipSuccess;
  switch (head_dim) {
    case 64:
      hipLaunchKernelGGL((reduce_kernel<OT, 64>), dim3((unsigned)((R + 3) / 4)), dim3(64), 0,
                         stream, p);
      break;
    case 128:
      hipLaunchKernelGGL((reduce_kernel<OT, 128>), dim3((unsigned)((R + 1) / 2)), dim3(64), 0,
                         stream, p);
      break;
    case 256:
      hipLaunchKernelGGL((reduce_kernel<OT, 256>), dim3((unsigned)R), dim3(64), 0, stream, p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_reduce(const Params& p, int o_dtype, int head_dim, hipStream_t stream) {
  return o_dtype == UA_F16 ? launch_reduce_t<UA_F16>(p, head_dim, stream)
                           : launch_reduce_t<UA_BF16>(p, head_dim, stream);
}

}  // namespace ua
