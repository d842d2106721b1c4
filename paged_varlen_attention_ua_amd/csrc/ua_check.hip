// Input checker for gfx950: verifies on the device the data preconditions the
// forward entry points assume without checking (cumulative query offsets,
// per-sequence lengths against the host bounds, block-table entries of every
// block a sequence uses), and reports violations as bits, never by faulting.
// One workgroup; every read is inside the arrays the ABI sizes (cu_seqlens_q
// [num_seqs + 1], seq_lens [num_seqs], block_table rows of max_blocks_per_seq
// entries, of which at most ceil(kv_len / block_size) are read, kv_len clamped
// to the row).

#include "ua_internal.h"

namespace ua {
namespace {

__global__ __launch_bounds__(256) void check_kernel(const int32_t* __restrict__ cu,
                                                    const int32_t* __restrict__ seq_lens,
                                                    const int32_t* __restrict__ block_table,
                                                    int32_t* flags, int num_seqs, int total_q,
                                                    int max_q, int max_k, int block_size,
                                                    int max_blocks, int64_t num_blocks) {
  __shared__ int32_t bits;
  const int tid = threadIdx.x;
  if (tid == 0) bits = 0;
  __syncthreads();
  int local = 0;
  if (tid == 0 && (cu[0] != 0 || cu[num_seqs] != total_q)) local |= UA_CHECK_CU;
  for (int s = tid; s < num_seqs; s += 256) {
    const int a = cu[s], b = cu[s + 1];
    if (b < a) local |= UA_CHECK_CU;
    const int ql = b - a;
    if (ql > max_q) local |= UA_CHECK_QLEN;
    const int kv = seq_lens[s];
    if (kv < 0 || kv < ql || kv > max_k) local |= UA_CHECK_KVLEN;
  }
  const int64_t row_keys = (int64_t)max_blocks * block_size;
  for (int s = 0; s < num_seqs; ++s) {
    const int64_t kv = min<int64_t>(max<int64_t>(seq_lens[s], 0), row_keys);
    const int nb = (int)((kv + block_size - 1) / block_size);
    const int32_t* row = block_table + (int64_t)s * max_blocks;
    for (int j = tid; j < nb; j += 256) {
      const int32_t e = row[j];
      if (e < 0 || (int64_t)e >= num_blocks) local |= UA_CHECK_BLOCK;
    }
  }
  if (local) atomicOr(&bits, local);
  __syncthreads();
  if (tid == 0) flags[0] = bits;
}

}  // namespace

hipError_t launch_check(const ua_problem* p, const ua_args* a, int32_t* flags,
                        hipStream_t stream) {
  hipLaunchKernelGGL(check_kernel, dim3(1), dim3(256), 0, stream, a->cu_seqlens_q, a->seq_lens,
                     a->block_table, flags, p->num_seqs, p->total_q, p->max_seqlen_q,
                     p->max_seqlen_k, p->block_size, p->max_blocks_per_seq, p->num_blocks);
  return hipGetLastError();
}

}  // namespace ua
