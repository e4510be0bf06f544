// Merge of two partial attention results over disjoint key sets.
//
// Page "Optimize context parallel attention layouts and gradient accumulation",
// "Private C++ FROST P2P" (CP over point-to-point exchanges: each step attends to one
// K/V block), and page "Support and performance optimization for Hopper (H200)
// architecture?" (the P2P ring communications of the folding model's CP).
//
// A step over key set A returns O_A (the softmax over A applied to V) and LSE_A (the
// log-sum-exp of the scores over A).  The result over A and B is
//   LSE = log(e^LSE_A + e^LSE_B),   O = e^(LSE_A - LSE) O_A + e^(LSE_B - LSE) O_B,
// because e^(LSE_X - LSE) is the share of the total softmax mass on X.  A row with no
// visible key in a set has LSE_X = -inf and O_X = 0 and merges as nothing.
#include "common.h"
#include "launch.h"

namespace cpattn {

// One thread per 8 head-dim values of one (chunk row, head); consecutive threads walk
// D, then heads, then rows, so each row's heads are read and written contiguously.
__global__ __launch_bounds__(kThreads) void merge_kernel(const MergeArgs a) {
  if (*a.dev_err) return;
  const int per_pair = a.D / 8;
  const int pairs_per_wg = kThreads / per_pair;
  const int c = blockIdx.x / a.blocks_per_chunk;
  const int blk = blockIdx.x % a.blocks_per_chunk;
  const Chunk ch = load_chunk_uniform(a.chunks, c);
  const int pair = blk * pairs_per_wg + threadIdx.x / per_pair;
  if (pair >= ch.len * a.hq) return;  // no barriers in this kernel
  const int r = pair / a.hq, h = pair % a.hq;
  const int64_t row = (int64_t)ch.q_row + r;
  const int64_t si = (int64_t)h * a.q_rows + row;
  const float la = a.lse_a[si], lb = a.lse_b[si];
  const float m = fmaxf(la, lb);
  const int64_t off = (row * a.q_pitch + h) * a.D + (threadIdx.x % per_pair) * 8;
  const u32x4 va = ld16(a.o_a + off), vb = ld16(a.o_b + off);
  float wa = 0.f, wb = 0.f, lse = -INFINITY;
  if (m > -INFINITY) {
    wa = __expf(la - m);
    wb = __expf(lb - m);
    const float sum = wa + wb;
    lse = m + __logf(sum);
    const float inv = 1.f / sum;
    wa *= inv;
    wb *= inv;
  }
  u32x4 out;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    out[i] = pack_bf16x2(fmaf(wa, bf16_lo(va[i]), wb * bf16_lo(vb[i])),
                         fmaf(wa, bf16_hi(va[i]), wb * bf16_hi(vb[i])));
  st16(a.o + off, out);
  if (threadIdx.x % per_pair == 0) a.lse[si] = lse;
}

hipError_t launch_merge(const MergeArgs& a, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL(merge_kernel, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace cpattn
