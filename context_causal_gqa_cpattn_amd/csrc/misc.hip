// Device promise check and the BHSD <-> THD layout copies.
//
// Page "Optimize context parallel attention layouts and gradient accumulation",
// "Changes": the promised sequence lengths and physical offsets are checked on the
// device on every execution and an invalid promise is reported as a device error;
// BF16 pack/unpack layout copies keep physical sequence origins.
#include "common.h"
#include "launch.h"
#include "../../include/cpattn.h"

namespace cpattn {

// One workgroup; overwrites *dev_err with the bits of every broken promise.
__global__ __launch_bounds__(1024) void validate_kernel(const ValidateArgs a) {
  __shared__ int bits_sm;
  if (threadIdx.x == 0) bits_sm = 0;
  __syncthreads();
  int bits = 0;
  for (int b = threadIdx.x; b < a.num_seqs; b += blockDim.x) {
    const int L = a.seq_lens[b];
    const int64_t off = a.seq_offsets[b];
    if (L < 0 || L > a.max_kv_len) bits |= CPATTN_DEV_ESEQ_LEN;
    if (off < 0 || off + (L > 0 ? L : 0) > a.rows) bits |= CPATTN_DEV_ESEQ_RANGE;
    if (b + 1 < a.num_seqs && off + (L > 0 ? L : 0) > (int64_t)a.seq_offsets[b + 1])
      bits |= CPATTN_DEV_ESEQ_RANGE;
    if (a.bias_len > 0 && L > a.bias_len) bits |= CPATTN_DEV_EBIAS;
    if (a.s_pitch > 0 && L > a.s_pitch) bits |= CPATTN_DEV_ELAYOUT;
  }
  int64_t ds = 0;  // this thread's share of the dS store's blocks per head
  for (int c = threadIdx.x; c < a.num_chunks; c += blockDim.x) {
    const Chunk ch = load_chunk(a.chunks, c);
    if (ch.seq < 0 || ch.seq >= a.num_seqs) { bits |= CPATTN_DEV_ECHUNK_SEQ; continue; }
    if (c + 1 < a.num_chunks && a.chunks[4 * (c + 1)] < ch.seq) bits |= CPATTN_DEV_ECHUNK_SEQ;
    const int L = a.seq_lens[ch.seq];
    const bool pos_ok = !(ch.len < 0 || ch.len > a.max_chunk_len || ch.pos0 < 0 ||
                          (int64_t)ch.pos0 + ch.len > (int64_t)L);
    if (!pos_ok) bits |= CPATTN_DEV_ECHUNK_POS;
    const int64_t n = ch.len > 0 ? ch.len : 0;
    if (ch.q_row < 0 || (int64_t)ch.q_row + n > a.q_rows) bits |= CPATTN_DEV_ECHUNK_ROWS;
    if (c + 1 < a.num_chunks && (int64_t)ch.q_row + n > (int64_t)a.chunks[4 * (c + 1) + 1])
      bits |= CPATTN_DEV_ECHUNK_ROWS;
    if (pos_ok) ds += (int64_t)((ch.len + 31) >> 5) * ds_chunk_kb(ch, L, a.causal != 0);
  }
  if (a.ds_blocks > 0) {  // block sum of ds, in a fixed order
    __shared__ int64_t part_sm[32];
    for (int m = 32; m >= 1; m >>= 1) ds += __shfl_xor(ds, m, 64);
    if ((threadIdx.x & 63) == 0) part_sm[threadIdx.x >> 6] = ds;
    __syncthreads();
    if (threadIdx.x == 0) {
      int64_t total = 0;
      for (int w = 0; w < (int)(blockDim.x >> 6); ++w) total += part_sm[w];
      if (total > a.ds_blocks) bits |= CPATTN_DEV_EDS_BLOCKS;
    }
  }
  if (bits) atomicOr(&bits_sm, bits);
  __syncthreads();
  if (threadIdx.x == 0) *a.dev_err = bits_sm;
}

// One workgroup of 1024 threads: the chunks in rounds of 1024, each round an inclusive
// scan in LDS plus the running total of the rounds before.
__global__ __launch_bounds__(1024) void ds_table_kernel(const DsTableArgs a) {
  if (*a.dev_err) return;
  __shared__ int64_t sm[1024];
  int64_t carry = 0;
  const int t = threadIdx.x;
  if (t < 128) st16(a.zero + 8 * t, u32x4{0u, 0u, 0u, 0u});
  for (int c0 = 0; c0 < a.num_chunks; c0 += 1024) {
    const int c = c0 + t;
    int64_t v = 0;
    if (c < a.num_chunks) {
      const Chunk ch = load_chunk(a.chunks, c);
      v = (int64_t)((ch.len + 31) >> 5) * ds_chunk_kb(ch, a.seq_lens[ch.seq], a.causal != 0);
    }
    sm[t] = v;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
      const int64_t add = t >= d ? sm[t - d] : 0;
      __syncthreads();
      sm[t] += add;
      __syncthreads();
    }
    if (c < a.num_chunks) a.tab[c] = carry + sm[t] - v;  // exclusive
    carry += sm[1023];
    __syncthreads();
  }
}

hipError_t launch_ds_table(const DsTableArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(ds_table_kernel, dim3(1), dim3(1024), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_validate(const ValidateArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(validate_kernel, dim3(1), dim3(1024), 0, s, a);
  return hipGetLastError();
}

// Layout copy: grid (pieces / (256*4), B).  A piece is 16 bytes of one row.
constexpr int kLayoutUnroll = 4;

__global__ __launch_bounds__(kThreads) void layout_kernel(const LayoutArgs a) {
  if (*a.dev_err) return;
  const int b = blockIdx.y;
  const int L = a.seq_lens[b];
  const int64_t off = a.seq_offsets[b];
  const int D8 = a.D / 8;
  const int64_t per_row = (int64_t)a.H * D8;  // pieces per THD row
  const int64_t total = (int64_t)L * per_row;
  const int64_t base = (int64_t)blockIdx.x * kThreads * kLayoutUnroll + threadIdx.x;
  u32x4 val[kLayoutUnroll];
  int64_t dsto[kLayoutUnroll];
#pragma unroll
  for (int u = 0; u < kLayoutUnroll; ++u) {
    const int64_t i = base + (int64_t)u * kThreads;  // piece index in THD order
    dsto[u] = -1;
    if (i < total) {
      const int64_t t = i / per_row;
      const int rem = (int)(i % per_row);
      const int h = rem / D8, c = rem % D8;
      const int64_t thd = ((off + t) * a.H + h) * a.D + c * 8;
      const int64_t bhsd = (((int64_t)b * a.H + h) * a.S_pitch + t) * a.D + c * 8;
      val[u] = ld16(a.src + (a.unpack ? thd : bhsd));
      dsto[u] = a.unpack ? bhsd : thd;
    }
  }
#pragma unroll
  for (int u = 0; u < kLayoutUnroll; ++u)
    if (dsto[u] >= 0) st16(a.dst + dsto[u], val[u]);
}

hipError_t launch_layout(const LayoutArgs& a, hipStream_t s) {
  const int64_t pieces = (int64_t)a.S_pitch * a.H * (a.D / 8);
  const int64_t per_block = (int64_t)kThreads * kLayoutUnroll;
  const int64_t gx = (pieces + per_block - 1) / per_block;
  if (gx <= 0 || a.B <= 0) return hipSuccess;
  hipLaunchKernelGGL(layout_kernel, dim3((unsigned)gx, (unsigned)a.B), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace cpattn
