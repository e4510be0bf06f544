// Copies around the all-to-all (A2A) head <-> sequence swap of context parallelism.
//
// Page "Optimize context parallel attention layouts and gradient accumulation",
// "Description" and "Changes" (vectorised BF16 A2A pack/unpack copies inside the
// swap, used by both attention backends), "Validation and performance" (the CP4/A2A
// run those copies sped up).
//
// Rank r of cp holds the rows of its chunks of every sequence with all H heads.  Before
// attention, split_heads cuts each row into cp head groups of Hc = H / cp heads (block j
// goes to rank j) and, after the exchange, scatter_rows puts the rows received from
// rank s at their places in the sequence-ordered tensor (row q_row + i of chunk
// {seq, q_row, pos0, len} of rank s -> row seq_offsets[seq] + pos0 + i).  After
// attention, gather_rows and merge_heads undo the two.
//
// The head copies give each workgroup whole rows: the row side is one contiguous run
// and the block side cp runs of (rows per workgroup) x Hc D elements.  The row copies
// move a whole chunk, a run contiguous on both sides.  Each lane moves 16-byte pieces,
// four in flight, a workgroup 16 KB.  Loads and stores are nontemporal: every byte is
// touched once, and streaming it past the caches measured about 10% faster than plain
// accesses for 1 GiB copies (6.2 against 5.5 TB/s).  Nothing here computes; HBM
// bandwidth bounds it.
#include "common.h"
#include "launch.h"
#include "../../include/cpattn.h"

namespace cpattn {

constexpr int kA2aUnroll = 4;
constexpr int kA2aPieces = kThreads * kA2aUnroll;  // 16-byte pieces per workgroup

__device__ __forceinline__ u32x4 ld16_nt(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16_nt(uint16_t* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// Moves the n 16-byte pieces of a run from src to dst.
__device__ __forceinline__ void copy_run(const uint16_t* src, uint16_t* dst, int n) {
  for (int base = threadIdx.x; base < n; base += kA2aPieces) {
    u32x4 v[kA2aUnroll];
#pragma unroll
    for (int u = 0; u < kA2aUnroll; ++u) {
      const int p = base + u * kThreads;
      if (p < n) v[u] = ld16_nt(src + (int64_t)p * 8);
    }
#pragma unroll
    for (int u = 0; u < kA2aUnroll; ++u) {
      const int p = base + u * kThreads;
      if (p < n) st16_nt(dst + (int64_t)p * 8, v[u]);
    }
  }
}

// Grid (row tiles).  Workgroup x moves every head group of rows_per_wg rows.  Piece p of
// the tile is piece e = p % row_pieces of row t = p / row_pieces of the row layout, and
// piece e % seg of head group e / seg: in the block layout, row r0 + t of block j.
__global__ __launch_bounds__(kThreads) void a2a_heads_kernel(const A2aHeadsArgs a) {
  const int64_t r0 = (int64_t)blockIdx.x * a.rows_per_wg;
  const int nr = (int)min((int64_t)a.rows_per_wg, a.rows - r0);
  if (nr <= 0) return;
  const int Hc = a.H / a.cp;
  const int seg = Hc * a.D / 8;        // pieces of one row's head group
  const int row_pieces = a.H * a.D / 8;
  const int64_t seg_el = (int64_t)Hc * a.D;
  const int64_t rows_base = r0 * row_pieces * 8;
  const int total = nr * row_pieces;
  for (int base = threadIdx.x; base < total; base += kA2aPieces) {
    u32x4 v[kA2aUnroll];
    int64_t bo[kA2aUnroll];
#pragma unroll
    for (int u = 0; u < kA2aUnroll; ++u) {
      const int p = base + u * kThreads;
      if (p < total) {
        const int t = p / row_pieces, e = p - t * row_pieces;
        const int j = e / seg, f = e - j * seg;
        bo[u] = ((int64_t)j * a.rows + r0 + t) * seg_el + f * 8;
        v[u] = ld16_nt(a.src + (a.merge ? bo[u] : rows_base + (int64_t)p * 8));
      }
    }
#pragma unroll
    for (int u = 0; u < kA2aUnroll; ++u) {
      const int p = base + u * kThreads;
      if (p < total) st16_nt(a.dst + (a.merge ? rows_base + (int64_t)p * 8 : bo[u]), v[u]);
    }
  }
}

hipError_t launch_a2a_heads(const A2aHeadsArgs& a, hipStream_t s) {
  const int64_t tiles = (a.rows + a.rows_per_wg - 1) / a.rows_per_wg;
  if (tiles <= 0 || a.cp <= 0) return hipSuccess;
  hipLaunchKernelGGL(a2a_heads_kernel, dim3((unsigned)tiles), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

// One workgroup of 1024 threads: overwrites *dev_err with the bits of every broken
// promise of the rank maps (bounds only; chunks may come in any order).
__global__ __launch_bounds__(1024) void a2a_validate_kernel(const A2aRowsArgs a) {
  __shared__ int bits_sm;
  if (threadIdx.x == 0) bits_sm = 0;
  __syncthreads();
  int bits = 0;
  for (int b = threadIdx.x; b < a.num_seqs; b += blockDim.x) {
    const int64_t off = a.seq_offsets[b];
    const int L = a.seq_lens[b];
    if (L < 0) bits |= CPATTN_DEV_ESEQ_LEN;
    if (off < 0 || off + (L > 0 ? L : 0) > a.full_rows) bits |= CPATTN_DEV_ESEQ_RANGE;
  }
  const int n = a.cp * a.chunks_per_rank;
  for (int c = threadIdx.x; c < n; c += blockDim.x) {
    const Chunk ch = load_chunk(a.maps, c);
    if (ch.seq < 0 || ch.seq >= a.num_seqs) { bits |= CPATTN_DEV_ECHUNK_SEQ; continue; }
    const int L = a.seq_lens[ch.seq];
    if (ch.len < 0 || ch.len > a.max_chunk_len || ch.pos0 < 0 || (int64_t)ch.pos0 + ch.len > (int64_t)L)
      bits |= CPATTN_DEV_ECHUNK_POS;
    if (ch.q_row < 0 || (int64_t)ch.q_row + (ch.len > 0 ? ch.len : 0) > a.rows_per_rank)
      bits |= CPATTN_DEV_ECHUNK_ROWS;
  }
  if (bits) atomicOr(&bits_sm, bits);
  __syncthreads();
  if (threadIdx.x == 0) *a.dev_err = bits_sm;
}

// Grid (wg_per_chunk * cp * chunks_per_rank).  Workgroup (chunk, part) moves pieces
// [part * kA2aPieces, +kA2aPieces) of the chunk's run.
__global__ __launch_bounds__(kThreads) void a2a_rows_kernel(const A2aRowsArgs a) {
  if (*a.dev_err) return;
  const int c = blockIdx.x / a.wg_per_chunk;
  const int part = blockIdx.x % a.wg_per_chunk;
  const Chunk ch = load_chunk(a.maps, c);
  const int s = c / a.chunks_per_rank;
  const int seg = a.heads * a.D / 8;  // pieces per row
  const int64_t pieces = (int64_t)ch.len * seg;
  const int64_t p0 = (int64_t)part * kA2aPieces;
  if (p0 >= pieces) return;
  const int64_t row_el = (int64_t)a.heads * a.D;
  const int64_t blk_off = ((int64_t)s * a.rows_per_rank + ch.q_row) * row_el + p0 * 8;
  const int64_t full_off = ((int64_t)a.seq_offsets[ch.seq] + ch.pos0) * row_el + p0 * 8;
  const int np = (int)min((int64_t)kA2aPieces, pieces - p0);
  copy_run(a.src + (a.gather ? full_off : blk_off), a.dst + (a.gather ? blk_off : full_off), np);
}

hipError_t launch_a2a_rows(const A2aRowsArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(a2a_validate_kernel, dim3(1), dim3(1024), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t wgs = (int64_t)a.wg_per_chunk * a.cp * a.chunks_per_rank;
  if (wgs <= 0) return hipSuccess;
  hipLaunchKernelGGL(a2a_rows_kernel, dim3((unsigned)wgs), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace cpattn
