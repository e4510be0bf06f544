// Backward pre-pass: the dO.O row dot and the transposed Q/dO tiles for dK/dV.
//
// Page "Optimize context parallel attention layouts and gradient accumulation":
//  - "CP8 AllGather: composition with first-gradient reuse": the pre-pass row dot
//    of dO and O, loaded at their physical pitch, with 64-bit addressing
//    ("Related optimization work" mentions the 64-bit fix of that dot helper);
//  - "Changes": GQA, causal THD with physical offsets.
//
// Delta = rowsum(dO * O) enters dS = P * (dP - Delta) in dK/dV and dQ.
#include "common.h"
#include "launch.h"

namespace cpattn {

// ---------------------------------------------------------------- pre-pass
//
// One workgroup per (chunk, 32-query tile, query head), the head varying fastest in the
// launch order, so that workgroups running together read neighbouring heads of the same
// rows (whole rows of the [rows, heads, D] tensors):
//  - Delta[h, r] = sum_d dO[r,h,d] O[r,h,d] in fp32 for the tile's rows, from 16-byte
//    loads of O and dO at their physical pitch with 64-bit addressing;
//  - the tile's Q and dO transposed to [D][32] (rows past the chunk are zero), the
//    layout in which dK/dV contracts over queries with 16-byte LDS reads.  Within each
//    half of 16 queries, position p holds query sigma16(p): the order in which a
//    32x32 accumulator lists one lane's rows, so that dK/dV's P and dS registers are
//    B operands as they are.  Granule g of row d is stored at g ^ tswz(d).
// Q, O and dO are read once here (the backward reads the transposed tiles instead), so
// their loads are non-temporal.  The transposed tiles are assembled in LDS and written
// as contiguous 16-byte pieces, 1 KB per wave instruction.
// Tile qt of chunk c is stored at slot tile_slot(c, q_row, qt).

constexpr int kTileQ = 32;

template <int D>
__global__ __launch_bounds__(kThreads) void prepass_kernel(const AttnArgs a) {
  if (*a.dev_err) return;
  constexpr int DG = D / 8;       // 16-byte granules per row
  constexpr int TASKS = DG * 4;   // (8-row group, granule) tasks per tensor
  __shared__ __attribute__((aligned(16))) uint16_t stage[2][D * kTileQ];
  const int tid = threadIdx.x;
  const int lin = blockIdx.x + gridDim.x * blockIdx.y;
  const int h = lin % a.hq;
  const int c = (lin / a.hq) / a.blocks_per_chunk;
  const int qt = (lin / a.hq) % a.blocks_per_chunk;
  const Chunk ch = load_chunk_uniform(a.chunks, c);
  const int r0 = qt * kTileQ;
  if (r0 >= ch.len) return;  // the whole workgroup
  const int nq = min(kTileQ, ch.len - r0);
  const int64_t tile = tile_slot(c, ch.q_row, qt);
  if (tid < 2 * TASKS) {
    const int tensor = tid / TASKS;  // 0: Q, 1: dO
    const int task = tid % TASKS;
    const int qg = task / DG, dg = task % DG;  // qg: output granule; dg varies fastest
    // the 8 queries of output granule qg, in stored order
    const int qbase = (qg >> 1) * 16, qsub = (qg & 1) * 8;
    const int64_t rs = a.q_pitch * D;
    const int64_t off = ((int64_t)ch.q_row + r0) * rs + (int64_t)h * D + dg * 8;
    const uint16_t* src = (tensor ? a.dout : a.q) + off;
    auto ld_once = [](const uint16_t* p) {
      return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    };
    u32x4 rows[8], cols[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int qi = qbase + sigma16(qsub + e);
      rows[e] = qi < nq ? ld_once(src + qi * rs) : u32x4{0u, 0u, 0u, 0u};
    }
    if (tensor == 1) {
      float ds[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int qi = qbase + sigma16(qsub + e);
        const u32x4 ov = qi < nq ? ld_once(a.o + off + qi * rs) : u32x4{0u, 0u, 0u, 0u};
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          acc = fmaf(bf16_lo(ov[w]), bf16_lo(rows[e][w]), acc);
          acc = fmaf(bf16_hi(ov[w]), bf16_hi(rows[e][w]), acc);
        }
        ds[e] = acc;
      }
#pragma unroll
      for (int m = DG / 2; m >= 1; m >>= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e) ds[e] += __shfl_xor(ds[e], m, 64);
      if (dg == 0) {
        // the tile's row statistics for dK/dV: log2(e) LSE (+inf past the chunk end, so
        // that those rows' probabilities come out 0), then Delta (0 past the end)
        float* st = a.stats_out + (tile * a.hq + h) * 64;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int qi = qbase + sigma16(qsub + e);
          const int64_t row = (int64_t)h * a.q_rows + ch.q_row + r0 + qi;
          if (qi < nq) a.delta_out[row] = ds[e];
          st[qi] = qi < nq ? a.lse[row] * kLog2e : INFINITY;
          st[32 + qi] = qi < nq ? ds[e] : 0.f;
        }
      }
    }
    transpose8x8(rows, cols);  // cols[d]: the granule's 8 queries at dimension dg*8 + d
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const int dd = dg * 8 + d;
      *reinterpret_cast<u32x4*>(&stage[tensor][dd * kTileQ + ((qg ^ tswz(dd)) * 8)]) = cols[d];
    }
  }
  __syncthreads();
  constexpr int PIECES = D * kTileQ / 8;  // 16-byte pieces per tile
  uint16_t* dst_q = a.qt_out + (tile * a.hq + h) * D * kTileQ;
  uint16_t* dst_do = a.dot_out + (tile * a.hq + h) * D * kTileQ;
#pragma unroll
  for (int i = tid; i < 2 * PIECES; i += kThreads) {
    const int t = i / PIECES, p = i % PIECES;
    st16((t ? dst_do : dst_q) + p * 8, *reinterpret_cast<const u32x4*>(&stage[t][p * 8]));
  }
}

hipError_t launch_prepass(const AttnArgs& a, int D, dim3 grid, hipStream_t s) {
  switch (D) {
    case 32: hipLaunchKernelGGL(prepass_kernel<32>, grid, dim3(kThreads), 0, s, a); break;
    case 64: hipLaunchKernelGGL(prepass_kernel<64>, grid, dim3(kThreads), 0, s, a); break;
    case 128: hipLaunchKernelGGL(prepass_kernel<128>, grid, dim3(kThreads), 0, s, a); break;
    case 256: hipLaunchKernelGGL(prepass_kernel<256>, grid, dim3(kThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace cpattn
