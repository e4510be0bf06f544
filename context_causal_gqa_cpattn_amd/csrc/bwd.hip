// Backward kernels: the dO.O pre-pass, dK/dV (KV-parallel) and dQ (Q-parallel).
//
// Page "Optimize context parallel attention layouts and gradient accumulation":
//  - "CP8 AllGather: composition with first-gradient reuse": the pre-pass row dot
//    of dO and O, loaded at their physical pitch, with 64-bit addressing
//    ("Related optimization work" mentions the 64-bit fix of that dot helper);
//  - "CP8 first-gradient accumulator reuse": the first dK/dV contribution is the
//    accumulator (STORE, no zero fill) and the later one is added (ADD);
//  - "Changes": GQA, causal THD with physical offsets, output zeroing removed.
//
// With P = exp(scale S - LSE), dP = dO V^T, Delta = rowsum(dO * O) and
// dS = P * (dP - Delta):  dV = P^T dO, dK = scale dS^T Q, dQ = scale dS K.
#include "common.h"
#include "launch.h"

namespace cpattn {

// ---------------------------------------------------------------- pre-pass
//
// One workgroup per (chunk, 32-query tile, query head):
//  - Delta[h, r] = sum_d dO[r,h,d] O[r,h,d] in fp32 for the tile's rows, from 16-byte
//    loads of O and dO at their physical pitch with 64-bit addressing;
//  - the tile's Q and dO transposed to [D][32] (rows past the chunk are zero), the
//    layout in which dK/dV contracts over queries with 16-byte LDS reads.  Within each
//    half of 16 queries, position p holds query sigma16(p): the order in which a
//    32x32 accumulator lists one lane's rows, so that dK/dV's P and dS registers are
//    B operands as they are.  Granule g of row d is stored at g ^ tswz(d).
// Tile qt of chunk c is stored at slot tile_slot(c, q_row, qt).

constexpr int kTileQ = 32;

template <int D>
__global__ __launch_bounds__(kThreads) void prepass_kernel(const AttnArgs a) {
  if (*a.dev_err) return;
  constexpr int DG = D / 8;       // 16-byte granules per row
  constexpr int TASKS = DG * 4;   // (8-row group, granule) tasks per tensor
  const int tid = threadIdx.x;
  const int c = blockIdx.x / a.blocks_per_chunk;
  const int qt = blockIdx.x % a.blocks_per_chunk;
  const int h = blockIdx.y;
  const Chunk ch = load_chunk(a.chunks, c);
  const int r0 = qt * kTileQ;
  if (r0 >= ch.len || tid >= 2 * TASKS) return;  // no barriers below
  const int nq = min(kTileQ, ch.len - r0);
  const int64_t tile = tile_slot(c, ch.q_row, qt);
  const int tensor = tid / TASKS;  // 0: Q, 1: dO
  const int task = tid % TASKS;
  const int qg = task / DG, dg = task % DG;  // qg: output granule; dg varies fastest
  // the 8 queries of output granule qg, in stored order
  const int qbase = (qg >> 1) * 16, qsub = (qg & 1) * 8;
  const int64_t rs = (int64_t)a.hq * D;
  const int64_t off = ((int64_t)ch.q_row + r0) * rs + (int64_t)h * D + dg * 8;
  const uint16_t* src = (tensor ? a.dout : a.q) + off;
  u32x4 rows[8], cols[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int qi = qbase + sigma16(qsub + e);
    rows[e] = qi < nq ? ld16(src + qi * rs) : u32x4{0u, 0u, 0u, 0u};
  }
  if (tensor == 1) {
    float ds[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int qi = qbase + sigma16(qsub + e);
      const u32x4 ov = qi < nq ? ld16(a.o + off + qi * rs) : u32x4{0u, 0u, 0u, 0u};
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
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int qi = qbase + sigma16(qsub + e);
        if (qi < nq) a.delta_out[(int64_t)h * a.q_rows + ch.q_row + r0 + qi] = ds[e];
      }
    }
  }
  transpose8x8(rows, cols);  // cols[d]: the granule's 8 queries at dimension dg*8 + d
  uint16_t* dst = (tensor ? a.dot_out : a.qt_out) + (tile * a.hq + h) * D * kTileQ;
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    const int dd = dg * 8 + d;
    st16(dst + dd * kTileQ + ((qg ^ tswz(dd)) * 8), cols[d]);
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

// ---------------------------------------------------------------- dQ
//
// Same decomposition as the forward: a wave owns 32 query rows of one head and keeps Q
// and dO in registers; K and V tiles of 64 keys are DMA'd into LDS (double buffer).
//   S^T = K Q^T,  dP^T = V dO^T   (A = K / V rows, 16-byte LDS reads)
//   dS^T = P^T (dP^T - Delta)     (lane = query)
//   dQ^T += K^T dS^T              (A = K^T by transposing reads of the same K tile)

constexpr int kBNq = 64;  // keys per KV tile in the dQ kernel

// dS^T = P^T (dP^T - Delta) for one 64-key tile, in place in dp (lane = query).
template <bool BIAS, bool MASK, bool CAUSAL>
__device__ __forceinline__ void ds_tile(f32x16 (&s)[2], f32x16 (&dp)[2], float c, const float* bias_row,
                                        int key0, int L, int qpos, int kg, int bias_len, float lse2,
                                        float dlt) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kbi = key0 + kb * 32 + i * 8 + kg * 4;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kk = kbi + j;
        float x;
        if (BIAS)
          x = fmaf(bias_row[min(kk, bias_len - 1)], kLog2e, s[kb][i * 4 + j] * c) - lse2;
        else
          x = fmaf(s[kb][i * 4 + j], c, -lse2);
        if (MASK) x = ((kk < L) && (!CAUSAL || kk <= qpos)) ? x : -INFINITY;
        const float p = exp2f_fast(x);  // branch-free: a masked score is exp2(-inf) = 0
        dp[kb][i * 4 + j] = p * (dp[kb][i * 4 + j] - dlt);
      }
    }
}

template <int D, bool CAUSAL, bool BIAS>
__global__ __launch_bounds__(kThreads) void dq_kernel(const AttnArgs a) {
  constexpr int NST = D / 16;
  constexpr int NDB = D / 32;
  __shared__ __attribute__((aligned(1024))) uint16_t lds_k[2][kBNq * D];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_v[2][kBNq * D];

  if (*a.dev_err) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kg = lane >> 5, col = lane & 31;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int n_hg = a.hq / a.hpw;
  const int pb = logical % a.blocks_per_chunk;
  const int rest = logical / a.blocks_per_chunk;
  const int hg = rest % n_hg;
  const int c = rest / n_hg;
  const Chunk ch = load_chunk(a.chunks, c);
  const int segs = 4 / a.hpw;
  const int wg_row0 = pb * 32 * segs;
  if (wg_row0 >= ch.len) return;
  const int h = hg * a.hpw + (wave % a.hpw);
  const int g = h / a.group;
  const int row0 = wg_row0 + (wave / a.hpw) * 32;
  const int nrows = max(0, min(32, ch.len - row0));
  const int L = a.seq_lens[ch.seq];
  const int64_t koff = a.seq_offsets[ch.seq];
  const int wg_last_pos = ch.pos0 + min(ch.len, wg_row0 + 32 * segs) - 1;
  const int kv_end = CAUSAL ? min(L, wg_last_pos + 1) : L;
  const int n_tiles = (kv_end + kBNq - 1) / kBNq;
  const int wave_first_pos = ch.pos0 + row0;
  const int wave_last_pos = wave_first_pos + nrows - 1;
  const int qpos = wave_first_pos + col;
  const bool qok = col < nrows;
  const int64_t qrow = (int64_t)ch.q_row + row0 + col;

  u32x4 qf[NST], dof[NST];
  {
    const int64_t off = (qrow * a.hq + h) * D + kg * 8;
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      qf[st] = qok ? ld16(a.q + off + st * 16) : u32x4{0u, 0u, 0u, 0u};
      dof[st] = qok ? ld16(a.dout + off + st * 16) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  const float lse2 = qok ? a.lse[(int64_t)h * a.q_rows + qrow] * kLog2e : INFINITY;
  const float dlt = qok ? a.delta[(int64_t)h * a.q_rows + qrow] : 0.f;
  const float* bias_row = nullptr;
  if (BIAS) bias_row = a.bias + ((int64_t)h * a.bias_len + min(qpos, a.bias_len - 1)) * a.bias_len;

  f32x16 dqt[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dqt[db] = f32x16{};
  const TrOffsets<D> tro(lane);

  const int64_t kv_stride = (int64_t)a.hkv * D;
  const uint16_t* kbase = a.k + koff * kv_stride + (int64_t)g * D;
  const uint16_t* vbase = a.v + koff * kv_stride + (int64_t)g * D;

  if (n_tiles > 0) {
    dma_rows<D, kBNq>(lds_k[0], kbase, kv_stride, L, wave, lane);
    dma_rows<D, kBNq>(lds_v[0], vbase, kv_stride, L, wave, lane);
  }
  wait_vm_all();
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int key0 = t * kBNq;
    const int buf = t & 1;
    if (t + 1 < n_tiles) {
      const int64_t nxt = (int64_t)(key0 + kBNq) * kv_stride;
      dma_rows<D, kBNq>(lds_k[buf ^ 1], kbase + nxt, kv_stride, L - key0 - kBNq, wave, lane);
      dma_rows<D, kBNq>(lds_v[buf ^ 1], vbase + nxt, kv_stride, L - key0 - kBNq, wave, lane);
    }
    if (nrows > 0 && !(CAUSAL && key0 > wave_last_pos)) {
      const uint16_t* kt = lds_k[buf];
      const uint16_t* vt = lds_v[buf];
      f32x16 s[2], dp[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
        dp[kb] = f32x16{};
#pragma unroll
        for (int st = 0; st < NST; ++st) {
          s[kb] = mfma32(lds_row16<D>(kt, kb * 32 + col, st * 2 + kg), qf[st], s[kb]);
          dp[kb] = mfma32(lds_row16<D>(vt, kb * 32 + col, st * 2 + kg), dof[st], dp[kb]);
        }
      }
      const bool need_mask = (key0 + kBNq > L) || (CAUSAL && key0 + kBNq - 1 > wave_first_pos);
      if (need_mask) {
        asm volatile("" ::: "memory");
        ds_tile<BIAS, true, CAUSAL>(s, dp, a.scale_log2, bias_row, key0, L, qpos, kg, a.bias_len, lse2, dlt);
      } else {
        ds_tile<BIAS, false, CAUSAL>(s, dp, a.scale_log2, bias_row, key0, L, qpos, kg, a.bias_len, lse2, dlt);
      }
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const u32x4 dsf = to_bf16x8(dp[st >> 1], (st & 1) * 8);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          dqt[db] = mfma32(tr_frag_at<D>(kt, tro, st, db), dsf, dqt[db]);
      }
    }
    wait_vm_all();
    __syncthreads();
  }

  if (!qok) return;
  uint16_t* op = a.dq + (qrow * a.hq + h) * D + kg * 4;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x2 w;
      w[0] = pack_bf16x2(dqt[db][i * 4 + 0] * a.scale, dqt[db][i * 4 + 1] * a.scale);
      w[1] = pack_bf16x2(dqt[db][i * 4 + 2] * a.scale, dqt[db][i * 4 + 3] * a.scale);
      st8(op + db * 32 + i * 8, w);
    }
}

// ---------------------------------------------------------------- launchers

hipError_t launch_dq(const AttnArgs& a, int D, bool causal, bool bias, dim3 grid, hipStream_t s) {
  CPATTN_BWD_DISPATCH(dq_kernel)
}

}  // namespace cpattn
