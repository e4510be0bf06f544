// dQ kernel of the attention backward (Q-parallel, with recompute).
//
// Page "Optimize context parallel attention layouts and gradient accumulation":
// "Changes" (GQA, causal THD with physical offsets) and "Related optimization work"
// (the backward is where the providers differ; here dQ recomputes S and dP rather than
// accumulating dQ with atomics).
//
// With P = exp(scale S - LSE), dP = dO V^T, Delta = rowsum(dO * O) and
// dS = P * (dP - Delta):  dQ = scale dS K, summed over the keys each query sees.
//
// Workgroup = (chunk, block of positions, `hpw` query heads that share one KV head),
// eight waves of 16 query rows each, two waves per SIMD: one wave's VALU and LDS work
// issues while the other's MFMAs run.  A wave keeps Q^T and dO^T of its rows in
// registers as B operands and dQ^T (D x 16 queries, fp32) as accumulators.  K and V
// tiles of 64 keys are copied into LDS one tile ahead (double buffer) and shared by the
// eight waves.  Per tile, with 16x16x32 MFMAs (C layout: lane = query, 4 key rows per
// lane and block):
//   S^T = K Q^T,  dP^T = V dO^T    (A = K / V rows, 16-byte LDS reads)
//   dS^T = P^T (dP^T - Delta)      (lane = query)
//   dQ^T += K^T dS^T               (A = K^T by transposing reads of the K tile,
//                                   B = dS^T as packed in-lane)
#include "common.h"
#include "launch.h"

namespace cpattn {

namespace {

constexpr int kKeys = 64;    // keys per K/V tile
constexpr int kRows = 16;    // query rows per wave
constexpr int kWavesQ = 8;   // waves per workgroup
constexpr int kThreadsQ = kWavesQ * 64;

// K and V tiles are stored with the kind-3 granule swizzle: the S^T / dP^T operand reads
// (lane group g of 16 lanes reads sixteen consecutive rows at granule 4 st + g) and the
// transposing reads below (eight consecutive rows x two adjacent granules per 32 lanes)
// are both free of bank conflicts.
constexpr int kSwz = 3;

// Lane parts of the transposing reads that gather the K^T A operand (16 dimensions x
// 32 keys) from the row-major, swizzled K tile.  In 16-lane group g, source lane
// 4 j + m reads key row k0 + 4 g + j (k0 = 32 ks + 16 r for read r of key step ks) at
// dimensions 16 db + 4 m + [0, 4); the output lane i then holds dimension 16 db + i of
// keys k0 + 4 g + [0, 4).  The row's swizzle depends on 4 g + j only and touches
// granule bits 0-3, so dimension block db = 8 a + b enters as 128 a + off[b].
template <int D>
struct KtOffsets {
  static constexpr int NB = (D / 16) < 8 ? (D / 16) : 8;
  int off[NB];
  __device__ __forceinline__ explicit KtOffsets(int lane) {
    const int g = lane >> 4, j = (lane >> 2) & 3, m = lane & 3;
    const int row = 4 * g + j;
#pragma unroll
    for (int b = 0; b < NB; ++b)
      off[b] = row * D + (((2 * b + (m >> 1)) ^ swz<D, kSwz>(row)) << 3) + 4 * (m & 1);
  }
};

template <int D>
__device__ __forceinline__ u32x4 kt_frag(const uint16_t* kt, const KtOffsets<D>& o, int ks, int db) {
  const uint16_t* b = kt + (32 * ks) * D + (db >> 3) * 128 + o.off[db & 7];
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(CPATTN_LDS(v4i16, b));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(CPATTN_LDS(v4i16, b + 16 * D));
  const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
  return u32x4{l2[0], l2[1], h2[0], h2[1]};
}

// dS^T = P^T (dP^T - Delta) for one 64-key tile, in place in dp (lane = query).
// Element j of block kb is key key0 + 16 kb + 4 g + j; with MASK, keys outside [lo, hi)
// (and past the query position when causal) give 0.
template <bool BIAS, bool MASK, bool CAUSAL>
__device__ __forceinline__ void ds_tile(const f32x4 (&s)[4], f32x4 (&dp)[4], float c,
                                        const float* bias_row, int key0, int lo, int hi, int qpos,
                                        int g, int bias_len, float lse2, float dlt) {
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kk = key0 + 16 * kb + 4 * g + j;
      float x;
      if (BIAS)
        x = fmaf(bias_row[min(kk, bias_len - 1)], kLog2e, s[kb][j] * c) - lse2;
      else
        x = fmaf(s[kb][j], c, -lse2);
      if (MASK) x = ((kk >= lo) && (kk < hi) && (!CAUSAL || kk <= qpos)) ? x : -INFINITY;
      const float p = exp2f_fast(x);  // a masked score is exp2(-inf) = 0
      dp[kb][j] = p * (dp[kb][j] - dlt);
    }
}

}  // namespace

template <int D, bool CAUSAL, bool BIAS>
__global__ __launch_bounds__(kThreadsQ) void dq_kernel(const AttnArgs a) {
  constexpr int NST = D / 32;  // 32-deep k-steps over the head dim
  constexpr int NDB = D / 16;  // 16-row blocks of dQ^T
  __shared__ __attribute__((aligned(1024))) uint16_t lds_k[2][kKeys * D];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_v[2][kKeys * D];

  if (*a.dev_err) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, q = lane & 15;  // lane group, query within the wave
  const int logical = xcd_group_order(blockIdx.x, gridDim.x / a.blocks_per_chunk, a.blocks_per_chunk, a.hq / a.hpw);
  const int n_hg = a.hq / a.hpw;
  const int pb = logical % a.blocks_per_chunk;
  const int rest = logical / a.blocks_per_chunk;
  const int hg = rest % n_hg;
  const int c = rest / n_hg;
  const Chunk ch = load_chunk_uniform(a.chunks, c);
  const int wg_pos = kRows * (kWavesQ / a.hpw);  // positions per workgroup
  const int wg_row0 = pb * wg_pos;
  if (wg_row0 >= ch.len) return;  // uniform over the workgroup, before any barrier
  const int h = hg * a.hpw + (wave % a.hpw);
  const int kvh = h / a.group;
  const int row0 = wg_row0 + (wave / a.hpw) * kRows;  // first chunk row of this wave
  const int nrows = max(0, min(kRows, ch.len - row0));
  const int L = rfl(a.seq_lens[ch.seq]);
  const int64_t koff = rfl(a.seq_offsets[ch.seq]);
  const int wg_last_pos = ch.pos0 + min(ch.len, wg_row0 + wg_pos) - 1;
  // Keys [kv_lo, kv_end): the key window (the whole sequence without one), cut at the
  // workgroup's last position when causal.
  const int kv_lo = a.kv_lo;
  const int kv_hi = min(L, a.kv_hi);
  const int kv_end = min(CAUSAL ? min(L, wg_last_pos + 1) : L, kv_hi);
  const int t_first = kv_lo / kKeys;               // first tile (absolute index)
  const int n_tiles = (kv_end + kKeys - 1) / kKeys;  // one past the last tile
  const int wave_first_pos = ch.pos0 + row0;
  const int wave_last_pos = wave_first_pos + nrows - 1;
  const int qpos = wave_first_pos + q;
  const bool qok = q < nrows;
  const int64_t qrow = (int64_t)ch.q_row + row0 + q;

  // Q^T and dO^T as B operands: lane (g, q) holds query q, dimensions 32 st + 8 g + [0, 8).
  u32x4 qf[NST], dof[NST];
  {
    const int64_t off = (qrow * a.q_pitch + h) * D + g * 8;
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      qf[st] = qok ? ld16(a.q + off + st * 32) : u32x4{0u, 0u, 0u, 0u};
      dof[st] = qok ? ld16(a.dout + off + st * 32) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  const float lse2 = qok ? a.lse[(int64_t)h * a.q_rows + qrow] * kLog2e : INFINITY;
  const float dlt = qok ? a.delta[(int64_t)h * a.q_rows + qrow] : 0.f;
  const float* bias_row = nullptr;
  if (BIAS) bias_row = a.bias + ((int64_t)h * a.bias_len + min(qpos, a.bias_len - 1)) * a.bias_len;

  f32x4 dqt[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dqt[db] = f32x4{};
  const KtOffsets<D> kto(lane);

  const int64_t kv_stride = a.kv_pitch * D;
  const uint16_t* kbase = a.k + koff * kv_stride + (int64_t)kvh * D;
  const uint16_t* vbase = a.v + koff * kv_stride + (int64_t)kvh * D;

  if (n_tiles > t_first) {
    const int64_t first = (int64_t)t_first * kKeys * kv_stride;
    dma_rows<D, kKeys, kWavesQ, kSwz>(lds_k[0], kbase + first, kv_stride, L - t_first * kKeys, wave, lane);
    dma_rows<D, kKeys, kWavesQ, kSwz>(lds_v[0], vbase + first, kv_stride, L - t_first * kKeys, wave, lane);
  }
  wait_vm_all();
  __syncthreads();

  for (int t = t_first; t < n_tiles; ++t) {
    const int key0 = t * kKeys;
    const int buf = (t - t_first) & 1;
    if (t + 1 < n_tiles) {
      const int64_t nxt = (int64_t)(key0 + kKeys) * kv_stride;
      dma_rows<D, kKeys, kWavesQ, kSwz>(lds_k[buf ^ 1], kbase + nxt, kv_stride, L - key0 - kKeys, wave, lane);
      dma_rows<D, kKeys, kWavesQ, kSwz>(lds_v[buf ^ 1], vbase + nxt, kv_stride, L - key0 - kKeys, wave, lane);
    }
    if (nrows > 0 && !(CAUSAL && key0 > wave_last_pos)) {
      const uint16_t* kt = lds_k[buf];
      const uint16_t* vt = lds_v[buf];
      // S^T and dP^T: four 16-key blocks; A operand = key row 16 kb + q, granule 4 st + g.
      f32x4 s[4], dp[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        s[kb] = f32x4{};
        dp[kb] = f32x4{};
      }
#pragma unroll
      for (int st = 0; st < NST; ++st)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          s[kb] = mfma16(lds_row16<D, kSwz>(kt, 16 * kb + q, 4 * st + g), qf[st], s[kb]);
          dp[kb] = mfma16(lds_row16<D, kSwz>(vt, 16 * kb + q, 4 * st + g), dof[st], dp[kb]);
        }
      const bool need_mask = (key0 + kKeys > kv_hi) || (key0 < kv_lo) ||
                             (CAUSAL && key0 + kKeys - 1 > wave_first_pos);
      if (need_mask)
        ds_tile<BIAS, true, CAUSAL>(s, dp, a.scale_log2, bias_row, key0, kv_lo, kv_hi, qpos, g, a.bias_len,
                                    lse2, dlt);
      else
        ds_tile<BIAS, false, CAUSAL>(s, dp, a.scale_log2, bias_row, key0, kv_lo, kv_hi, qpos, g, a.bias_len,
                                     lse2, dlt);
      // dQ^T += K^T dS^T over two 32-key steps; k-position 8 g + e of step ks is key
      // 32 ks + 16 (e / 4) + 4 g + e % 4, i.e. element e % 4 of blocks 2 ks and 2 ks + 1.
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const u32x4 dsf = {pack_bf16x2(dp[2 * ks][0], dp[2 * ks][1]), pack_bf16x2(dp[2 * ks][2], dp[2 * ks][3]),
                           pack_bf16x2(dp[2 * ks + 1][0], dp[2 * ks + 1][1]),
                           pack_bf16x2(dp[2 * ks + 1][2], dp[2 * ks + 1][3])};
#pragma unroll
        for (int db = 0; db < NDB; ++db) dqt[db] = mfma16(kt_frag<D>(kt, kto, ks, db), dsf, dqt[db]);
      }
    }
    wait_vm_all();
    __syncthreads();
  }

  if (!qok) return;
  // element j of block db is dimension 16 db + 4 g + j; with dq_accumulate the existing
  // BF16 value is added in fp32 and the sum rounded once (a key window's contribution)
  uint16_t* op = a.dq + (qrow * a.q_pitch + h) * D + g * 4;
  if (a.dq_accumulate) {
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const u32x2 old = ld8(op + db * 16);
      st8(op + db * 16,
          u32x2{pack_bf16x2(fmaf(dqt[db][0], a.scale, bf16_lo(old[0])), fmaf(dqt[db][1], a.scale, bf16_hi(old[0]))),
                pack_bf16x2(fmaf(dqt[db][2], a.scale, bf16_lo(old[1])), fmaf(dqt[db][3], a.scale, bf16_hi(old[1])))});
    }
  } else {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      st8(op + db * 16, u32x2{pack_bf16x2(dqt[db][0] * a.scale, dqt[db][1] * a.scale),
                              pack_bf16x2(dqt[db][2] * a.scale, dqt[db][3] * a.scale)});
  }
}

hipError_t launch_dq(const AttnArgs& a, int D, bool causal, bool bias, dim3 grid, hipStream_t s) {
  constexpr int kThreads = kThreadsQ;
  CPATTN_BWD_DISPATCH(dq_kernel)
}

}  // namespace cpattn
