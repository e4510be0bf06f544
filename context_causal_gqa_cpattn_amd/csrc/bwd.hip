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
//    layout in which dK/dV contracts over queries with 16-byte LDS reads.
// Tiles are numbered per chunk through tile_base (prefix sums of ceil(len/32)).

constexpr int kTileQ = 32;

__global__ __launch_bounds__(1024) void tile_scan_kernel(const int32_t* chunks, int num_chunks,
                                                          int32_t* tile_base, const int32_t* dev_err) {
  if (*dev_err) return;
  __shared__ int part[1024];
  const int t = threadIdx.x;
  const int per = (num_chunks + 1023) / 1024;
  const int c0 = min(num_chunks, t * per), c1 = min(num_chunks, c0 + per);
  int sum = 0;
  for (int c = c0; c < c1; ++c) sum += (max(chunks[4 * c + 3], 0) + kTileQ - 1) / kTileQ;
  part[t] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int run = part[t] - sum;
  for (int c = c0; c < c1; ++c) {
    tile_base[c] = run;
    run += (max(chunks[4 * c + 3], 0) + kTileQ - 1) / kTileQ;
  }
  if (t == 1023) tile_base[num_chunks] = part[1023];
}

hipError_t launch_tile_scan(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(tile_scan_kernel, dim3(1), dim3(1024), 0, s, a.chunks, a.num_chunks,
                     a.tile_base_out, a.dev_err);
  return hipGetLastError();
}

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
  const int tile = a.tile_base[c] + qt;
  const int tensor = tid / TASKS;  // 0: Q, 1: dO
  const int task = tid % TASKS;
  const int qg = task / DG, dg = task % DG;  // dg varies fastest within a wave
  const int64_t rs = (int64_t)a.hq * D;
  const int64_t off = ((int64_t)ch.q_row + r0) * rs + (int64_t)h * D + dg * 8;
  const uint16_t* src = (tensor ? a.dout : a.q) + off;
  u32x4 rows[8], cols[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int qi = qg * 8 + e;
    rows[e] = qi < nq ? ld16(src + qi * rs) : u32x4{0u, 0u, 0u, 0u};
  }
  if (tensor == 1) {
    float ds[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int qi = qg * 8 + e;
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
      for (int e = 0; e < 8; ++e)
        if (qg * 8 + e < nq) a.delta_out[(int64_t)h * a.q_rows + ch.q_row + r0 + qg * 8 + e] = ds[e];
    }
  }
  transpose8x8(rows, cols);  // cols[d]: the 8 queries of dimension dg*8 + d
  uint16_t* dst = (tensor ? a.dot_out : a.qt_out) + ((int64_t)tile * a.hq + h) * D * kTileQ;
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

// ---------------------------------------------------------------- dK / dV
//
// Workgroup = (sequence, 128-key tile, KV head g) with eight waves; wave w owns keys
// [16w, 16w+16) of the tile and keeps them in registers as B operands (K^T, V^T) for
// the whole loop, with dK^T and dV^T (16 keys x D) accumulating in fp32 (16x16x32 MFMA
// tiles keep that at 2*D/16*4 registers per lane).  The loop runs over every (chunk of
// the sequence, query head of the group, 32-query tile) that sees the key tile; Q and
// dO tiles (and their LSE/Delta) are DMA'd into LDS one iteration ahead.  Per tile:
//   S  = Q K^T     A = Q rows (16-byte LDS reads), B = K^T registers
//   dP = dO V^T    A = dO rows, B = V^T registers
//   P = exp(scale S - LSE), dS = P (dP - Delta)    (C layout: lane = key, rows = queries)
//   dV^T += dO^T P   A = rows of the pre-pass's transposed dO tile (16-byte reads),
//                    B = P (already in B layout)
//   dK^T += Q^T dS   A = rows of the transposed Q tile, B = dS
// The S/dP row order is chosen so that lane group g of P and dS holds the eight
// contiguous queries 8g..8g+7, the order of one 16-byte granule of a transposed row.
// The GQA sum over the group's query heads and the sum over chunks happen in the fp32
// accumulators; dK = scale dK^T and dV are rounded to BF16 once (STORE), or added to
// the existing BF16 values and rounded once (ADD).

constexpr int kBM = 32;          // queries per tile
constexpr int kDkdvWaves = 8;    // waves per dK/dV workgroup (16 keys each)
constexpr int kDkdvThreads = kDkdvWaves * 64;

struct QTileIter {
  int c, hh, qt, qt_first, n_qt;
  Chunk ch;
};

// Advance to the next chunk (from c) that has query tiles seeing keys >= key0.
template <bool CAUSAL>
__device__ __forceinline__ bool seek_chunk(const AttnArgs& a, QTileIter& it, int c_end, int key0) {
  for (; it.c < c_end; ++it.c) {
    it.ch = load_chunk(a.chunks, it.c);
    const int first_row = CAUSAL ? max(0, key0 - it.ch.pos0) : 0;
    if (first_row < it.ch.len) {
      it.qt_first = first_row / kBM;
      it.n_qt = (it.ch.len + kBM - 1) / kBM;
      it.qt = it.qt_first;
      it.hh = 0;
      return true;
    }
  }
  return false;
}

template <bool CAUSAL>
__device__ __forceinline__ bool advance(const AttnArgs& a, QTileIter& it, int c_end, int key0) {
  if (++it.qt < it.n_qt) return true;
  it.qt = it.qt_first;
  if (++it.hh < a.group) return true;
  ++it.c;
  return seek_chunk<CAUSAL>(a, it, c_end, key0);
}

template <int D>
__device__ __forceinline__ void dma_q_do(uint16_t* lq, uint16_t* ldo, uint16_t* lqt, uint16_t* ldot,
                                         const AttnArgs& a, const QTileIter& it, int g, int wave,
                                         int lane) {
  const int h = g * a.group + it.hh;
  const int64_t rs = (int64_t)a.hq * D;
  const int64_t off = ((int64_t)it.ch.q_row + it.qt * kBM) * rs + (int64_t)h * D;
  const int nq = min(kBM, it.ch.len - it.qt * kBM);
  dma_rows<D, kBM, kDkdvWaves, 2>(lq, a.q + off, rs, nq, wave, lane);
  dma_rows<D, kBM, kDkdvWaves, 2>(ldo, a.dout + off, rs, nq, wave, lane);
  // transposed tiles: already swizzled by the pre-pass, copied as they are
  const int64_t toff = ((int64_t)(a.tile_base[it.c] + it.qt) * a.hq + h) * D * kTileQ;
  constexpr int NI = D * kTileQ * 2 / 1024;
  for (int i = __builtin_amdgcn_readfirstlane(wave); i < NI; i += kDkdvWaves) {
    dma16(a.qt + toff + i * 512 + lane * 8, lqt + i * 512);
    dma16(a.dot + toff + i * 512 + lane * 8, ldot + i * 512);
  }
}

// LSE (as base-2) and Delta of tile row `r` (clamped to the valid rows).
__device__ __forceinline__ void load_stats(const AttnArgs& a, const QTileIter& it, int g, int r,
                                           float& lse2, float& dl) {
  const int h = g * a.group + it.hh;
  const int nq = min(kBM, it.ch.len - it.qt * kBM);
  const int64_t idx = (int64_t)h * a.q_rows + it.ch.q_row + it.qt * kBM + min(r, nq - 1);
  lse2 = a.lse[idx] * kLog2e;
  dl = a.delta[idx];
}

template <int D, bool CAUSAL, bool BIAS>
__global__ __launch_bounds__(kDkdvThreads) void dkdv_kernel(const AttnArgs a) {
  constexpr int NS = D / 32;   // 32-wide k-steps of S and dP
  constexpr int NDB = D / 16;  // 16-row d blocks of dK^T and dV^T
  __shared__ __attribute__((aligned(1024))) uint16_t lds_q[2][kBM * D];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_do[2][kBM * D];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_qt[2][D * kBM];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_dot[2][D * kBM];
  __shared__ __attribute__((aligned(16))) float lds_lse[2][kBM];
  __shared__ __attribute__((aligned(16))) float lds_dl[2][kBM];

  if (*a.dev_err) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 4, n = lane & 15;
  // S/dP A-operand row n of block mb is tile query 8*(n/4) + 4*mb + n%4
  const int qrow_a = 8 * (n >> 2) + (n & 3);
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int kt = logical % a.kv_tiles;
  const int rest = logical / a.kv_tiles;
  const int g = rest % a.hkv;
  const int b = rest / a.hkv;
  const int L = a.seq_lens[b];
  const int wg_key0 = kt * kDkdvKeys;
  if (wg_key0 >= L) return;
  const int64_t koff = a.seq_offsets[b];
  const int wkey0 = wg_key0 + wave * 16;
  const int nk = max(0, min(16, L - wkey0));
  const int key = wkey0 + n;  // this lane's key (column of S, dP; of dK^T, dV^T)

  // K and V as B operands (columns = keys), held for the whole loop.
  const int64_t kv_stride = (int64_t)a.hkv * D;
  u32x4 kf[NS], vf[NS];
  {
    const int64_t off = (koff + min(key, L - 1)) * kv_stride + (int64_t)g * D + lg * 8;
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      kf[st] = (n < nk) ? ld16(a.k + off + st * 32) : u32x4{0u, 0u, 0u, 0u};
      vf[st] = (n < nk) ? ld16(a.v + off + st * 32) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  f32x4 dkt[NDB], dvt[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) { dkt[db] = f32x4{}; dvt[db] = f32x4{}; }

  const int c_end = chunk_lower_bound(a.chunks, a.num_chunks, b + 1);
  QTileIter cur;
  cur.c = chunk_lower_bound(a.chunks, a.num_chunks, b);
  bool have = seek_chunk<CAUSAL>(a, cur, c_end, wg_key0);
  float st_lse = 0.f, st_dl = 0.f;  // stats staged for the next tile (threads < kBM)
  if (have) {
    dma_q_do<D>(lds_q[0], lds_do[0], lds_qt[0], lds_dot[0], a, cur, g, wave, lane);
    if (tid < kBM) {
      load_stats(a, cur, g, tid, st_lse, st_dl);
      lds_lse[0][tid] = st_lse;
      lds_dl[0][tid] = st_dl;
    }
  }
  wait_vm_all();
  __syncthreads();

  int buf = 0;
  while (have) {
    QTileIter nxt = cur;
    const bool have_next = advance<CAUSAL>(a, nxt, c_end, wg_key0);
    if (have_next) {
      dma_q_do<D>(lds_q[buf ^ 1], lds_do[buf ^ 1], lds_qt[buf ^ 1], lds_dot[buf ^ 1], a, nxt, g,
                  wave, lane);
      if (tid < kBM) load_stats(a, nxt, g, tid, st_lse, st_dl);
    }

    const int nq = min(kBM, cur.ch.len - cur.qt * kBM);
    const int tile_pos0 = cur.ch.pos0 + cur.qt * kBM;
    if (nk > 0 && !(CAUSAL && tile_pos0 + nq - 1 < wkey0)) {
      const uint16_t* qt_l = lds_q[buf];
      const uint16_t* dt_l = lds_do[buf];
      f32x4 s[2], dp[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        s[mb] = f32x4{};
        dp[mb] = f32x4{};
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          s[mb] = mfma16(lds_row16<D, 2>(qt_l, qrow_a + 4 * mb, st * 4 + lg), kf[st], s[mb]);
          dp[mb] = mfma16(lds_row16<D, 2>(dt_l, qrow_a + 4 * mb, st * 4 + lg), vf[st], dp[mb]);
        }
      }
      const bool need_mask = (nk < 16) || (nq < kBM) || (CAUSAL && tile_pos0 < wkey0 + 15);
      const float* bias_h = BIAS ? a.bias + (int64_t)(g * a.group + cur.hh) * a.bias_len * a.bias_len : nullptr;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int q4 = lg * 8 + mb * 4;  // element j is tile query q4 + j
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&lds_lse[buf][q4]);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&lds_dl[buf][q4]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int qi = q4 + j;
          float x = s[mb][j] * a.scale_log2;
          if (BIAS)
            x = fmaf(bias_h[(int64_t)min(tile_pos0 + qi, a.bias_len - 1) * a.bias_len + min(key, a.bias_len - 1)],
                     kLog2e, x);
          bool vis = true;
          if (need_mask) vis = (n < nk) && (qi < nq) && (!CAUSAL || key <= tile_pos0 + qi);
          const float p = vis ? exp2f_fast(x - l4[j]) : 0.f;
          s[mb][j] = p;
          dp[mb][j] = p * (dp[mb][j] - d4[j]);
        }
      }
      const u32x4 pf = {pack_bf16x2(s[0][0], s[0][1]), pack_bf16x2(s[0][2], s[0][3]),
                        pack_bf16x2(s[1][0], s[1][1]), pack_bf16x2(s[1][2], s[1][3])};
      const u32x4 dsf = {pack_bf16x2(dp[0][0], dp[0][1]), pack_bf16x2(dp[0][2], dp[0][3]),
                         pack_bf16x2(dp[1][0], dp[1][1]), pack_bf16x2(dp[1][2], dp[1][3])};
      const uint16_t* qtt = lds_qt[buf];
      const uint16_t* dtt = lds_dot[buf];
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int d = db * 16 + n;
        const int o = d * kBM + ((lg ^ tswz(d)) * 8);
        dvt[db] = mfma16(ld16(dtt + o), pf, dvt[db]);
        dkt[db] = mfma16(ld16(qtt + o), dsf, dkt[db]);
      }
    }
    if (have_next && tid < kBM) {
      lds_lse[buf ^ 1][tid] = st_lse;
      lds_dl[buf ^ 1][tid] = st_dl;
    }
    wait_vm_all();
    __syncthreads();
    cur = nxt;
    have = have_next;
    buf ^= 1;
  }

  if (n >= nk) return;
  const int64_t off = (koff + key) * kv_stride + (int64_t)g * D + lg * 4;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int64_t o = off + db * 16;
    float k0 = dkt[db][0] * a.scale, k1 = dkt[db][1] * a.scale;
    float k2 = dkt[db][2] * a.scale, k3 = dkt[db][3] * a.scale;
    float v0 = dvt[db][0], v1 = dvt[db][1], v2 = dvt[db][2], v3 = dvt[db][3];
    if (a.accumulate) {
      const u32x2 ok = ld8(a.dk + o), ov = ld8(a.dv + o);
      k0 += bf16_lo(ok[0]); k1 += bf16_hi(ok[0]); k2 += bf16_lo(ok[1]); k3 += bf16_hi(ok[1]);
      v0 += bf16_lo(ov[0]); v1 += bf16_hi(ov[0]); v2 += bf16_lo(ov[1]); v3 += bf16_hi(ov[1]);
    }
    st8(a.dk + o, u32x2{pack_bf16x2(k0, k1), pack_bf16x2(k2, k3)});
    st8(a.dv + o, u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)});
  }
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
        float x = s[kb][i * 4 + j] * c;
        if (BIAS) x = fmaf(bias_row[min(kk, bias_len - 1)], kLog2e, x);
        bool vis = true;
        if (MASK) vis = (kk < L) && (!CAUSAL || kk <= qpos);
        const float p = vis ? exp2f_fast(x - lse2) : 0.f;
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
          dqt[db] = mfma32(tr_frag<D>(kt, st * 16, db, lane), dsf, dqt[db]);
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

#define CPATTN_BWD_DISPATCH(KERNEL)                                                          \
  if (bias) {                                                                                \
    if (causal) return hipErrorInvalidValue;                                                 \
    switch (D) {                                                                             \
      case 32: hipLaunchKernelGGL((KERNEL<32, false, true>), grid, dim3(kThreads), 0, s, a); break;   \
      case 64: hipLaunchKernelGGL((KERNEL<64, false, true>), grid, dim3(kThreads), 0, s, a); break;   \
      case 128: hipLaunchKernelGGL((KERNEL<128, false, true>), grid, dim3(kThreads), 0, s, a); break; \
      default: return hipErrorInvalidValue;                                                  \
    }                                                                                        \
  } else if (causal) {                                                                       \
    switch (D) {                                                                             \
      case 32: hipLaunchKernelGGL((KERNEL<32, true, false>), grid, dim3(kThreads), 0, s, a); break;   \
      case 64: hipLaunchKernelGGL((KERNEL<64, true, false>), grid, dim3(kThreads), 0, s, a); break;   \
      case 128: hipLaunchKernelGGL((KERNEL<128, true, false>), grid, dim3(kThreads), 0, s, a); break; \
      case 256: hipLaunchKernelGGL((KERNEL<256, true, false>), grid, dim3(kThreads), 0, s, a); break; \
      default: return hipErrorInvalidValue;                                                  \
    }                                                                                        \
  } else {                                                                                   \
    switch (D) {                                                                             \
      case 32: hipLaunchKernelGGL((KERNEL<32, false, false>), grid, dim3(kThreads), 0, s, a); break;   \
      case 64: hipLaunchKernelGGL((KERNEL<64, false, false>), grid, dim3(kThreads), 0, s, a); break;   \
      case 128: hipLaunchKernelGGL((KERNEL<128, false, false>), grid, dim3(kThreads), 0, s, a); break; \
      case 256: hipLaunchKernelGGL((KERNEL<256, false, false>), grid, dim3(kThreads), 0, s, a); break; \
      default: return hipErrorInvalidValue;                                                  \
    }                                                                                        \
  }                                                                                          \
  return hipGetLastError();

hipError_t launch_dkdv(const AttnArgs& a, int D, bool causal, bool bias, dim3 grid, hipStream_t s) {
  constexpr int kThreads = kDkdvThreads;
  CPATTN_BWD_DISPATCH(dkdv_kernel)
}

hipError_t launch_dq(const AttnArgs& a, int D, bool causal, bool bias, dim3 grid, hipStream_t s) {
  CPATTN_BWD_DISPATCH(dq_kernel)
}

}  // namespace cpattn
