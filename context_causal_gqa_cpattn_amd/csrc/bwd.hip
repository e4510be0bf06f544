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

template <int D>
__global__ __launch_bounds__(kThreads) void prepass_kernel(const AttnArgs a) {
  if (*a.dev_err) return;
  constexpr int TPP = D / 8;  // threads per (row, head) pair, 8 elements each
  const int tid = threadIdx.x;
  const int c = blockIdx.x / a.blocks_per_chunk;
  const int rb = blockIdx.x % a.blocks_per_chunk;
  const Chunk ch = load_chunk(a.chunks, c);
  const int r0 = rb * kPrepassRows;
  if (r0 >= ch.len) return;
  const int nr = min(kPrepassRows, ch.len - r0);
  const int pairs = nr * a.hq;
  const int sub = tid % TPP;
  for (int p = tid / TPP; p < pairs; p += kThreads / TPP) {
    const int row = p / a.hq, h = p % a.hq;
    const int64_t qr = (int64_t)ch.q_row + r0 + row;
    const int64_t off = (qr * a.hq + h) * D + sub * 8;
    const u32x4 ov = ld16(a.o + off), dv = ld16(a.dout + off);
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc = fmaf(bf16_lo(ov[w]), bf16_lo(dv[w]), acc);
      acc = fmaf(bf16_hi(ov[w]), bf16_hi(dv[w]), acc);
    }
#pragma unroll
    for (int m = TPP / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
    if (sub == 0) a.delta_out[(int64_t)h * a.q_rows + qr] = acc;
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

template <int D>
struct DkdvSmem {
  static constexpr int NS = D + 8;   // natural [query][d] stride
  static constexpr int TS = 32 + 8;  // transposed [d][query slot] stride
  uint16_t q[32 * NS];
  uint16_t dO[32 * NS];
  uint16_t qt[D * TS];
  uint16_t dOt[D * TS];
  float lse2[32];
  float delta[32];
};

// Stage 32 chunk rows of Q and dO for head h: natural and transposed (sigma slots).
template <int D>
__device__ __forceinline__ void stage_q_do(DkdvSmem<D>& sm, const AttnArgs& a, int64_t qrow0,
                                           int nq, int h, int tid) {
  constexpr int D8 = D / 8;
  constexpr int NBLK = 4 * D8;  // 8x8 blocks per tensor
  const int64_t rs = (int64_t)a.hq * D;
  for (int i = tid; i < 2 * NBLK; i += kThreads) {
    const int tsel = i / NBLK, j = i % NBLK;
    const int pg = j & 3, dg = j >> 2;
    const uint16_t* base = (tsel ? a.dout : a.q) + qrow0 * rs + (int64_t)h * D + dg * 8;
    uint16_t* nat = tsel ? sm.dO : sm.q;
    uint16_t* tr = tsel ? sm.dOt : sm.qt;
    u32x4 rows[8], cols[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int qi = (pg >> 1) * 16 + sigma16((pg & 1) * 8 + e);
      rows[e] = (qi < nq) ? ld16(base + (int64_t)qi * rs) : u32x4{0u, 0u, 0u, 0u};
      st16(&nat[qi * DkdvSmem<D>::NS + dg * 8], rows[e]);
    }
    transpose8x8(rows, cols);
#pragma unroll
    for (int d = 0; d < 8; ++d) st16(&tr[(dg * 8 + d) * DkdvSmem<D>::TS + pg * 8], cols[d]);
  }
  if (tid < 32) {
    const bool ok = tid < nq;
    const int64_t idx = (int64_t)h * a.q_rows + qrow0 + tid;
    sm.lse2[tid] = ok ? a.lse[idx] * kLog2e : INFINITY;
    sm.delta[tid] = ok ? a.delta[idx] : 0.f;
  }
}

template <int D, bool CAUSAL, bool BIAS>
__global__ __launch_bounds__(kThreads) void dkdv_kernel(const AttnArgs a) {
  constexpr int NST = D / 16;
  constexpr int NDB = D / 32;
  __shared__ DkdvSmem<D> sm;

  if (*a.dev_err) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kg = lane >> 5, col = lane & 31;
  const int b = blockIdx.x / a.kv_tiles;
  const int kt = blockIdx.x % a.kv_tiles;
  const int g = blockIdx.y;
  const int L = a.seq_lens[b];
  const int wg_key0 = kt * kDkdvKeys;
  if (wg_key0 >= L) return;
  const int64_t koff = a.seq_offsets[b];
  const int wkey0 = wg_key0 + wave * 32;
  const int nk = max(0, min(32, L - wkey0));
  const int key = wkey0 + col;  // this lane's key (column of S, dP; of dK^T, dV^T)

  // K and V as B operands (columns = keys), held for the whole loop.
  const int64_t kv_stride = (int64_t)a.hkv * D;
  u32x4 kf[NST], vf[NST];
  {
    const int64_t off = (koff + key) * kv_stride + (int64_t)g * D + kg * 8;
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      kf[st] = (col < nk) ? ld16(a.k + off + st * 16) : u32x4{0u, 0u, 0u, 0u};
      vf[st] = (col < nk) ? ld16(a.v + off + st * 16) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  f32x16 dkt[NDB], dvt[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) { dkt[db] = f32x16{}; dvt[db] = f32x16{}; }

  const int c_begin = chunk_lower_bound(a.chunks, a.num_chunks, b);
  const int c_end = chunk_lower_bound(a.chunks, a.num_chunks, b + 1);
  for (int c = c_begin; c < c_end; ++c) {
    const Chunk ch = load_chunk(a.chunks, c);
    const int first_row = CAUSAL ? max(0, wg_key0 - ch.pos0) : 0;
    if (first_row >= ch.len) continue;
    const int n_qt = (ch.len + 31) / 32;
    for (int hh = 0; hh < a.group; ++hh) {
      const int h = g * a.group + hh;
      const float* bias_h = BIAS ? a.bias + (int64_t)h * a.bias_len * a.bias_len : nullptr;
      for (int qt = first_row / 32; qt < n_qt; ++qt) {
        const int nq = min(32, ch.len - qt * 32);
        const int64_t qrow0 = (int64_t)ch.q_row + qt * 32;
        const int tile_pos0 = ch.pos0 + qt * 32;
        __syncthreads();
        stage_q_do<D>(sm, a, qrow0, nq, h, tid);
        __syncthreads();
        if (nk == 0) continue;
        if (CAUSAL && tile_pos0 + nq - 1 < wkey0) continue;

        f32x16 s = f32x16{}, dp = f32x16{};
        const uint16_t* qa = &sm.q[col * DkdvSmem<D>::NS + kg * 8];
        const uint16_t* da = &sm.dO[col * DkdvSmem<D>::NS + kg * 8];
#pragma unroll
        for (int st = 0; st < NST; ++st) {
          s = mfma32(ld16(qa + st * 16), kf[st], s);
          dp = mfma32(ld16(da + st * 16), vf[st], dp);
        }
        // P and dS; element r of s is query 8*(r/4) + 4*kg + r%4 of the tile.
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qi = (r >> 2) * 8 + kg * 4 + (r & 3);
          const int qpos = tile_pos0 + qi;
          float x = s[r] * a.scale_log2;
          if (BIAS) x += bias_h[(int64_t)min(qpos, a.bias_len - 1) * a.bias_len + min(key, a.bias_len - 1)] * kLog2e;
          const bool vis = (col < nk) && (!CAUSAL || key <= qpos);
          const float p = vis ? exp2f_fast(x - sm.lse2[qi]) : 0.f;
          s[r] = p;
          dp[r] = p * (dp[r] - sm.delta[qi]);
        }
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const u32x4 pf = to_bf16x8(s, st * 8);
          const u32x4 dsf = to_bf16x8(dp, st * 8);
          const uint16_t* dta = &sm.dOt[col * DkdvSmem<D>::TS + st * 16 + kg * 8];
          const uint16_t* qta = &sm.qt[col * DkdvSmem<D>::TS + st * 16 + kg * 8];
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            dvt[db] = mfma32(ld16(dta + db * 32 * DkdvSmem<D>::TS), pf, dvt[db]);
            dkt[db] = mfma32(ld16(qta + db * 32 * DkdvSmem<D>::TS), dsf, dkt[db]);
          }
        }
      }
    }
  }

  if (col >= nk) return;
  const int64_t off = (koff + key) * kv_stride + (int64_t)g * D + kg * 4;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t o = off + db * 32 + i * 8;
      float k0 = dkt[db][i * 4 + 0] * a.scale, k1 = dkt[db][i * 4 + 1] * a.scale;
      float k2 = dkt[db][i * 4 + 2] * a.scale, k3 = dkt[db][i * 4 + 3] * a.scale;
      float v0 = dvt[db][i * 4 + 0], v1 = dvt[db][i * 4 + 1];
      float v2 = dvt[db][i * 4 + 2], v3 = dvt[db][i * 4 + 3];
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

constexpr int kBNq = 64;  // keys per KV tile in the dQ kernel

template <int D>
struct DqSmem {
  static constexpr int NS = D + 8;
  static constexpr int TS = kBNq + 8;
  uint16_t k[kBNq * NS];
  uint16_t v[kBNq * NS];
  uint16_t kt[D * TS];
};

template <int D>
__device__ __forceinline__ void stage_kv_dq(DqSmem<D>& sm, const uint16_t* __restrict__ kbase,
                                            const uint16_t* __restrict__ vbase, int64_t rs,
                                            int key0, int L, int tid) {
  constexpr int D8 = D / 8;
  // K: natural rows and the transpose (sigma slots), from one load.
  for (int i = tid; i < (kBNq / 8) * D8; i += kThreads) {
    const int pg = i % (kBNq / 8), dg = i / (kBNq / 8);
    u32x4 rows[8], cols[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int kl = (pg >> 1) * 16 + sigma16((pg & 1) * 8 + e);
      const int key = key0 + kl;
      rows[e] = (key < L) ? ld16(kbase + (int64_t)key * rs + dg * 8) : u32x4{0u, 0u, 0u, 0u};
      st16(&sm.k[kl * DqSmem<D>::NS + dg * 8], rows[e]);
    }
    transpose8x8(rows, cols);
#pragma unroll
    for (int d = 0; d < 8; ++d) st16(&sm.kt[(dg * 8 + d) * DqSmem<D>::TS + pg * 8], cols[d]);
  }
  for (int i = tid; i < kBNq * D8; i += kThreads) {
    const int r = i / D8, c = i % D8;
    const int key = key0 + r;
    st16(&sm.v[r * DqSmem<D>::NS + c * 8],
         (key < L) ? ld16(vbase + (int64_t)key * rs + c * 8) : u32x4{0u, 0u, 0u, 0u});
  }
}

template <int D, bool CAUSAL, bool BIAS>
__global__ __launch_bounds__(kThreads) void dq_kernel(const AttnArgs a) {
  constexpr int NST = D / 16;
  constexpr int NDB = D / 32;
  __shared__ DqSmem<D> sm;

  if (*a.dev_err) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kg = lane >> 5, col = lane & 31;
  const int c = blockIdx.x / a.blocks_per_chunk;
  const int pb = blockIdx.x % a.blocks_per_chunk;
  const Chunk ch = load_chunk(a.chunks, c);
  const int segs = 4 / a.hpw;
  const int wg_row0 = pb * 32 * segs;
  if (wg_row0 >= ch.len) return;
  const int h = blockIdx.y * a.hpw + (wave % a.hpw);
  const int g = h / a.group;
  const int row0 = wg_row0 + (wave / a.hpw) * 32;
  const int nrows = max(0, min(32, ch.len - row0));
  const int L = a.seq_lens[ch.seq];
  const int64_t koff = a.seq_offsets[ch.seq];
  const int wg_last_pos = ch.pos0 + min(ch.len, wg_row0 + 32 * segs) - 1;
  const int kv_end = CAUSAL ? min(L, wg_last_pos + 1) : L;
  const int n_tiles = (kv_end + kBNq - 1) / kBNq;
  const int wave_last_pos = ch.pos0 + row0 + nrows - 1;
  const int qpos = ch.pos0 + row0 + col;
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

  for (int t = 0; t < n_tiles; ++t) {
    const int key0 = t * kBNq;
    __syncthreads();
    stage_kv_dq<D>(sm, kbase, vbase, kv_stride, key0, L, tid);
    __syncthreads();
    if (nrows == 0) continue;
    if (CAUSAL && key0 > wave_last_pos) continue;

    f32x16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      dp[kb] = f32x16{};
      const uint16_t* kp = &sm.k[(kb * 32 + col) * DqSmem<D>::NS + kg * 8];
      const uint16_t* vp = &sm.v[(kb * 32 + col) * DqSmem<D>::NS + kg * 8];
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        s[kb] = mfma32(ld16(kp + st * 16), qf[st], s[kb]);
        dp[kb] = mfma32(ld16(vp + st * 16), dof[st], dp[kb]);
      }
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kbase_i = key0 + kb * 32 + i * 8 + kg * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int kk = kbase_i + j;
          float x = s[kb][i * 4 + j] * a.scale_log2;
          if (BIAS) x += bias_row[min(kk, a.bias_len - 1)] * kLog2e;
          const bool vis = (kk < L) && (!CAUSAL || kk <= qpos);
          const float p = vis ? exp2f_fast(x - lse2) : 0.f;
          dp[kb][i * 4 + j] = p * (dp[kb][i * 4 + j] - dlt);
        }
      }
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const u32x4 dsf = to_bf16x8(dp[st >> 1], (st & 1) * 8);
      const uint16_t* kta = &sm.kt[col * DqSmem<D>::TS + st * 16 + kg * 8];
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        dqt[db] = mfma32(ld16(kta + db * 32 * DqSmem<D>::TS), dsf, dqt[db]);
    }
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
  CPATTN_BWD_DISPATCH(dkdv_kernel)
}

hipError_t launch_dq(const AttnArgs& a, int D, bool causal, bool bias, dim3 grid, hipStream_t s) {
  CPATTN_BWD_DISPATCH(dq_kernel)
}

}  // namespace cpattn
