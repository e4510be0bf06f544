// Forward kernel: blockwise causal GQA attention over one rank's chunk map.
//
// Page "Optimize context parallel attention layouts and gradient accumulation",
// "Description"/"Changes": causal THD attention with physical offsets, GQA,
// head dims 128/256, and the softmax statistics (LSE) kept for the backward.
//
// Work decomposition
//   workgroup = 4 waves = (one chunk, one block of positions, `hpw` query heads
//   that share one KV head).  Each wave owns 32 query rows of one head and keeps
//   its Q tile in registers for the whole KV loop.  K and V tiles of 64 keys are
//   staged in LDS once per workgroup and read by all four waves (GQA sharing).
//
// Transposed formulation (no cross-lane shuffles for P):
//   S^T = K Q^T         A = K rows from LDS, B = Q^T from registers
//   O^T += V^T P^T      A = V^T from LDS (transposed while staging), B = P^T made
//                       in-lane from the S^T accumulator
//   so every lane owns one query (column) of S^T and of O^T, and the online
//   softmax (running max m, running sum l in fp32, base-2 with log2(e)*scale
//   folded into the scores) needs only one exchange between the two lanes of a
//   query per KV tile.
#include "common.h"
#include "launch.h"

namespace cpattn {

constexpr int kBN = 64;  // keys per KV tile

template <int D>
struct FwdSmem {
  static constexpr int KS = D + 8;    // K tile row stride (elements)
  static constexpr int VS = kBN + 8;  // V^T tile row stride (elements)
  uint16_t k[kBN * KS];
  uint16_t vt[D * VS];
};

// Stage K rows [key0, key0+64) (natural) and V^T (transposed, sigma order) into LDS.
template <int D>
__device__ __forceinline__ void stage_kv(FwdSmem<D>& sm, const uint16_t* __restrict__ kbase,
                                         const uint16_t* __restrict__ vbase, int64_t row_stride,
                                         int key0, int L, int tid) {
  constexpr int D8 = D / 8;
  // K: 16-byte pieces, row-major.
  for (int i = tid; i < kBN * D8; i += kThreads) {
    const int r = i / D8, c = i % D8;
    const int key = key0 + r;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (key < L) val = ld16(kbase + (int64_t)key * row_stride + c * 8);
    st16(&sm.k[r * FwdSmem<D>::KS + c * 8], val);
  }
  // V: 8 keys x 8 dims per thread, transposed into V^T[d][slot].
  for (int i = tid; i < (kBN / 8) * D8; i += kThreads) {
    const int pg = i % (kBN / 8), dg = i / (kBN / 8);
    u32x4 rows[8], cols[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int key = key0 + (pg >> 1) * 16 + sigma16((pg & 1) * 8 + e);
      rows[e] = (key < L) ? ld16(vbase + (int64_t)key * row_stride + dg * 8) : u32x4{0u, 0u, 0u, 0u};
    }
    transpose8x8(rows, cols);
#pragma unroll
    for (int d = 0; d < 8; ++d) st16(&sm.vt[(dg * 8 + d) * FwdSmem<D>::VS + pg * 8], cols[d]);
  }
}

template <int D, bool CAUSAL, bool BIAS>
__global__ __launch_bounds__(kThreads) void attn_fwd_kernel(const AttnArgs a) {
  constexpr int NST = D / 16;  // 16-wide k-steps over the head dim
  constexpr int NDB = D / 32;  // 32-row blocks of O^T
  __shared__ FwdSmem<D> sm;

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
  const int row0 = wg_row0 + (wave / a.hpw) * 32;  // first chunk row of this wave
  const int nrows = max(0, min(32, ch.len - row0));
  const int L = a.seq_lens[ch.seq];
  const int64_t koff = a.seq_offsets[ch.seq];

  const int wg_last_pos = ch.pos0 + min(ch.len, wg_row0 + 32 * segs) - 1;
  const int kv_end = CAUSAL ? min(L, wg_last_pos + 1) : L;
  const int n_tiles = (kv_end + kBN - 1) / kBN;
  const int wave_last_pos = ch.pos0 + row0 + nrows - 1;
  const int qpos = ch.pos0 + row0 + col;  // this lane's query position

  // Q^T as B operand: lane holds query `col`, dims [16*st + 8*kg, +8).
  u32x4 qf[NST];
  {
    const uint16_t* qp = a.q + ((int64_t)(ch.q_row + row0 + col) * a.hq + h) * D + kg * 8;
#pragma unroll
    for (int st = 0; st < NST; ++st)
      qf[st] = (col < nrows) ? ld16(qp + st * 16) : u32x4{0u, 0u, 0u, 0u};
  }

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  const float* bias_row = nullptr;
  if (BIAS) bias_row = a.bias + ((int64_t)h * a.bias_len + min(qpos, a.bias_len - 1)) * a.bias_len;

  const int64_t kv_stride = (int64_t)a.hkv * D;
  const uint16_t* kbase = a.k + koff * kv_stride + (int64_t)g * D;
  const uint16_t* vbase = a.v + koff * kv_stride + (int64_t)g * D;

  for (int t = 0; t < n_tiles; ++t) {
    const int key0 = t * kBN;
    __syncthreads();
    stage_kv<D>(sm, kbase, vbase, kv_stride, key0, L, tid);
    __syncthreads();
    if (nrows == 0) continue;
    if (CAUSAL && key0 > wave_last_pos) continue;

    // S^T for two 32-key blocks.
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      const uint16_t* kp = &sm.k[(kb * 32 + col) * FwdSmem<D>::KS + kg * 8];
#pragma unroll
      for (int st = 0; st < NST; ++st) s[kb] = mfma32(ld16(kp + st * 16), qf[st], s[kb]);
    }

    // Scale (base 2), bias, mask; tile row max.
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kbase_i = key0 + kb * 32 + i * 8 + kg * 4;
        f32x4 bv = {0.f, 0.f, 0.f, 0.f};
        if (BIAS) {
          if (kbase_i + 3 < L && (a.bias_len & 3) == 0)
            bv = *reinterpret_cast<const f32x4*>(bias_row + kbase_i);
          else {
#pragma unroll
            for (int j = 0; j < 4; ++j) bv[j] = (kbase_i + j < L) ? bias_row[kbase_i + j] : 0.f;
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = kbase_i + j;
          float x = s[kb][i * 4 + j] * a.scale_log2;
          if (BIAS) x += bv[j] * kLog2e;
          const bool vis = (key < L) && (!CAUSAL || key <= qpos);
          x = vis ? x : -INFINITY;
          s[kb][i * 4 + j] = x;
          mx = fmaxf(mx, x);
        }
      }
    }
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f_fast(m_run - m_use);
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2f_fast(s[kb][r] - m_use);
        s[kb][r] = p;
        rs += p;
      }
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;

    // O^T += V^T P^T over four 16-key steps.
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const u32x4 pf = to_bf16x8(s[st >> 1], (st & 1) * 8);
      const uint16_t* vp = &sm.vt[col * FwdSmem<D>::VS + st * 16 + kg * 8];
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        oacc[db] = mfma32(ld16(vp + db * 32 * FwdSmem<D>::VS), pf, oacc[db]);
    }
  }

  if (col >= nrows) return;
  const float l = l_run + xor32(l_run);
  const float inv = 1.f / l;
  uint16_t* op = a.o_out + ((int64_t)(ch.q_row + row0 + col) * a.hq + h) * D + kg * 4;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x2 w;
      w[0] = pack_bf16x2(oacc[db][i * 4 + 0] * inv, oacc[db][i * 4 + 1] * inv);
      w[1] = pack_bf16x2(oacc[db][i * 4 + 2] * inv, oacc[db][i * 4 + 3] * inv);
      st8(op + db * 32 + i * 8, w);
    }
  if (kg == 0) a.lse_out[(int64_t)h * a.q_rows + ch.q_row + row0 + col] = (m_run + log2f_fast(l)) * kLn2;
}

template <int D, bool CAUSAL, bool BIAS>
static void launch_fwd_t(const AttnArgs& a, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, BIAS>), grid, dim3(kThreads), 0, s, a);
}

hipError_t launch_fwd(const AttnArgs& a, int D, bool causal, bool bias, dim3 grid, hipStream_t s) {
  if (bias) {
    if (causal) return hipErrorInvalidValue;
    switch (D) {
      case 32: launch_fwd_t<32, false, true>(a, grid, s); break;
      case 64: launch_fwd_t<64, false, true>(a, grid, s); break;
      case 128: launch_fwd_t<128, false, true>(a, grid, s); break;
      default: return hipErrorInvalidValue;
    }
  } else if (causal) {
    switch (D) {
      case 32: launch_fwd_t<32, true, false>(a, grid, s); break;
      case 64: launch_fwd_t<64, true, false>(a, grid, s); break;
      case 128: launch_fwd_t<128, true, false>(a, grid, s); break;
      case 256: launch_fwd_t<256, true, false>(a, grid, s); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (D) {
      case 32: launch_fwd_t<32, false, false>(a, grid, s); break;
      case 64: launch_fwd_t<64, false, false>(a, grid, s); break;
      case 128: launch_fwd_t<128, false, false>(a, grid, s); break;
      case 256: launch_fwd_t<256, false, false>(a, grid, s); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

}  // namespace cpattn
