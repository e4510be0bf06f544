// dBias for pair-biased row attention: dBias[h, p, j] = sum over every chunk row at
// position p of dS[row, h, j], with dS = P * (dP - Delta) recomputed per row.
//
// Page "Support and performance optimization for Hopper (H200) architecture?"
// (maintainer reply): triangle attention, whose pair bias is shared by every row of
// the pair tensor, so its gradient is a reduction over rows.
//
// A workgroup owns a 128-position x 64-key tile of one head's dBias and walks one
// unit (a fixed range of consecutive chunks) of the chunk list in order, keeping the
// tile's partial sum in registers; a second kernel adds the units' partial tiles in
// unit order.  The unit count depends on the bias size and the chunk count only, so
// the result depends neither on scheduling nor on how the heads are split over calls.
#include "common.h"
#include "launch.h"

namespace cpattn {

template <int D>
__global__ __launch_bounds__(kThreads) void dbias_kernel(const AttnArgs a) {
  constexpr int NST = D / 16;
  if (*a.dev_err) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kg = lane >> 5, col = lane & 31;
  const int BL = a.bias_len;
  const int key_tiles = (BL + kDbiasKeys - 1) / kDbiasKeys;
  const int key0 = (blockIdx.x % key_tiles) * kDbiasKeys;
  const int part = blockIdx.x / key_tiles;
  const int wpos0 = blockIdx.y * kDbiasPos + wave * 32;
  const int h = blockIdx.z;
  const int per = (a.num_chunks + a.parts - 1) / a.parts;
  const int c_begin = part * per, c_end = min(a.num_chunks, c_begin + per);
  const int g = h / a.group;
  const int qpos = wpos0 + col;

  // Bias tile in base-2 units: element r of block kb is key key0+32kb+8(r/4)+4kg+r%4.
  f32x16 bias2[2];
  {
    const float* br = a.bias + ((int64_t)h * BL + min(qpos, BL - 1)) * BL;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = key0 + kb * 32 + (r >> 2) * 8 + kg * 4 + (r & 3);
        bias2[kb][r] = (kk < BL) ? br[kk] * kLog2e : 0.f;
      }
  }
  f32x16 acc[2] = {f32x16{}, f32x16{}};
  const int64_t kv_stride = a.kv_pitch * D;

  if (wpos0 < BL) {
    for (int c = c_begin; c < c_end; ++c) {
      const Chunk ch = load_chunk(a.chunks, c);
      if (ch.pos0 >= wpos0 + 32 || ch.pos0 + ch.len <= wpos0) continue;
      const int L = a.seq_lens[ch.seq];
      if (key0 >= L) continue;
      const int64_t koff = a.seq_offsets[ch.seq];
      const bool qok = qpos >= ch.pos0 && qpos < ch.pos0 + ch.len;
      const int64_t qrow = (int64_t)ch.q_row + (qpos - ch.pos0);
      u32x4 qf[NST], dof[NST];
      const int64_t qoff = (qrow * a.q_pitch + h) * D + kg * 8;
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        qf[st] = qok ? ld16(a.q + qoff + st * 16) : u32x4{0u, 0u, 0u, 0u};
        dof[st] = qok ? ld16(a.dout + qoff + st * 16) : u32x4{0u, 0u, 0u, 0u};
      }
      const float lse2 = qok ? a.lse[(int64_t)h * a.q_rows + qrow] * kLog2e : INFINITY;
      const float dlt = qok ? a.delta[(int64_t)h * a.q_rows + qrow] : 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int krow = key0 + kb * 32 + col;  // A-operand row of this lane
        const bool kok = krow < L;
        const int64_t koff_l = (koff + krow) * kv_stride + (int64_t)g * D + kg * 8;
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int st = 0; st < NST; ++st) {
          const u32x4 ka = kok ? ld16(a.k + koff_l + st * 16) : u32x4{0u, 0u, 0u, 0u};
          const u32x4 va = kok ? ld16(a.v + koff_l + st * 16) : u32x4{0u, 0u, 0u, 0u};
          s = mfma32(ka, qf[st], s);
          dp = mfma32(va, dof[st], dp);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = key0 + kb * 32 + (r >> 2) * 8 + kg * 4 + (r & 3);
          const float x = s[r] * a.scale_log2 + bias2[kb][r] - lse2;
          const float p = (kk < L) ? exp2f_fast(x) : 0.f;
          acc[kb][r] += p * (dp[r] - dlt);
        }
      }
    }
  }

  if (qpos >= BL) return;
  float* dst = a.dbias + (int64_t)part * a.hq * BL * BL + ((int64_t)h * BL + qpos) * BL;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kk = key0 + kb * 32 + i * 8 + kg * 4;
      if (kk + 3 < BL && (BL & 3) == 0) {
        *reinterpret_cast<f32x4*>(dst + kk) =
            f32x4{acc[kb][i * 4 + 0], acc[kb][i * 4 + 1], acc[kb][i * 4 + 2], acc[kb][i * 4 + 3]};
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (kk + j < BL) dst[kk + j] = acc[kb][i * 4 + j];
      }
    }
}

hipError_t launch_dbias(const AttnArgs& a, int D, dim3 grid, hipStream_t s) {
  switch (D) {
    case 32: hipLaunchKernelGGL(dbias_kernel<32>, grid, dim3(kThreads), 0, s, a); break;
    case 64: hipLaunchKernelGGL(dbias_kernel<64>, grid, dim3(kThreads), 0, s, a); break;
    case 128: hipLaunchKernelGGL(dbias_kernel<128>, grid, dim3(kThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// dbias_out[i] = sum over parts of partial[part][i], in part order.
__global__ __launch_bounds__(kThreads) void dbias_reduce_kernel(const float* __restrict__ partial,
                                                                float* __restrict__ out, int64_t n,
                                                                int parts, const int32_t* dev_err) {
  if (*dev_err) return;
  const int64_t i = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 4;
  if (i + 3 < n && (n & 3) == 0) {
    f32x4 s = *reinterpret_cast<const f32x4*>(partial + i);
    for (int p = 1; p < parts; ++p) s += *reinterpret_cast<const f32x4*>(partial + (int64_t)p * n + i);
    *reinterpret_cast<f32x4*>(out + i) = s;
  } else {
    for (int64_t j = i; j < n; ++j) {
      float s = partial[j];
      for (int p = 1; p < parts; ++p) s += partial[(int64_t)p * n + j];
      out[j] = s;
    }
  }
}

hipError_t launch_dbias_reduce(const float* partial, float* out, int64_t n, int parts,
                               const int32_t* dev_err, hipStream_t s) {
  const int64_t blocks = (n + kThreads * 4 - 1) / (kThreads * 4);
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(dbias_reduce_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, partial, out,
                     n, parts, dev_err);
  return hipGetLastError();
}

}  // namespace cpattn

namespace cpattn {

// dBias from the stored dS: with the dS store filled by dK/dV (BF16 blocks of 32 keys x
// 32 queries per (chunk tile, head, 32-key block)), dBias[h, p, k] is the sum over
// every chunk row at position p of that row's dS[h, k]: a streaming reduction over the
// blocks instead of forming S, P and dP again.
//
// Workgroup = (head h, 32 positions from P0, 32 keys from K0, unit of consecutive
// chunks), 128 threads; thread t owns key row n = t / 4 and granule v = t % 4 of a
// block, i.e. key K0 + n and the 8 queries 16 (v / 2) + 8 (i / 4) + 4 (v % 2) + i % 4
// (i = 0..7) of a 32-query tile.  A chunk whose first position is a multiple of 32
// covers the positions [P0, P0 + 32) with one of its tiles, and the thread adds its
// 16 bytes of that tile's block; the chunks are read four at a time, added in chunk
// order.  A unit with any other chunk is summed element by element (same order).  Only
// blocks that dK/dV stored are read: a tile with rows and a key block below the
// sequence length (the kernel runs without causal masking only).
__global__ __launch_bounds__(128) void dbias_ds_kernel(const AttnArgs a) {
  if (*a.dev_err) return;
  const int t = threadIdx.x, n = t >> 2, v = t & 3;
  const int BL = a.bias_len;
  const int kblocks = (BL + 31) / 32;
  const int kb = blockIdx.x % kblocks;
  const int part = blockIdx.x / kblocks;
  const int P0 = blockIdx.y * 32, K0 = kb * 32;
  const int h = blockIdx.z;
  const int per = (a.num_chunks + a.parts - 1) / a.parts;
  const int c_begin = part * per, c_end = min(a.num_chunks, c_begin + per);
  // the thread's 8 query slots within a tile
  int qq[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) qq[i] = 16 * (v >> 1) + 8 * (i >> 2) + 4 * (v & 1) + (i & 3);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

  auto chunk_at = [&](int c) {
    const int32_t* m = a.chunks + 4 * __builtin_amdgcn_readfirstlane(c);
    return Chunk{m[0], m[1], m[2], m[3]};
  };
  auto block_ptr = [&](int c, const Chunk& ch, int tile) {
    const int kbc = ds_chunk_kb(ch, a.seq_lens[ch.seq], false);
    return a.ds + (ds_block0(a.ds_tab[c], kbc, tile, h, a.hq) + kb) * 1024;
  };
  // Does the unit hold a chunk whose tiles do not line up with 32-position tiles?
  bool aligned = true;
  for (int c = c_begin; c < c_end; ++c) aligned &= (chunk_at(c).pos0 & 31) == 0;

  if (aligned) {
    for (int c0 = c_begin; c0 < c_end; c0 += 4) {
      u32x4 w[4];
      bool use[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = c0 + j;
        use[j] = false;
        w[j] = u32x4{0u, 0u, 0u, 0u};
        if (c < c_end) {
          const Chunk ch = chunk_at(c);
          if (P0 >= ch.pos0 && P0 < ch.pos0 + ch.len && K0 < a.seq_lens[ch.seq]) {
            use[j] = true;
            w[j] = ld16(block_ptr(c, ch, (P0 - ch.pos0) >> 5) + n * 32 + v * 8);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (use[j]) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[2 * i] += bf16_lo(w[j][i]);
            acc[2 * i + 1] += bf16_hi(w[j][i]);
          }
        }
    }
  } else {
    for (int c = c_begin; c < c_end; ++c) {
      const Chunk ch = chunk_at(c);
      if (ch.pos0 >= P0 + 32 || ch.pos0 + ch.len <= P0 || K0 >= a.seq_lens[ch.seq]) continue;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = P0 + qq[i] - ch.pos0;  // chunk row of this query slot
        if (r < 0 || r >= ch.len) continue;
        const int q = r & 31, e = q >> 4, wq = q & 15;
        const int off = (2 * e + ((wq >> 2) & 1)) * 8 + 4 * (wq >> 3) + (wq & 3);
        const uint16_t bits = block_ptr(c, ch, r >> 5)[n * 32 + off];
        acc[i] += __uint_as_float((uint32_t)bits << 16);
      }
    }
  }

  const int k = K0 + n;
  if (k >= BL) return;
  float* dst = a.dbias + (int64_t)part * a.hq * BL * BL + (int64_t)h * BL * BL + k;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int p = P0 + qq[i];
    if (p < BL) dst[(int64_t)p * BL] = acc[i];
  }
}

hipError_t launch_dbias_ds(const AttnArgs& a, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL(dbias_ds_kernel, grid, dim3(128), 0, s, a);
  return hipGetLastError();
}

}  // namespace cpattn
