// Device helpers and kernel argument blocks shared by the cpattn HIP kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kThreads = 256;  // four wave64s per workgroup

// One 32x32x16 BF16 MFMA with fp32 accumulation.
//  A (32 x 16): lane l holds row l%32, the 8 k-values of lane group l/32.
//  B (16 x 32): lane l holds column l%32, the same 8 k-values.
//  C (32 x 32): lane l holds column l%32; element r is row 8*(r/4) + 4*(l/32) + r%4.
// A and B share the k-numbering, so any bijection between (lane group, element)
// and the contracted index gives the same product; the kernels use that freedom
// to make the C layout of one product the B layout of the next.
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(uint16_t* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ u32x2 ld8(const uint16_t* p) {
  return *reinterpret_cast<const u32x2*>(p);
}
__device__ __forceinline__ void st8(uint16_t* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }

// fp32 -> packed BF16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Elements [base, base+8) of an accumulator as eight BF16 values.
__device__ __forceinline__ u32x4 to_bf16x8(const f32x16& v, int base) {
  u32x4 r;
  r[0] = pack_bf16x2(v[base + 0], v[base + 1]);
  r[1] = pack_bf16x2(v[base + 2], v[base + 3]);
  r[2] = pack_bf16x2(v[base + 4], v[base + 5]);
  r[3] = pack_bf16x2(v[base + 6], v[base + 7]);
  return r;
}

// 8x8 transpose of 16-bit values: in[e] is row e (8 values), out[d] is column d.
__device__ __forceinline__ void transpose8x8(const u32x4 in[8], u32x4 out[8]) {
#pragma unroll
  for (int m = 0; m < 4; ++m) {
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const uint32_t a = in[2 * n][m], b = in[2 * n + 1][m];
      out[2 * m][n] = (a & 0xffffu) | (b << 16);
      out[2 * m + 1][n] = (a >> 16) | (b & 0xffff0000u);
    }
  }
}

// Within each group of 16 contracted indices, storage slot s (= 8*lane group + element)
// holds index sigma(s): bits 2 and 3 swapped.  This is the order in which the C layout
// of a 32x32 product lists its rows for one lane group, so an accumulator converts to
// a B operand without any cross-lane movement.
__device__ __forceinline__ int sigma16(int s) {
  return (s & ~12) | ((s & 4) << 1) | ((s & 8) >> 1);
}

__device__ __forceinline__ float exp2f_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2f_fast(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float xor32(float v) { return __shfl_xor(v, 32, 64); }

struct Chunk {
  int seq, q_row, pos0, len;
};
__device__ __forceinline__ Chunk load_chunk(const int32_t* map, int c) {
  const int4 v = reinterpret_cast<const int4*>(map)[c];
  return Chunk{v.x, v.y, v.z, v.w};
}

// First chunk index whose seq is >= b (chunks are listed with non-decreasing seq).
__device__ __forceinline__ int chunk_lower_bound(const int32_t* map, int num_chunks, int b) {
  int lo = 0, hi = num_chunks;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (map[4 * mid] < b) lo = mid + 1; else hi = mid;
  }
  return lo;
}

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* bias;
  const uint16_t* o;     // forward output (backward pre-pass input)
  const float* lse;      // forward output [hq, q_rows]
  const uint16_t* dout;  // dO
  const float* delta;    // [hq, q_rows]
  uint16_t* o_out;       // forward: O
  float* lse_out;        // forward: LSE
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* dbias;          // dBias (or the partial-sum slab when parts > 1)
  float* delta_out;      // pre-pass output
  const int32_t* seq_offsets;
  const int32_t* seq_lens;
  const int32_t* chunks;
  const int32_t* dev_err;
  int64_t q_rows;
  int num_seqs, num_chunks;
  int hq, hkv, group, hpw;  // group = hq/hkv; hpw = query heads per workgroup
  int blocks_per_chunk;     // position blocks per chunk (forward / dQ / pre-pass)
  int kv_tiles;             // KV tiles per sequence (dK/dV)
  int bias_len;
  int accumulate;           // dK/dV: 0 store, 1 add
  int parts;                // dBias partitions of the chunk list
  float scale;
  float scale_log2;         // scale * log2(e)
};

}  // namespace cpattn
