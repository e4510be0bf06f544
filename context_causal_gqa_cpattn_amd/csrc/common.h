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

// Max and sum over the two 32-lane halves of a wave (lanes l and l ^ 32), by one
// v_permlane32_swap (a VALU lane swap; no LDS round trip): swapping the upper half of
// one copy with the lower half of another leaves [lo, lo] and [hi, hi].
__device__ __forceinline__ float halves_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
#define CPATTN_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt fields at their no-wait maxima), through the
// builtin so that the compiler knows every earlier vector-memory load has completed.
__device__ __forceinline__ void wait_vm_all() {
  __builtin_amdgcn_s_waitcnt(0x0F70);
  asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(N): at most N vector-memory operations of this wave still pending
// (vmcnt is 6 bits: bits 3-0 and 15-14 of the immediate).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
  asm volatile("" ::: "memory");
}

// Physical block id -> logical work item, so that consecutive logical items (which
// share K/V) run on the same XCD (blocks are dealt to the 8 XCDs round robin) and
// hit that XCD's L2.
__device__ __forceinline__ int xcd_remap(int pid, int n) {
  const int per = n >> 3;
  return pid < per * 8 ? (pid & 7) * per + (pid >> 3) : pid;
}

// Logical work item (group * per_group + item) of physical block pid, for a launch of
// n_groups groups of per_group items, where a group's items share their inputs through
// L2 (the query blocks of one chunk and head group, the key tiles of one sequence and KV
// head).  Groups are numbered with the head index fastest, over n_heads heads.  With
// n_heads a multiple of 8, XCD x takes the groups of heads x, x + 8, ... of every chunk or
// sequence, each group's items consecutively, so every XCD gets the same share of work
// however unequal the sequences are.  Otherwise (dealing by group index would then
// follow the chunk order, e.g. put every short chunk on half the XCDs) each XCD takes a
// contiguous range (xcd_remap).
__device__ __forceinline__ int xcd_group_order(int pid, int n_groups, int per_group, int n_heads) {
  if ((n_heads & 7) == 0) {
    const int x = pid & 7, j = pid >> 3;
    return (x + 8 * (j / per_group)) * per_group + j % per_group;
  }
  return xcd_remap(pid, n_groups * per_group);
}

// LDS tiles [rows][D] of BF16 are written by LDS DMA (1 KB contiguous per wave
// instruction, so rows are unpadded) and read two ways: 16-byte row reads (A operands
// whose contracted index runs along D) and transposing 8-byte reads (A operands whose
// contracted index runs along the rows).  Granule g (16 bytes) of row r is stored at
// granule g ^ swz(r), swz(r) = (r & 3) * 4 + ((r >> 2) & 3): sixteen consecutive rows
// read at one granule hit sixteen distinct bank groups, and the 4 rows x 64 bytes of
// one transposing read also do.
template <int D, int KIND = 0>
__device__ __forceinline__ int swz(int r) {
  constexpr int G = D / 8;
  if (KIND == 0) return (((r & 3) << 2) | ((r >> 2) & 3)) & (G - 1);
  if (KIND == 1) return (((r & 7) << 1) | ((r >> 3) & 1)) & (G - 1);
  // KIND 2: rows read sixteen at a time as {8a + 4b' + c : a, c in 0..3} for a fixed b'
  // (the dK/dV query order) land in sixteen distinct bank groups.
  if (KIND == 2) return ((r & 3) | (((r >> 3) & 3) << 2)) & (G - 1);
  // KIND 3: kind 1 with bit 2 of the row flipped by bit 3 before the shift.  A 16-byte
  // read serves its 64 lanes in four passes of 16; in each 32-lane half, the lanes whose
  // quad index (lane bits 2-4) has even parity form one pass.  When lane group g of 16
  // lanes reads rows r0 + [0, 16) at one granule per group, a pass holds rows
  // {0-3, 12-15} of one group and rows 4-11 of the next, and this swizzle maps the two
  // sets to complementary bank groups.  Eight consecutive rows x two adjacent granules
  // (a transposing read) stay conflict-free, as under kind 1.
  return (((((r & 7) ^ ((r >> 1) & 4)) << 1) | ((r >> 3) & 1))) & (G - 1);
}

// A pointer that is the same in every lane, forced into scalar registers.
__device__ __forceinline__ const char* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const char*>(((uint64_t)hi << 32) | lo);
}

// One 16-byte LDS DMA per lane (global_load_lds_dwordx4): lane l's 16 bytes from
// base + off (base the same in every lane, off the lane's byte offset) land at
// lds + 16 l bytes.  It is issued from inline assembly so that the compiler does not
// track it as an LDS write: the compiler waits for every pending LDS DMA before an LDS
// read it cannot prove disjoint (a transposing read always), which would serialise the
// DMA of the next tile with the compute on the current one.  The kernels order DMA and
// reads themselves: a DMA'd buffer is read only after wait_vm_all() and a workgroup
// barrier, and is refilled only after the barrier that follows its last read.  M0
// holds the LDS address (no compiler-generated code in these kernels uses M0); the
// s_nop separates the M0 write from its use.
__device__ __forceinline__ void dma16_at(const char* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds), "v"(off), "s"(base)
               : "memory", "m0");
}

// The same copy with the LDS address given as a wave-uniform base plus a constant
// lds_off (known at compile time once the caller's loops are unrolled): M0 is formed by
// one scalar add with a literal inside the block, instead of a constant materialised in
// a scalar register and an add.
__device__ __forceinline__ void dma16_add(const char* base, uint32_t off, uint32_t lds,
                                          uint32_t lds_off) {
  asm volatile("s_add_u32 m0, %0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds), "v"(off), "s"(base), "i"(lds_off)
               : "memory", "m0", "scc");
}

// 4 bytes per lane: lane i's dword from base + off lands at LDS address lds + 4 i.
__device__ __forceinline__ void dma4_at(const char* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
               :
               : "s"(lds), "v"(off), "s"(base)
               : "memory", "m0");
}

// The same copy with the non-temporal hint, for data read once (a stream that should not
// push reused tiles out of L2).
__device__ __forceinline__ void dma16_nt_at(const char* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
               :
               : "s"(lds), "v"(off), "s"(base)
               : "memory", "m0");
}
__device__ __forceinline__ void dma16_nt_add(const char* base, uint32_t off, uint32_t lds,
                                             uint32_t lds_off) {
  asm volatile("s_add_u32 m0, %0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
               :
               : "s"(lds), "v"(off), "s"(base), "i"(lds_off)
               : "memory", "m0", "scc");
}

// 32-bit LDS address of a shared-memory pointer that is the same in every lane.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)CPATTN_LDS(const void, p));
}

__device__ __forceinline__ void dma16(const char* base, uint32_t off, const void* lds) {
  dma16_at(base, off, lds_addr(lds));
}

// DMA a contiguous block of NI KB into LDS, instructions dealt round robin over NW waves.
// Addresses are a scalar base plus the lane's 16-byte slot.
template <int NI, int NW = 4>
__device__ __forceinline__ void dma_flat(uint16_t* lds, const uint16_t* src, int wave, int lane) {
  const char* b = uniform_ptr(src);
  const uint32_t l0 = lds_addr(lds);
  const uint32_t lo = (uint32_t)lane * 16u;
  for (int i = __builtin_amdgcn_readfirstlane(wave); i < NI; i += NW)
    dma16_at(b + i * 1024, lo, l0 + i * 1024);
}

// DMA an R-row tile: tile row r comes from base + min(r, nvalid-1) * rs (rows past
// the valid ones repeat the last valid row: finite data, masked by the caller).
// Instruction i of the tile carries rows [i RPI, i RPI + RPI) (RPI = 64 / (D/8)); wave w
// issues i = w, w + NW, ...  For a full tile the row part of each address is scalar and
// the lane part (row within the instruction, swizzled granule) repeats with period 2
// in the wave's instruction index, since the swizzle depends on the row mod 16; so the
// lane parts are computed once.  R rows of rs elements span less than 2 GiB.
template <int D, int R, int NW = 4, int KIND = 0>
__device__ __forceinline__ void dma_rows(uint16_t* lds, const uint16_t* base, int64_t rs,
                                         int nvalid, int wave, int lane) {
  constexpr int G = D / 8;
  constexpr int RPI = 64 / G;          // rows per instruction
  constexpr int NI = R * G / 64;       // instructions per tile
  constexpr int NK = (NI + NW - 1) / NW;
  static_assert((2 * NW * RPI) % 16 == 0, "lane offsets repeat with period 2");
  static_assert(KIND != 2, "swizzles of kinds 0, 1 and 3 depend on the row mod 16 only");
  const char* b = uniform_ptr(base);
  const uint32_t rs_bytes = (uint32_t)(rs * 2);
  const uint32_t l0 = lds_addr(lds);
  const int w = __builtin_amdgcn_readfirstlane(wave);
  const int lr = lane / G, p = lane % G;
  if (nvalid >= R) {
    uint32_t o[2];
#pragma unroll
    for (int e = 0; e < 2; ++e)
      o[e] = (uint32_t)lr * rs_bytes + (uint32_t)((p ^ swz<D, KIND>((w + NW * e) * RPI + lr)) * 16);
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      const int i = w + NW * k;
      if (NI % NW == 0 || i < NI)
        dma16_at(b + (uint64_t)(i * RPI) * rs_bytes, o[k & 1], l0 + i * 1024);
    }
  } else {
    for (int i = w; i < NI; i += NW) {
      const int r = i * RPI + lr;
      const uint32_t row = (uint32_t)min(r, nvalid - 1);
      dma16_at(b, row * rs_bytes + (uint32_t)((p ^ swz<D, KIND>(r)) * 16), l0 + i * 1024);
    }
  }
}

// 16-byte read of logical granule g of row r.
template <int D, int KIND = 0>
__device__ __forceinline__ u32x4 lds_row16(const uint16_t* t, int r, int g) {
  return ld16(t + r * D + ((g ^ swz<D, KIND>(r)) * 8));
}

// A operand (32 x 16) whose rows are 32 columns [32*db, +32) of the tile and whose 16
// contracted values are tile rows kr0 + sigma16(8*(lane/32) + e): two transposing reads.
// Lane l gets tile[kr0 + 4*(l/32) + j][32*db + l%32] for j = 0..3, then the same + 8.
template <int D>
__device__ __forceinline__ u32x4 tr_frag(const uint16_t* t, int kr0, int db, int lane) {
  const int r = kr0 + (lane >> 5) * 4 + ((lane & 15) >> 2);
  const int d = db * 32 + ((lane >> 4) & 1) * 16 + 4 * (lane & 3);
  const int gl = d >> 3, off = d & 7;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      CPATTN_LDS(v4i16, t + r * D + ((gl ^ swz<D>(r)) << 3) + off));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      CPATTN_LDS(v4i16, t + (r + 8) * D + ((gl ^ swz<D>(r + 8)) << 3) + off));
  const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
  return u32x4{l2[0], l2[1], h2[0], h2[1]};
}

// Lane parts of the tr_frag addresses, computed once per kernel (three registers).  The
// fragment for rows [16 st, +16) and columns [32 db, +32) of a tile sits at element
// 16 st D + 128 (db / 4) + lo(db % 4), its second read hi_delta further on:
//  - the swizzle depends on the row mod 16 only and touches granule bits 0-3, so st and
//    db / 4 enter as constants;
//  - granule 4 m + gsub of row rr (rr < 8) is stored at (4 m + gsub) ^ swz(rr), which
//    splits into bits 2-3, m ^ t with t = swz(rr) >> 2, and bits 0-1 from the lane alone:
//    lo(m) = base + 32 (m ^ t) elements;
//  - the second read's rows are the first's + 8, whose swizzle is the first's with bit 1
//    set (rows below 8 have it clear), and bit 1 of the granule index comes from the lane
//    alone, so the two reads differ by one lane constant: 8 D + 16 elements when that bit
//    is clear, 8 D - 16 when set.
template <int D>
struct TrOffsets {
  static constexpr int NM = (D / 32) < 4 ? (D / 32) : 4;
  int base, t, hi_delta;
  __device__ __forceinline__ explicit TrOffsets(int lane) {
    const int rr = (lane >> 5) * 4 + ((lane & 15) >> 2);
    const int gsub = ((lane >> 4) & 1) * 2 + ((lane & 3) >> 1);
    const int off = (lane & 1) * 4;
    base = rr * D + ((gsub ^ (swz<D>(rr) & 3)) << 3) + off;
    t = swz<D>(rr) >> 2;
    hi_delta = 8 * D + ((gsub & 2) ? -16 : 16);
  }
  __device__ __forceinline__ int lo(int m) const { return base + ((m ^ t) << 5); }
};

// tr_frag(t, 16 st, db, lane) with the lane parts precomputed.
template <int D>
__device__ __forceinline__ u32x4 tr_frag_at(const uint16_t* t, const TrOffsets<D>& o, int st, int db) {
  const uint16_t* b = t + st * 16 * D + (db >> 2) * 128 + o.lo(db & 3);
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(CPATTN_LDS(v4i16, b));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(CPATTN_LDS(v4i16, b + o.hi_delta));
  const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
  return u32x4{l2[0], l2[1], h2[0], h2[1]};
}

// One 16x16x32 BF16 MFMA with fp32 accumulation.
//  A (16 x 32): lane l holds row l%16, the 8 k-values of lane group l/16.
//  B (32 x 16): lane l holds column l%16, the same 8 k-values.
//  C (16 x 16): lane l holds column l%16; element j is row 4*(l/16) + j.
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// A operand (16 x 32) of a 16x16x32 product whose rows are columns [16*dblk, +16) of a
// 32-row tile and whose contracted values are the tile's rows in the order of two stacked
// 16x16 accumulators: lane group g, element e -> row 16*(e/4) + 4*g + e%4.  Two
// transposing reads; lane l gets tile[4*(l/16) + j][16*dblk + l%16], then rows + 16.
template <int D>
__device__ __forceinline__ u32x4 tr_frag16(const uint16_t* t, int dblk, int lane) {
  const int r = (lane >> 4) * 4 + ((lane & 15) >> 2);
  const int d = dblk * 16 + 4 * (lane & 3);
  const int gl = d >> 3, off = d & 7;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      CPATTN_LDS(v4i16, t + r * D + ((gl ^ swz<D, 1>(r)) << 3) + off));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      CPATTN_LDS(v4i16, t + (r + 16) * D + ((gl ^ swz<D, 1>(r + 16)) << 3) + off));
  const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
  return u32x4{l2[0], l2[1], h2[0], h2[1]};
}

struct Chunk {
  int seq, q_row, pos0, len;
};
__device__ __forceinline__ Chunk load_chunk(const int32_t* map, int c) {
  const int4 v = reinterpret_cast<const int4*>(map)[c];
  return Chunk{v.x, v.y, v.z, v.w};
}

// The same for a chunk index that is the same in every lane (from the block index or a
// workgroup-uniform loop): the fields go to scalar registers, so that loops and tests on
// them compile to scalar branches instead of exec-masked vector code, and take no VGPRs.
__device__ __forceinline__ int rfl(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ Chunk load_chunk_uniform(const int32_t* map, int c) {
  const Chunk ch = load_chunk(map, c);
  return Chunk{rfl(ch.seq), rfl(ch.q_row), rfl(ch.pos0), rfl(ch.len)};
}

// First chunk index whose seq is >= b (chunks are listed with non-decreasing seq).
__device__ __forceinline__ int chunk_lower_bound(const int32_t* map, int num_chunks, int b) {
  int lo = 0, hi = num_chunks;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (rfl(map[4 * mid]) < b) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// Transposed 32-query tiles [D][32] (query-contiguous rows of 64 bytes) written by the
// pre-pass and read by dK/dV with 16-byte reads: granule g of row d is stored at
// g ^ ((d >> 2) & 3), so 16 consecutive rows read at one granule hit 16 bank groups.
__device__ __forceinline__ int tswz(int d) { return (d >> 2) & 3; }

// Slot of query tile qt (32 rows) of chunk c whose first Q row is q_row.  Chunks are
// ordered by Q row and do not overlap, so slots are distinct, and they stay below
// ceil(q_rows / 32) + num_chunks.
__device__ __forceinline__ int64_t tile_slot(int c, int q_row, int qt) {
  return (int64_t)(q_row >> 5) + c + qt;
}

// The dS store keeps, for every 32-query tile and query head of a chunk, the 32-key
// blocks that the chunk's last row sees: ceil(K_c / 32) of them, K_c = pos0 + len with
// causal masking, else the sequence length L.  Chunk c's blocks start at block
// ds_tab[c] * hq (ds_tab: the running sum of ceil(len / 32) * ceil(K_c / 32) over the
// chunks before c), ordered [tile][head][key block].
__device__ __forceinline__ int ds_chunk_kb(const Chunk& ch, int L, bool causal) {
  return ((causal ? ch.pos0 + ch.len : L) + 31) >> 5;
}
// First block of (tile qt, head h) of a chunk whose store starts at tab * hq.
__device__ __forceinline__ int64_t ds_block0(int64_t tab, int kb_c, int qt, int h, int hq) {
  return (tab + (int64_t)qt * kb_c) * hq + (int64_t)h * kb_c;
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
  uint16_t* qt_out;      // pre-pass output: transposed Q tiles
  uint16_t* dot_out;     // pre-pass output: transposed dO tiles
  const uint16_t* qt;    // transposed Q tiles [slot][hq][D][32]
  const uint16_t* dot;   // transposed dO tiles
  float* stats_out;      // pre-pass output: per-tile row statistics [slot][hq][64]
  const float* stats;    // the same, read by dK/dV: log2(e) LSE (+inf past the end), Delta
  uint16_t* ds_out;      // dK/dV: where to store dS blocks (null: not stored)
  const uint16_t* ds;    // dQ from stored dS: the dS blocks
  const int64_t* ds_tab; // per chunk: first dS block / hq (see ds_block0)
  const uint16_t* ds_zero;  // a dS block of zeros (read for blocks that a tile does not use)
  int64_t q_pitch;       // heads per row in memory: Q, O, dO, dQ
  int64_t kv_pitch;      // heads per row in memory: K, V, dK, dV
  int kv_lo, kv_hi;      // key window [kv_lo, kv_hi) in sequence positions (0, INT_MAX: all)
  int dq_accumulate;     // dQ: 0 store, 1 add to the existing values
  const int32_t* seq_offsets;
  const int32_t* seq_lens;
  const int32_t* chunks;
  const int32_t* dev_err;
  int64_t q_rows;
  int num_seqs, num_chunks;
  int hq, hkv, group, hpw;  // group = hq/hkv; hpw = query heads per workgroup
  int blocks_per_chunk;     // position blocks per chunk (forward / dQ / pre-pass)
  int kv_tiles;             // KV tiles per sequence (dK/dV): workgroups per (sequence, KV head)
  int kv_pair;              // dK/dV: each workgroup takes two key tiles (see dkdv_kernel)
  int bias_len;
  int accumulate;           // dK/dV: 0 store, 1 add
  int parts;                // dBias partitions of the chunk list
  float scale;
  float scale_log2;         // scale * log2(e)
};

// Launch KERNEL<D, CAUSAL, BIAS> with kThreads threads for the supported combinations
// (a bias only without causal masking and with D <= 128); returns the launch status.
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

}  // namespace cpattn
