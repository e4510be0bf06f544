// dK/dV kernel of the attention backward (KV-parallel).
//
// Page "Optimize context parallel attention layouts and gradient accumulation":
//  - "CP8 first-gradient accumulator reuse": the first dK/dV contribution is the
//    accumulator (STORE, no zero fill) and the later one is added (ADD);
//  - "Changes": GQA, causal THD with physical offsets.
//
// With P = exp(scale S - LSE), dP = dO V^T, Delta = rowsum(dO * O) and
// dS = P * (dP - Delta):  dV = P^T dO and dK = scale dS^T Q, summed over every query
// that sees the key, over the chunks of the sequence and over the group's query heads.
//
// Workgroup = (sequence, 128-key tile, KV head g), four waves with one wave per SIMD;
// wave w owns keys [32w, 32w+32) of the tile.  It keeps K^T and V^T of its keys in
// registers as B operands and dK^T, dV^T (D x 32 keys, fp32) as MFMA accumulators for
// the whole loop.  The loop runs over every (chunk of the sequence, query head of the
// group, 32-query tile) that sees the key tile.  The pre-pass's transposed tiles Q^T and
// dO^T ([D][32], contiguous) are DMA'd into LDS one step ahead, three buffers deep.
// Per tile, with 32x32x16 MFMAs (C layout: lane = key, 16 query rows per lane):
//   S  = Q K^T,  dP = dO V^T           (A = Q / dO rows: two transposing reads of the
//                                       transposed tiles; B = K^T / V^T registers)
//   P = exp2(S scale log2e - LSE log2e), dS = P (dP - Delta)
//   dV^T += dO^T P,  dK^T += Q^T dS    (A = 16-byte reads of the transposed tiles,
//                                       B = P / dS as packed)
// The pre-pass stores the transposed tiles in the query order of the accumulator rows,
// so P and dS become B operands without any data movement.  The steps are software
// pipelined: while the S/dP products of tile i are done, the softmax of tile i runs
// between the dV/dK products of tile i-1, so that VALU work issues while the matrix
// cores are busy.  dK = scale dK^T and dV are rounded to BF16 once (STORE), or added to
// the existing BF16 values and rounded once (ADD).
//
// Rounding P and dS to BF16 for the dV/dK products costs up to 2^-9 of each term.  Where
// single probabilities are large (queries with few visible keys: the first positions of a
// sequence, or a peaked row), those few terms dominate the largest dV/dK elements, and
// their rounding comes on top of the final BF16 rounding of the output.  So where any P
// of a wave's tile reaches 2^-5, the wave repeats that tile's dV/dK products with the
// rounding residues P - bf16(P) and dS - bf16(dS) as B operands (exact to about 2^-17);
// smaller probabilities add at most about 1e-3 in total.
#include "common.h"
#include "launch.h"

namespace cpattn {

namespace {

constexpr int kTq = 32;     // queries per tile
constexpr int kBufs = 3;    // LDS tile buffers (DMA one step ahead + the step before)
constexpr int kWaves = 4;   // waves per workgroup, 32 keys each
constexpr int kKvThreads = kWaves * 64;
static_assert(kWaves * 32 == kDkdvKeys, "keys per workgroup");

// The workgroup's walk over (chunk, query head of the group, query tile): tile qt
// innermost, then the head, then the chunks of the sequence.  Besides the position it
// carries the running indices that the step needs, so that a step costs a few scalar
// additions: the tile's unit (tile slot * hq + query head: its index among the
// transposed tiles and their statistics) and its first dS block.
struct QTileIter {
  int c, hh, qt, qt_first, n_qt;
  Chunk ch;
  int unit, ubase;        // this tile's unit; the unit of (qt_first, head 0 of the group)
  int64_t ds, dsbase;     // dS block of (this tile, head, key block 0); of (qt_first, head 0)
  int64_t ds_step;        // dS blocks from one tile to the next (ceil(K_c / 32) hq)
  int kbc;                // dS blocks per (tile, head) of the chunk
};

// Advance to the next chunk (from it.c) that has query tiles seeing keys >= key0.  h0:
// the group's first query head; L: the sequence length.
template <bool CAUSAL>
__device__ __forceinline__ bool seek_chunk(const AttnArgs& a, QTileIter& it, int c_end, int key0,
                                           int h0, int L) {
  for (; it.c < c_end; ++it.c) {
    it.ch = load_chunk_uniform(a.chunks, it.c);
    const int first_row = CAUSAL ? max(0, key0 - it.ch.pos0) : 0;
    if (first_row < it.ch.len) {
      it.qt_first = first_row / kTq;
      it.n_qt = (it.ch.len + kTq - 1) / kTq;
      it.qt = it.qt_first;
      it.hh = 0;
      it.ubase = (int)tile_slot(it.c, it.ch.q_row, it.qt_first) * a.hq + h0;
      it.unit = it.ubase;
      if (a.ds_out != nullptr) {
        it.kbc = ds_chunk_kb(it.ch, L, CAUSAL);
        const int64_t* t = a.ds_tab + it.c;
        const int64_t tab = (int64_t)(((uint64_t)rfl((int)(*t >> 32)) << 32) | (uint32_t)rfl((int)*t));
        it.dsbase = ds_block0(tab, it.kbc, it.qt_first, h0, a.hq);
        it.ds = it.dsbase;
        it.ds_step = (int64_t)it.kbc * a.hq;
      }
      return true;
    }
  }
  return false;
}

template <bool CAUSAL>
__device__ __forceinline__ bool advance(const AttnArgs& a, QTileIter& it, int c_end, int key0, int h0,
                                        int L) {
  if (++it.qt < it.n_qt) {
    it.unit += a.hq;
    it.ds += it.ds_step;
    return true;
  }
  it.qt = it.qt_first;
  if (++it.hh < a.group) {
    it.unit = it.ubase + it.hh;
    it.ds = it.dsbase + (int64_t)it.hh * it.kbc;
    return true;
  }
  ++it.c;
  return seek_chunk<CAUSAL>(a, it, c_end, key0, h0, L);
}

template <int D>
__device__ __forceinline__ void dma_tiles(uint16_t* lqt, uint16_t* ldot, const AttnArgs& a,
                                          const QTileIter& it, int wave, int lane) {
  dma_flat<D * kTq * 2 / 1024, kWaves>(lqt, a.qt + (int64_t)it.unit * D * kTq, wave, lane);
  dma_flat<D * kTq * 2 / 1024, kWaves>(ldot, a.dot + (int64_t)it.unit * D * kTq, wave, lane);
}

// The tile's row statistics (64 floats: log2(e) LSE of its 32 rows, +inf past the chunk
// end, then Delta) into LDS, one dword per lane; issued by one wave.
__device__ __forceinline__ void dma_stats(uint32_t lds, const AttnArgs& a, int unit, int lane) {
  dma4_at(uniform_ptr(a.stats + (int64_t)unit * 64), (uint32_t)lane * 4u, lds);
}

// P and dS of accumulator elements [r0, r0 + n) of a lane, in place (s -> P, dp -> dS).
// Element r is query 8 (r / 4) + 4 hl + r % 4 of the tile; the lane's key is `key`.
// With MASK the causal / length mask is applied (pipelined tiles always apply it: the
// few VALU operations issue under the MFMAs).
// bv: the bias of the lane's 16 elements (loaded a step ahead).
template <int N, bool MASK, bool CAUSAL, bool BIAS>
__device__ __forceinline__ void softmax_part(f32x16& s, f32x16& dp, int r0, const float* lse,
                                             const float* dl, int hl, float c, int key,
                                             bool key_ok, int nq, int tile_pos0,
                                             const float (&bv)[16]) {
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const int r = r0 + k, qi = 8 * (r >> 2) + 4 * hl + (r & 3);
    float x;
    if (BIAS)
      x = fmaf(bv[r], kLog2e, s[r] * c) - lse[qi];
    else
      x = fmaf(s[r], c, -lse[qi]);
    if (MASK) {
      const bool vis = key_ok && qi < nq && (!CAUSAL || key <= tile_pos0 + qi);
      x = vis ? x : -INFINITY;
    }
    const float p = exp2f_fast(x);
    s[r] = p;
    dp[r] = p * (dp[r] - dl[qi]);
  }
}

// Probability from which a tile's dV/dK products are repeated with the BF16 residues.
constexpr float kResidueP = 0.03125f;

// The BF16 residues x - bf16(x) of accumulator elements [base, base + 8), given their
// packed BF16 values hi (the difference is exact in fp32).
__device__ __forceinline__ u32x4 residue_bf16x8(const f32x16& v, const u32x4& hi, int base) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = pack_bf16x2(v[base + 2 * i] - bf16_lo(hi[i]), v[base + 2 * i + 1] - bf16_hi(hi[i]));
  return r;
}

// Whether any probability of the wave's tile (P in the accumulator) reaches kResidueP.
// P is not negative (an exponential, or 0 where masked), so its bits order like its
// value as signed integers: the maximum is integer max3 steps (no NaN quieting), and the
// result is a wave-uniform scalar.
__device__ __forceinline__ uint32_t wave_has_large_p(const f32x16& p) {
  int m = max(__float_as_int(p[0]), __float_as_int(p[1]));
#pragma unroll
  for (int r = 2; r < 16; ++r) m = max(m, __float_as_int(p[r]));
  const uint64_t b = __builtin_amdgcn_ballot_w64(m >= __float_as_int(kResidueP));
  return (uint32_t)b | (uint32_t)(b >> 32);  // nonzero iff some lane's P reaches it
}

}  // namespace

// A 16-byte LDS read at a 32-bit LDS address (the dV/dK operand addresses are formed as
// integers once per step and shared with the residue products' assembly).
using lds_u32x4_cptr = const __attribute__((address_space(3))) u32x4*;
__device__ __forceinline__ u32x4 lds16(uint32_t addr) { return *(lds_u32x4_cptr)(uintptr_t)addr; }

// S and dP products in arch VGPRs.  At D = 256 the dK^T/dV^T accumulators fill all 256
// accumulation registers, and the compiler places every MFMA result there, so S and dP
// would displace one dK/dV block per step (96 register moves).  Inline assembly pins
// their destinations to VGPRs.  A chain accumulates into the same registers (no wait
// states needed between dependent products of one shape); xdl_fence covers the wait
// states before VALU reads the results (at least 11 after an 8-pass product; 12 given,
// counted from the fence alone).
__device__ __forceinline__ f32x16 mfma32_v0(u32x4 a, u32x4 b) {
  f32x16 d;
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  return d;
}
__device__ __forceinline__ void mfma32_v(f32x16& c, u32x4 a, u32x4 b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void xdl_fence(f32x16& x) {
  asm volatile("s_nop 7\n\ts_nop 3" : "+v"(x));
}
__device__ __forceinline__ void xdl_fence2(f32x16& x, f32x16& y) {
  asm volatile("s_nop 7\n\ts_nop 3" : "+v"(x), "+v"(y));
}

// The residue products of one tile, dV^T += dO^T rp and dK^T += Q^T rd for every 32-row
// block, only when flag (wave-uniform) is non-zero.  The branch and the products are one
// assembly block: the compiler then sees no control flow around the accumulators (at
// D = 256 they take all 256 accumulation registers, and with a branch around compiler
// products it shuffled them through the arch registers and spilled), and the common case
// costs one taken branch per step.  The block reads its A operands itself (16-byte reads
// of the transposed tiles at the lane addresses a0 / a1 of k-steps 0 / 1; the dO^T tile
// is TB bytes after the Q^T tile, block b 2048 bytes after block 0), two blocks' reads in
// flight, and runs before the tile's ordinary products, so that the last writer of every
// accumulator is a product the compiler placed (and whose hazards it tracks); consecutive
// products accumulating into exactly the same registers need no wait states.  The
// s_waitcnt at entry drains the compiler's outstanding LDS / scalar loads, so the counts
// inside refer to this block's reads only.
template <int NB, int TB>
__device__ __forceinline__ void residue_products(f32x16 (&dvt)[NB], f32x16 (&dkt)[NB], uint32_t a0,
                                                 uint32_t a1, const u32x4 (&rp)[2], const u32x4 (&rd)[2],
                                                 uint32_t flag_in) {
  static_assert(TB + (NB - 1) * 2048 < 65536, "ds_read offsets are 16 bits");
  const uint32_t flag = flag_in;  // wave-uniform (a ballot), kept in a scalar register
  u32x4 t[4], u[4];
  (void)u;
  if constexpr (NB == 1) {
    asm volatile(
        "s_cmp_eq_u32 %[flag], 0\n\t"
        "s_cbranch_scc1 9f\n\t"
        "s_waitcnt lgkmcnt(0)\n\t"
        "s_nop 1\n\t"
        "ds_read_b128 %[t0], %[a0] offset:%c[od0]\n\t"
        "ds_read_b128 %[t1], %[a1] offset:%c[od0]\n\t"
        "ds_read_b128 %[t2], %[a0] offset:%c[oq0]\n\t"
        "ds_read_b128 %[t3], %[a1] offset:%c[oq0]\n\t"
        "s_waitcnt lgkmcnt(0)\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dv0], %[t0], %[rp0], %[dv0]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dv0], %[t1], %[rp1], %[dv0]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dk0], %[t2], %[rd0], %[dk0]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dk0], %[t3], %[rd1], %[dk0]\n\t"
        "9:"
        : [dv0] "+a"(dvt[0]), [dk0] "+a"(dkt[0]), [t0] "=&v"(t[0]), [t1] "=&v"(t[1]), [t2] "=&v"(t[2]), [t3] "=&v"(t[3])
        : [a0] "v"(a0), [a1] "v"(a1), [rp0] "v"(rp[0]), [rp1] "v"(rp[1]), [rd0] "v"(rd[0]), [rd1] "v"(rd[1]), [flag] "s"(flag), [od0] "i"(TB + 0 * 2048), [oq0] "i"(0 * 2048)
        : "scc");
  }
  if constexpr (NB == 2) {
    asm volatile(
        "s_cmp_eq_u32 %[flag], 0\n\t"
        "s_cbranch_scc1 9f\n\t"
        "s_waitcnt lgkmcnt(0)\n\t"
        "s_nop 1\n\t"
        "ds_read_b128 %[t0], %[a0] offset:%c[od0]\n\t"
        "ds_read_b128 %[t1], %[a1] offset:%c[od0]\n\t"
        "ds_read_b128 %[t2], %[a0] offset:%c[oq0]\n\t"
        "ds_read_b128 %[t3], %[a1] offset:%c[oq0]\n\t"
        "ds_read_b128 %[u0], %[a0] offset:%c[od1]\n\t"
        "ds_read_b128 %[u1], %[a1] offset:%c[od1]\n\t"
        "ds_read_b128 %[u2], %[a0] offset:%c[oq1]\n\t"
        "ds_read_b128 %[u3], %[a1] offset:%c[oq1]\n\t"
        "s_waitcnt lgkmcnt(4)\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dv0], %[t0], %[rp0], %[dv0]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dv0], %[t1], %[rp1], %[dv0]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dk0], %[t2], %[rd0], %[dk0]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dk0], %[t3], %[rd1], %[dk0]\n\t"
        "s_waitcnt lgkmcnt(0)\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dv1], %[u0], %[rp0], %[dv1]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dv1], %[u1], %[rp1], %[dv1]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dk1], %[u2], %[rd0], %[dk1]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dk1], %[u3], %[rd1], %[dk1]\n\t"
        "9:"
        : [dv0] "+a"(dvt[0]), [dk0] "+a"(dkt[0]), [dv1] "+a"(dvt[1]), [dk1] "+a"(dkt[1]), [t0] "=&v"(t[0]), [t1] "=&v"(t[1]), [t2] "=&v"(t[2]), [t3] "=&v"(t[3]), [u0] "=&v"(u[0]), [u1] "=&v"(u[1]), [u2] "=&v"(u[2]), [u3] "=&v"(u[3])
        : [a0] "v"(a0), [a1] "v"(a1), [rp0] "v"(rp[0]), [rp1] "v"(rp[1]), [rd0] "v"(rd[0]), [rd1] "v"(rd[1]), [flag] "s"(flag), [od0] "i"(TB + 0 * 2048), [oq0] "i"(0 * 2048), [od1] "i"(TB + 1 * 2048), [oq1] "i"(1 * 2048)
        : "scc");
  }
  if constexpr (NB == 4) {
    asm volatile(
        "s_cmp_eq_u32 %[flag], 0\n\t"
        "s_cbranch_scc1 9f\n\t"
        "s_waitcnt lgkmcnt(0)\n\t"
        "s_nop 1\n\t"
        "ds_read_b128 %[t0], %[a0] offset:%c[od0]\n\t"
        "ds_read_b128 %[t1], %[a1] offset:%c[od0]\n\t"
        "ds_read_b128 %[t2], %[a0] offset:%c[oq0]\n\t"
        "ds_read_b128 %[t3], %[a1] offset:%c[oq0]\n\t"
        "ds_read_b128 %[u0], %[a0] offset:%c[od1]\n\t"
        "ds_read_b128 %[u1], %[a1] offset:%c[od1]\n\t"
        "ds_read_b128 %[u2], %[a0] offset:%c[oq1]\n\t"
        "ds_read_b128 %[u3], %[a1] offset:%c[oq1]\n\t"
        "s_waitcnt lgkmcnt(4)\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dv0], %[t0], %[rp0], %[dv0]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dv0], %[t1], %[rp1], %[dv0]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dk0], %[t2], %[rd0], %[dk0]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dk0], %[t3], %[rd1], %[dk0]\n\t"
        "ds_read_b128 %[t0], %[a0] offset:%c[od2]\n\t"
        "ds_read_b128 %[t1], %[a1] offset:%c[od2]\n\t"
        "ds_read_b128 %[t2], %[a0] offset:%c[oq2]\n\t"
        "ds_read_b128 %[t3], %[a1] offset:%c[oq2]\n\t"
        "s_waitcnt lgkmcnt(4)\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dv1], %[u0], %[rp0], %[dv1]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dv1], %[u1], %[rp1], %[dv1]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dk1], %[u2], %[rd0], %[dk1]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dk1], %[u3], %[rd1], %[dk1]\n\t"
        "ds_read_b128 %[u0], %[a0] offset:%c[od3]\n\t"
        "ds_read_b128 %[u1], %[a1] offset:%c[od3]\n\t"
        "ds_read_b128 %[u2], %[a0] offset:%c[oq3]\n\t"
        "ds_read_b128 %[u3], %[a1] offset:%c[oq3]\n\t"
        "s_waitcnt lgkmcnt(4)\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dv2], %[t0], %[rp0], %[dv2]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dv2], %[t1], %[rp1], %[dv2]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dk2], %[t2], %[rd0], %[dk2]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dk2], %[t3], %[rd1], %[dk2]\n\t"
        "s_waitcnt lgkmcnt(0)\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dv3], %[u0], %[rp0], %[dv3]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dv3], %[u1], %[rp1], %[dv3]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dk3], %[u2], %[rd0], %[dk3]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dk3], %[u3], %[rd1], %[dk3]\n\t"
        "9:"
        : [dv0] "+a"(dvt[0]), [dk0] "+a"(dkt[0]), [dv1] "+a"(dvt[1]), [dk1] "+a"(dkt[1]), [dv2] "+a"(dvt[2]), [dk2] "+a"(dkt[2]), [dv3] "+a"(dvt[3]), [dk3] "+a"(dkt[3]), [t0] "=&v"(t[0]), [t1] "=&v"(t[1]), [t2] "=&v"(t[2]), [t3] "=&v"(t[3]), [u0] "=&v"(u[0]), [u1] "=&v"(u[1]), [u2] "=&v"(u[2]), [u3] "=&v"(u[3])
        : [a0] "v"(a0), [a1] "v"(a1), [rp0] "v"(rp[0]), [rp1] "v"(rp[1]), [rd0] "v"(rd[0]), [rd1] "v"(rd[1]), [flag] "s"(flag), [od0] "i"(TB + 0 * 2048), [oq0] "i"(0 * 2048), [od1] "i"(TB + 1 * 2048), [oq1] "i"(1 * 2048), [od2] "i"(TB + 2 * 2048), [oq2] "i"(2 * 2048), [od3] "i"(TB + 3 * 2048), [oq3] "i"(3 * 2048)
        : "scc");
  }
  if constexpr (NB == 8) {
    asm volatile(
        "s_cmp_eq_u32 %[flag], 0\n\t"
        "s_cbranch_scc1 9f\n\t"
        "s_waitcnt lgkmcnt(0)\n\t"
        "s_nop 1\n\t"
        "ds_read_b128 %[t0], %[a0] offset:%c[od0]\n\t"
        "ds_read_b128 %[t1], %[a1] offset:%c[od0]\n\t"
        "ds_read_b128 %[t2], %[a0] offset:%c[oq0]\n\t"
        "ds_read_b128 %[t3], %[a1] offset:%c[oq0]\n\t"
        "ds_read_b128 %[u0], %[a0] offset:%c[od1]\n\t"
        "ds_read_b128 %[u1], %[a1] offset:%c[od1]\n\t"
        "ds_read_b128 %[u2], %[a0] offset:%c[oq1]\n\t"
        "ds_read_b128 %[u3], %[a1] offset:%c[oq1]\n\t"
        "s_waitcnt lgkmcnt(4)\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dv0], %[t0], %[rp0], %[dv0]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dv0], %[t1], %[rp1], %[dv0]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dk0], %[t2], %[rd0], %[dk0]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dk0], %[t3], %[rd1], %[dk0]\n\t"
        "ds_read_b128 %[t0], %[a0] offset:%c[od2]\n\t"
        "ds_read_b128 %[t1], %[a1] offset:%c[od2]\n\t"
        "ds_read_b128 %[t2], %[a0] offset:%c[oq2]\n\t"
        "ds_read_b128 %[t3], %[a1] offset:%c[oq2]\n\t"
        "s_waitcnt lgkmcnt(4)\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dv1], %[u0], %[rp0], %[dv1]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dv1], %[u1], %[rp1], %[dv1]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dk1], %[u2], %[rd0], %[dk1]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dk1], %[u3], %[rd1], %[dk1]\n\t"
        "ds_read_b128 %[u0], %[a0] offset:%c[od3]\n\t"
        "ds_read_b128 %[u1], %[a1] offset:%c[od3]\n\t"
        "ds_read_b128 %[u2], %[a0] offset:%c[oq3]\n\t"
        "ds_read_b128 %[u3], %[a1] offset:%c[oq3]\n\t"
        "s_waitcnt lgkmcnt(4)\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dv2], %[t0], %[rp0], %[dv2]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dv2], %[t1], %[rp1], %[dv2]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dk2], %[t2], %[rd0], %[dk2]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dk2], %[t3], %[rd1], %[dk2]\n\t"
        "ds_read_b128 %[t0], %[a0] offset:%c[od4]\n\t"
        "ds_read_b128 %[t1], %[a1] offset:%c[od4]\n\t"
        "ds_read_b128 %[t2], %[a0] offset:%c[oq4]\n\t"
        "ds_read_b128 %[t3], %[a1] offset:%c[oq4]\n\t"
        "s_waitcnt lgkmcnt(4)\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dv3], %[u0], %[rp0], %[dv3]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dv3], %[u1], %[rp1], %[dv3]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dk3], %[u2], %[rd0], %[dk3]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dk3], %[u3], %[rd1], %[dk3]\n\t"
        "ds_read_b128 %[u0], %[a0] offset:%c[od5]\n\t"
        "ds_read_b128 %[u1], %[a1] offset:%c[od5]\n\t"
        "ds_read_b128 %[u2], %[a0] offset:%c[oq5]\n\t"
        "ds_read_b128 %[u3], %[a1] offset:%c[oq5]\n\t"
        "s_waitcnt lgkmcnt(4)\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dv4], %[t0], %[rp0], %[dv4]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dv4], %[t1], %[rp1], %[dv4]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dk4], %[t2], %[rd0], %[dk4]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dk4], %[t3], %[rd1], %[dk4]\n\t"
        "ds_read_b128 %[t0], %[a0] offset:%c[od6]\n\t"
        "ds_read_b128 %[t1], %[a1] offset:%c[od6]\n\t"
        "ds_read_b128 %[t2], %[a0] offset:%c[oq6]\n\t"
        "ds_read_b128 %[t3], %[a1] offset:%c[oq6]\n\t"
        "s_waitcnt lgkmcnt(4)\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dv5], %[u0], %[rp0], %[dv5]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dv5], %[u1], %[rp1], %[dv5]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dk5], %[u2], %[rd0], %[dk5]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dk5], %[u3], %[rd1], %[dk5]\n\t"
        "ds_read_b128 %[u0], %[a0] offset:%c[od7]\n\t"
        "ds_read_b128 %[u1], %[a1] offset:%c[od7]\n\t"
        "ds_read_b128 %[u2], %[a0] offset:%c[oq7]\n\t"
        "ds_read_b128 %[u3], %[a1] offset:%c[oq7]\n\t"
        "s_waitcnt lgkmcnt(4)\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dv6], %[t0], %[rp0], %[dv6]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dv6], %[t1], %[rp1], %[dv6]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dk6], %[t2], %[rd0], %[dk6]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dk6], %[t3], %[rd1], %[dk6]\n\t"
        "s_waitcnt lgkmcnt(0)\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dv7], %[u0], %[rp0], %[dv7]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dv7], %[u1], %[rp1], %[dv7]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dk7], %[u2], %[rd0], %[dk7]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[dk7], %[u3], %[rd1], %[dk7]\n\t"
        "9:"
        : [dv0] "+a"(dvt[0]), [dk0] "+a"(dkt[0]), [dv1] "+a"(dvt[1]), [dk1] "+a"(dkt[1]), [dv2] "+a"(dvt[2]), [dk2] "+a"(dkt[2]), [dv3] "+a"(dvt[3]), [dk3] "+a"(dkt[3]), [dv4] "+a"(dvt[4]), [dk4] "+a"(dkt[4]), [dv5] "+a"(dvt[5]), [dk5] "+a"(dkt[5]), [dv6] "+a"(dvt[6]), [dk6] "+a"(dkt[6]), [dv7] "+a"(dvt[7]), [dk7] "+a"(dkt[7]), [t0] "=&v"(t[0]), [t1] "=&v"(t[1]), [t2] "=&v"(t[2]), [t3] "=&v"(t[3]), [u0] "=&v"(u[0]), [u1] "=&v"(u[1]), [u2] "=&v"(u[2]), [u3] "=&v"(u[3])
        : [a0] "v"(a0), [a1] "v"(a1), [rp0] "v"(rp[0]), [rp1] "v"(rp[1]), [rd0] "v"(rd[0]), [rd1] "v"(rd[1]), [flag] "s"(flag), [od0] "i"(TB + 0 * 2048), [oq0] "i"(0 * 2048), [od1] "i"(TB + 1 * 2048), [oq1] "i"(1 * 2048), [od2] "i"(TB + 2 * 2048), [oq2] "i"(2 * 2048), [od3] "i"(TB + 3 * 2048), [oq3] "i"(3 * 2048), [od4] "i"(TB + 4 * 2048), [oq4] "i"(4 * 2048), [od5] "i"(TB + 5 * 2048), [oq5] "i"(5 * 2048), [od6] "i"(TB + 6 * 2048), [oq6] "i"(6 * 2048), [od7] "i"(TB + 7 * 2048), [oq7] "i"(7 * 2048)
        : "scc");
  }

}

// One side of the residue products, for the step order that runs all dV^T products
// before all dK^T products: acc += X^T r for every 32-row block, X^T the tile OFF bytes
// after the lane addresses a0 / a1 (k-steps 0 / 1), only when flag (wave-uniform) is
// non-zero.  The same conventions as residue_products.
template <int NB, int OFF>
__device__ __forceinline__ void residue_half(f32x16 (&acc)[NB], uint32_t a0, uint32_t a1,
                                             const u32x4 (&r)[2], uint32_t flag_in) {
  static_assert(NB == 8 && OFF + (NB - 1) * 2048 < 65536, "ds_read offsets are 16 bits");
  const uint32_t flag = flag_in;  // wave-uniform (a ballot), kept in a scalar register
  u32x4 t[2], u[2];
  if constexpr (NB == 8) {
    asm volatile(
        "s_cmp_eq_u32 %[flag], 0\n\t"
        "s_cbranch_scc1 9f\n\t"
        "s_waitcnt lgkmcnt(0)\n\t"
        "s_nop 1\n\t"
        "ds_read_b128 %[t0], %[a0] offset:%c[o0]\n\t"
        "ds_read_b128 %[t1], %[a1] offset:%c[o0]\n\t"
        "ds_read_b128 %[u0], %[a0] offset:%c[o1]\n\t"
        "ds_read_b128 %[u1], %[a1] offset:%c[o1]\n\t"
        "s_waitcnt lgkmcnt(2)\n\t"
        "v_mfma_f32_32x32x16_bf16 %[c0], %[t0], %[r0], %[c0]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[c0], %[t1], %[r1], %[c0]\n\t"
        "ds_read_b128 %[t0], %[a0] offset:%c[o2]\n\t"
        "ds_read_b128 %[t1], %[a1] offset:%c[o2]\n\t"
        "s_waitcnt lgkmcnt(2)\n\t"
        "v_mfma_f32_32x32x16_bf16 %[c1], %[u0], %[r0], %[c1]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[c1], %[u1], %[r1], %[c1]\n\t"
        "ds_read_b128 %[u0], %[a0] offset:%c[o3]\n\t"
        "ds_read_b128 %[u1], %[a1] offset:%c[o3]\n\t"
        "s_waitcnt lgkmcnt(2)\n\t"
        "v_mfma_f32_32x32x16_bf16 %[c2], %[t0], %[r0], %[c2]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[c2], %[t1], %[r1], %[c2]\n\t"
        "ds_read_b128 %[t0], %[a0] offset:%c[o4]\n\t"
        "ds_read_b128 %[t1], %[a1] offset:%c[o4]\n\t"
        "s_waitcnt lgkmcnt(2)\n\t"
        "v_mfma_f32_32x32x16_bf16 %[c3], %[u0], %[r0], %[c3]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[c3], %[u1], %[r1], %[c3]\n\t"
        "ds_read_b128 %[u0], %[a0] offset:%c[o5]\n\t"
        "ds_read_b128 %[u1], %[a1] offset:%c[o5]\n\t"
        "s_waitcnt lgkmcnt(2)\n\t"
        "v_mfma_f32_32x32x16_bf16 %[c4], %[t0], %[r0], %[c4]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[c4], %[t1], %[r1], %[c4]\n\t"
        "ds_read_b128 %[t0], %[a0] offset:%c[o6]\n\t"
        "ds_read_b128 %[t1], %[a1] offset:%c[o6]\n\t"
        "s_waitcnt lgkmcnt(2)\n\t"
        "v_mfma_f32_32x32x16_bf16 %[c5], %[u0], %[r0], %[c5]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[c5], %[u1], %[r1], %[c5]\n\t"
        "ds_read_b128 %[u0], %[a0] offset:%c[o7]\n\t"
        "ds_read_b128 %[u1], %[a1] offset:%c[o7]\n\t"
        "s_waitcnt lgkmcnt(2)\n\t"
        "v_mfma_f32_32x32x16_bf16 %[c6], %[t0], %[r0], %[c6]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[c6], %[t1], %[r1], %[c6]\n\t"
        "s_waitcnt lgkmcnt(0)\n\t"
        "v_mfma_f32_32x32x16_bf16 %[c7], %[u0], %[r0], %[c7]\n\t"
        "v_mfma_f32_32x32x16_bf16 %[c7], %[u1], %[r1], %[c7]\n\t"
        "9:"
        : [c0] "+a"(acc[0]), [c1] "+a"(acc[1]), [c2] "+a"(acc[2]), [c3] "+a"(acc[3]), [c4] "+a"(acc[4]), [c5] "+a"(acc[5]), [c6] "+a"(acc[6]), [c7] "+a"(acc[7]), [t0] "=&v"(t[0]), [t1] "=&v"(t[1]), [u0] "=&v"(u[0]), [u1] "=&v"(u[1])
        : [a0] "v"(a0), [a1] "v"(a1), [r0] "v"(r[0]), [r1] "v"(r[1]), [flag] "s"(flag), [o0] "i"(OFF + 0 * 2048), [o1] "i"(OFF + 1 * 2048), [o2] "i"(OFF + 2 * 2048), [o3] "i"(OFF + 3 * 2048), [o4] "i"(OFF + 4 * 2048), [o5] "i"(OFF + 5 * 2048), [o6] "i"(OFF + 6 * 2048), [o7] "i"(OFF + 7 * 2048)
        : "scc");
  }

}

template <int D, bool CAUSAL, bool BIAS>
__global__ __launch_bounds__(kKvThreads) void dkdv_kernel(const AttnArgs a) {
  constexpr int NS = D / 16;       // 16-deep k-steps of S and dP
  constexpr int NB = D / 32;       // 32-row blocks of dK^T and dV^T
  constexpr int TE = D * kTq;      // elements of one transposed tile
  constexpr int EPB = 16 / NB;     // softmax elements per dV/dK block
  // Up to D = 128 the steps are software pipelined: a tile's softmax runs under the
  // previous tile's dV/dK products.  At D = 256 the accumulators fill the accumulation
  // registers and two tiles' P / dS do not fit; a step then orders its own products so
  // that its softmax runs under its dP and dV products (SPLIT).
  constexpr bool SPLIT = D == 256;
  constexpr bool PIPE = !SPLIT;
  __shared__ __attribute__((aligned(1024))) uint16_t lds_t[kBufs][2][TE];  // [buf][Q^T, dO^T]
  // per buffer: log2(e) LSE of the tile's rows, then their Delta
  __shared__ __attribute__((aligned(16))) float lds_st[kBufs][2 * kTq];

  if (*a.dev_err) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, n = lane & 31;
  const int logical = xcd_group_order(blockIdx.x, gridDim.x / a.kv_tiles, a.kv_tiles, a.hkv);
  const int kslot = logical % a.kv_tiles;
  const int rest = logical / a.kv_tiles;
  const int g = rest % a.hkv;
  const int b = rest / a.hkv;
  const int L = rfl(a.seq_lens[b]);
  // With a.kv_pair (causal masking) the workgroup takes two key tiles of its sequence,
  // kslot and nt - 1 - kslot (nt = the sequence's tiles), one after the other: a tile's
  // work falls with its position, and the pairs even it out across workgroups.
  const int nt = (L + kDkdvKeys - 1) / kDkdvKeys;
  for (int pass = 0; pass < (a.kv_pair ? 2 : 1); ++pass) {
    const int kt = !a.kv_pair ? kslot : pass == 0 ? (kslot < (nt + 1) / 2 ? kslot : -1)
                                                  : (kslot < nt / 2 ? nt - 1 - kslot : -1);
    if (kt < 0) continue;
    if (pass > 0) __syncthreads();  // the first pass's last reads of the tile buffers are done
    const int wg_key0 = kt * kDkdvKeys;
    // no key of the tile in the sequence or in the key window [kv_lo, kv_hi)
    if (wg_key0 >= L || wg_key0 >= a.kv_hi || wg_key0 + kDkdvKeys <= a.kv_lo) continue;
    const int64_t koff = rfl(a.seq_offsets[b]);
    const int wkey0 = wg_key0 + wave * 32;
    const int nk = max(0, min(32, L - wkey0));
    const int key = wkey0 + n;  // this lane's key (column of S, dP, dK^T, dV^T)
    const bool key_ok = n < nk && key >= a.kv_lo && key < a.kv_hi;  // in the sequence and the window
    // The wave-level tests (keys past the sequence end or outside the key window) from a
    // scalar copy of the wave's first key, for the per-step decisions (mask fix-up, dS
    // store), so that they are scalar branches.
    const int wkey0_u = wg_key0 + __builtin_amdgcn_readfirstlane(wave) * 32;
    const bool wave_masked_u = min(32, L - wkey0_u) < 32 || wkey0_u < a.kv_lo || wkey0_u + 32 > a.kv_hi;

    // K and V as B operands: lane (hl, n) holds key n, dimensions 16 st + 8 hl + [0, 8).
    // Lanes past the sequence end load its last key (finite values; their P and dS are 0).
    const int64_t kv_stride = a.kv_pitch * D;
    u32x4 kf[NS], vf[NS];
    {
      const int64_t off = (koff + min(key, L - 1)) * kv_stride + (int64_t)g * D + hl * 8;
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        kf[st] = ld16(a.k + off + st * 16);
        vf[st] = ld16(a.v + off + st * 16);
      }
    }
    f32x16 dkt[NB], dvt[NB];
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      dkt[blk] = f32x16{};
      dvt[blk] = f32x16{};
    }
    // S/dP A operand, k-step st: row n of S is tile query n; its 8 values are dimensions
    // 16 st + 8 hl + 4 r + j (r = 0, 1 reads), gathered by transposing reads in which
    // source lane 4 j + m of each 16-lane group reads dimension row 16 st + 8 hl + 4 r + j
    // at stored query positions c0 .. c0 + 3, c0 = 16 (group & 1) + 4 swap2(m) (the stored
    // order sigma16 within 16 queries, undone).  The row's granule swizzle is
    // tswz = 2 hl + r, the same for every st.
    int tra[2];
    {
      const int grp = lane >> 4, j = (lane >> 2) & 3, m = lane & 3;
      const int sm = ((m & 1) << 1) | (m >> 1);
      const int gq = 2 * (grp & 1) + (sm >> 1);
#pragma unroll
      for (int r = 0; r < 2; ++r)
        tra[r] = (8 * hl + 4 * r + j) * kTq + ((gq ^ (2 * hl + r)) * 8) + 4 * (sm & 1);
    }
    // dV/dK A operand, k-step t: row 32 blk + n, granule (2 t + hl) ^ tswz(n).
    const int tr_off0 = n * kTq + ((hl ^ tswz(n)) * 8);
    const int tr_off1 = n * kTq + (((2 + hl) ^ tswz(n)) * 8);

    const int c_end = chunk_lower_bound(a.chunks, a.num_chunks, b + 1);
    const int h0 = g * a.group;  // the group's first query head
    QTileIter cur;
    cur.c = chunk_lower_bound(a.chunks, a.num_chunks, b);
    bool have = seek_chunk<CAUSAL>(a, cur, c_end, wg_key0, h0, L);
    // With a bias: the lane's 16 bias values of a tile (element r is query 8 (r / 4) +
    // 4 hl + r % 4 of the tile, key `key`), loaded one step ahead so that their latency
    // is spent under the previous step's products; used only after the step's wait.
    float bias_cur[16] = {}, bias_nxt[16] = {};
    auto load_bias = [&](const QTileIter& it, float (&bv)[16]) {
      const float* bh = a.bias + (int64_t)(g * a.group + it.hh) * a.bias_len * a.bias_len;
      const int tp0 = it.ch.pos0 + it.qt * kTq;
      const int kk = min(key, a.bias_len - 1);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = 8 * (r >> 2) + 4 * hl + (r & 3);
        bv[r] = bh[(int64_t)min(tp0 + qi, a.bias_len - 1) * a.bias_len + kk];
      }
    };
    if (BIAS && have) load_bias(cur, bias_cur);
    // the wave that copies each step's row statistics
    const bool stats_wave = __builtin_amdgcn_readfirstlane(wave) == kWaves - 1;
    if (have) {
      dma_tiles<D>(lds_t[0][0], lds_t[0][1], a, cur, wave, lane);
      if (stats_wave) dma_stats(lds_addr(lds_st[0]), a, cur.unit, lane);
    }
    wait_vm_all();
    __syncthreads();

    // Lane addresses of the dV/dK A operands, k-steps 0 / 1, in buffer 0 (the residue
    // products and the ordinary ones share them, plus the buffer's offset).
    const uint32_t lds_st0 = lds_addr(lds_st[0]);
    const uint32_t res_a0 = lds_addr(lds_t[0][0]) + 2u * (uint32_t)tr_off0;
    const uint32_t res_a1 = lds_addr(lds_t[0][0]) + 2u * (uint32_t)tr_off1;
    // dV/dK products of one tile: A operands from buffer pb, B = packed P / dS.  The
    // operand stream (per block: dO^T steps 0 and 1, then Q^T steps 0 and 1) is read
    // three products ahead.  Between the blocks, body(blk) issues independent work.
    auto dvdk = [&](int pb, const u32x4 (&pp)[2], const u32x4 (&pd)[2], auto&& body) {
      const uint32_t boff = (uint32_t)pb * (2u * TE * 2u);
      const uint32_t a0 = res_a0 + boff, a1 = res_a1 + boff;
      constexpr int NOP = 4 * NB;
      auto operand = [&](int i) {
        const int blk = i >> 2, which = i & 3;
        return lds16(((which & 1) ? a1 : a0) + (uint32_t)((which < 2 ? TE * 2 : 0) + blk * 32 * kTq * 2));
      };
      u32x4 f[4];
      f[0] = operand(0);
      f[1] = operand(1);
      f[2] = operand(2);
#pragma unroll
      for (int i = 0; i < NOP; ++i) {
        if (i + 3 < NOP) f[(i + 3) & 3] = operand(i + 3);
        const int blk = i >> 2, which = i & 3;
        if (which < 2) dvt[blk] = mfma32(f[i & 3], pp[which], dvt[blk]);
        else dkt[blk] = mfma32(f[i & 3], pd[which & 1], dkt[blk]);
        if (which == 3) body(blk);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    u32x4 pp[2] = {}, pd[2] = {};  // packed P and dS of the previous tile
    u32x4 rp[2] = {}, rd[2] = {};  // their BF16 residues, when res_prev
    int buf = 0, pbuf = 0;
    bool have_prev = false;
    uint32_t res_prev = 0;
    auto nop = [](int) {};
    // Residue products of the tile in buffer pb (lane addresses of its k-step 0 / 1 operands).
    auto residue = [&](int pb, const u32x4 (&rp)[2], const u32x4 (&rd)[2], uint32_t flag) {
      const uint32_t boff = (uint32_t)pb * (2u * TE * 2u);
      residue_products<NB, TE * 2>(dvt, dkt, res_a0 + boff, res_a1 + boff, rp, rd, flag);
    };
    // Tile copies of the next step: for D >= 128 one instruction every other S/dP k-step
    // (every wave issues D / 32 of them; without a next tile the current one is re-copied
    // into the free buffer), for smaller D all at once.  Copy k of a tensor by this wave
    // moves the tile's 1 KB piece i = wave + kWaves k: the lane offsets are fixed.
    constexpr bool SPREAD = D >= 128;
    constexpr int TI = SPREAD ? D * kTq * 2 / 1024 / kWaves : 1;  // copies per wave per tensor
    const int wu = __builtin_amdgcn_readfirstlane(wave);
    uint32_t voff[SPREAD ? TI : 1];
#pragma unroll
    for (int k = 0; k < (SPREAD ? TI : 1); ++k) voff[k] = (uint32_t)lane * 16u + (uint32_t)(wu + kWaves * k) * 1024u;
    const char* const qt_base = uniform_ptr(a.qt);
    const char* const dot_base = uniform_ptr(a.dot);
    // D = 256: the first three A operands of a step (S, k-steps 0-2, from its Q^T tile)
    // are read right after the previous step's barrier, so that their latency passes
    // under the step's scalar set-up instead of delaying its first product.
    auto s_opnd = [&](const uint16_t* t, int st) {
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(CPATTN_LDS(v4i16, t + st * 16 * kTq + tra[0]));
      const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(CPATTN_LDS(v4i16, t + st * 16 * kTq + tra[1]));
      const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
      return u32x4{l2[0], l2[1], h2[0], h2[1]};
    };
    u32x4 ring0[3];
    if constexpr (SPLIT) {
#pragma unroll
      for (int k = 0; k < 3; ++k) ring0[k] = s_opnd(lds_t[0][0], k);
    }
    while (have) {
      QTileIter nxt = cur;
      const bool have_next = advance<CAUSAL>(a, nxt, c_end, wg_key0, h0, L);
      const int nbuf = (buf + 1 == kBufs) ? 0 : buf + 1;
      const int src_unit = have_next ? nxt.unit : cur.unit;
      const int64_t src_off = (int64_t)src_unit * (D * kTq * 2);
      const char* cb[2] = {qt_base + src_off, dot_base + src_off};
      const uint32_t clw = lds_addr(lds_t[nbuf][0]) + (uint32_t)wu * 1024u;
      auto copy_one = [&](int p) {  // p < 2 TI: tensor p / TI, copy p % TI
        const int which = p / TI, k = p % TI;
        dma16_add(cb[which], voff[k], clw, (uint32_t)(which * TE * 2 + k * kWaves * 1024));
      };
      // (the LDS address as an integer: a pointer into lds_st converted per step costs
      // 64-bit arithmetic and a null test)
      if (stats_wave) dma_stats(lds_st0 + (uint32_t)nbuf * (2u * kTq * 4u), a, src_unit, lane);
      if (BIAS && have_next) load_bias(nxt, bias_nxt);
      if (!SPREAD && have_next) dma_tiles<D>(lds_t[nbuf][0], lds_t[nbuf][1], a, nxt, wave, lane);

      // Every wave runs every tile of the loop: tiles that a wave's keys do not see (at the
      // causal diagonal, or past the sequence end) give P = dS = 0 and add nothing.
      const int nq = min(kTq, cur.ch.len - cur.qt * kTq);
      const int tile_pos0 = cur.ch.pos0 + cur.qt * kTq;
      uint32_t res_cur = 0;

      // A operand of the S / dP products, k-step st, from the transposed tile t.
      auto tr_a = [&](const uint16_t* t, int st) {
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(CPATTN_LDS(v4i16, t + st * 16 * kTq + tra[0]));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(CPATTN_LDS(v4i16, t + st * 16 * kTq + tra[1]));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        return u32x4{l2[0], l2[1], h2[0], h2[1]};
      };
      if constexpr (SPLIT) {
        // One tile as a stream of 64 products in four phases, so that the softmax runs on
        // the vector ALU while the matrix core works: (1) S, (2) dP, with P = exp2(S c - LSE)
        // formed element by element under it, (3) dV^T += dO^T P, with dS = P (dP - Delta)
        // formed under it, (4) dK^T += Q^T dS.  The A operands of the stream are read from
        // LDS three products ahead.
        static_assert(!BIAS, "no bias term at this head dimension");
        const uint16_t* qtt = lds_t[buf][0];
        const uint16_t* dtt = lds_t[buf][1];
        const uint32_t a0 = res_a0 + (uint32_t)buf * (2u * TE * 2u), a1 = a0 + (res_a1 - res_a0);
        // Elements that a mask may hide this step: the causal diagonal, and keys past the
        // sequence end or outside the key window (queries past the chunk end have LSE =
        // +inf, so their P is 0 already).  Element r is visible iff c(r) >= thr, with
        // c(r) = 8 (r / 4) + r % 4 its query less 4 hl.
        const bool fix = (CAUSAL && tile_pos0 < wkey0_u + 31) || wave_masked_u;
        const int thr = !key_ok ? (1 << 20) : CAUSAL ? key - tile_pos0 - 4 * hl : -(1 << 20);
        // the lane's 16 LSE / Delta values (element r: query 8 (r / 4) + 4 hl + r % 4)
        auto row16 = [&](const float* x, float (&out)[16]) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(x + 8 * i + 4 * hl);
#pragma unroll
            for (int j = 0; j < 4; ++j) out[4 * i + j] = v[j];
          }
        };
        auto opnd = [&](int i) -> u32x4 {
          if (i < NS) return tr_a(qtt, i);
          if (i < 2 * NS) return tr_a(dtt, i - NS);
          const int j = i & 15;  // (3) dO^T, (4) Q^T: block j / 2, k-step j % 2
          return lds16(((j & 1) ? a1 : a0) + (uint32_t)((i < 48 ? TE * 2 : 0) + (j >> 1) * 32 * kTq * 2));
        };
        static_assert(2 * NS == 32 && 4 * NB == 32, "64 products per step");
        f32x16 s, dp;
        float lv[16], dlv[16];
        u32x4 sp[2], sd[2];  // BF16 residues of P and dS (set when flag)
        uint32_t flag = 0;
        u32x4 ring[4];
        ring[0] = ring0[0];
        ring[1] = ring0[1];
        ring[2] = ring0[2];
        // product i of the stream: its A operand, with the read of product i + 3 issued
        auto next_a = [&](int i) {
          if (i + 3 < 64) ring[(i + 3) & 3] = opnd(i + 3);
          return ring[i & 3];
        };
        // (1) S; the next tile's copies every other k-step
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const u32x4 A = next_a(i);
          if ((i & 1) == 0) copy_one(i >> 1);
          if (i == 0)
            s = mfma32_v0(A, kf[0]);
          else
            mfma32_v(s, A, kf[i]);
          if (i == 12) row16(lds_st[buf], lv);
          __builtin_amdgcn_sched_barrier(0);
        }
        // (2) dP; P two elements per product, then the mask, the packing, the residue decision
#pragma unroll
        for (int st = 0; st < 16; ++st) {
          const u32x4 A = next_a(16 + st);
          if (st == 0) {
            dp = mfma32_v0(A, vf[0]);
            xdl_fence(s);
          } else {
            mfma32_v(dp, A, vf[st]);
          }
          if (st >= 1 && st <= 8) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const int r = 2 * (st - 1) + e;
              s[r] = exp2f_fast(fmaf(s[r], a.scale_log2, -lv[r]));
            }
          }
          if (st == 9 && fix) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[r] = (8 * (r >> 2) + (r & 3) >= thr) ? s[r] : 0.f;
          }
          if (st == 10) {
            pp[0] = to_bf16x8(s, 0);
            pp[1] = to_bf16x8(s, 8);
          }
          if (st == 11) flag = wave_has_large_p(s);
          if (st == 12) row16(lds_st[buf] + kTq, dlv);
          if (st == 13 && flag) {
            sp[0] = residue_bf16x8(s, pp[0], 0);
            sp[1] = residue_bf16x8(s, pp[1], 8);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        // (3) dV^T += dO^T P; dS two elements per product, its packing and residues
        residue_half<NB, TE * 2>(dvt, a0, a1, sp, flag);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const u32x4 A = next_a(32 + j);
          dvt[j >> 1] = mfma32(A, pp[j & 1], dvt[j >> 1]);
          if (j == 0) xdl_fence(dp);
          if (j >= 1 && j <= 8) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const int r = 2 * (j - 1) + e;
              dp[r] = s[r] * (dp[r] - dlv[r]);
            }
          }
          if (j == 9) {
            pd[0] = to_bf16x8(dp, 0);
            pd[1] = to_bf16x8(dp, 8);
          }
          if (j == 10 && flag) {
            sd[0] = residue_bf16x8(dp, pd[0], 0);
            sd[1] = residue_bf16x8(dp, pd[1], 8);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        // (4) dK^T += Q^T dS
        residue_half<NB, 0>(dkt, a0, a1, sd, flag);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const u32x4 A = next_a(48 + j);
          dkt[j >> 1] = mfma32(A, pd[j & 1], dkt[j >> 1]);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        // S and dP of this tile; each A operand is read one k-step ahead.
        f32x16 s = {}, dp = {};
        {
          const uint16_t* qtt = lds_t[buf][0];
          const uint16_t* dtt = lds_t[buf][1];
          u32x4 fq = tr_a(qtt, 0), fd = tr_a(dtt, 0);
#pragma unroll
          for (int st = 0; st < NS; ++st) {
            if (SPREAD && (st & 1) == 0) copy_one(st >> 1);
            u32x4 nq_ = fq, nd_ = fd;
            if (st + 1 < NS) {
              nq_ = tr_a(qtt, st + 1);
              nd_ = tr_a(dtt, st + 1);
            }
            if (st == 0) {
              s = mfma32_v0(fq, kf[0]);
              dp = mfma32_v0(fd, vf[0]);
            } else {
              mfma32_v(s, fq, kf[st]);
              mfma32_v(dp, fd, vf[st]);
            }
            fq = nq_;
            fd = nd_;
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        xdl_fence2(s, dp);

        // Softmax of this tile, between the dV/dK products of the previous one, without a
        // mask; on the steps that need one (the causal diagonal, keys past the sequence
        // end or outside the key window: element r is visible iff c(r) >= thr, c(r) =
        // 8 (r / 4) + r % 4 its query less 4 hl) the hidden elements' P and dS are set to
        // 0 afterwards.  Queries past the chunk end have LSE = +inf: P = 0 already.
        const bool fix = (CAUSAL && tile_pos0 < wkey0_u + 31) || wave_masked_u;
        const int thr = !key_ok ? (1 << 20) : CAUSAL ? key - tile_pos0 - 4 * hl : -(1 << 20);
        const float* lse = lds_st[buf];
        const float* dl = lds_st[buf] + kTq;
        auto sm_block = [&](int blk) {
          softmax_part<EPB, false, CAUSAL, BIAS>(s, dp, blk * EPB, lse, dl, hl, a.scale_log2, key, key_ok,
                                                 nq, tile_pos0, bias_cur);
        };
        if (have_prev) {
          residue(pbuf, rp, rd, res_prev);
          dvdk(pbuf, pp, pd, sm_block);
        } else {
#pragma unroll
          for (int blk = 0; blk < NB; ++blk) sm_block(blk);
        }
        if (fix) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const bool vis = 8 * (r >> 2) + (r & 3) >= thr;
            s[r] = vis ? s[r] : 0.f;
            dp[r] = vis ? dp[r] : 0.f;
          }
        }
        // k-step t of the dV/dK products = accumulator rows 8t .. 8t+7 of each lane
        pp[0] = to_bf16x8(s, 0);
        pp[1] = to_bf16x8(s, 8);
        pd[0] = to_bf16x8(dp, 0);
        pd[1] = to_bf16x8(dp, 8);
        res_cur = wave_has_large_p(s);
        if (res_cur) {  // kept for the next step, with pp / pd
          rp[0] = residue_bf16x8(s, pp[0], 0);
          rp[1] = residue_bf16x8(s, pp[1], 8);
          rd[0] = residue_bf16x8(dp, pd[0], 0);
          rd[1] = residue_bf16x8(dp, pd[1], 8);
        }
      }

      wait_vm_all();
      __syncthreads();
      // Stored dS for the dQ product: block (tile, head, key block of this wave), key row
      // n, granules 2 e + hl (pd[e]).  Only blocks with a visible pair are stored; they are
      // the blocks that dQ reads.  Issued after the step's wait for its copies, so that the
      // stores complete during the next step instead of extending this one.
      if (a.ds_out != nullptr && wkey0_u < L && (!CAUSAL || wkey0_u <= tile_pos0 + nq - 1)) {
        uint16_t* dst = a.ds_out + (cur.ds + (wkey0_u >> 5)) * 1024 + n * 32 + hl * 8;
        // streaming stores: dS is read back only by the dQ product, long after
        __builtin_nontemporal_store(pd[0], reinterpret_cast<u32x4*>(dst));
        __builtin_nontemporal_store(pd[1], reinterpret_cast<u32x4*>(dst + 16));
      }
      cur = nxt;
      if (BIAS) {
#pragma unroll
        for (int r = 0; r < 16; ++r) bias_cur[r] = bias_nxt[r];
      }
      have = have_next;
      have_prev = true;
      res_prev = res_cur;
      pbuf = buf;
      buf = nbuf;
      if constexpr (SPLIT) {  // (after the last step: reads of a re-copied tile, unused)
#pragma unroll
        for (int k = 0; k < 3; ++k) ring0[k] = s_opnd(lds_t[buf][0], k);
      }
    }
    if (PIPE && have_prev) {
      residue(pbuf, rp, rd, res_prev);
      dvdk(pbuf, pp, pd, nop);
    }

    if (!key_ok) continue;  // (no barrier follows in this pass)
    // element r of block blk is dimension 32 blk + 8 (r / 4) + 4 hl + r % 4
    const int64_t off = (koff + key) * kv_stride + (int64_t)g * D + hl * 4;
    if (a.accumulate) {
#pragma unroll
      for (int blk = 0; blk < NB; ++blk)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t o = off + blk * 32 + i * 8;
          const u32x2 ok = ld8(a.dk + o), ov = ld8(a.dv + o);
          const float k0 = fmaf(dkt[blk][4 * i], a.scale, bf16_lo(ok[0]));
          const float k1 = fmaf(dkt[blk][4 * i + 1], a.scale, bf16_hi(ok[0]));
          const float k2 = fmaf(dkt[blk][4 * i + 2], a.scale, bf16_lo(ok[1]));
          const float k3 = fmaf(dkt[blk][4 * i + 3], a.scale, bf16_hi(ok[1]));
          st8(a.dk + o, u32x2{pack_bf16x2(k0, k1), pack_bf16x2(k2, k3)});
          st8(a.dv + o, u32x2{pack_bf16x2(dvt[blk][4 * i] + bf16_lo(ov[0]), dvt[blk][4 * i + 1] + bf16_hi(ov[0])),
                              pack_bf16x2(dvt[blk][4 * i + 2] + bf16_lo(ov[1]), dvt[blk][4 * i + 3] + bf16_hi(ov[1]))});
        }
    } else {
#pragma unroll
      for (int blk = 0; blk < NB; ++blk)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t o = off + blk * 32 + i * 8;
          st8(a.dk + o, u32x2{pack_bf16x2(dkt[blk][4 * i] * a.scale, dkt[blk][4 * i + 1] * a.scale),
                              pack_bf16x2(dkt[blk][4 * i + 2] * a.scale, dkt[blk][4 * i + 3] * a.scale)});
          st8(a.dv + o, u32x2{pack_bf16x2(dvt[blk][4 * i], dvt[blk][4 * i + 1]),
                              pack_bf16x2(dvt[blk][4 * i + 2], dvt[blk][4 * i + 3])});
        }
    }
  }
}

hipError_t launch_dkdv(const AttnArgs& a, int D, bool causal, bool bias, dim3 grid, hipStream_t s) {
  constexpr int kThreads = kKvThreads;
  CPATTN_BWD_DISPATCH(dkdv_kernel)
}

}  // namespace cpattn
