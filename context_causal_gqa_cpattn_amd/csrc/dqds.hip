// dQ from stored dS: the backward's last product when the workspace holds dS.
//
// Page "Optimize context parallel attention layouts and gradient accumulation":
// "Changes" (GQA, causal THD with physical offsets) and "Related optimization work"
// (the backward is where the providers differ).
//
// dK/dV already forms dS = P (dP - Delta) for every (32-key block, 32-query tile, query
// head) that has a visible pair, and in this mode stores it in BF16, the precision in
// which both dK and dQ multiply it.  dQ = scale dS K is then a product over the visible
// key blocks alone: S, P and dP are not formed a second time.
//
// dS block (2 KB, written by dK/dV): 32 key rows of 64 bytes; granule v = 2 e + hl of key
// row n holds queries 16 e + 8 (i / 4) + 4 hl + i % 4, i = 0..7 (the order in which a
// 32x32 accumulator lane holds its rows).  Block kb of (tile qt of chunk c, head h) is
// block ds_block0(ds_tab[c], ceil(K_c / 32), qt, h, hq) + kb of the dS area (the chunk's
// blocks in [tile][head][key block] order, K_c the keys its last row sees).
//
// With a key window [kv_lo, kv_hi) only the window's key blocks are multiplied, and
// with dq_accumulate the result is added to the existing BF16 dQ (one rounding): a ring
// step's dQ share from the dS that its window's dK/dV stored.
//
// Workgroup = (chunk, block of positions, hpw query heads that share one KV head) with
// four slots of (head, two 32-query tiles).  For D >= 128 two waves share a slot, each
// keeping half of dQ^T (D/2 x 64 queries, fp32) in registers, two waves per SIMD (one
// wave's copies and LDS reads issue while the other's MFMAs run); for D <= 64 one wave
// per slot.  Each 32-key step, the K tile (32 x D, kind-0 swizzle) and the slots' dS
// blocks are copied into LDS three steps ahead (four stages: the dS stream comes from
// HBM, read once, with the non-temporal hint so that the K tiles stay in L2); the copy
// instructions are spread between the step's MFMAs rather than issued
// together after the barrier, where all waves would queue on the address unit at once.
// With 32x32x16 MFMAs:
//   dQ^T += K^T dS^T    A = K^T by transposing reads of the K tile (as V^T in the forward),
//                       B = dS^T by transposing reads of the dS block.
#include "common.h"
#include "launch.h"

namespace cpattn {

namespace {

constexpr int kStages = 4;
constexpr int kBlk = 32;              // keys per dS block and per step
constexpr int kBlkElems = 32 * 32;    // BF16 elements of a dS block
constexpr int kSlots = 4;             // (head, two-tile) slots per workgroup

// Waves per workgroup: each slot's D columns are split over kSplit waves, two waves per
// SIMD for D >= 128 (128 accumulation registers each), one for D <= 64.
template <int D>
struct DsCfg {
  static constexpr int kSplit = D >= 128 ? 2 : 1;
  static constexpr int kWaves = kSlots * kSplit;
  static constexpr int kThreads = kWaves * 64;
};

// Lane part of the transposing reads that give the B operand dS^T of k-step st (16 keys
// x 32 queries): lane l holds query l % 32 and keys 16 st + 8 (e / 4) + 4 (l / 32) + e % 4
// for e = 0..7, the contracted order of the K^T operand.  In 16-lane group G of a read,
// source lane 4 j + u gives the four queries of unit 4 (G % 2) + u at key row 4 (G / 2) + j
// (+ 8 for the second read); unit U (queries 4 U .. 4 U + 3) is half (U / 2) % 2 of
// granule 2 (U / 4) + U % 2.  The 32 lanes of one pass touch four key rows x four
// granules, sixteen distinct bank groups.
__device__ __forceinline__ int ds_tr_off(int lane) {
  const int i = lane & 15, G = lane >> 4;
  const int j = i >> 2, u = i & 3;
  return (4 * (G >> 1) + j) * 32 + (2 * (G & 1) + (u & 1)) * 8 + (u >> 1) * 4;
}

}  // namespace

template <int D, bool CAUSAL>
__global__ __launch_bounds__(DsCfg<D>::kThreads) void dq_ds_kernel(const AttnArgs a) {
  constexpr int kSplit = DsCfg<D>::kSplit;
  constexpr int kWaves = DsCfg<D>::kWaves;
  constexpr int NDB = D / 32 / kSplit;                 // 32-row blocks of dQ^T per wave
  // K-tile copy instructions (1 KB each) per tile and per wave.  At D = 32 the 2 KB tile is
  // two instructions for four waves: waves w and w + 2 copy the same kilobyte (identical
  // bytes to the same place), so that every wave issues the same number of copies.
  constexpr int KTI = kBlk * D * 2 / 1024;
  constexpr int KI = KTI >= kWaves ? KTI / kWaves : 1;
  constexpr int PER = KI + 4 / kSplit;                 // copy instructions per wave per step
  static_assert(KTI % kWaves == 0 || kWaves % KTI == 0, "K tile split evenly over the waves");
  static_assert(2 * PER < 64, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) uint16_t lds_k[kStages][kBlk * D];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_s[kStages][kSlots * 2 * kBlkElems];

  if (*a.dev_err) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = rfl(tid >> 6);  // wave-uniform, so that everything derived from it is scalar
  const int slot = wave / kSplit, part = wave % kSplit;
  const int logical = xcd_group_order(blockIdx.x, gridDim.x / a.blocks_per_chunk, a.blocks_per_chunk, a.hq / a.hpw);
  const int n_hg = a.hq / a.hpw;
  const int pb = logical % a.blocks_per_chunk;
  const int rest = logical / a.blocks_per_chunk;
  const int hg = rest % n_hg;
  const int c = rest / n_hg;
  const Chunk ch = load_chunk_uniform(a.chunks, c);
  const int wg_pos = 64 * (kSlots / a.hpw);  // positions per workgroup
  const int wg_row0 = pb * wg_pos;
  if (wg_row0 >= ch.len) return;  // uniform over the workgroup, before any barrier
  const int h = hg * a.hpw + (slot % a.hpw);
  const int kvh = rfl(h / a.group);
  const int row0 = wg_row0 + (slot / a.hpw) * 64;  // first chunk row of this slot (a tile start)
  const int L = rfl(a.seq_lens[ch.seq]);
  const int64_t koff = rfl(a.seq_offsets[ch.seq]);
  const int wg_last_pos = ch.pos0 + min(ch.len, wg_row0 + wg_pos) - 1;
  // Key blocks [kb_first, n_steps): those with a visible key, within the key window
  // [kv_lo, kv_hi) (the whole sequence without one).
  const int kv_end = min(min(L, CAUSAL ? wg_last_pos + 1 : L), a.kv_hi);
  const int kb_first = a.kv_lo / kBlk;
  const int n_steps = (kv_end + kBlk - 1) / kBlk;

  // The slot's two tiles: rows, key blocks with a visible pair, first dS block.
  const int kbc = ds_chunk_kb(ch, L, CAUSAL);
  const int64_t tab = (int64_t)(((uint64_t)rfl((int)(a.ds_tab[c] >> 32)) << 32) | (uint32_t)rfl((int)a.ds_tab[c]));
  int nq[2], nkb[2];
  const uint16_t* dsrc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = row0 + 32 * i;
    nq[i] = max(0, min(32, ch.len - r));
    const int last = ch.pos0 + r + nq[i] - 1;
    nkb[i] = nq[i] > 0 ? (min(min(L, CAUSAL ? last + 1 : L), a.kv_hi) + kBlk - 1) / kBlk : 0;
    dsrc[i] = a.ds_zero;
    if (nq[i] > 0)
      dsrc[i] = a.ds + ds_block0(tab, kbc, r / 32, h, a.hq) * kBlkElems;
  }

  const int64_t kv_stride = a.kv_pitch * D;
  const uint16_t* kbase = a.k + koff * kv_stride + (int64_t)kvh * D;
  // Copy instruction p (0 <= p < PER) of this wave for step kb into its stage:
  // the K tile (rows past L repeat the last key), then the slot's dS blocks (with two
  // waves per slot, wave `part` copies tile `part`).  For a block that the tile does not
  // use (no visible pair: dK/dV did not store it) a block of zeros is copied, so that
  // the products need no mask and every wave issues PER copies per step; steps past the
  // last re-copy the last step into a free stage.
  const int wu = wave;
  const uint32_t rs_bytes = (uint32_t)(kv_stride * 2);
  // The lane's source offset of K-tile copy p (row * row stride + swizzled granule; the
  // granule is below the row stride, so clamping the row is a min of the offsets), and
  // the granule part alone.
  constexpr int KG = D / 8, KRPI = 64 / KG;
  uint32_t kroff[KI], kgran[KI];
#pragma unroll
  for (int p = 0; p < KI; ++p) {
    const int i = KTI >= kWaves ? wu + kWaves * p : wu % KTI;  // instruction of the tile
    const int r = i * KRPI + lane / KG;                        // tile row of this lane
    kgran[p] = (uint32_t)(((lane % KG) ^ swz<D, 0>(r)) * 16);
    kroff[p] = (uint32_t)r * rs_bytes + kgran[p];
  }
  // Stage of step kb: (kb - kb_first) mod kStages (the loop below is unrolled over the
  // stages, so that LDS addresses are constants).
  // LDS addresses of stage 0 (converted once; a stage's are constants further on) and the
  // dS sources as wave-uniform byte pointers (a block past a tile's visible ones is taken
  // from the zero block by a select, not a branch).
  const uint32_t lk0 = lds_addr(lds_k[0]);
  const uint32_t ls0 = lds_addr(lds_s[0]) + (uint32_t)(slot * 2 * kBlkElems * 2);
  const char* const zsrc = uniform_ptr(a.ds_zero);
  const char* const dsrc_b[2] = {uniform_ptr(dsrc[0]), uniform_ptr(dsrc[1])};
  // LDS destinations as a wave-uniform base plus a constant (folded into the M0 write):
  // K tile instruction i = wave + kWaves p (or wave mod KTI), dS block ti of the slot
  const uint32_t lkw = lk0 + (uint32_t)((KTI >= kWaves ? wu : wu % KTI) * 1024);
  const uint32_t lsw = ls0 + (uint32_t)(kSplit == 2 ? part * kBlkElems * 2 : 0);
  // Source offsets without a multiply by a clamped step index: step kb's K rows start
  // kb * k_stride bytes after kbase; steps past the last re-copy the last one, and only
  // the last step can have fewer than kBlk valid keys.
  const int64_t k_stride = (int64_t)kBlk * kv_stride * 2;
  const int kb_last = max(n_steps - 1, 0);
  const char* const kbase_b = uniform_ptr(kbase);
  const uint32_t klast_full = (uint32_t)(kBlk - 1) * rs_bytes;
  const uint32_t klast_tail = (uint32_t)min(L - kb_last * kBlk - 1, kBlk - 1) * rs_bytes;
  auto issue_one = [&](int kb_req, int p, int sb) {
    const bool past = kb_req >= kb_last;
    const int kb = past ? kb_last : kb_req;
    if (p < KI) {
      const uint32_t last = past ? klast_tail : klast_full;
      const char* b = kbase_b + (past ? (int64_t)kb_last * k_stride : (int64_t)kb_req * k_stride);
      dma16_add(b, min(kroff[p], last + kgran[p]), lkw,
                (uint32_t)(sb * kBlk * D * 2 + (KTI >= kWaves ? kWaves * p : 0) * 1024));
    } else {
      const int q = p - KI;
      const int ti = kSplit == 2 ? part : (q >> 1);
      const int half = q & 1;
      const uint64_t blk = (uint64_t)(uintptr_t)(dsrc_b[ti] + (int64_t)kb * (kBlkElems * 2));
      const uint64_t m = 0 - (uint64_t)(kb < nkb[ti]);  // all ones when the block is stored
      const char* src = (const char*)(uintptr_t)((blk & m) | ((uint64_t)(uintptr_t)zsrc & ~m));
      dma16_nt_add(src + half * 1024, (uint32_t)lane * 16u, lsw,
                   (uint32_t)(sb * kSlots * 2 * kBlkElems * 2 + (kSplit == 2 ? 0 : (q >> 1)) * kBlkElems * 2 +
                              half * 1024));
    }
  };
  f32x16 acc[2][NDB];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NDB; ++j) acc[i][j] = f32x16{};
  // Transposing-read offsets of this wave's K^T blocks db = part * NDB + j.
  int klo[NDB], khi[NDB];
  {
    const TrOffsets<D> tro(lane);
#pragma unroll
    for (int j = 0; j < NDB; ++j) {
      const int db = part * NDB + j;
      klo[j] = tro.lo(db & 3) + (db >> 2) * 128;
      khi[j] = klo[j] + tro.hi_delta;
    }
  }
  // LDS reads as lane pointers plus constants (stage, k-step, block).
  using lds_p = __attribute__((address_space(3))) uint16_t*;
  lds_p klp[NDB], khp[NDB];
#pragma unroll
  for (int j = 0; j < NDB; ++j) {
    klp[j] = CPATTN_LDS(uint16_t, lds_k[0]) + klo[j];
    khp[j] = CPATTN_LDS(uint16_t, lds_k[0]) + khi[j];
  }
  auto kfrag = [&](int sb, int st, int j) {
    const int o = sb * kBlk * D + st * 16 * D;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<__attribute__((address_space(3))) v4i16*>(klp[j] + o));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<__attribute__((address_space(3))) v4i16*>(khp[j] + o));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return u32x4{l2[0], l2[1], h2[0], h2[1]};
  };
  // dS^T fragment of tile i, k-step st, stage sb
  const lds_p dsp = CPATTN_LDS(uint16_t, lds_s[0]) + (slot * 2) * kBlkElems + ds_tr_off(lane);
  auto dsfrag = [&](int sb, int i, int st) {
    const int o = sb * kSlots * 2 * kBlkElems + i * kBlkElems + st * 16 * 32;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<__attribute__((address_space(3))) v4i16*>(dsp + o));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<__attribute__((address_space(3))) v4i16*>(dsp + o + 8 * 32));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return u32x4{l2[0], l2[1], h2[0], h2[1]};
  };

  if (n_steps > kb_first) {
#pragma unroll
    for (int s = 0; s < kStages - 1; ++s)
#pragma unroll
      for (int p = 0; p < PER; ++p) issue_one(kb_first + s, p, s);
  }

  for (int kb0 = kb_first; kb0 < n_steps; kb0 += kStages)
#pragma unroll
  for (int sb = 0; sb < kStages; ++sb) {
    const int kb = kb0 + sb;
    if (kb >= n_steps) break;
    wait_vm<(kStages - 2) * PER>();  // stage sb has landed (later stages may be in flight)
    __syncthreads();                 // stage sb is in LDS for every wave; the previous one is free

    // A tile without a visible pair in this block multiplies the zero block copied in
    // its place.  The copies of step kb + kStages - 1 are spread between the products.
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const u32x4 b0 = dsfrag(sb, 0, st), b1 = dsfrag(sb, 1, st);
      u32x4 ka = kfrag(sb, st, 0);
#pragma unroll
      for (int j = 0; j < NDB; ++j) {
        const int it = st * NDB + j;
#pragma unroll
        for (int p = 0; p < PER; ++p)
          if (p * 2 * NDB / PER == it) issue_one(kb + kStages - 1, p, (sb + kStages - 1) % kStages);
        u32x4 nk = ka;
        if (j + 1 < NDB) nk = kfrag(sb, st, j + 1);
        acc[0][j] = mfma32(ka, b0, acc[0][j]);
        acc[1][j] = mfma32(ka, b1, acc[1][j]);
        ka = nk;
      }
    }
  }
  wait_vm<0>();  // no copy into LDS outlives the workgroup

  // element r of block j is dimension 32 (part NDB + j) + 8 (r / 4) + 4 (lane / 32) + r % 4
  // of query lane % 32
  const int col = lane & 31;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const bool ok = col < nq[i];
    const int64_t qrow = (int64_t)ch.q_row + row0 + 32 * i + (ok ? col : 0);
    uint16_t* op = a.dq + (qrow * a.q_pitch + h) * D + part * NDB * 32 + (lane >> 5) * 4;
#pragma unroll
    for (int j = 0; j < NDB; ++j)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        float r4[4] = {acc[i][j][4 * i4] * a.scale, acc[i][j][4 * i4 + 1] * a.scale,
                       acc[i][j][4 * i4 + 2] * a.scale, acc[i][j][4 * i4 + 3] * a.scale};
        if (a.dq_accumulate && ok) {  // add to the existing BF16 values, one rounding
          const u32x2 old = ld8(op + j * 32 + i4 * 8);
          r4[0] += bf16_lo(old[0]);
          r4[1] += bf16_hi(old[0]);
          r4[2] += bf16_lo(old[1]);
          r4[3] += bf16_hi(old[1]);
        }
        const u32x2 w{pack_bf16x2(r4[0], r4[1]), pack_bf16x2(r4[2], r4[3])};
        if (ok) st8(op + j * 32 + i4 * 8, w);
        __builtin_amdgcn_sched_barrier(0);  // one block's registers at a time
      }
  }
}

hipError_t launch_dq_ds(const AttnArgs& a, int D, bool causal, dim3 grid, hipStream_t s) {
  if (causal) {
    switch (D) {
      case 32: hipLaunchKernelGGL((dq_ds_kernel<32, true>), grid, dim3(DsCfg<32>::kThreads), 0, s, a); break;
      case 64: hipLaunchKernelGGL((dq_ds_kernel<64, true>), grid, dim3(DsCfg<64>::kThreads), 0, s, a); break;
      case 128: hipLaunchKernelGGL((dq_ds_kernel<128, true>), grid, dim3(DsCfg<128>::kThreads), 0, s, a); break;
      case 256: hipLaunchKernelGGL((dq_ds_kernel<256, true>), grid, dim3(DsCfg<256>::kThreads), 0, s, a); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (D) {
      case 32: hipLaunchKernelGGL((dq_ds_kernel<32, false>), grid, dim3(DsCfg<32>::kThreads), 0, s, a); break;
      case 64: hipLaunchKernelGGL((dq_ds_kernel<64, false>), grid, dim3(DsCfg<64>::kThreads), 0, s, a); break;
      case 128: hipLaunchKernelGGL((dq_ds_kernel<128, false>), grid, dim3(DsCfg<128>::kThreads), 0, s, a); break;
      case 256: hipLaunchKernelGGL((dq_ds_kernel<256, false>), grid, dim3(DsCfg<256>::kThreads), 0, s, a); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

}  // namespace cpattn
