// Forward kernel: blockwise causal GQA attention over one rank's chunk map.
//
// Page "Optimize context parallel attention layouts and gradient accumulation",
// "Description"/"Changes": causal THD attention with physical offsets, GQA,
// head dims 128/256, and the softmax statistics (LSE) kept for the backward.
//
// Work decomposition
//   workgroup = 4 waves = (one chunk, one block of positions, `hpw` query heads
//   that share one KV head).  Each wave owns 32 query rows of one head and keeps
//   its Q tile in registers for the whole KV loop.  K and V tiles of 64 keys go
//   HBM -> LDS by direct LDS DMA (no register staging), double-buffered so the
//   next tile streams in while the current one is computed, and are shared by
//   the four waves (GQA sharing).
//
// Transposed formulation (no cross-lane movement for P):
//   S^T = K Q^T      A = K rows from LDS, B = Q^T from registers
//   O^T += V^T P^T   A = V^T read from the natural-layout V tile with transposing
//                    LDS reads, B = P^T made in-lane from the S^T accumulator
//   Every lane owns one query (a column of S^T and O^T).  The online softmax
//   (running max m, running sum l, fp32, base 2 with log2(e)*scale folded in)
//   rescales O only when the running max grows by more than 2^8, so most tiles
//   skip the rescale; O/l is unchanged by that choice of reference max.
#include "common.h"
#include "launch.h"

namespace cpattn {

// Keys per K/V tile, waves per workgroup and K/V buffers.  D <= 128: 64-key tiles, four
// waves, double-buffered (the tiles leave room for a second workgroup per CU).  D = 256:
// 32-key tiles and eight waves, two per SIMD: a 64-key tile pair (128 KB of LDS) would
// leave one wave per SIMD, and a tile now serves 256 query rows instead of 128, half the
// copied bytes per FLOP.  A 32-key tile is computed in about a microsecond, less than
// the latency of its copy from L2 or HBM, so the tiles are copied AHEAD = STAGES - 1
// tiles ahead (three 32 KB stages: 3% faster than two on the 64 x 8192 D256 rank share;
// a fourth gains nothing).
template <int D>
struct FwdShape {
  static constexpr int BN = D == 256 ? 32 : 64;
  static constexpr int NW = D == 256 ? 8 : 4;
  static constexpr int STAGES = D == 256 ? 3 : 2;
  static constexpr int AHEAD = STAGES - 1;
  static constexpr bool PAIR = D <= 128;  // with causal masking: two position blocks each
};

// Scores of one 64-key tile in base 2 (+ bias), masked when MASK (keys outside
// [lo, hi), and past the query position when causal); returns the lane max (four
// independent running maxima, so the chain is a quarter as long).  Without a bias the
// scores stay unscaled (the positive scale is applied to the max and inside the
// exponential's FMA); with one they are scaled and biased here.
// Element r of block kb is key key0 + 32 kb + 8 (r/4) + 4 kg + r%4.
// The lane's bias values of the tile at key0 (element r of block kb: key
// key0 + 32 kb + 8 (r/4) + 4 kg + r%4), as groups of four; keys past L read as 0.
__device__ __forceinline__ void load_bias_tile(f32x4 (&bv)[8], const float* bias_row, int key0, int L,
                                               int kg, int bias_len) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)  // bias only with 64-key tiles (D <= 128)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kbi = key0 + kb * 32 + i * 8 + kg * 4;
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (kbi + 3 < L && (bias_len & 3) == 0)
        v = *reinterpret_cast<const f32x4*>(bias_row + kbi);
      else {
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = (kbi + j < L) ? bias_row[kbi + j] : 0.f;
      }
      bv[kb * 4 + i] = v;
    }
}

template <bool BIAS, bool MASK, bool CAUSAL, int NKB>
__device__ __forceinline__ void scale_tile(f32x16 (&s)[NKB], float c, const f32x4 (&btile)[8], int key0,
                                           int lo, int hi, int qpos, int kg, float& mx) {
  float mj[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kbi = key0 + kb * 32 + i * 8 + kg * 4;
      const f32x4 bv = btile[kb * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float x = s[kb][i * 4 + j];
        if (BIAS) x = fmaf(bv[j], kLog2e, x * c);
        if (MASK) {
          const int key = kbi + j;
          x = ((key >= lo) && (key < hi) && (!CAUSAL || key <= qpos)) ? x : -INFINITY;
        }
        s[kb][i * 4 + j] = x;
        mj[j] = fmaxf(mj[j], x);
      }
    }
  mx = fmaxf(fmaxf(mx, fmaxf(mj[0], mj[1])), fmaxf(mj[2], mj[3]));
}

template <int D, bool CAUSAL, bool BIAS>
__global__ __launch_bounds__(FwdShape<D>::NW * 64) void attn_fwd_kernel(const AttnArgs a) {
  constexpr int kBN = FwdShape<D>::BN;  // keys per K/V tile
  constexpr int NW = FwdShape<D>::NW;   // waves per workgroup
  constexpr int NKB = kBN / 32;         // 32-key blocks of S^T
  constexpr int NST = D / 16;  // 16-wide k-steps over the head dim
  constexpr int NDB = D / 32;  // 32-row blocks of O^T
  constexpr int STAGES = FwdShape<D>::STAGES;
  constexpr int AHEAD = FwdShape<D>::AHEAD;  // tiles copied ahead of the one computed
  static_assert(AHEAD >= 1, "at least one tile ahead");
  static_assert(!BIAS || kBN == 64, "bias tiles are 64 keys");
  // With a bias each tile's bias loads are issued before its copies, and the tile-end
  // wait below counts on the copies being the only newer vector-memory operations.
  static_assert(!BIAS || AHEAD == 1, "bias tiles double-buffered");
  __shared__ __attribute__((aligned(1024))) uint16_t lds_k[STAGES][kBN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_v[STAGES][kBN * D];

  if (*a.dev_err) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kg = lane >> 5, col = lane & 31;

  const int logical = xcd_group_order(blockIdx.x, gridDim.x / a.blocks_per_chunk, a.blocks_per_chunk, a.hq / a.hpw);
  const int n_hg = a.hq / a.hpw;
  const int pslot = logical % a.blocks_per_chunk;
  const int rest = logical / a.blocks_per_chunk;
  const int hg = rest % n_hg;
  const int c = rest / n_hg;
  const Chunk ch = load_chunk_uniform(a.chunks, c);
  const int segs = NW / a.hpw;
  // With causal masking and D <= 128, in a chunk whose last block sees more than twice
  // the keys of its first (one that starts near its sequence's start), workgroup pslot
  // < nb / 2 takes position blocks pslot and nb - 1 - pslot (nb = the chunk's blocks),
  // one after the other, and the other workgroups of the chunk exit: a block's work
  // grows with its position, and the pairs even it out.  (At D = 256 the registers the
  // second pass would hold are not there.)
  constexpr bool PAIR = FwdShape<D>::PAIR && CAUSAL;
  const int nb = (ch.len + 32 * segs - 1) / (32 * segs);
  const bool pair = PAIR && ch.pos0 + ch.len > 2 * (ch.pos0 + 32 * segs);
  for (int pass = 0; pass < (PAIR ? 2 : 1); ++pass) {
    const int pb = !pair ? (pass == 0 ? pslot : -1)
                         : pass == 0 ? (pslot < (nb + 1) / 2 ? pslot : -1)
                                     : (pslot < nb / 2 ? nb - 1 - pslot : -1);
    if (pb < 0) continue;
    if (pass > 0) __syncthreads();  // the first pass's last reads of the K/V buffers are done
    const int wg_row0 = pb * 32 * segs;
    if (wg_row0 >= ch.len) continue;
    const int h = hg * a.hpw + (wave % a.hpw);
    const int g = rfl(hg * a.hpw / a.group);  // hpw divides the group: one KV head per workgroup
    const int row0 = wg_row0 + (wave / a.hpw) * 32;  // first chunk row of this wave
    const int nrows = max(0, min(32, ch.len - row0));
    const int L = rfl(a.seq_lens[ch.seq]);
    const int64_t koff = rfl(a.seq_offsets[ch.seq]);

    const int wg_last_pos = ch.pos0 + min(ch.len, wg_row0 + 32 * segs) - 1;
    // Keys [kv_lo, kv_end) are visible to some row of the workgroup: the key window
    // (the whole sequence without one) cut at the last position when causal.
    const int kv_lo = a.kv_lo;
    const int kv_hi = min(L, a.kv_hi);
    const int kv_end = min(CAUSAL ? min(L, wg_last_pos + 1) : L, kv_hi);
    const int t_first = kv_lo / kBN;                // first tile (absolute index)
    const int n_tiles = (kv_end + kBN - 1) / kBN;   // one past the last tile
    const int wave_first_pos = ch.pos0 + row0;
    const int wave_last_pos = wave_first_pos + nrows - 1;
    // A scalar copy for the per-tile mask decision, so that its two paths (vector work
    // only) are a scalar branch instead of an exec-mask if/else.
    const int wave_first_pos_u = rfl(wave_first_pos);
    const int qpos = wave_first_pos + col;  // this lane's query position

    // Q^T as B operand: lane holds query `col`, dims [16*st + 8*kg, +8).
    u32x4 qf[NST];
    {
      const uint16_t* qp = a.q + ((int64_t)(ch.q_row + row0 + col) * a.q_pitch + h) * D + kg * 8;
#pragma unroll
      for (int st = 0; st < NST; ++st)
        qf[st] = (col < nrows) ? ld16(qp + st * 16) : u32x4{0u, 0u, 0u, 0u};
    }

    // Without a bias the scale is folded in after the max (max(c s) = c max(s) for c > 0)
    // and into the FMA before each exponential; a negative scale is applied as |c| with Q
    // negated (exact in BF16), a zero one as a tiny positive one (every score 0 either way).
    const float c_eff = BIAS ? a.scale_log2 : fmaxf(fabsf(a.scale_log2), 1e-30f);
    if (!BIAS && a.scale_log2 < 0.f) {
#pragma unroll
      for (int st = 0; st < NST; ++st) qf[st] ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
    }

    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;

    // LDS operand reads as a lane pointer plus a constant (the tile loop is unrolled over
    // the K/V buffers, so the buffer, the k-step and the block are all offset-field
    // constants and a read costs no address arithmetic).
    //  K (A operand of S^T): row 32 kb + col, logical granule 2 st + kg, stored at granule
    //    g ^ swz(row); swz(row) < 16 and depends on the row mod 16, so kb and the granule's
    //    bit 4 (st >= 8) enter as constants: KN lane pointers for st mod 8.
    //  V^T (A operand of O^T): the tr_frag_at addresses, four lane parts lo(m) (m = db
    //    mod 4) and their second reads hi_delta further on.
    constexpr int KN = NST < 8 ? NST : 8;
    constexpr int TILE_BYTES = kBN * D * 2;
    using lds_cptr = const __attribute__((address_space(3))) char*;
    lds_cptr kp[KN];
#pragma unroll
    for (int j = 0; j < KN; ++j)
      kp[j] = CPATTN_LDS(const char, lds_k[0]) + (col * D + (((2 * j + kg) ^ swz<D>(col)) << 3)) * 2;
    constexpr int VM = TrOffsets<D>::NM;
    lds_cptr vlo[VM], vhi[VM];
    {
      const TrOffsets<D> tro(lane);
#pragma unroll
      for (int m = 0; m < VM; ++m) {
        vlo[m] = CPATTN_LDS(const char, lds_v[0]) + tro.lo(m) * 2;
        vhi[m] = vlo[m] + tro.hi_delta * 2;
      }
    }
    // K fragment of block kb, k-step st, buffer u
    auto kread = [&](int u, int st, int kb) -> u32x4 {
      return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
          kp[st & 7] + u * TILE_BYTES + (st >> 3) * 256 + kb * 64 * D);
    };
    // V^T fragment of rows [16 st, +16) and columns [32 db, +32), buffer u
    auto vread = [&](int u, int st, int db) -> u32x4 {
      const int off = u * TILE_BYTES + st * 32 * D + (db >> 2) * 256;
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          reinterpret_cast<__attribute__((address_space(3))) v4i16*>(const_cast<__attribute__((address_space(3))) char*>(vlo[db & 3] + off)));
      const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          reinterpret_cast<__attribute__((address_space(3))) v4i16*>(const_cast<__attribute__((address_space(3))) char*>(vhi[db & 3] + off)));
      const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
      return u32x4{l2[0], l2[1], h2[0], h2[1]};
    };

    // With a bias, each tile's bias values are loaded one tile ahead (their latency is
    // spent under the previous tile's products) and used after that tile's wait.
    const float* bias_row = nullptr;
    f32x4 bias_cur[8] = {}, bias_nxt[8] = {};
    if (BIAS) {
      bias_row = a.bias + ((int64_t)h * a.bias_len + min(qpos, a.bias_len - 1)) * a.bias_len;
      if (n_tiles > t_first) load_bias_tile(bias_cur, bias_row, t_first * kBN, L, kg, a.bias_len);
    }

    const int64_t kv_stride = a.kv_pitch * D;
    const uint16_t* kbase = a.k + koff * kv_stride + (int64_t)g * D;
    const uint16_t* vbase = a.v + koff * kv_stride + (int64_t)g * D;

    // Copies of tile t + STAGES - 1, one instruction at a time between the S^T products of
    // tile t: CPW per wave (K then V, CPW / 2 each), one every NST / CPW k-steps.  Copy p
    // of a tensor is tile instruction i = w + NW p, rows i RPI + lane / G (clamped to the
    // valid rows), swizzled granule of the row.  Tiles past the last re-copy the last one
    // into a free buffer, so that the loop has no branch and every wave issues CPW copies
    // per tile.
    constexpr int G = D / 8, RPI = 64 / G;
    constexpr int CPW = 2 * (kBN * G / 64 / NW);
    static_assert(CPW >= 2 && NST % CPW == 0, "copies spread evenly over the S^T k-steps");
    constexpr int CEVERY = NST / CPW;
    const int wu = __builtin_amdgcn_readfirstlane(wave);
    const int lane_row = lane / G;
    const uint32_t rs_bytes = (uint32_t)(kv_stride * 2);
    uint32_t gran[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) gran[e] = (uint32_t)(((lane % G) ^ swz<D>((wu + NW * e) * RPI + lane_row)) * 16);
    // the lane's source offset of copy pp of a tensor (row * row stride + granule; the
    // granule is below the row stride, so clamping the row is a min of the offsets)
    uint32_t roff[CPW / 2];
#pragma unroll
    for (int pp = 0; pp < CPW / 2; ++pp)
      roff[pp] = (uint32_t)((wu + NW * pp) * RPI + lane_row) * rs_bytes + gran[pp & 1];
    struct CopyStep {
      const char* bk;
      const char* bv;
      uint32_t lk, lv;
      uint32_t lim[2];  // offset of the last valid row's granule (clamp)
    };
    // Source offsets without a multiply per tile: tile t's K/V rows start tile_stride * t
    // bytes after kbase / vbase; tiles past the last re-copy the last one, and only the last
    // tile can have fewer than kBN valid rows.
    const int64_t tile_stride = (int64_t)kBN * kv_stride * 2;
    const int64_t last_off = (int64_t)max(n_tiles - 1, 0) * tile_stride;
    const uint32_t last_full = (uint32_t)(kBN - 1) * rs_bytes;
    const uint32_t last_tail = (uint32_t)min(L - max(n_tiles - 1, 0) * kBN - 1, kBN - 1) * rs_bytes;
    const char* const kbase_b = uniform_ptr(kbase);
    const char* const vbase_b = uniform_ptr(vbase);
    auto copy_step = [&](int t_next, int buf_next) {
      const bool past = t_next >= n_tiles - 1;  // the last tile (or past it: the last again)
      const int64_t off = past ? last_off : (int64_t)t_next * tile_stride;
      CopyStep c;
      c.bk = kbase_b + off;
      c.bv = vbase_b + off;
      c.lk = lds_addr(lds_k[buf_next]) + (uint32_t)wu * 1024u;  // this wave's first instruction
      c.lv = lds_addr(lds_v[buf_next]) + (uint32_t)wu * 1024u;
      const uint32_t last = past ? last_tail : last_full;
#pragma unroll
      for (int e = 0; e < 2; ++e) c.lim[e] = last + gran[e];
      return c;
    };
    auto copy_one = [&](const CopyStep& c, int p) {
      const bool is_v = p >= CPW / 2;
      const int pp = is_v ? p - CPW / 2 : p;
      dma16_add(is_v ? c.bv : c.bk, min(roff[pp], c.lim[pp & 1]), is_v ? c.lv : c.lk, (uint32_t)(NW * pp * 1024));
    };

    // The copies are inline assembly, which the compiler's wait-count bookkeeping does
    // not see; it does see the Q (and bias) loads above.  A full wait here, after the
    // first tile's copies, shows it that Q has landed.  (With a partial count it places a
    // wait for Q inside the loop, which then also drains the copies in flight.)
    if (n_tiles > t_first) {
      const CopyStep c0 = copy_step(t_first, 0);
#pragma unroll
      for (int p = 0; p < CPW; ++p) copy_one(c0, p);
    }
    wait_vm_all();  // Q and the first tile have landed
    if (n_tiles > t_first) {
      for (int j = 1; j < AHEAD; ++j) {
        const CopyStep c0 = copy_step(t_first + j, j);
#pragma unroll
        for (int p = 0; p < CPW; ++p) copy_one(c0, p);
      }
    }
    __syncthreads();

    // The tile loop, unrolled over the STAGES buffers: tile t uses buffer u = (t - t_first)
    // mod STAGES.
    for (int t0 = t_first; t0 < n_tiles; t0 += STAGES)
#pragma unroll
    for (int buf = 0; buf < STAGES; ++buf) {
      const int t = t0 + buf;
      if (t >= n_tiles) break;
      const int key0 = t * kBN;
      const int buf_fill = (buf + AHEAD) % STAGES;  // tile t + AHEAD
      const CopyStep cs = copy_step(t + AHEAD, buf_fill);
      if (BIAS && t + 1 < n_tiles) load_bias_tile(bias_nxt, bias_row, key0 + kBN, L, kg, a.bias_len);
      const bool active = nrows > 0 && !(CAUSAL && key0 > wave_last_pos);
      if (active) {
        // S^T for the tile's 32-key blocks, as interleaved accumulator chains; the LDS
        // fragments for step st+1 are requested before the MFMAs of step st.  (One
        // branch for the products and the softmax: split in two, the S^T registers
        // would have to hold zeros on the other path, 23 moves per tile.)
        f32x16 s[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
        // scheduling hint: interleave the step's MFMAs with its LDS reads and VALU work
        // (on the 64x8192 D256 rank share: 10% faster than no hint; strategy 1 another
        // 0.7% over strategy 0)
        if (D != 256) __builtin_amdgcn_iglp_opt(1);
        {
          u32x4 kf[NKB];
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) kf[kb] = kread(buf, 0, kb);
#pragma unroll
          for (int st = 0; st < NST; ++st) {
            u32x4 nf[NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
              nf[kb] = kf[kb];
              if (st + 1 < NST) nf[kb] = kread(buf, st + 1, kb);
            }
            if (st % CEVERY == 0) copy_one(cs, st / CEVERY);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) s[kb] = mfma32(kf[kb], qf[st], s[kb]);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) kf[kb] = nf[kb];
          }
        }
        // Scale to base 2, bias, mask (diagonal or tail tiles only); tile row max.  The
        // masked and unmasked tiles take separate, wave-uniform paths.
        const bool need_mask = (key0 + kBN > kv_hi) || (key0 < kv_lo) ||
                               (CAUSAL && key0 + kBN - 1 > wave_first_pos_u);
        float mx = -INFINITY;
        if (need_mask) {
          asm volatile("" ::: "memory");
          scale_tile<BIAS, true, CAUSAL, NKB>(s, a.scale_log2, bias_cur, key0, kv_lo, kv_hi, qpos, kg, mx);
        } else {
          scale_tile<BIAS, false, CAUSAL, NKB>(s, a.scale_log2, bias_cur, key0, kv_lo, kv_hi, qpos, kg, mx);
        }
        mx = halves_max(mx);
        if (!BIAS) mx *= c_eff;
        // Lazy rescale: move the reference max only when it grows by more than 8 (x256).
        if (__builtin_expect(__any(mx > m_run + 8.f), 0)) {
          // A real branch: the rescale must not be if-converted into every tile.
          asm volatile("" ::: "memory");
          const float m_new = fmaxf(m_run, mx);
          const float alpha = (m_new == -INFINITY) ? 1.f : exp2f_fast(m_run - m_new);
#pragma unroll
          for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
          l_run *= alpha;
          m_run = m_new;
        }
        const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
        float rs[2] = {0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = BIAS ? exp2f_fast(s[kb][r] - m_use) : exp2f_fast(fmaf(s[kb][r], c_eff, -m_use));
            s[kb][r] = p;
            rs[r & 1] += p;
          }
        l_run += rs[0] + rs[1];

        // O^T += V^T P^T over the tile's 16-key steps; the V^T fragment of the next MFMA is
        // requested before the current one issues.
        {
          constexpr int NPS = kBN / 16;
          u32x4 pf[NPS];
#pragma unroll
          for (int st = 0; st < NPS; ++st) pf[st] = to_bf16x8(s[st >> 1], (st & 1) * 8);
          u32x4 va = vread(buf, 0, 0);
#pragma unroll
          for (int it = 0; it < NPS * NDB; ++it) {
            const int st = it / NDB, db = it % NDB;
            u32x4 nv = va;
            if (it + 1 < NPS * NDB) nv = vread(buf, (it + 1) / NDB, (it + 1) % NDB);
            oacc[db] = mfma32(va, pf[st], oacc[db]);
            va = nv;
          }
        }
      } else {
#pragma unroll
        for (int p = 0; p < CPW; ++p) copy_one(cs, p);
      }
      // tile t + 1 has landed in every wave's share (later tiles may be in flight), and
      // every wave is past its last read of buffer `buf`, which the next copies fill
      wait_vm<(AHEAD - 1) * CPW>();
      __syncthreads();
      if (BIAS) {
#pragma unroll
        for (int i = 0; i < 8; ++i) bias_cur[i] = bias_nxt[i];
      }
    }
    wait_vm_all();  // no copy into LDS outlives the workgroup

    if (col >= nrows) continue;  // (no barrier follows in this pass)
    // A row with no visible key in the window: O = 0 and LSE = -inf (merges as nothing).
    const float l = halves_sum(l_run);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    uint16_t* op = a.o_out + ((int64_t)(ch.q_row + row0 + col) * a.q_pitch + h) * D + kg * 4;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x2 w;
        w[0] = pack_bf16x2(oacc[db][i * 4 + 0] * inv, oacc[db][i * 4 + 1] * inv);
        w[1] = pack_bf16x2(oacc[db][i * 4 + 2] * inv, oacc[db][i * 4 + 3] * inv);
        st8(op + db * 32 + i * 8, w);
      }
    if (kg == 0)
      a.lse_out[(int64_t)h * a.q_rows + ch.q_row + row0 + col] = l > 0.f ? (m_run + log2f_fast(l)) * kLn2 : -INFINITY;
  }
}

template <int D, bool CAUSAL, bool BIAS>
static void launch_fwd_t(const AttnArgs& a, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, BIAS>), grid, dim3(FwdShape<D>::NW * 64), 0, s, a);
}

int fwd_waves(int D) { return D == 256 ? FwdShape<256>::NW : FwdShape<128>::NW; }

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
