/*
 * cpattn: blockwise causal grouped-query softmax attention, forward and
 * backward in BF16, on one context-parallel rank's share of a packed THD batch,
 * for AMD MI355X (gfx950).
 *
 * The operations follow the page "Optimize context parallel attention layouts
 * and gradient accumulation" (TransformerEngine PR 3683): its "Description" and
 * "Changes" sections (equal-length and padded THD inputs with physical offsets,
 * separate Q/K/V, GQA, head dims 128/256, the on-device check of the promised
 * lengths and offsets, output zeroing removed, the BF16 layout copies), its
 * "CP8 first-gradient accumulator reuse" section (the first dK/dV contribution
 * is the accumulator, the later one is added) and its "CP8 AllGather:
 * composition with first-gradient reuse" section (the dO.O row-dot pre-pass);
 * and the triangle (pair-biased row) attention named on the page "Support and
 * performance optimization for Hopper (H200) architecture?".
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *    allocates no memory and keeps no state between calls, except the static
 *    scratch array of cpattn_bwd_noalloc (part of its code object, one per GPU)
 *    and that array's device address, looked up once per GPU.
 *  - BF16 tensors are passed as raw 16-bit patterns, contiguous, head dim
 *    innermost, 16-byte aligned:
 *        Q, O, dO, dQ : [q_rows,  hq,  head_dim]
 *        K, V, dK, dV : [kv_rows, hkv, head_dim]
 *    LSE and the pre-pass output Delta are fp32 [hq, q_rows].
 *    The pair bias and dBias are fp32 [hq, bias_len, bias_len].
 *  - Sequence and chunk descriptors live in device memory:
 *        seq_offsets int32 [num_seqs]: K/V row holding position 0 of sequence b
 *        seq_lens    int32 [num_seqs]: valid length L_b of sequence b
 *        q_chunk_map int32 [num_chunks][4] = {seq, q_row, pos0, len}: Q rows
 *            [q_row, q_row+len) hold positions [pos0, pos0+len) of `seq`.
 *    Promises checked on the device on every call (cpattn_validate):
 *        0 <= L_b <= max_kv_len; sequences lie in [0, kv_rows), in ascending
 *        order, without overlap; chunks are listed with non-decreasing `seq`
 *        and ascending, non-overlapping Q rows inside [0, q_rows);
 *        0 <= len <= max_chunk_len; pos0 >= 0 and pos0+len <= L_seq; with a
 *        bias, every L_b <= bias_len.
 *  - Rows of Q/O/dO/dQ that no chunk covers and K/V/dK/dV rows past L_b
 *    (padding) are never read or written.
 *  - Causal visibility: the query at position p of a sequence sees key j iff
 *    j < L and (not causal or j <= p).  GQA maps query head h to KV head
 *    h / (hq / hkv).
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream) and never synchronizes.
 *  - Host-detectable errors return a non-zero status before anything is
 *    enqueued: CPATTN_EINVAL for null or misaligned pointers, bad sizes,
 *    hq % hkv != 0, a workspace that is too small, or any output byte range
 *    that overlaps an input or another output (pointer-alias audit);
 *    CPATTN_EUNSUPPORTED for unsupported head dims or variants;
 *    CPATTN_EHIP when a launch fails.  cpattn_last_error() describes it.
 *  - Device-detectable errors: the validation step overwrites *dev_err (a
 *    caller-owned device int32) with the CPATTN_DEV_* bits of every broken
 *    promise, 0 if none.  Every later kernel of the same call reads *dev_err
 *    first and writes nothing when it is non-zero (fail closed).  The caller
 *    reads it back after synchronizing.
 */
#ifndef CPATTN_H
#define CPATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* cpattn_stream_t; /* same type as hipStream_t */

typedef enum cpattn_status {
  CPATTN_OK = 0,
  CPATTN_EINVAL = 1,
  CPATTN_EUNSUPPORTED = 2,
  CPATTN_EHIP = 3
} cpattn_status;

/* Bits of the device error word. */
#define CPATTN_DEV_ESEQ_LEN    0x01 /* a seq_lens entry < 0 or > max_kv_len            */
#define CPATTN_DEV_ESEQ_RANGE  0x02 /* a sequence outside [0,kv_rows), unordered or overlapping */
#define CPATTN_DEV_ECHUNK_SEQ  0x04 /* chunk seq out of range or decreasing             */
#define CPATTN_DEV_ECHUNK_ROWS 0x08 /* chunk Q rows outside [0,q_rows), unordered or overlapping */
#define CPATTN_DEV_ECHUNK_POS  0x10 /* len < 0, len > max_chunk_len, pos0 < 0 or pos0+len > L */
#define CPATTN_DEV_EBIAS       0x20 /* a sequence longer than bias_len                 */
#define CPATTN_DEV_ELAYOUT     0x40 /* pack/unpack: L_b > S_pitch or THD rows out of range */
#define CPATTN_DEV_EDS_BLOCKS  0x80 /* stored-dS backward: the chunks need more than ds_blocks */

/* Shape and variant of one rank share. */
typedef struct cpattn_problem {
  int32_t num_seqs;      /* B */
  int32_t hq;            /* query heads */
  int32_t hkv;           /* key/value heads; hq % hkv == 0 */
  int32_t head_dim;      /* D: 64, 128 or 256 (causal or not); 32, 64 or 128 with a bias */
  int64_t q_rows;        /* physical Q rows, padding included */
  int64_t kv_rows;       /* physical K/V rows, padding included */
  int32_t num_chunks;    /* C */
  int32_t max_chunk_len; /* host-known bound on every chunk len (sizes the grids) */
  int32_t max_kv_len;    /* host-known bound on every L_b (sizes the grids) */
  int32_t causal;        /* 1: causal by position; 0: every key of the sequence */
  float scale;           /* score scale, usually 1/sqrt(head_dim) */
  int32_t bias_len;      /* 0: no bias; else bias is fp32 [hq, bias_len, bias_len]
                            indexed [h, query position, key position]; needs causal = 0 */
  int32_t q_head_pitch;  /* heads per row in the memory of Q, O, dO, dQ (0: hq); >= hq */
  int32_t kv_head_pitch; /* heads per row in the memory of K, V, dK, dV (0: hkv); >= hkv */
  int64_t ds_blocks;     /* host-known bound that sizes the stored-dS backward's dS store:
                            the sum over chunks of ceil(len / 32) * ceil(K_c / 32), where
                            K_c is the keys the chunk's last row sees (causal: pos0 + len;
                            else L of its sequence).  0: no bound known, every query-tile
                            slot is sized for ceil(max_kv_len / 32) key blocks.  Checked on
                            the device (CPATTN_DEV_EDS_BLOCKS). */
} cpattn_problem;
/* Head pitches let one call cover a group of heads of larger tensors in place ("First-
 * gradient buffer reuse" / head partitioning: H16/H8 head-group calls on strided
 * views that reuse one workspace): pass pointers to the group's first query head and
 * first KV head, hq/hkv the group's head counts, and the full tensors' heads per row
 * as the pitches.  Row r, head h of Q is then at q + (r * q_head_pitch + h) * D.  LSE
 * and Delta stay [hq, q_rows] per call (a head slice of a larger LSE is contiguous);
 * the workspace scales with the call's hq. */

#define CPATTN_OP_FWD 0
#define CPATTN_OP_BWD 1
#define CPATTN_OP_BWD_DS 2

/* Text of a status code. */
const char* cpattn_status_str(int status);

/* Description of the last host-side failure of the calling thread ("" if none). */
const char* cpattn_last_error(void);

/* Library version: major*10000 + minor*100 + patch. */
int cpattn_version(void);

/* Bytes of caller-provided device workspace that cpattn_fwd (op = CPATTN_OP_FWD)
 * or cpattn_bwd (op = CPATTN_OP_BWD) needs for `p`.  The backward workspace holds,
 * each part starting on a 256-byte boundary: Delta (fp32 [hq, q_rows], at offset
 * 0); Q^T and dO^T as BF16 tiles [slot][hq][head_dim][32 queries, in an internal
 * order] with ceil(q_rows/32) + num_chunks slots (tile t of chunk c is slot
 * floor(q_row_c / 32) + c + t; queries past the chunk end are zero); the tiles' row
 * statistics, fp32 [slot][hq][64] (log2(e) * LSE of the 32 rows, +inf past the chunk
 * end, then Delta, 0 past the end); and, with a bias, the per-partition dBias partial
 * sums.
 * op = CPATTN_OP_BWD_DS: the backward workspace followed by the chunks' dS store
 * offsets (int64 per chunk), a 2 KB block of zeros and the dS store, BF16 blocks of
 * 32 keys x 32 queries
 * (2 KB, internal order), one per (chunk tile, query head, 32-key block the chunk
 * sees): with it dK/dV stores dS and dQ is a product with the stored dS instead of
 * a second pass that forms S, P and dP again.  It is hq * ds_blocks blocks (hq *
 * (ceil(q_rows/32) + num_chunks) * ceil(max_kv_len/32) when ds_blocks is 0): e.g.
 * 18.3 GB for 64 sequences of 8192 keys holding two 512-row chunks each (one at the
 * start, one at the end), 32 heads and causal masking, against 36.5 GB without the
 * bound.  Every supported head dim (32 to 256).
 * Returns 0 for an invalid problem (check it with the entry point for the reason). */
size_t cpattn_workspace_size(const cpattn_problem* p, int op);

/* The device promise check alone ("Changes": promised sequence lengths and
 * physical offsets checked on the device on every execution).  Overwrites
 * *dev_err with the CPATTN_DEV_* bits. */
int cpattn_validate(const cpattn_problem* p, const int32_t* seq_offsets, const int32_t* seq_lens,
                    const int32_t* q_chunk_map, int32_t* dev_err, cpattn_stream_t stream);

/* Forward.  For every chunk row and query head: O = softmax(scale Q K^T (+bias)) V
 * over the visible keys (BF16, round to nearest even) and LSE = natural-log
 * log-sum-exp of the scaled scores (fp32, the "Stats" layout [hq, q_rows]).
 * Writes O and LSE on chunk rows only.  ws may be NULL when
 * cpattn_workspace_size(p, CPATTN_OP_FWD) is 0. */
int cpattn_fwd(const cpattn_problem* p, const void* q, const void* k, const void* v,
               const int32_t* seq_offsets, const int32_t* seq_lens, const int32_t* q_chunk_map,
               const float* bias, void* o, float* lse, void* ws, size_t ws_bytes,
               int32_t* dev_err, cpattn_stream_t stream);

/* Forward over a key window ("Private C++ FROST P2P": CP over point-to-point steps,
 * each attending to one K/V block): as cpattn_fwd with the visible keys further
 * restricted to sequence positions [kv_lo, kv_hi).  O (BF16) is the softmax over
 * the window's visible keys applied to V and LSE (fp32) their log-sum-exp; a row
 * with no visible key in the window gets O = 0 and LSE = -inf.  Two results over
 * disjoint windows combine with cpattn_merge.  kv_lo = 0, kv_hi >= every L_b is
 * cpattn_fwd.  EINVAL for kv_lo < 0 or kv_hi < kv_lo. */
int cpattn_fwd_window(const cpattn_problem* p, const void* q, const void* k, const void* v,
                      const int32_t* seq_offsets, const int32_t* seq_lens,
                      const int32_t* q_chunk_map, const float* bias, int32_t kv_lo, int32_t kv_hi,
                      void* o, float* lse, int32_t* dev_err, cpattn_stream_t stream);

/* Merge of two partial results over disjoint key sets A and B (the ring step's LSE
 * correction): on every chunk row and head, LSE = log(e^lse_a + e^lse_b) and
 * O = e^(lse_a - LSE) o_a + e^(lse_b - LSE) o_b in fp32, rounded to BF16 once; rows
 * whose two LSEs are -inf get O = 0, LSE = -inf.  o may equal o_a and lse may equal
 * lse_a (the running result updated in place); any other overlap is EINVAL.  Does
 * not validate (call cpattn_validate first on the same stream with the same dev_err);
 * does nothing when *dev_err is set. */
int cpattn_merge(const cpattn_problem* p, const int32_t* q_chunk_map, const void* o_a,
                 const float* lse_a, const void* o_b, const float* lse_b, void* o, float* lse,
                 const int32_t* dev_err, cpattn_stream_t stream);

/* Backward: validate, the Delta pre-pass, dK/dV, then dQ.
 *  dQ (BF16) is written on chunk rows.
 *  dK/dV (BF16) are the sums over all chunks of each sequence and over the
 *  hq/hkv query heads of each KV head, accumulated in fp32 and rounded once.
 *  dkv_accumulate = 0 (first contribution): every valid K/V row of every
 *  sequence is STORED (0 where no query attends), so dK/dV need no zero fill.
 *  dkv_accumulate = 1 (second addition): the existing BF16 dK/dV values are
 *  read, this call's contribution is added in fp32 and the sum is rounded once.
 *  dbias (fp32, with a bias only, may be NULL to skip it) is STORED: the sum of
 *  dS over every chunk row, unscaled, with dS formed in fp32 (cpattn_bwd_dbias,
 *  whichever dQ path is taken: a sum over many rows of BF16-rounded dS drifts by
 *  the rows' rounding errors).  O and LSE are the forward's outputs.
 *  ws must hold cpattn_workspace_size(p, CPATTN_OP_BWD) bytes.  When it holds
 *  cpattn_workspace_size(p, CPATTN_OP_BWD_DS) bytes (nonzero), dK/dV stores dS in
 *  it and dQ multiplies the stored dS (cpattn_bwd_dkdv_ds, cpattn_bwd_dq_ds);
 *  otherwise dQ forms S, P and dP again (cpattn_bwd_dkdv, cpattn_bwd_dq).  Both
 *  give dQ = scale dS K with dS rounded to BF16 before the product. */
int cpattn_bwd(const cpattn_problem* p, const void* q, const void* k, const void* v,
               const int32_t* seq_offsets, const int32_t* seq_lens, const int32_t* q_chunk_map,
               const float* bias, const void* o, const float* lse, const void* dout,
               void* dq, void* dk, void* dv, float* dbias, int dkv_accumulate,
               void* ws, size_t ws_bytes, int32_t* dev_err, cpattn_stream_t stream);

/* Backward over a key window: the contribution of the keys at sequence positions
 * [kv_lo, kv_hi), with O and LSE the complete forward results (merged over all
 * windows), so P = exp(S - LSE) and Delta = rowsum(dO * O) are those of the whole
 * attention.  dK/dV are written for the window's valid keys only (STORE, or ADD with
 * dkv_accumulate = 1; other rows untouched).  dQ gets the window's share of
 * scale dS K: STORE (dq_accumulate = 0) or added to the existing BF16 values and
 * rounded once (dq_accumulate = 1), so dQ summed over disjoint windows covering
 * every key is the full dQ.  prepass = 1 validates and runs the Delta pre-pass into
 * ws (cpattn_workspace_size(p, CPATTN_OP_BWD) bytes, without the dBias partials);
 * prepass = 0 reuses the pre-pass results an earlier call left in ws for the same O,
 * dO and chunks.  When ws holds cpattn_workspace_size(p, CPATTN_OP_BWD_DS) bytes, dK/dV
 * store the window's dS and the dQ share multiplies it (the dS store is reused by the
 * next window); otherwise dS is formed again for dQ.  No dBias is produced. */
int cpattn_bwd_window(const cpattn_problem* p, const void* q, const void* k, const void* v,
                      const int32_t* seq_offsets, const int32_t* seq_lens,
                      const int32_t* q_chunk_map, const float* bias, const void* o, const float* lse,
                      const void* dout, int32_t kv_lo, int32_t kv_hi, int prepass, void* dq,
                      int dq_accumulate, void* dk, void* dv, int dkv_accumulate, void* ws,
                      size_t ws_bytes, int32_t* dev_err, cpattn_stream_t stream);

/* The backward's steps one by one, for callers that schedule them (and for
 * timing each kernel).  None of them validates: call cpattn_validate first on
 * the same stream with the same dev_err.  All take the backward workspace
 * (cpattn_workspace_size(p, CPATTN_OP_BWD) bytes; without dBias the partial
 * sums may be left off, so ws_bytes may be that size minus them).
 *  cpattn_bwd_prepass: writes Delta[h, r] = sum_d dO[r,h,d] O[r,h,d] (fp32) on
 *      chunk rows ("CP8 AllGather: composition with first-gradient reuse": the
 *      row dot of dO and O, loaded at their physical pitch), the transposed
 *      32-query tiles of Q and dO that dK/dV multiplies with, and each tile's row
 *      statistics (LSE, the forward's output, and Delta).
 *  cpattn_bwd_dkdv: dK/dV as in cpattn_bwd from the pre-pass results.
 *  cpattn_bwd_dq: dQ as in cpattn_bwd from the pre-pass results.
 *  cpattn_bwd_dbias: dBias as in cpattn_bwd from the pre-pass results; ws must
 *      also hold the partial sums.
 *  cpattn_bwd_dkdv_ds: cpattn_bwd_dkdv that also stores dS (BF16) in the dS store
 *      of ws (cpattn_workspace_size(p, CPATTN_OP_BWD_DS) bytes): every block with a
 *      visible (key, query) pair, the others are left as they are.
 *  cpattn_bwd_dq_ds: dQ = scale dS K from the dS store that cpattn_bwd_dkdv_ds
 *      filled for the same problem and chunks (reads K and the dS store only).
 *  cpattn_bwd_dbias_ds: dBias (fp32, with a bias) as the sum over chunk rows of the
 *      dS that cpattn_bwd_dkdv_ds stored (page "Support and performance optimization
 *      for Hopper (H200) architecture?": the pair bias is shared by every row, so its
 *      gradient is a reduction over rows).  The rows are summed in the same fixed
 *      partition units and order as cpattn_bwd_dbias; the result differs from it only
 *      by the BF16 rounding of the stored dS (about 2^-9 |dS| per row, adding up over
 *      the rows like a random walk), in exchange for reading 2 bytes per pair instead
 *      of forming S and dP again.  ws must hold the dBias partial sums and the dS
 *      store (cpattn_workspace_size(p, CPATTN_OP_BWD_DS) bytes); reads the
 *      descriptors and the dS store only. */
int cpattn_bwd_prepass(const cpattn_problem* p, const void* q, const int32_t* q_chunk_map,
                       const void* o, const void* dout, const float* lse, void* ws,
                       size_t ws_bytes, const int32_t* dev_err, cpattn_stream_t stream);
int cpattn_bwd_dkdv(const cpattn_problem* p, const void* q, const void* k, const void* v,
                    const int32_t* seq_offsets, const int32_t* seq_lens,
                    const int32_t* q_chunk_map, const float* bias, const float* lse,
                    const void* dout, const void* ws, size_t ws_bytes, void* dk, void* dv,
                    int dkv_accumulate, const int32_t* dev_err, cpattn_stream_t stream);
int cpattn_bwd_dq(const cpattn_problem* p, const void* q, const void* k, const void* v,
                  const int32_t* seq_offsets, const int32_t* seq_lens,
                  const int32_t* q_chunk_map, const float* bias, const float* lse,
                  const void* dout, const void* ws, size_t ws_bytes, void* dq,
                  const int32_t* dev_err, cpattn_stream_t stream);
int cpattn_bwd_dbias(const cpattn_problem* p, const void* q, const void* k, const void* v,
                     const int32_t* seq_offsets, const int32_t* seq_lens,
                     const int32_t* q_chunk_map, const float* bias, const float* lse,
                     const void* dout, void* ws, size_t ws_bytes, float* dbias,
                     const int32_t* dev_err, cpattn_stream_t stream);
int cpattn_bwd_dkdv_ds(const cpattn_problem* p, const void* q, const void* k, const void* v,
                       const int32_t* seq_offsets, const int32_t* seq_lens,
                       const int32_t* q_chunk_map, const float* bias, const float* lse,
                       const void* dout, void* ws, size_t ws_bytes, void* dk, void* dv,
                       int dkv_accumulate, const int32_t* dev_err, cpattn_stream_t stream);
int cpattn_bwd_dq_ds(const cpattn_problem* p, const void* k, const int32_t* seq_offsets,
                     const int32_t* seq_lens, const int32_t* q_chunk_map, const void* ws,
                     size_t ws_bytes, void* dq, const int32_t* dev_err, cpattn_stream_t stream);
int cpattn_bwd_dbias_ds(const cpattn_problem* p, const int32_t* seq_offsets, const int32_t* seq_lens,
                        const int32_t* q_chunk_map, void* ws, size_t ws_bytes, float* dbias,
                        const int32_t* dev_err, cpattn_stream_t stream);

/* Bytes of the static scratch array behind cpattn_bwd_noalloc (64 MiB per GPU). */
#define CPATTN_NOALLOC_SCRATCH_BYTES (64u << 20)

/* cpattn_bwd without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, outputs, checks and kernels as cpattn_bwd; the
 * workspace is a static device array of CPATTN_NOALLOC_SCRATCH_BYTES held by each GPU
 * the library runs on until the process ends.  It takes the stored-dS backward when
 * cpattn_workspace_size(p, CPATTN_OP_BWD_DS) fits in the array, else the backward that
 * forms dS again for dQ when cpattn_workspace_size(p, CPATTN_OP_BWD) fits (results
 * bit-identical to cpattn_bwd with a workspace of that size), else returns
 * CPATTN_EUNSUPPORTED with nothing enqueued.  Calls no allocating routine; the first
 * call on a device looks up the array's device address (hipGetSymbolAddress) with the
 * current device, which must be the stream's.  Nothing in the array needs clearing
 * between calls.  Calls that overlap in time on one GPU share the array and race:
 * serialize them (one stream, or the caller's own ordering). */
int cpattn_bwd_noalloc(const cpattn_problem* p, const void* q, const void* k, const void* v,
                       const int32_t* seq_offsets, const int32_t* seq_lens,
                       const int32_t* q_chunk_map, const float* bias, const void* o,
                       const float* lse, const void* dout, void* dq, void* dk, void* dv,
                       float* dbias, int dkv_accumulate, int32_t* dev_err,
                       cpattn_stream_t stream);

/* Layout copies ("Changes": vectorised BF16 pack/unpack copies that keep
 * physical sequence origins).  BHSD is [B, H, S_pitch, D]; THD is
 * [thd_rows, H, D].  pack: thd[seq_offsets[b]+s, h, :] = bhsd[b, h, s, :] for
 * s < seq_lens[b]; unpack is the inverse.  Only valid rows are copied; the
 * other destination rows keep their contents.  D must be a multiple of 8.
 * The promises (L_b <= S_pitch, ascending non-overlapping THD ranges inside
 * [0, thd_rows)) are checked on the device; on a violation *dev_err gets
 * CPATTN_DEV_ELAYOUT (plus the sequence bits) and nothing is copied. */
int cpattn_pack(const void* bhsd, void* thd, int32_t B, int32_t H, int32_t S_pitch, int32_t D,
                int64_t thd_rows, const int32_t* seq_offsets, const int32_t* seq_lens,
                int32_t* dev_err, cpattn_stream_t stream);
int cpattn_unpack(const void* thd, void* bhsd, int32_t B, int32_t H, int32_t S_pitch, int32_t D,
                  int64_t thd_rows, const int32_t* seq_offsets, const int32_t* seq_lens,
                  int32_t* dev_err, cpattn_stream_t stream);

/* Copies around the all-to-all (A2A) head <-> sequence swap of context parallelism
 * (page "Optimize context parallel attention layouts and gradient accumulation",
 * "Changes": BF16 A2A pack/unpack copies inside the swap; "Validation and
 * performance": the CP4/A2A run they sped up).  Rank r of cp ranks holds the rows of
 * its chunks of every sequence with all H heads; the swap gives every rank whole
 * sequences of Hc = H / cp heads.  Before attention: split_heads, the exchange (block
 * j to rank j), scatter_rows.  After attention: gather_rows, the exchange,
 * merge_heads.  The exchange itself (an RCCL all-to-all) is not part of this library.
 * All tensors are BF16 with the head dim innermost; D must be a multiple of 8 and
 * every tensor pointer 16-byte aligned.  Source and destination must not overlap. */

/* split_heads: dst[j, t, h, :] = src[t, j*Hc + h, :], src [rows, H, D] -> dst
 * [cp, rows, Hc, D] (block j is contiguous: the send buffer for rank j).
 * merge_heads is the inverse, src [cp, rows, Hc, D] -> dst [rows, H, D].  Every row is
 * copied.  H must be a multiple of cp; cp <= 65535.  No device promise is involved. */
int cpattn_a2a_split_heads(const void* src, void* dst, int64_t rows, int32_t H, int32_t D, int32_t cp,
                           cpattn_stream_t stream);
int cpattn_a2a_merge_heads(const void* src, void* dst, int64_t rows, int32_t H, int32_t D, int32_t cp,
                           cpattn_stream_t stream);

/* Sizes of a row copy between the exchange's blocks and the sequence-ordered tensor. */
typedef struct {
  int32_t cp;              /* ranks: blocks of the exchange                           */
  int32_t chunks_per_rank; /* entries per rank map (unused entries: len = 0)         */
  int32_t num_seqs;
  int32_t max_chunk_len;   /* bound on every len (checked on the device)             */
  int64_t rows_per_rank;   /* rows of each block                                     */
  int64_t full_rows;       /* rows of the sequence-ordered tensor                    */
  int32_t heads;           /* heads per row on both sides (Hc)                       */
  int32_t head_dim;
} cpattn_a2a_rows;

/* scatter_rows: blocks [cp, rows_per_rank, heads, D] -> full [full_rows, heads, D].
 * rank_maps is int32 [cp][chunks_per_rank][4] of {seq, q_row, pos0, len} in device
 * memory: chunk {seq, q_row, pos0, len} of rank s moves rows [q_row, q_row + len) of
 * block s to rows seq_offsets[seq] + pos0 + [0, len) of full.  gather_rows is the
 * inverse (full -> blocks).  Rows no chunk names keep their contents.  Checked on the
 * device (*dev_err overwritten; nothing copied on a violation): seq in range
 * (CPATTN_DEV_ECHUNK_SEQ), 0 <= len <= max_chunk_len and [pos0, pos0 + len) inside
 * [0, seq_lens[seq]) (CPATTN_DEV_ECHUNK_POS), [q_row, q_row + len) inside the block
 * (CPATTN_DEV_ECHUNK_ROWS), seq_lens >= 0 (CPATTN_DEV_ESEQ_LEN) and every sequence
 * inside [0, full_rows) (CPATTN_DEV_ESEQ_RANGE).  Chunks may come in any order; two
 * chunks naming the same destination row leave that row with either one's data. */
int cpattn_a2a_scatter_rows(const cpattn_a2a_rows* p, const void* blocks, void* full,
                            const int32_t* rank_maps, const int32_t* seq_offsets,
                            const int32_t* seq_lens, int32_t* dev_err, cpattn_stream_t stream);
int cpattn_a2a_gather_rows(const cpattn_a2a_rows* p, const void* full, void* blocks,
                           const int32_t* rank_maps, const int32_t* seq_offsets,
                           const int32_t* seq_lens, int32_t* dev_err, cpattn_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* CPATTN_H */
