// Internal launchers (host side) for the cpattn kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpattn {

struct AttnArgs;

struct ValidateArgs {
  const int32_t* seq_offsets;
  const int32_t* seq_lens;
  const int32_t* chunks;  // may be null (layout copies)
  int32_t* dev_err;
  int64_t rows;           // kv_rows (attention) or thd_rows (layout copies)
  int64_t q_rows;
  int num_seqs, num_chunks, max_chunk_len, max_kv_len, bias_len;
  int s_pitch;            // layout copies: BHSD pitch (0 for attention)
  int causal;
  int64_t ds_blocks;      // promised dS store bound (0: none to check)
};

// Per-chunk first dS block (divided by hq) of the stored-dS backward: the running sum of
// ceil(len / 32) * ceil(K_c / 32) over the chunks before each one.
struct DsTableArgs {
  const int32_t* seq_lens;
  const int32_t* chunks;
  const int32_t* dev_err;
  int64_t* tab;
  uint16_t* zero;  // 2 KB set to zero
  int num_chunks, causal;
};
hipError_t launch_ds_table(const DsTableArgs& a, hipStream_t s);

struct LayoutArgs {
  const uint16_t* src;
  uint16_t* dst;
  const int32_t* seq_offsets;
  const int32_t* seq_lens;
  const int32_t* dev_err;
  int B, H, S_pitch, D;
  int unpack;  // 0: BHSD -> THD, 1: THD -> BHSD
};

struct MergeArgs {
  const uint16_t* o_a;  // partial O over key set A, [q_rows, hq, D] BF16
  const float* lse_a;   // its LSE, [hq, q_rows]
  const uint16_t* o_b;
  const float* lse_b;
  uint16_t* o;          // merged O (may be o_a)
  float* lse;           // merged LSE (may be lse_a)
  const int32_t* chunks;
  const int32_t* dev_err;
  int64_t q_rows;
  int64_t q_pitch;      // heads per row in memory
  int hq, D, blocks_per_chunk;
};
// Head-group copies of the A2A swap: [rows, H, D] <-> [cp, rows, H / cp, D].
struct A2aHeadsArgs {
  const uint16_t* src;
  uint16_t* dst;
  int64_t rows;
  int H, D, cp;
  int merge;        // 0: rows -> blocks (split), 1: blocks -> rows (merge)
  int rows_per_wg;
};

// Row copies of the A2A swap between [cp, rows_per_rank, heads, D] blocks and the
// sequence-ordered [full_rows, heads, D] tensor, driven by per-rank chunk maps.
struct A2aRowsArgs {
  const uint16_t* src;   // blocks (scatter) or the full tensor (gather)
  uint16_t* dst;         // the full tensor (scatter) or blocks (gather)
  const int32_t* maps;   // [cp][chunks_per_rank][4] {seq, q_row, pos0, len}
  const int32_t* seq_offsets;
  const int32_t* seq_lens;
  int32_t* dev_err;
  int64_t full_rows, rows_per_rank;
  int cp, chunks_per_rank, num_seqs, max_chunk_len, heads, D;
  int gather;            // 0: blocks -> full (scatter), 1: full -> blocks (gather)
  int wg_per_chunk;
};

hipError_t launch_a2a_heads(const A2aHeadsArgs& a, hipStream_t s);
hipError_t launch_a2a_rows(const A2aRowsArgs& a, hipStream_t s);
hipError_t launch_validate(const ValidateArgs& a, hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, dim3 grid, hipStream_t s);
hipError_t launch_layout(const LayoutArgs& a, hipStream_t s);
hipError_t launch_fwd(const AttnArgs& a, int D, bool causal, bool bias, dim3 grid, hipStream_t s);
// Waves per forward workgroup at head dim D (each wave: 32 query rows of one head).
int fwd_waves(int D);
hipError_t launch_prepass(const AttnArgs& a, int D, dim3 grid, hipStream_t s);
hipError_t launch_dkdv(const AttnArgs& a, int D, bool causal, bool bias, dim3 grid, hipStream_t s);
hipError_t launch_dq(const AttnArgs& a, int D, bool causal, bool bias, dim3 grid, hipStream_t s);
hipError_t launch_dq_ds(const AttnArgs& a, int D, bool causal, dim3 grid, hipStream_t s);
hipError_t launch_dbias(const AttnArgs& a, int D, dim3 grid, hipStream_t s);
// dBias summed from the stored dS (grid: 32-key blocks x parts, 32-position tiles, heads).
hipError_t launch_dbias_ds(const AttnArgs& a, dim3 grid, hipStream_t s);
hipError_t launch_dbias_reduce(const float* partial, float* out, int64_t n, int parts,
                               const int32_t* dev_err, hipStream_t s);

// Rows of a chunk handled by one pre-pass workgroup (one query tile).
constexpr int kPrepassRows = 32;
// Keys per stored dS block (one dK/dV wave) and query rows per dQ-from-dS workgroup
// wave (two 32-query tiles).
constexpr int kDsBlockKeys = 32;
constexpr int kDqDsRows = 64;
// Keys per dK/dV workgroup (four waves of 32 keys).
constexpr int kDkdvKeys = 128;
// dBias tile: 128 query positions x 64 keys per workgroup.
constexpr int kDbiasPos = 128;
constexpr int kDbiasKeys = 64;

}  // namespace cpattn
