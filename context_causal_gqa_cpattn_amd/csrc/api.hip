// C-ABI of the cpattn library: host-side argument checks, the pointer-alias audit,
// grid sizing and kernel dispatch.  Every entry point enqueues on the caller's stream
// and returns without synchronizing.
//
// Page "Optimize context parallel attention layouts and gradient accumulation":
// "Changes" (promise checked on the device, explicit contract instead of private
// switches as asked under "Remaining before ready"), "CP8 AllGather: composition
// with first-gradient reuse" (pointer-alias audits outside the timed region).
// Page on the ws2 tensor/sequence/context-parallel block ("Scope / Known
// limitations"): unsupported shapes and dtypes raise instead of falling back.
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>
#include <vector>

#include "../../include/cpattn.h"
#include "common.h"
#include "launch.h"

using namespace cpattn;

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(CPATTN_EHIP, "%s: %s", what, hipGetErrorString(e));
  return CPATTN_OK;
}

struct Range {
  const char* name;
  uintptr_t lo, hi;  // span [lo, hi)
  bool output;
  int64_t pitch = 0;  // > 0: the bytes are rows of `row` bytes every `pitch` bytes
  int64_t row = 0;
};

int64_t floor_div(int64_t x, int64_t y) { return x >= 0 ? x / y : -((-x + y - 1) / y); }

// Whether two ranges share a byte.  Two row sets with one pitch (head slices of one
// tensor) are tested exactly: rows i of A and j of B meet iff -row_b < d + (j - i) pitch
// < row_a with d = lo_b - lo_a; any other pair is tested by its spans.
bool overlaps(const Range& a, const Range& b) {
  if (!(a.lo < b.hi && b.lo < a.hi)) return false;
  if (a.pitch <= 0 || a.pitch != b.pitch) return true;
  const int64_t P = a.pitch, d = (int64_t)(b.lo - a.lo);
  const int64_t na = ((int64_t)(a.hi - a.lo) - a.row) / P + 1, nb = ((int64_t)(b.hi - b.lo) - b.row) / P + 1;
  const int64_t m_lo = std::max(floor_div(-b.row - d, P) + 1, 1 - na);
  const int64_t m_hi = std::min(-floor_div(d - a.row, P) - 1, nb - 1);
  return m_lo <= m_hi;
}

// Every output range must be disjoint from every other range.
int alias_audit(const std::vector<Range>& rs) {
  for (size_t i = 0; i < rs.size(); ++i) {
    if (!rs[i].output || rs[i].lo == rs[i].hi) continue;
    for (size_t j = 0; j < rs.size(); ++j) {
      if (i == j || rs[j].lo == rs[j].hi) continue;
      if (rs[j].output && j < i) continue;  // output pairs checked once
      if (overlaps(rs[i], rs[j]))
        return fail(CPATTN_EINVAL, "pointer alias: output %s overlaps %s %s", rs[i].name,
                    rs[j].output ? "output" : "input", rs[j].name);
    }
  }
  return CPATTN_OK;
}

Range rng(const char* name, const void* p, uint64_t bytes, bool out) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{name, lo, p ? lo + bytes : lo, out};
}

// rows of `row` bytes every `pitch` bytes; `span` = bytes from the first to the last byte
Range rng_rows(const char* name, const void* p, int64_t span, int64_t pitch, int64_t row, bool out) {
  Range r = rng(name, p, span, out);
  r.pitch = pitch;
  r.row = row;
  return r;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_ptr(const void* p, uint64_t bytes, size_t align, const char* name) {
  if (bytes == 0) return CPATTN_OK;
  if (!p) return fail(CPATTN_EINVAL, "%s is NULL", name);
  if (!aligned(p, align)) return fail(CPATTN_EINVAL, "%s is not %zu-byte aligned", name, align);
  return CPATTN_OK;
}

constexpr int64_t kGridMax = 0x7fffffff;

struct Plan;
Range rq(const Plan& pl, const char* name, const void* p, bool out);
Range rkv(const Plan& pl, const char* name, const void* p, bool out);

struct Plan {
  int D, G, hpw, hq, hkv;
  int64_t qp, kvp;  // heads per row in memory (Q side, K/V side)
  bool bias;
  int64_t q_bytes, kv_bytes, stat_bytes, bias_bytes;
  int64_t delta_bytes;  // rounded to 256
  int parts;            // dBias partitions
  int64_t partial_bytes;
  // backward workspace: delta | Q^T tiles | dO^T tiles | tile statistics | dBias partials |
  // dS store (per-chunk offsets, then the blocks)
  int64_t off_qt, off_dot, off_stats, off_partials, ws_core;
  bool ds_ok;            // the stored-dS backward applies (every supported head_dim, 32 to 256)
  int64_t ds_head_blocks;  // dS blocks per query head
  int64_t off_ds, off_ds_zero, off_ds_blocks, ds_bytes;  // ds_bytes: offsets, zero block, blocks
  dim3 grid_fwd, grid_fwd1d, grid_fwdk, grid_prepass, grid_dkdv, grid_dbias, grid_dbias_ds, grid_dqds;
  int bpc_fwd, bpc_fwdk, bpc_prepass, bpc_dqds, kv_tiles, kv_slots;
};

int64_t round256(int64_t x) { return (x + 255) / 256 * 256; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

Range rq(const Plan& pl, const char* name, const void* p, bool out) {
  return rng_rows(name, p, pl.q_bytes, pl.qp * pl.D * 2, (int64_t)pl.hq * pl.D * 2, out);
}
Range rkv(const Plan& pl, const char* name, const void* p, bool out) {
  return rng_rows(name, p, pl.kv_bytes, pl.kvp * pl.D * 2, (int64_t)pl.hkv * pl.D * 2, out);
}

int make_plan(const cpattn_problem* p, Plan& pl) {
  if (!p) return fail(CPATTN_EINVAL, "problem is NULL");
  if (p->num_seqs < 0 || p->num_chunks < 0 || p->q_rows < 0 || p->kv_rows < 0 ||
      p->max_chunk_len < 0 || p->max_kv_len < 0 || p->bias_len < 0)
    return fail(CPATTN_EINVAL, "negative size in problem");
  if (p->hq <= 0 || p->hkv <= 0) return fail(CPATTN_EINVAL, "hq and hkv must be positive");
  if (p->hq % p->hkv) return fail(CPATTN_EINVAL, "hq (%d) is not a multiple of hkv (%d)", p->hq, p->hkv);
  if (!std::isfinite(p->scale)) return fail(CPATTN_EINVAL, "scale is not finite");
  if (p->causal != 0 && p->causal != 1) return fail(CPATTN_EINVAL, "causal must be 0 or 1");
  const int D = p->head_dim;
  pl.bias = p->bias_len > 0;
  if (pl.bias) {
    if (p->causal) return fail(CPATTN_EUNSUPPORTED, "a pair bias is supported without causal masking only");
    if (D != 32 && D != 64 && D != 128)
      return fail(CPATTN_EUNSUPPORTED, "head_dim %d unsupported with a bias (32, 64, 128)", D);
  } else if (D != 32 && D != 64 && D != 128 && D != 256) {
    return fail(CPATTN_EUNSUPPORTED, "head_dim %d unsupported (32, 64, 128, 256)", D);
  }
  if (p->max_chunk_len > (1 << 30) || p->max_kv_len > (1 << 30) || p->bias_len > (1 << 20))
    return fail(CPATTN_EUNSUPPORTED, "length bound too large");
  if (p->q_rows > (int64_t(1) << 31) || p->kv_rows > (int64_t(1) << 31))
    return fail(CPATTN_EUNSUPPORTED, "row count exceeds 2^31 (chunk map rows are int32)");
  pl.D = D;
  pl.G = p->hq / p->hkv;
  pl.hpw = (pl.G % 4 == 0) ? 4 : (pl.G % 2 == 0) ? 2 : 1;
  if (p->q_head_pitch < 0 || (p->q_head_pitch > 0 && p->q_head_pitch < p->hq) || p->kv_head_pitch < 0 ||
      (p->kv_head_pitch > 0 && p->kv_head_pitch < p->hkv))
    return fail(CPATTN_EINVAL, "head pitches (%d, %d) below the head counts (%d, %d)", p->q_head_pitch,
                p->kv_head_pitch, p->hq, p->hkv);
  pl.hq = p->hq;
  pl.hkv = p->hkv;
  pl.qp = p->q_head_pitch > 0 ? p->q_head_pitch : p->hq;
  pl.kvp = p->kv_head_pitch > 0 ? p->kv_head_pitch : p->hkv;
  // a K/V tile's row offsets are 32-bit byte offsets (64 rows x 4096 heads x 512 B < 2^32)
  if (pl.qp > 4096 || pl.kvp > 4096) return fail(CPATTN_EUNSUPPORTED, "more than 4096 heads per row");
  // bytes from the first element of a Q-side (K/V-side) tensor to the end of its last head
  pl.q_bytes = p->q_rows > 0 ? ((p->q_rows - 1) * pl.qp + p->hq) * (int64_t)D * 2 : 0;
  pl.kv_bytes = p->kv_rows > 0 ? ((p->kv_rows - 1) * pl.kvp + p->hkv) * (int64_t)D * 2 : 0;
  pl.stat_bytes = (int64_t)p->hq * p->q_rows * 4;
  pl.bias_bytes = pl.bias ? (int64_t)p->hq * p->bias_len * p->bias_len * 4 : 0;
  pl.delta_bytes = round256(pl.stat_bytes);

  // dQ (forming dS again): four waves of 32 rows; the forward: fwd_waves(D) waves
  const int64_t pos_per_wg = 32 * (4 / pl.hpw);
  pl.bpc_fwd = (int)cdiv(p->max_chunk_len, pos_per_wg);
  pl.bpc_fwdk = (int)cdiv(p->max_chunk_len, (int64_t)32 * (fwd_waves(D) / pl.hpw));
  pl.bpc_prepass = (int)cdiv(p->max_chunk_len, kPrepassRows);
  pl.kv_tiles = (int)cdiv(p->max_kv_len, kDkdvKeys);
  const int64_t gx_fwd = (int64_t)p->num_chunks * pl.bpc_fwd;
  const int64_t gx_pre = (int64_t)p->num_chunks * pl.bpc_prepass;
  // causal: a dK/dV workgroup takes key tiles j and n - 1 - j of its sequence
  pl.kv_slots = p->causal ? (int)cdiv(pl.kv_tiles, 2) : pl.kv_tiles;
  const int64_t gx_kv = (int64_t)p->num_seqs * pl.kv_slots;
  if (gx_fwd > kGridMax || gx_pre > kGridMax || gx_kv > kGridMax || p->hq / pl.hpw > 65535 ||
      p->hkv > 65535)
    return fail(CPATTN_EUNSUPPORTED, "problem too large for one launch");
  pl.grid_fwd = dim3((unsigned)gx_fwd, (unsigned)(p->hq / pl.hpw));
  if (gx_fwd * (p->hq / pl.hpw) > kGridMax) return fail(CPATTN_EUNSUPPORTED, "problem too large for one launch");
  pl.grid_fwd1d = dim3((unsigned)(gx_fwd * (p->hq / pl.hpw)));
  pl.grid_fwdk = dim3((unsigned)((int64_t)p->num_chunks * pl.bpc_fwdk * (p->hq / pl.hpw)));
  if (gx_kv * p->hkv > kGridMax) return fail(CPATTN_EUNSUPPORTED, "problem too large for one launch");
  pl.grid_dkdv = dim3((unsigned)(gx_kv * p->hkv));

  pl.parts = 1;
  pl.partial_bytes = 0;
  if (pl.bias) {
    // The rows are reduced in `parts` units of consecutive chunks, each unit's partial
    // summed in chunk order and the units' partials added in unit order.  The unit
    // count depends on the bias size and the chunk count only, never on the heads of
    // the call, so head-group calls and the call over all heads give the same bits.
    const int64_t tiles_per_head = cdiv(p->bias_len, kDbiasKeys) * cdiv(p->bias_len, kDbiasPos);
    const int64_t parts = std::max<int64_t>(
        1, std::min<int64_t>({cdiv(512, tiles_per_head), 16, std::max(1, p->num_chunks)}));
    pl.parts = (int)parts;
    if (pl.parts > 1) pl.partial_bytes = round256((int64_t)pl.parts * pl.bias_bytes);
    pl.grid_dbias = dim3((unsigned)(cdiv(p->bias_len, kDbiasKeys) * pl.parts),
                         (unsigned)cdiv(p->bias_len, kDbiasPos), (unsigned)p->hq);
    // from the stored dS: 32-key blocks x parts, 32-position tiles, heads (same units)
    if (cdiv(p->bias_len, 32) > 65535 || cdiv(p->bias_len, 32) * pl.parts > kGridMax)
      return fail(CPATTN_EUNSUPPORTED, "bias too large for one launch");
    pl.grid_dbias_ds = dim3((unsigned)(cdiv(p->bias_len, 32) * pl.parts),
                            (unsigned)cdiv(p->bias_len, 32), (unsigned)p->hq);
  }
  // Transposed 32-query tiles: at most ceil(q_rows/32) + C of them.
  const int64_t max_tiles = cdiv(p->q_rows, kPrepassRows) + p->num_chunks;
  const int64_t tile_bytes = max_tiles * p->hq * (int64_t)D * kPrepassRows * 2;
  pl.off_qt = pl.delta_bytes;
  pl.off_dot = pl.off_qt + round256(tile_bytes);
  // per tile and head: log2(e) LSE of its 32 rows, then their Delta (fp32)
  pl.off_stats = pl.off_dot + round256(tile_bytes);
  pl.off_partials = pl.off_stats + round256(max_tiles * p->hq * 64 * 4);
  pl.ws_core = pl.off_partials;
  // the pre-pass numbers its workgroups linearly (head fastest)
  if (gx_pre * p->hq > kGridMax) return fail(CPATTN_EUNSUPPORTED, "problem too large for one launch");
  pl.grid_prepass = dim3((unsigned)gx_pre, (unsigned)p->hq);
  // Stored dS: 2 KB per (chunk tile, head, 32-key block the chunk sees), the chunks'
  // block count promised in ds_blocks (checked on the device); without a promise every
  // tile slot is sized for the longest sequence.
  if (p->ds_blocks < 0) return fail(CPATTN_EINVAL, "ds_blocks is negative");
  pl.ds_ok = D >= 32;
  pl.ds_head_blocks = p->ds_blocks > 0 ? p->ds_blocks : max_tiles * cdiv(p->max_kv_len, kDsBlockKeys);
  if (pl.ds_head_blocks > (int64_t(1) << 40) / std::max(1, p->hq))
    return fail(CPATTN_EUNSUPPORTED, "dS store too large");
  pl.off_ds = pl.ws_core + pl.partial_bytes;
  pl.off_ds_zero = pl.off_ds + round256((int64_t)p->num_chunks * 8);
  pl.off_ds_blocks = pl.off_ds_zero + kDsBlockKeys * kPrepassRows * 2;
  pl.ds_bytes = pl.ds_ok ? (pl.off_ds_blocks - pl.off_ds) +
                               round256(pl.ds_head_blocks * p->hq * kDsBlockKeys * kPrepassRows * 2)
                         : 0;
  pl.bpc_dqds = (int)cdiv(p->max_chunk_len, (int64_t)kDqDsRows * (4 / pl.hpw));
  const int64_t gx_dqds = (int64_t)p->num_chunks * pl.bpc_dqds * (p->hq / pl.hpw);
  if (gx_dqds > kGridMax) return fail(CPATTN_EUNSUPPORTED, "problem too large for one launch");
  pl.grid_dqds = dim3((unsigned)gx_dqds);
  return CPATTN_OK;
}

AttnArgs base_args(const cpattn_problem* p, const Plan& pl) {
  AttnArgs a{};
  a.q_rows = p->q_rows;
  a.num_seqs = p->num_seqs;
  a.num_chunks = p->num_chunks;
  a.hq = p->hq;
  a.hkv = p->hkv;
  a.group = pl.G;
  a.hpw = pl.hpw;
  a.kv_tiles = pl.kv_tiles;
  a.bias_len = p->bias_len;
  a.parts = pl.parts;
  a.scale = p->scale;
  a.scale_log2 = p->scale * kLog2e;
  a.q_pitch = pl.qp;
  a.kv_pitch = pl.kvp;
  a.kv_lo = 0;
  a.kv_hi = INT_MAX;
  a.dq_accumulate = 0;
  return a;
}

int check_descriptors(const cpattn_problem* p, const int32_t* so, const int32_t* sl, const int32_t* cm,
                      const int32_t* dev_err) {
  int r;
  if ((r = check_ptr(so, (uint64_t)p->num_seqs * 4, 4, "seq_offsets"))) return r;
  if ((r = check_ptr(sl, (uint64_t)p->num_seqs * 4, 4, "seq_lens"))) return r;
  if ((r = check_ptr(cm, (uint64_t)p->num_chunks * 16, 16, "q_chunk_map"))) return r;
  if ((r = check_ptr(dev_err, 4, 4, "dev_err"))) return r;
  return CPATTN_OK;
}

void add_descriptor_ranges(std::vector<Range>& rs, const cpattn_problem* p, const int32_t* so,
                           const int32_t* sl, const int32_t* cm, const int32_t* dev_err,
                           bool dev_err_written) {
  rs.push_back(rng("seq_offsets", so, (uint64_t)p->num_seqs * 4, false));
  rs.push_back(rng("seq_lens", sl, (uint64_t)p->num_seqs * 4, false));
  rs.push_back(rng("q_chunk_map", cm, (uint64_t)p->num_chunks * 16, false));
  rs.push_back(rng("dev_err", dev_err, 4, dev_err_written));
}

int run_validate(const cpattn_problem* p, const int32_t* so, const int32_t* sl, const int32_t* cm,
                 int32_t* dev_err, hipStream_t s) {
  ValidateArgs v{};
  v.seq_offsets = so;
  v.seq_lens = sl;
  v.chunks = cm;
  v.dev_err = dev_err;
  v.rows = p->kv_rows;
  v.q_rows = p->q_rows;
  v.num_seqs = p->num_seqs;
  v.num_chunks = p->num_chunks;
  v.max_chunk_len = p->max_chunk_len;
  v.max_kv_len = p->max_kv_len;
  v.bias_len = p->bias_len;
  v.s_pitch = 0;
  v.causal = p->causal;
  v.ds_blocks = p->ds_blocks;
  return hip_check(launch_validate(v, s), "validate launch");
}

bool empty(dim3 g) { return g.x == 0 || g.y == 0 || g.z == 0; }

}  // namespace

extern "C" {

const char* cpattn_status_str(int status) {
  switch (status) {
    case CPATTN_OK: return "CPATTN_OK";
    case CPATTN_EINVAL: return "CPATTN_EINVAL: invalid argument";
    case CPATTN_EUNSUPPORTED: return "CPATTN_EUNSUPPORTED: unsupported problem";
    case CPATTN_EHIP: return "CPATTN_EHIP: HIP runtime error";
    default: return "unknown cpattn status";
  }
}

const char* cpattn_last_error(void) { return g_last_error.c_str(); }

__attribute__((visibility("hidden"))) int cpattn_internal_fail(int status, const char* msg) {
  return fail(status, "%s", msg);
}

int cpattn_version(void) { return 10100; }

size_t cpattn_workspace_size(const cpattn_problem* p, int op) {
  Plan pl;
  if (make_plan(p, pl)) return 0;
  if (op == CPATTN_OP_FWD) return 0;
  if (op == CPATTN_OP_BWD) return (size_t)(pl.ws_core + pl.partial_bytes);
  if (op == CPATTN_OP_BWD_DS) return pl.ds_ok ? (size_t)(pl.off_ds + pl.ds_bytes) : 0;
  return 0;
}

int cpattn_validate(const cpattn_problem* p, const int32_t* seq_offsets, const int32_t* seq_lens,
                    const int32_t* q_chunk_map, int32_t* dev_err, cpattn_stream_t stream) {
  g_last_error.clear();
  Plan pl;
  int r;
  if ((r = make_plan(p, pl))) return r;
  if ((r = check_descriptors(p, seq_offsets, seq_lens, q_chunk_map, dev_err))) return r;
  std::vector<Range> rs;
  add_descriptor_ranges(rs, p, seq_offsets, seq_lens, q_chunk_map, dev_err, true);
  if ((r = alias_audit(rs))) return r;
  return run_validate(p, seq_offsets, seq_lens, q_chunk_map, dev_err, (hipStream_t)stream);
}

namespace {
int fwd_impl(const cpattn_problem* p, const void* q, const void* k, const void* v,
             const int32_t* seq_offsets, const int32_t* seq_lens, const int32_t* q_chunk_map,
             const float* bias, int32_t kv_lo, int32_t kv_hi, void* o, float* lse,
             int32_t* dev_err, cpattn_stream_t stream) {
  g_last_error.clear();
  Plan pl;
  int r;
  if ((r = make_plan(p, pl))) return r;
  if ((r = check_ptr(q, pl.q_bytes, 16, "q")) || (r = check_ptr(k, pl.kv_bytes, 16, "k")) ||
      (r = check_ptr(v, pl.kv_bytes, 16, "v")) || (r = check_ptr(o, pl.q_bytes, 16, "o")) ||
      (r = check_ptr(lse, pl.stat_bytes, 4, "lse")) ||
      (r = check_ptr(bias, pl.bias_bytes, 16, "bias")))
    return r;
  if (!pl.bias && bias) return fail(CPATTN_EINVAL, "bias given but bias_len is 0");
  if (kv_lo < 0 || kv_hi < kv_lo) return fail(CPATTN_EINVAL, "key window [%d, %d) is invalid", kv_lo, kv_hi);
  if ((r = check_descriptors(p, seq_offsets, seq_lens, q_chunk_map, dev_err))) return r;
  std::vector<Range> rs = {rq(pl, "q", q, false), rkv(pl, "k", k, false),
                           rkv(pl, "v", v, false), rng("bias", bias, pl.bias_bytes, false),
                           rq(pl, "o", o, true), rng("lse", lse, pl.stat_bytes, true)};
  add_descriptor_ranges(rs, p, seq_offsets, seq_lens, q_chunk_map, dev_err, true);
  if ((r = alias_audit(rs))) return r;

  hipStream_t s = (hipStream_t)stream;
  if ((r = run_validate(p, seq_offsets, seq_lens, q_chunk_map, dev_err, s))) return r;
  if (empty(pl.grid_fwdk)) return CPATTN_OK;
  AttnArgs a = base_args(p, pl);
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.bias = bias;
  a.o_out = (uint16_t*)o;
  a.lse_out = lse;
  a.seq_offsets = seq_offsets;
  a.seq_lens = seq_lens;
  a.chunks = q_chunk_map;
  a.dev_err = dev_err;
  a.blocks_per_chunk = pl.bpc_fwdk;
  a.kv_lo = kv_lo;
  a.kv_hi = kv_hi;
  return hip_check(launch_fwd(a, pl.D, p->causal != 0, pl.bias, pl.grid_fwdk, s), "forward launch");
}
}  // namespace

int cpattn_fwd(const cpattn_problem* p, const void* q, const void* k, const void* v,
               const int32_t* seq_offsets, const int32_t* seq_lens, const int32_t* q_chunk_map,
               const float* bias, void* o, float* lse, void* ws, size_t ws_bytes,
               int32_t* dev_err, cpattn_stream_t stream) {
  (void)ws;
  (void)ws_bytes;
  return fwd_impl(p, q, k, v, seq_offsets, seq_lens, q_chunk_map, bias, 0, INT_MAX, o, lse, dev_err,
                  stream);
}

int cpattn_fwd_window(const cpattn_problem* p, const void* q, const void* k, const void* v,
                      const int32_t* seq_offsets, const int32_t* seq_lens,
                      const int32_t* q_chunk_map, const float* bias, int32_t kv_lo, int32_t kv_hi,
                      void* o, float* lse, int32_t* dev_err, cpattn_stream_t stream) {
  return fwd_impl(p, q, k, v, seq_offsets, seq_lens, q_chunk_map, bias, kv_lo, kv_hi, o, lse, dev_err,
                  stream);
}

int cpattn_merge(const cpattn_problem* p, const int32_t* q_chunk_map, const void* o_a,
                 const float* lse_a, const void* o_b, const float* lse_b, void* o, float* lse,
                 const int32_t* dev_err, cpattn_stream_t stream) {
  g_last_error.clear();
  Plan pl;
  int r;
  if ((r = make_plan(p, pl))) return r;
  if ((r = check_ptr(o_a, pl.q_bytes, 16, "o_a")) || (r = check_ptr(o_b, pl.q_bytes, 16, "o_b")) ||
      (r = check_ptr(o, pl.q_bytes, 16, "o")) || (r = check_ptr(lse_a, pl.stat_bytes, 4, "lse_a")) ||
      (r = check_ptr(lse_b, pl.stat_bytes, 4, "lse_b")) || (r = check_ptr(lse, pl.stat_bytes, 4, "lse")) ||
      (r = check_ptr(q_chunk_map, (uint64_t)p->num_chunks * 16, 16, "q_chunk_map")) ||
      (r = check_ptr(dev_err, 4, 4, "dev_err")))
    return r;
  // o may be o_a and lse may be lse_a (the running result updated in place); every other
  // overlap is rejected.
  std::vector<Range> rs = {rq(pl, "o_b", o_b, false), rng("lse_b", lse_b, pl.stat_bytes, false),
                           rq(pl, "o", o, true), rng("lse", lse, pl.stat_bytes, true),
                           rng("q_chunk_map", q_chunk_map, (uint64_t)p->num_chunks * 16, false),
                           rng("dev_err", dev_err, 4, false)};
  if (o_a != o) rs.push_back(rq(pl, "o_a", o_a, false));
  if (lse_a != lse) rs.push_back(rng("lse_a", lse_a, pl.stat_bytes, false));
  if ((r = alias_audit(rs))) return r;
  const int pairs_per_wg = kThreads / (pl.D / 8);
  const int64_t bpc = cdiv((int64_t)p->max_chunk_len * p->hq, pairs_per_wg);
  const int64_t gx = (int64_t)p->num_chunks * bpc;
  if (gx > kGridMax) return fail(CPATTN_EUNSUPPORTED, "problem too large for one launch");
  if (gx == 0) return CPATTN_OK;
  MergeArgs m{};
  m.o_a = (const uint16_t*)o_a;
  m.lse_a = lse_a;
  m.o_b = (const uint16_t*)o_b;
  m.lse_b = lse_b;
  m.o = (uint16_t*)o;
  m.lse = lse;
  m.chunks = q_chunk_map;
  m.dev_err = dev_err;
  m.q_rows = p->q_rows;
  m.hq = p->hq;
  m.q_pitch = pl.qp;
  m.D = pl.D;
  m.blocks_per_chunk = (int)bpc;
  return hip_check(launch_merge(m, dim3((unsigned)gx), (hipStream_t)stream), "merge launch");
}

// ---------------------------------------------------------------- backward steps

namespace {

int bwd_common_checks(const cpattn_problem* p, const Plan& pl, const void* q, const void* k,
                      const void* v, const float* bias, const float* lse, const void* dout,
                      const int32_t* so, const int32_t* sl, const int32_t* cm, const int32_t* dev_err) {
  int r;
  if ((r = check_ptr(q, pl.q_bytes, 16, "q")) || (r = check_ptr(k, pl.kv_bytes, 16, "k")) ||
      (r = check_ptr(v, pl.kv_bytes, 16, "v")) || (r = check_ptr(lse, pl.stat_bytes, 4, "lse")) ||
      (r = check_ptr(dout, pl.q_bytes, 16, "dout")) ||
      (r = check_ptr(bias, pl.bias_bytes, 16, "bias")))
    return r;
  if (!pl.bias && bias) return fail(CPATTN_EINVAL, "bias given but bias_len is 0");
  return check_descriptors(p, so, sl, cm, dev_err);
}

AttnArgs bwd_args(const cpattn_problem* p, const Plan& pl, const void* q, const void* k, const void* v,
                  const int32_t* so, const int32_t* sl, const int32_t* cm, const float* bias,
                  const float* lse, const void* dout, const void* ws, const int32_t* dev_err) {
  AttnArgs a = base_args(p, pl);
  const char* w = (const char*)ws;
  const float* delta = (const float*)w;
  a.qt = (const uint16_t*)(w + pl.off_qt);
  a.dot = (const uint16_t*)(w + pl.off_dot);
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.bias = bias;
  a.lse = lse;
  a.dout = (const uint16_t*)dout;
  a.delta = delta;
  a.stats = (const float*)(w + pl.off_stats);
  a.seq_offsets = so;
  a.seq_lens = sl;
  a.chunks = cm;
  a.dev_err = dev_err;
  return a;
}

int enqueue_prepass(const cpattn_problem* p, const Plan& pl, const int32_t* cm, const void* q,
                    const void* o, const void* dout, const float* lse, void* ws, const int32_t* dev_err,
                    hipStream_t s) {
  AttnArgs a = base_args(p, pl);
  char* w = (char*)ws;
  a.q = (const uint16_t*)q;
  a.o = (const uint16_t*)o;
  a.dout = (const uint16_t*)dout;
  a.delta_out = (float*)w;
  a.qt_out = (uint16_t*)(w + pl.off_qt);
  a.dot_out = (uint16_t*)(w + pl.off_dot);
  a.stats_out = (float*)(w + pl.off_stats);
  a.lse = lse;
  a.chunks = cm;
  a.dev_err = dev_err;
  a.blocks_per_chunk = pl.bpc_prepass;
  if (empty(pl.grid_prepass)) return CPATTN_OK;
  return hip_check(launch_prepass(a, pl.D, pl.grid_prepass, s), "pre-pass launch");
}

// ds_area: the dS part of the workspace (offsets, then blocks), or null to store no dS.
int enqueue_dkdv(const cpattn_problem* p, const Plan& pl, AttnArgs a, void* dk, void* dv, int acc,
                 hipStream_t s, void* ds_area = nullptr) {
  if (empty(pl.grid_dkdv)) return CPATTN_OK;
  a.dk = (uint16_t*)dk;
  a.dv = (uint16_t*)dv;
  a.accumulate = acc ? 1 : 0;
  a.kv_tiles = pl.kv_slots;
  a.kv_pair = pl.kv_slots != pl.kv_tiles;
  if (ds_area) {
    DsTableArgs t{};
    t.seq_lens = a.seq_lens;
    t.chunks = a.chunks;
    t.dev_err = a.dev_err;
    t.tab = (int64_t*)ds_area;
    t.zero = (uint16_t*)((char*)ds_area + (pl.off_ds_zero - pl.off_ds));
    t.num_chunks = p->num_chunks;
    t.causal = p->causal;
    int r = hip_check(launch_ds_table(t, s), "dS table launch");
    if (r) return r;
    a.ds_tab = (const int64_t*)ds_area;
    a.ds_out = (uint16_t*)((char*)ds_area + (pl.off_ds_blocks - pl.off_ds));
  }
  return hip_check(launch_dkdv(a, pl.D, p->causal != 0, pl.bias, pl.grid_dkdv, s), "dK/dV launch");
}

int enqueue_dq(const cpattn_problem* p, const Plan& pl, AttnArgs a, void* dq, hipStream_t s) {
  if (empty(pl.grid_fwd1d)) return CPATTN_OK;
  a.dq = (uint16_t*)dq;
  a.blocks_per_chunk = pl.bpc_fwd;
  return hip_check(launch_dq(a, pl.D, p->causal != 0, pl.bias, pl.grid_fwd1d, s), "dQ launch");
}

int enqueue_dq_ds(const cpattn_problem* p, const Plan& pl, AttnArgs a, const void* ws, void* dq,
                  hipStream_t s) {
  if (empty(pl.grid_dqds)) return CPATTN_OK;
  a.dq = (uint16_t*)dq;
  a.ds_tab = (const int64_t*)((const char*)ws + pl.off_ds);
  a.ds_zero = (const uint16_t*)((const char*)ws + pl.off_ds_zero);
  a.ds = (const uint16_t*)((const char*)ws + pl.off_ds_blocks);
  a.blocks_per_chunk = pl.bpc_dqds;
  return hip_check(launch_dq_ds(a, pl.D, p->causal != 0, pl.grid_dqds, s), "dQ (stored dS) launch");
}

int enqueue_dbias(const cpattn_problem* p, const Plan& pl, AttnArgs a, float* dbias, void* ws,
                  hipStream_t s) {
  if (!pl.bias || empty(pl.grid_dbias)) return CPATTN_OK;
  float* partial = pl.parts > 1 ? (float*)((char*)ws + pl.off_partials) : dbias;
  a.dbias = partial;
  int r = hip_check(launch_dbias(a, pl.D, pl.grid_dbias, s), "dBias launch");
  if (r || pl.parts == 1) return r;
  return hip_check(launch_dbias_reduce(partial, dbias, pl.bias_bytes / 4, pl.parts, a.dev_err, s),
                   "dBias reduce launch");
}

// dBias as a sum over the dS blocks that dK/dV stored (same units and order of the
// partial sums as enqueue_dbias).
int enqueue_dbias_ds(const cpattn_problem* p, const Plan& pl, AttnArgs a, float* dbias, const void* ws,
                     hipStream_t s) {
  if (!pl.bias || empty(pl.grid_dbias_ds)) return CPATTN_OK;
  float* partial = pl.parts > 1 ? (float*)((char*)ws + pl.off_partials) : dbias;
  a.dbias = partial;
  a.ds_tab = (const int64_t*)((const char*)ws + pl.off_ds);
  a.ds = (const uint16_t*)((const char*)ws + pl.off_ds_blocks);
  int r = hip_check(launch_dbias_ds(a, pl.grid_dbias_ds, s), "dBias (stored dS) launch");
  if (r || pl.parts == 1) return r;
  return hip_check(launch_dbias_reduce(partial, dbias, pl.bias_bytes / 4, pl.parts, a.dev_err, s),
                   "dBias reduce launch");
}

}  // namespace

int cpattn_bwd(const cpattn_problem* p, const void* q, const void* k, const void* v,
               const int32_t* seq_offsets, const int32_t* seq_lens, const int32_t* q_chunk_map,
               const float* bias, const void* o, const float* lse, const void* dout,
               void* dq, void* dk, void* dv, float* dbias, int dkv_accumulate,
               void* ws, size_t ws_bytes, int32_t* dev_err, cpattn_stream_t stream) {
  g_last_error.clear();
  Plan pl;
  int r;
  if ((r = make_plan(p, pl))) return r;
  if ((r = bwd_common_checks(p, pl, q, k, v, bias, lse, dout, seq_offsets, seq_lens, q_chunk_map,
                             dev_err)))
    return r;
  if ((r = check_ptr(o, pl.q_bytes, 16, "o")) || (r = check_ptr(dq, pl.q_bytes, 16, "dq")) ||
      (r = check_ptr(dk, pl.kv_bytes, 16, "dk")) || (r = check_ptr(dv, pl.kv_bytes, 16, "dv")))
    return r;
  if (dbias && !pl.bias) return fail(CPATTN_EINVAL, "dbias given but bias_len is 0");
  if (dbias && !aligned(dbias, 16)) return fail(CPATTN_EINVAL, "dbias is not 16-byte aligned");
  if (dkv_accumulate != 0 && dkv_accumulate != 1) return fail(CPATTN_EINVAL, "dkv_accumulate must be 0 or 1");
  // With room for the dS store, dK/dV stores dS and dQ multiplies it (no recompute).
  const bool use_ds = pl.ds_ok && (int64_t)ws_bytes >= pl.off_ds + pl.ds_bytes;
  const int64_t need = use_ds ? pl.off_ds + pl.ds_bytes : pl.ws_core + (dbias ? pl.partial_bytes : 0);
  if ((int64_t)ws_bytes < need) return fail(CPATTN_EINVAL, "workspace too small: %zu < %lld", ws_bytes, (long long)need);
  if ((r = check_ptr(ws, need, 256, "ws"))) return r;
  const int64_t dbias_bytes = dbias ? pl.bias_bytes : 0;
  std::vector<Range> rs = {rq(pl, "q", q, false),        rkv(pl, "k", k, false),
                           rkv(pl, "v", v, false),        rng("bias", bias, pl.bias_bytes, false),
                           rq(pl, "o", o, false),         rng("lse", lse, pl.stat_bytes, false),
                           rq(pl, "dout", dout, false),   rq(pl, "dq", dq, true),
                           rkv(pl, "dk", dk, true),       rkv(pl, "dv", dv, true),
                           rng("dbias", dbias, dbias_bytes, true), rng("ws", ws, need, true)};
  add_descriptor_ranges(rs, p, seq_offsets, seq_lens, q_chunk_map, dev_err, true);
  if ((r = alias_audit(rs))) return r;

  hipStream_t s = (hipStream_t)stream;
  if ((r = run_validate(p, seq_offsets, seq_lens, q_chunk_map, dev_err, s))) return r;
  if ((r = enqueue_prepass(p, pl, q_chunk_map, q, o, dout, lse, ws, dev_err, s))) return r;
  AttnArgs a = bwd_args(p, pl, q, k, v, seq_offsets, seq_lens, q_chunk_map, bias, lse, dout, ws, dev_err);
  if (use_ds) {
    if ((r = enqueue_dkdv(p, pl, a, dk, dv, dkv_accumulate, s, (char*)ws + pl.off_ds))) return r;
    if ((r = enqueue_dq_ds(p, pl, a, ws, dq, s))) return r;
  } else {
    if ((r = enqueue_dkdv(p, pl, a, dk, dv, dkv_accumulate, s))) return r;
    if ((r = enqueue_dq(p, pl, a, dq, s))) return r;
  }
  // dBias from dS formed in fp32 on either path (the stored dS is BF16, and a sum of
  // many rows of it drifts by their rounding errors)
  if (dbias) return enqueue_dbias(p, pl, a, dbias, ws, s);
  return CPATTN_OK;
}

int cpattn_bwd_window(const cpattn_problem* p, const void* q, const void* k, const void* v,
                      const int32_t* seq_offsets, const int32_t* seq_lens,
                      const int32_t* q_chunk_map, const float* bias, const void* o, const float* lse,
                      const void* dout, int32_t kv_lo, int32_t kv_hi, int prepass, void* dq,
                      int dq_accumulate, void* dk, void* dv, int dkv_accumulate, void* ws,
                      size_t ws_bytes, int32_t* dev_err, cpattn_stream_t stream) {
  g_last_error.clear();
  Plan pl;
  int r;
  if ((r = make_plan(p, pl))) return r;
  if ((r = bwd_common_checks(p, pl, q, k, v, bias, lse, dout, seq_offsets, seq_lens, q_chunk_map,
                             dev_err)))
    return r;
  if ((r = check_ptr(o, pl.q_bytes, 16, "o")) || (r = check_ptr(dq, pl.q_bytes, 16, "dq")) ||
      (r = check_ptr(dk, pl.kv_bytes, 16, "dk")) || (r = check_ptr(dv, pl.kv_bytes, 16, "dv")))
    return r;
  if (kv_lo < 0 || kv_hi < kv_lo) return fail(CPATTN_EINVAL, "key window [%d, %d) is invalid", kv_lo, kv_hi);
  if ((prepass != 0 && prepass != 1) || (dq_accumulate != 0 && dq_accumulate != 1) ||
      (dkv_accumulate != 0 && dkv_accumulate != 1))
    return fail(CPATTN_EINVAL, "prepass, dq_accumulate and dkv_accumulate must be 0 or 1");
  if ((int64_t)ws_bytes < pl.ws_core)
    return fail(CPATTN_EINVAL, "workspace too small: %zu < %lld", ws_bytes, (long long)pl.ws_core);
  // With room for the dS store, dK/dV store the window's dS and the dQ share multiplies it.
  const bool use_ds = pl.ds_ok && (int64_t)ws_bytes >= pl.off_ds + pl.ds_bytes;
  const int64_t ws_used = use_ds ? pl.off_ds + pl.ds_bytes : pl.ws_core;
  if ((r = check_ptr(ws, ws_used, 256, "ws"))) return r;
  std::vector<Range> rs = {rq(pl, "q", q, false),        rkv(pl, "k", k, false),
                           rkv(pl, "v", v, false),        rng("bias", bias, pl.bias_bytes, false),
                           rq(pl, "o", o, false),         rng("lse", lse, pl.stat_bytes, false),
                           rq(pl, "dout", dout, false),   rq(pl, "dq", dq, true),
                           rkv(pl, "dk", dk, true),       rkv(pl, "dv", dv, true),
                           rng("ws", ws, pl.ws_core, prepass != 0)};
  if (use_ds) rs.push_back(rng("ws (dS area)", (char*)ws + pl.off_ds, pl.ds_bytes, true));
  add_descriptor_ranges(rs, p, seq_offsets, seq_lens, q_chunk_map, dev_err, prepass != 0);
  if ((r = alias_audit(rs))) return r;

  hipStream_t s = (hipStream_t)stream;
  if (prepass) {
    if ((r = run_validate(p, seq_offsets, seq_lens, q_chunk_map, dev_err, s))) return r;
    if ((r = enqueue_prepass(p, pl, q_chunk_map, q, o, dout, lse, ws, dev_err, s))) return r;
  }
  AttnArgs a = bwd_args(p, pl, q, k, v, seq_offsets, seq_lens, q_chunk_map, bias, lse, dout, ws, dev_err);
  a.kv_lo = kv_lo;
  a.kv_hi = kv_hi;
  a.dq_accumulate = dq_accumulate;
  if (use_ds) {
    if ((r = enqueue_dkdv(p, pl, a, dk, dv, dkv_accumulate, s, (char*)ws + pl.off_ds))) return r;
    return enqueue_dq_ds(p, pl, a, ws, dq, s);
  }
  if ((r = enqueue_dkdv(p, pl, a, dk, dv, dkv_accumulate, s))) return r;
  return enqueue_dq(p, pl, a, dq, s);
}

int cpattn_bwd_prepass(const cpattn_problem* p, const void* q, const int32_t* q_chunk_map,
                       const void* o, const void* dout, const float* lse, void* ws,
                       size_t ws_bytes, const int32_t* dev_err, cpattn_stream_t stream) {
  g_last_error.clear();
  Plan pl;
  int r;
  if ((r = make_plan(p, pl))) return r;
  if ((r = check_ptr(q, pl.q_bytes, 16, "q")) || (r = check_ptr(o, pl.q_bytes, 16, "o")) ||
      (r = check_ptr(dout, pl.q_bytes, 16, "dout")) || (r = check_ptr(lse, pl.stat_bytes, 4, "lse")) ||
      (r = check_ptr(q_chunk_map, (uint64_t)p->num_chunks * 16, 16, "q_chunk_map")) ||
      (r = check_ptr(dev_err, 4, 4, "dev_err")))
    return r;
  if ((int64_t)ws_bytes < pl.ws_core)
    return fail(CPATTN_EINVAL, "workspace too small: %zu < %lld", ws_bytes, (long long)pl.ws_core);
  if ((r = check_ptr(ws, pl.ws_core, 256, "ws"))) return r;
  std::vector<Range> rs = {rq(pl, "q", q, false), rq(pl, "o", o, false),
                           rq(pl, "dout", dout, false), rng("lse", lse, pl.stat_bytes, false),
                           rng("q_chunk_map", q_chunk_map, (uint64_t)p->num_chunks * 16, false),
                           rng("dev_err", dev_err, 4, false), rng("ws", ws, pl.ws_core, true)};
  if ((r = alias_audit(rs))) return r;
  return enqueue_prepass(p, pl, q_chunk_map, q, o, dout, lse, ws, dev_err, (hipStream_t)stream);
}

namespace {
// Shared checks of the dK/dV, dQ and dBias steps, which read the pre-pass workspace.
int step_checks(const cpattn_problem* p, const Plan& pl, const void* q, const void* k, const void* v,
                const int32_t* so, const int32_t* sl, const int32_t* cm, const float* bias,
                const float* lse, const void* dout, const void* ws, size_t ws_bytes, int64_t need,
                const int32_t* dev_err, std::vector<Range>& rs) {
  int r;
  if ((r = bwd_common_checks(p, pl, q, k, v, bias, lse, dout, so, sl, cm, dev_err))) return r;
  if ((int64_t)ws_bytes < need) return fail(CPATTN_EINVAL, "workspace too small: %zu < %lld", ws_bytes, (long long)need);
  if ((r = check_ptr(ws, need, 256, "ws"))) return r;
  rs = {rq(pl, "q", q, false),       rkv(pl, "k", k, false),
        rkv(pl, "v", v, false),       rng("bias", bias, pl.bias_bytes, false),
        rng("lse", lse, pl.stat_bytes, false), rq(pl, "dout", dout, false),
        rng("ws (pre-pass results)", ws, pl.ws_core, false)};
  add_descriptor_ranges(rs, p, so, sl, cm, dev_err, false);
  return CPATTN_OK;
}
}  // namespace

int cpattn_bwd_dkdv(const cpattn_problem* p, const void* q, const void* k, const void* v,
                    const int32_t* seq_offsets, const int32_t* seq_lens,
                    const int32_t* q_chunk_map, const float* bias, const float* lse,
                    const void* dout, const void* ws, size_t ws_bytes, void* dk, void* dv,
                    int dkv_accumulate, const int32_t* dev_err, cpattn_stream_t stream) {
  g_last_error.clear();
  Plan pl;
  int r;
  std::vector<Range> rs;
  if ((r = make_plan(p, pl))) return r;
  if ((r = step_checks(p, pl, q, k, v, seq_offsets, seq_lens, q_chunk_map, bias, lse, dout, ws,
                       ws_bytes, pl.ws_core, dev_err, rs)))
    return r;
  if ((r = check_ptr(dk, pl.kv_bytes, 16, "dk")) || (r = check_ptr(dv, pl.kv_bytes, 16, "dv"))) return r;
  if (dkv_accumulate != 0 && dkv_accumulate != 1) return fail(CPATTN_EINVAL, "dkv_accumulate must be 0 or 1");
  rs.push_back(rkv(pl, "dk", dk, true));
  rs.push_back(rkv(pl, "dv", dv, true));
  if ((r = alias_audit(rs))) return r;
  AttnArgs a = bwd_args(p, pl, q, k, v, seq_offsets, seq_lens, q_chunk_map, bias, lse, dout, ws, dev_err);
  return enqueue_dkdv(p, pl, a, dk, dv, dkv_accumulate, (hipStream_t)stream);
}

int cpattn_bwd_dq(const cpattn_problem* p, const void* q, const void* k, const void* v,
                  const int32_t* seq_offsets, const int32_t* seq_lens,
                  const int32_t* q_chunk_map, const float* bias, const float* lse,
                  const void* dout, const void* ws, size_t ws_bytes, void* dq,
                  const int32_t* dev_err, cpattn_stream_t stream) {
  g_last_error.clear();
  Plan pl;
  int r;
  std::vector<Range> rs;
  if ((r = make_plan(p, pl))) return r;
  if ((r = step_checks(p, pl, q, k, v, seq_offsets, seq_lens, q_chunk_map, bias, lse, dout, ws,
                       ws_bytes, pl.ws_core, dev_err, rs)))
    return r;
  if ((r = check_ptr(dq, pl.q_bytes, 16, "dq"))) return r;
  rs.push_back(rq(pl, "dq", dq, true));
  if ((r = alias_audit(rs))) return r;
  AttnArgs a = bwd_args(p, pl, q, k, v, seq_offsets, seq_lens, q_chunk_map, bias, lse, dout, ws, dev_err);
  return enqueue_dq(p, pl, a, dq, (hipStream_t)stream);
}

int cpattn_bwd_dkdv_ds(const cpattn_problem* p, const void* q, const void* k, const void* v,
                       const int32_t* seq_offsets, const int32_t* seq_lens,
                       const int32_t* q_chunk_map, const float* bias, const float* lse,
                       const void* dout, void* ws, size_t ws_bytes, void* dk, void* dv,
                       int dkv_accumulate, const int32_t* dev_err, cpattn_stream_t stream) {
  g_last_error.clear();
  Plan pl;
  int r;
  std::vector<Range> rs;
  if ((r = make_plan(p, pl))) return r;
  if (!pl.ds_ok) return fail(CPATTN_EUNSUPPORTED, "the stored-dS backward needs head_dim >= 32");
  if ((r = step_checks(p, pl, q, k, v, seq_offsets, seq_lens, q_chunk_map, bias, lse, dout, ws,
                       ws_bytes, pl.off_ds + pl.ds_bytes, dev_err, rs)))
    return r;
  if ((r = check_ptr(dk, pl.kv_bytes, 16, "dk")) || (r = check_ptr(dv, pl.kv_bytes, 16, "dv"))) return r;
  if (dkv_accumulate != 0 && dkv_accumulate != 1) return fail(CPATTN_EINVAL, "dkv_accumulate must be 0 or 1");
  rs.push_back(rkv(pl, "dk", dk, true));
  rs.push_back(rkv(pl, "dv", dv, true));
  rs.push_back(rng("ws (dS area)", (char*)ws + pl.off_ds, pl.ds_bytes, true));
  if ((r = alias_audit(rs))) return r;
  AttnArgs a = bwd_args(p, pl, q, k, v, seq_offsets, seq_lens, q_chunk_map, bias, lse, dout, ws, dev_err);
  return enqueue_dkdv(p, pl, a, dk, dv, dkv_accumulate, (hipStream_t)stream, (char*)ws + pl.off_ds);
}

int cpattn_bwd_dq_ds(const cpattn_problem* p, const void* k, const int32_t* seq_offsets,
                     const int32_t* seq_lens, const int32_t* q_chunk_map, const void* ws,
                     size_t ws_bytes, void* dq, const int32_t* dev_err, cpattn_stream_t stream) {
  g_last_error.clear();
  Plan pl;
  int r;
  if ((r = make_plan(p, pl))) return r;
  if (!pl.ds_ok) return fail(CPATTN_EUNSUPPORTED, "the stored-dS backward needs head_dim >= 32");
  if ((r = check_ptr(k, pl.kv_bytes, 16, "k")) || (r = check_ptr(dq, pl.q_bytes, 16, "dq"))) return r;
  if ((r = check_descriptors(p, seq_offsets, seq_lens, q_chunk_map, dev_err))) return r;
  const int64_t need = pl.off_ds + pl.ds_bytes;
  if ((int64_t)ws_bytes < need) return fail(CPATTN_EINVAL, "workspace too small: %zu < %lld", ws_bytes, (long long)need);
  if ((r = check_ptr(ws, need, 256, "ws"))) return r;
  std::vector<Range> rs = {rkv(pl, "k", k, false),
                           rng("ws (dS area)", (const char*)ws + pl.off_ds, pl.ds_bytes, false),
                           rq(pl, "dq", dq, true)};
  add_descriptor_ranges(rs, p, seq_offsets, seq_lens, q_chunk_map, dev_err, false);
  if ((r = alias_audit(rs))) return r;
  AttnArgs a = base_args(p, pl);
  a.k = (const uint16_t*)k;
  a.seq_offsets = seq_offsets;
  a.seq_lens = seq_lens;
  a.chunks = q_chunk_map;
  a.dev_err = dev_err;
  return enqueue_dq_ds(p, pl, a, ws, dq, (hipStream_t)stream);
}

int cpattn_bwd_dbias(const cpattn_problem* p, const void* q, const void* k, const void* v,
                     const int32_t* seq_offsets, const int32_t* seq_lens,
                     const int32_t* q_chunk_map, const float* bias, const float* lse,
                     const void* dout, void* ws, size_t ws_bytes, float* dbias,
                     const int32_t* dev_err, cpattn_stream_t stream) {
  g_last_error.clear();
  Plan pl;
  int r;
  std::vector<Range> rs;
  if ((r = make_plan(p, pl))) return r;
  if (!pl.bias) return fail(CPATTN_EINVAL, "dBias needs a bias (bias_len > 0)");
  if ((r = step_checks(p, pl, q, k, v, seq_offsets, seq_lens, q_chunk_map, bias, lse, dout, ws,
                       ws_bytes, pl.ws_core + pl.partial_bytes, dev_err, rs)))
    return r;
  if ((r = check_ptr(dbias, pl.bias_bytes, 16, "dbias"))) return r;
  rs.push_back(rng("dbias", dbias, pl.bias_bytes, true));
  rs.push_back(rng("ws partials", (char*)ws + pl.off_partials, pl.partial_bytes, true));
  if ((r = alias_audit(rs))) return r;
  AttnArgs a = bwd_args(p, pl, q, k, v, seq_offsets, seq_lens, q_chunk_map, bias, lse, dout, ws, dev_err);
  return enqueue_dbias(p, pl, a, dbias, ws, (hipStream_t)stream);
}

int cpattn_bwd_dbias_ds(const cpattn_problem* p, const int32_t* seq_offsets, const int32_t* seq_lens,
                        const int32_t* q_chunk_map, void* ws, size_t ws_bytes, float* dbias,
                        const int32_t* dev_err, cpattn_stream_t stream) {
  g_last_error.clear();
  Plan pl;
  int r;
  if ((r = make_plan(p, pl))) return r;
  if (!pl.bias) return fail(CPATTN_EINVAL, "dBias needs a bias (bias_len > 0)");
  if (!pl.ds_ok) return fail(CPATTN_EUNSUPPORTED, "the stored-dS backward needs head_dim >= 32");
  if ((r = check_descriptors(p, seq_offsets, seq_lens, q_chunk_map, dev_err))) return r;
  if ((r = check_ptr(dbias, pl.bias_bytes, 16, "dbias"))) return r;
  const int64_t need = pl.off_ds + pl.ds_bytes;
  if ((int64_t)ws_bytes < need) return fail(CPATTN_EINVAL, "workspace too small: %zu < %lld", ws_bytes, (long long)need);
  if ((r = check_ptr(ws, need, 256, "ws"))) return r;
  std::vector<Range> rs = {rng("ws (dS area)", (const char*)ws + pl.off_ds, pl.ds_bytes, false),
                           rng("ws partials", (char*)ws + pl.off_partials, pl.partial_bytes, true),
                           rng("dbias", dbias, pl.bias_bytes, true)};
  add_descriptor_ranges(rs, p, seq_offsets, seq_lens, q_chunk_map, dev_err, false);
  if ((r = alias_audit(rs))) return r;
  AttnArgs a = base_args(p, pl);
  a.seq_offsets = seq_offsets;
  a.seq_lens = seq_lens;
  a.chunks = q_chunk_map;
  a.dev_err = dev_err;
  return enqueue_dbias_ds(p, pl, a, dbias, ws, (hipStream_t)stream);
}

// ---------------------------------------------------------------- layout copies

static int layout_call(const void* src, void* dst, int32_t B, int32_t H, int32_t S_pitch, int32_t D,
                       int64_t thd_rows, const int32_t* so, const int32_t* sl, int32_t* dev_err,
                       hipStream_t s, int unpack) {
  g_last_error.clear();
  if (B < 0 || H <= 0 || S_pitch < 0 || D <= 0 || thd_rows < 0)
    return fail(CPATTN_EINVAL, "bad layout sizes");
  if (D % 8) return fail(CPATTN_EUNSUPPORTED, "D must be a multiple of 8 for the layout copies");
  if (B > 65535) return fail(CPATTN_EUNSUPPORTED, "more than 65535 sequences");
  const int64_t bhsd_bytes = (int64_t)B * H * S_pitch * D * 2;
  const int64_t thd_bytes = thd_rows * H * (int64_t)D * 2;
  int r;
  if ((r = check_ptr(src, unpack ? thd_bytes : bhsd_bytes, 16, "src")) ||
      (r = check_ptr(dst, unpack ? bhsd_bytes : thd_bytes, 16, "dst")) ||
      (r = check_ptr(so, (uint64_t)B * 4, 4, "seq_offsets")) ||
      (r = check_ptr(sl, (uint64_t)B * 4, 4, "seq_lens")) || (r = check_ptr(dev_err, 4, 4, "dev_err")))
    return r;
  std::vector<Range> rs = {rng("src", src, unpack ? thd_bytes : bhsd_bytes, false),
                           rng("dst", dst, unpack ? bhsd_bytes : thd_bytes, true),
                           rng("seq_offsets", so, (uint64_t)B * 4, false),
                           rng("seq_lens", sl, (uint64_t)B * 4, false), rng("dev_err", dev_err, 4, true)};
  if ((r = alias_audit(rs))) return r;
  ValidateArgs v{};
  v.seq_offsets = so;
  v.seq_lens = sl;
  v.chunks = nullptr;
  v.dev_err = dev_err;
  v.rows = thd_rows;
  v.num_seqs = B;
  v.max_kv_len = S_pitch;
  v.s_pitch = S_pitch > 0 ? S_pitch : 1;
  if ((r = hip_check(launch_validate(v, s), "validate launch"))) return r;
  LayoutArgs a{(const uint16_t*)src, (uint16_t*)dst, so, sl, dev_err, B, H, S_pitch, D, unpack};
  return hip_check(launch_layout(a, s), "layout launch");
}

int cpattn_pack(const void* bhsd, void* thd, int32_t B, int32_t H, int32_t S_pitch, int32_t D,
                int64_t thd_rows, const int32_t* seq_offsets, const int32_t* seq_lens,
                int32_t* dev_err, cpattn_stream_t stream) {
  return layout_call(bhsd, thd, B, H, S_pitch, D, thd_rows, seq_offsets, seq_lens, dev_err,
                     (hipStream_t)stream, 0);
}

int cpattn_unpack(const void* thd, void* bhsd, int32_t B, int32_t H, int32_t S_pitch, int32_t D,
                  int64_t thd_rows, const int32_t* seq_offsets, const int32_t* seq_lens,
                  int32_t* dev_err, cpattn_stream_t stream) {
  return layout_call(thd, bhsd, B, H, S_pitch, D, thd_rows, seq_offsets, seq_lens, dev_err,
                     (hipStream_t)stream, 1);
}

// ---------------------------------------------------------------- A2A swap copies

static int a2a_heads_call(const void* src, void* dst, int64_t rows, int32_t H, int32_t D, int32_t cp,
                          hipStream_t s, int merge) {
  g_last_error.clear();
  if (rows < 0 || H <= 0 || D <= 0 || cp <= 0) return fail(CPATTN_EINVAL, "bad A2A head-copy sizes");
  if (H % cp) return fail(CPATTN_EINVAL, "H (%d) is not a multiple of cp (%d)", H, cp);
  if (D % 8) return fail(CPATTN_EUNSUPPORTED, "D must be a multiple of 8 for the A2A copies");
  if (cp > 65535) return fail(CPATTN_EUNSUPPORTED, "cp above 65535");
  if ((int64_t)H * D > (1 << 24)) return fail(CPATTN_EUNSUPPORTED, "rows above 2^24 elements");
  const int64_t bytes = rows * H * (int64_t)D * 2;
  int r;
  if ((r = check_ptr(src, bytes, 16, "src")) || (r = check_ptr(dst, bytes, 16, "dst"))) return r;
  std::vector<Range> rs = {rng("src", src, bytes, false), rng("dst", dst, bytes, true)};
  if ((r = alias_audit(rs))) return r;
  A2aHeadsArgs a{};
  a.src = (const uint16_t*)src;
  a.dst = (uint16_t*)dst;
  a.rows = rows;
  a.H = H;
  a.D = D;
  a.cp = cp;
  a.merge = merge;
  a.rows_per_wg = std::max(1, kThreads * 4 / (H * D / 8));  // 16 KB of whole rows
  if ((rows + a.rows_per_wg - 1) / a.rows_per_wg > kGridMax) return fail(CPATTN_EUNSUPPORTED, "too many rows");
  return hip_check(launch_a2a_heads(a, s), "A2A head-copy launch");
}

int cpattn_a2a_split_heads(const void* src, void* dst, int64_t rows, int32_t H, int32_t D, int32_t cp,
                           cpattn_stream_t stream) {
  return a2a_heads_call(src, dst, rows, H, D, cp, (hipStream_t)stream, 0);
}

int cpattn_a2a_merge_heads(const void* src, void* dst, int64_t rows, int32_t H, int32_t D, int32_t cp,
                           cpattn_stream_t stream) {
  return a2a_heads_call(src, dst, rows, H, D, cp, (hipStream_t)stream, 1);
}

static int a2a_rows_call(const cpattn_a2a_rows* p, const void* src, void* dst, const int32_t* maps,
                         const int32_t* so, const int32_t* sl, int32_t* dev_err, hipStream_t s,
                         int gather) {
  g_last_error.clear();
  if (!p) return fail(CPATTN_EINVAL, "A2A row sizes are NULL");
  if (p->cp <= 0 || p->chunks_per_rank < 0 || p->num_seqs < 0 || p->max_chunk_len < 0 ||
      p->rows_per_rank < 0 || p->full_rows < 0 || p->heads <= 0 || p->head_dim <= 0)
    return fail(CPATTN_EINVAL, "bad A2A row-copy sizes");
  if (p->head_dim % 8) return fail(CPATTN_EUNSUPPORTED, "D must be a multiple of 8 for the A2A copies");
  if ((int64_t)p->heads * p->head_dim > (1 << 24) || p->max_chunk_len > (1 << 30))
    return fail(CPATTN_EUNSUPPORTED, "A2A row copy too large");
  const int64_t row_bytes = (int64_t)p->heads * p->head_dim * 2;
  const int64_t blk_bytes = (int64_t)p->cp * p->rows_per_rank * row_bytes;
  const int64_t full_bytes = p->full_rows * row_bytes;
  const int64_t n_chunks = (int64_t)p->cp * p->chunks_per_rank;
  if (n_chunks > (1 << 24)) return fail(CPATTN_EUNSUPPORTED, "more than 2^24 chunks");
  const int64_t seg = row_bytes / 16;
  const int64_t wg_per_chunk = std::max<int64_t>(1, (p->max_chunk_len * seg + kThreads * 4 - 1) / (kThreads * 4));
  if (wg_per_chunk * n_chunks > kGridMax) return fail(CPATTN_EUNSUPPORTED, "A2A row copy grid too large");
  const int64_t src_bytes = gather ? full_bytes : blk_bytes, dst_bytes = gather ? blk_bytes : full_bytes;
  int r;
  if ((r = check_ptr(src, src_bytes, 16, "src")) || (r = check_ptr(dst, dst_bytes, 16, "dst")) ||
      (r = check_ptr(maps, (uint64_t)n_chunks * 16, 16, "rank_maps")) ||
      (r = check_ptr(so, (uint64_t)p->num_seqs * 4, 4, "seq_offsets")) ||
      (r = check_ptr(sl, (uint64_t)p->num_seqs * 4, 4, "seq_lens")) || (r = check_ptr(dev_err, 4, 4, "dev_err")))
    return r;
  std::vector<Range> rs = {rng("src", src, src_bytes, false), rng("dst", dst, dst_bytes, true),
                           rng("rank_maps", maps, (uint64_t)n_chunks * 16, false),
                           rng("seq_offsets", so, (uint64_t)p->num_seqs * 4, false),
                           rng("seq_lens", sl, (uint64_t)p->num_seqs * 4, false),
                           rng("dev_err", dev_err, 4, true)};
  if ((r = alias_audit(rs))) return r;
  A2aRowsArgs a{};
  a.src = (const uint16_t*)src;
  a.dst = (uint16_t*)dst;
  a.maps = maps;
  a.seq_offsets = so;
  a.seq_lens = sl;
  a.dev_err = dev_err;
  a.full_rows = p->full_rows;
  a.rows_per_rank = p->rows_per_rank;
  a.cp = p->cp;
  a.chunks_per_rank = p->chunks_per_rank;
  a.num_seqs = p->num_seqs;
  a.max_chunk_len = p->max_chunk_len;
  a.heads = p->heads;
  a.D = p->head_dim;
  a.gather = gather;
  a.wg_per_chunk = (int)wg_per_chunk;
  return hip_check(launch_a2a_rows(a, s), "A2A row-copy launch");
}

int cpattn_a2a_scatter_rows(const cpattn_a2a_rows* p, const void* blocks, void* full,
                            const int32_t* rank_maps, const int32_t* seq_offsets,
                            const int32_t* seq_lens, int32_t* dev_err, cpattn_stream_t stream) {
  return a2a_rows_call(p, blocks, full, rank_maps, seq_offsets, seq_lens, dev_err, (hipStream_t)stream, 0);
}

int cpattn_a2a_gather_rows(const cpattn_a2a_rows* p, const void* full, void* blocks,
                           const int32_t* rank_maps, const int32_t* seq_offsets,
                           const int32_t* seq_lens, int32_t* dev_err, cpattn_stream_t stream) {
  return a2a_rows_call(p, full, blocks, rank_maps, seq_offsets, seq_lens, dev_err, (hipStream_t)stream, 1);
}

}  // extern "C"
