// C ABI entry points: argument checks (pure host code, before any HIP call),
// work tables, launches and the optional event-based per-kernel timing.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "ra.h"
#include "ra_internal.h"

using namespace ra;

namespace {

thread_local std::string g_err;

ra_status fail(ra_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

ra_status hip_fail(int rc, const char *what) {
  return fail(RA_E_HIP, "%s: %s", what, hipGetErrorString((hipError_t)rc));
}

// ---------------------------------------------------------------------------
// Argument checks
// ---------------------------------------------------------------------------
size_t elem_size(int dtype) { return dtype == RA_BF16 ? 2 : 4; }

ra_status check_tensor(const ra_tensor *t, const char *name, bool is_lse) {
  if (!t) return fail(RA_E_INVALID, "%s: null tensor descriptor", name);
  if (t->dtype != RA_BF16 && t->dtype != RA_F32) return fail(RA_E_UNSUPPORTED, "%s: unknown dtype %d", name, t->dtype);
  if (t->b < 0 || t->s < 0 || t->h <= 0 || t->d <= 0) return fail(RA_E_INVALID, "%s: bad sizes", name);
  if (t->s > INT32_MAX - 1 || t->b > INT32_MAX || t->h > 65535)
    return fail(RA_E_UNSUPPORTED, "%s: sizes beyond the supported range", name);
  if (t->sb < 0 || t->ss < 0 || t->sh < 0) return fail(RA_E_INVALID, "%s: negative stride", name);
  if (t->sh > INT32_MAX) return fail(RA_E_UNSUPPORTED, "%s: head stride beyond 2^31-1 elements", name);
  const bool nonempty = t->b > 0 && t->s > 0;
  if (nonempty && !t->data) return fail(RA_E_INVALID, "%s: null data pointer", name);
  if (is_lse) {
    if (t->d != 1) return fail(RA_E_INVALID, "%s: lse tensors have d = 1", name);
    if (t->dtype != RA_F32) return fail(RA_E_UNSUPPORTED, "%s: lse must be fp32", name);
    if (reinterpret_cast<uintptr_t>(t->data) % 4) return fail(RA_E_ALIGN, "%s: data not 4-byte aligned", name);
    return RA_OK;
  }
  const size_t es = elem_size(t->dtype);
  const int64_t vec = 16 / (int64_t)es;
  if (reinterpret_cast<uintptr_t>(t->data) % 16) return fail(RA_E_ALIGN, "%s: data not 16-byte aligned", name);
  if (t->sb % vec || t->ss % vec || t->sh % vec) return fail(RA_E_ALIGN, "%s: strides must be multiples of 16 bytes", name);
  return RA_OK;
}

ra_status check_qkv(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v) {
  ra_status st;
  if ((st = check_tensor(q, "q", false)) || (st = check_tensor(k, "k", false)) || (st = check_tensor(v, "v", false)))
    return st;
  if (q->dtype != k->dtype || q->dtype != v->dtype) return fail(RA_E_INVALID, "q, k, v must share one dtype");
  if (q->d != 64 && q->d != 128) return fail(RA_E_UNSUPPORTED, "head_dim %lld not supported (64 or 128)", (long long)q->d);
  if (k->d != q->d || v->d != q->d) return fail(RA_E_INVALID, "q, k, v head_dim mismatch");
  if (k->b != q->b || v->b != q->b) return fail(RA_E_INVALID, "batch mismatch");
  if (k->s != v->s || k->h != v->h) return fail(RA_E_INVALID, "k and v shapes differ");
  if (q->h % k->h) return fail(RA_E_INVALID, "Hq (%lld) must be a multiple of Hkv (%lld)", (long long)q->h, (long long)k->h);
  // The bf16 kernel addresses a K/V tile's rows as 32-bit byte offsets from
  // the tile's first row: (row * ss + column) * 2 with row < 32 keys.
  if (q->dtype == RA_BF16) {
    const int64_t max_ss = (INT32_MAX - q->d) / (kKTileBF16 - 1);
    if (k->ss > max_ss || v->ss > max_ss)
      return fail(RA_E_UNSUPPORTED, "k/v token stride beyond %lld elements (bf16)", (long long)max_ss);
  }
  // Work tiles of one launch are counted in 32 bits: (batch, head, 128-row
  // tile) triples plus a margin for per-item ragged tiles and key splits.
  const double tiles = (double)q->b * (double)q->h * ((double)q->s / 128.0 + 1024.0);
  if (tiles > (double)INT32_MAX)
    return fail(RA_E_UNSUPPORTED, "B x Hq x Sq too large for one launch's work-tile count");
  return RA_OK;
}

ra_status check_out(const ra_tensor *q, const ra_tensor *out, const ra_tensor *lse, const char *oname,
                    const char *lname) {
  ra_status st;
  if ((st = check_tensor(out, oname, false)) || (st = check_tensor(lse, lname, true))) return st;
  if (out->dtype != RA_F32) return fail(RA_E_UNSUPPORTED, "%s must be fp32", oname);
  if (out->b != q->b || out->s != q->s || out->h != q->h || out->d != q->d)
    return fail(RA_E_INVALID, "%s shape must be [B, Sq, Hq, d] of q", oname);
  if (lse->b != q->b || lse->s != q->s || lse->h != q->h)
    return fail(RA_E_INVALID, "%s shape must be [B, Sq, Hq] of q", lname);
  return RA_OK;
}

// ---------------------------------------------------------------------------
// Timing (events around each launch, off by default)
// ---------------------------------------------------------------------------
struct Prof {
  std::mutex mu;
  std::atomic<bool> on{false};  // read without the lock on every launch
  std::vector<hipEvent_t> pool;
  struct Rec {
    int kind;
    hipEvent_t a, b;
  };
  std::vector<Rec> recs;
  size_t next = 0;
} g_prof;

struct ProfScope {
  int kind;
  hipStream_t s;
  hipEvent_t b = nullptr;
  ProfScope(int kind_, void *stream) : kind(kind_), s((hipStream_t)stream) {
    if (!g_prof.on) return;
    std::lock_guard<std::mutex> lk(g_prof.mu);
    if (g_prof.next + 2 > g_prof.pool.size()) {
      for (int i = 0; i < 64; ++i) {
        hipEvent_t e;
        if (hipEventCreate(&e) != hipSuccess) return;
        g_prof.pool.push_back(e);
      }
    }
    hipEvent_t a = g_prof.pool[g_prof.next++];
    b = g_prof.pool[g_prof.next++];
    (void)hipEventRecord(a, s);  // instrumentation only: a failed record just loses this sample
    g_prof.recs.push_back({kind, a, b});
  }
  ~ProfScope() {
    if (b) (void)hipEventRecord(b, s);
  }
};

// ---------------------------------------------------------------------------
// Work tables
// ---------------------------------------------------------------------------
struct Geometry {
  int QT, KT;
};

// Tile geometry of the attention kernel for a dtype.
Geometry geometry(int dtype) {
  if (dtype != RA_BF16) return Geometry{kQTileF32, kKTileF32};
  return Geometry{kQTileBF16, kKTileBF16};
}

void fill_strides(AttnArgs &a, const ra_tensor *q, const ra_tensor *k, const ra_tensor *v) {
  a.q = q->data;
  a.k = k->data;
  a.v = v->data;
  a.q_sb = q->sb, a.q_ss = q->ss, a.q_sh = (int32_t)q->sh;
  a.k_sb = k->sb, a.k_ss = k->ss, a.k_sh = (int32_t)k->sh;
  a.v_sb = v->sb, a.v_ss = v->ss, a.v_sh = (int32_t)v->sh;
  a.B = (int32_t)q->b;
  a.Hq = (int32_t)q->h;
  a.Hkv = (int32_t)k->h;
  a.G = a.Hq / a.Hkv;
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)q->d));
}

void set_dest(AttnArgs &a, float *out, int64_t o_sb, int64_t o_ss, int64_t o_sh, float *lse, int64_t l_sb,
              int64_t l_ss, int64_t l_sh) {
  a.out = out, a.o_sb = o_sb, a.o_ss = o_ss, a.o_sh = (int32_t)o_sh;
  a.lse = lse, a.l_sb = l_sb, a.l_ss = l_ss, a.l_sh = (int32_t)l_sh;
}

// Packing of grouped query heads into tile rows: when the query block is
// shorter than a tile, the heads sharing one K/V head are packed as rows.
int choose_gp(int64_t q_len_max, int G, int QT) { return (q_len_max < QT && G > 1) ? G : 1; }

// Finalise tile counts and XCD split after items are filled in.
void finish_tiles(AttnArgs &a, int QT) {
  int tile = 0;
  for (int i = 0; i < a.nitems; ++i) {
    KItem &it = a.items[i];
    it.nqt = (int32_t)((int64_t(it.q_len) * a.GP + QT - 1) / QT);
    it.tile0 = tile;
    tile += it.nqt * it.nsplit;
  }
  a.nhb = a.Hq / a.GP;
  a.ntiles = tile;
  const int64_t nw = (int64_t)a.B * a.nhb * a.ntiles;
  a.n_work = (int32_t)nw;
  const int64_t pairs = (int64_t)a.B * a.nhb;
  if (pairs % 8 == 0) {  // whole (batch, head block) pairs per XCD
    a.per_xcd_pairs = (int32_t)(pairs / 8);
    a.per_xcd = a.per_xcd_pairs * a.ntiles;
  } else {  // consecutive work indices split over the XCDs
    a.per_xcd_pairs = 0;
    a.per_xcd = (int32_t)((nw + 7) / 8);
  }
}

KItem to_kitem(const ra_plan_item &p, int64_t o_row0) {
  KItem k{};
  k.q_start = (int32_t)p.q_start;
  k.q_len = (int32_t)p.q_len;
  k.qpos0 = (int32_t)p.q_pos0;
  k.o_row0 = (int32_t)o_row0;
  k.nsplit = 1;
  k.split_len = 0;
  k.nseg = p.nseg;
  k.first = p.first;
  int64_t work = 0;
  for (int s = 0; s < p.nseg; ++s) {
    k.seg[s].kv_start = (int32_t)p.seg[s].kv_start;
    k.seg[s].kv_len = (int32_t)p.seg[s].kv_len;
    k.seg[s].kpos0 = (int32_t)p.seg[s].kv_start;
    k.seg[s].causal = p.seg[s].causal;
    work += p.seg[s].causal ? p.seg[s].kv_len / 2 : p.seg[s].kv_len;
  }
  k.work = (int32_t)std::min<int64_t>(INT32_MAX, work * p.q_len / 1024 + 1);
  return k;
}

// Split-K sizing: enough work-groups to cover the chip twice.
struct Split {
  int nsplit = 1;
  int split_len = 0;
};

Split choose_split(int64_t wgs, int64_t kv_len, int KT) {
  Split s;
  const int64_t target = 2 * 256;
  if (wgs >= target || kv_len < 4 * KT) return s;
  int64_t ns = (target + wgs - 1) / wgs;
  ns = std::min<int64_t>(ns, kv_len / (2 * KT));
  if (ns < 2) return s;
  int64_t len = (kv_len + ns - 1) / ns;
  len = (len + KT - 1) / KT * KT;
  s.split_len = (int)len;
  s.nsplit = (int)((kv_len + len - 1) / len);
  return s;
}

size_t split_bytes(const Split &s, int64_t B, int64_t H, int64_t rows, int64_t D) {
  if (s.nsplit <= 1) return 0;
  return (size_t)s.nsplit * B * H * rows * (D + 1) * sizeof(float);
}

// Launch attention for one item, splitting the keys over work-groups when the
// item alone cannot fill the chip and scratch is available.  The result is
// written (mode kWrite) or merged (kMerge) into the destination held in `a`.
ra_status run_single_item(AttnArgs a, int dtype, int D, char *ws, size_t ws_bytes, void *stream) {
  KItem &it = a.items[0];
  const Geometry geo = geometry(dtype);
  const int64_t nqt = (int64_t(it.q_len) * a.GP + geo.QT - 1) / geo.QT;
  const int64_t wgs = (int64_t)a.B * (a.Hq / a.GP) * nqt;
  Split sp = (it.nseg == 1) ? choose_split(wgs, it.seg[0].kv_len, geo.KT) : Split{};
  const size_t need = split_bytes(sp, a.B, a.Hq, it.q_len, D);
  if (sp.nsplit > 1 && (ws == nullptr || ws_bytes < need)) sp = Split{};
  if (sp.nsplit <= 1) {
    finish_tiles(a, geo.QT);
    if (a.n_work == 0) return RA_OK;
    ProfScope ps(RA_KERNEL_ATTN, stream);
    const int rc = launch_attn(a, dtype, D, stream);
    return rc ? hip_fail(rc, "attention launch") : RA_OK;
  }
  it.nsplit = sp.nsplit;
  it.split_len = sp.split_len;
  SplitArgs s{};
  s.out = a.out, s.lse = a.lse;
  s.o_sb = a.o_sb, s.o_ss = a.o_ss, s.o_sh = a.o_sh;
  s.l_sb = a.l_sb, s.l_ss = a.l_ss, s.l_sh = a.l_sh;
  s.B = a.B, s.H = a.Hq, s.D = D, s.rows = it.q_len, s.nsplit = sp.nsplit;
  s.o_row0 = it.o_row0;
  s.mode = a.mode;
  s.first = it.first;
  float *po = reinterpret_cast<float *>(ws);
  float *pl = po + (size_t)sp.nsplit * a.B * a.Hq * it.q_len * D;
  s.part_out = po, s.part_lse = pl;
  a.part_out = po, a.part_lse = pl, a.part_rows = it.q_len;
  a.mode = kSplit;
  finish_tiles(a, geo.QT);
  {
    ProfScope ps(RA_KERNEL_ATTN, stream);
    const int rc = launch_attn(a, dtype, D, stream);
    if (rc) return hip_fail(rc, "attention launch");
  }
  ProfScope ps(RA_KERNEL_SPLIT_REDUCE, stream);
  const int rc = launch_split_reduce(s, stream);
  return rc ? hip_fail(rc, "split-reduce launch") : RA_OK;
}

size_t single_item_ws(int dtype, int64_t B, int64_t Hq, int GP, int64_t q_len, int64_t kv_len, int64_t D) {
  const Geometry geo = geometry(dtype);
  const int64_t nqt = (q_len * GP + geo.QT - 1) / geo.QT;
  const int64_t wgs = B * (Hq / GP) * nqt;
  return split_bytes(choose_split(wgs, kv_len, geo.KT), B, Hq, q_len, D);
}

// KV-sharded, fused: the P blocks are the ranks' shards.  Their partials do
// not depend on each other (each rank attends the broadcast queries to its
// own shard), so when one block's query tiles make only a few rounds of
// work-groups (a launch per block would spend much of its time in its last,
// partly filled round) all of them run in one launch, each cut into nsub
// sub-blocks when that is still short of two work-groups per CU, and one
// reduction merges the P * nsub partials into (out, lse): the gather-merge.
// Returns nsplit = 0 when the step-by-step path is used instead (P = 1, or
// at least kGatherMaxWgs work-groups per block).
constexpr int64_t kGatherMaxWgs = 2048;
Split choose_gather(int64_t wgs, int64_t block_len, int P, int KT) {
  Split g;
  g.nsplit = 0;
  const int64_t target = 2 * 256;
  if (P < 2 || wgs >= kGatherMaxWgs || block_len < 1) return g;
  if (wgs >= target || block_len < 2 * KT) {  // no sub-blocks
    g.nsplit = 1;
    g.split_len = (int)block_len;
    return g;
  }
  const int64_t want = (target + wgs - 1) / wgs;  // partials per row over all blocks
  int64_t ns = std::max<int64_t>(1, (want + P - 1) / P);
  ns = std::min<int64_t>(ns, std::max<int64_t>(1, block_len / (2 * KT)));
  int64_t len = (block_len + ns - 1) / ns;
  len = (len + KT - 1) / KT * KT;
  g.split_len = (int)len;
  g.nsplit = (int)((block_len + len - 1) / len);
  return g;
}

int64_t kv_sharded_wgs(int dtype, int64_t B, int64_t Hq, int GP, int64_t q_len) {
  const Geometry geo = geometry(dtype);
  return B * (Hq / GP) * ((q_len * GP + geo.QT - 1) / geo.QT);
}

size_t gather_ws(const Split &g, int P, int64_t B, int64_t Hq, int64_t q_len, int64_t D) {
  if (g.nsplit <= 0) return 0;
  return (size_t)P * g.nsplit * B * Hq * q_len * (D + 1) * sizeof(float);
}

// One attention launch over every block (partials to the workspace), then
// one split reduction that writes (out, lse).
ra_status run_gather(AttnArgs a, const std::vector<ra_plan_item> &items, const Split &g, int dtype, int D,
                     char *ws, void *stream) {
  const int P = (int)items.size();
  const int64_t rows = items[0].q_len;
  a.nitems = 0;
  for (int i = 0; i < P; ++i) {
    KItem k = to_kitem(items[i], items[i].q_start);
    k.nsplit = g.nsplit;
    k.split_len = g.split_len;
    k.split0 = i * g.nsplit;
    a.items[a.nitems++] = k;
  }
  const int nparts = P * g.nsplit;
  float *po = reinterpret_cast<float *>(ws);
  float *pl = po + (size_t)nparts * a.B * a.Hq * rows * D;
  a.part_out = po, a.part_lse = pl, a.part_rows = (int32_t)rows;
  SplitArgs s{};
  s.out = a.out, s.lse = a.lse;
  s.o_sb = a.o_sb, s.o_ss = a.o_ss, s.o_sh = a.o_sh;
  s.l_sb = a.l_sb, s.l_ss = a.l_ss, s.l_sh = a.l_sh;
  s.B = a.B, s.H = a.Hq, s.D = D, s.rows = (int32_t)rows, s.nsplit = nparts;
  s.o_row0 = (int32_t)items[0].q_start;
  s.mode = kWrite;
  s.first = 1;
  s.part_out = po, s.part_lse = pl;
  a.mode = kSplit;
  finish_tiles(a, geometry(dtype).QT);
  {
    ProfScope ps(RA_KERNEL_ATTN, stream);
    const int rc = launch_attn(a, dtype, D, stream);
    if (rc) return hip_fail(rc, "attention launch");
  }
  ProfScope ps(RA_KERNEL_SPLIT_REDUCE, stream);
  const int rc = launch_split_reduce(s, stream);
  return rc ? hip_fail(rc, "split-reduce launch") : RA_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// Public API
// ---------------------------------------------------------------------------
extern "C" {

int ra_version(void) { return RA_VERSION; }

const char *ra_status_str(int st) {
  switch (st) {
    case RA_OK: return "RA_OK";
    case RA_E_INVALID: return "RA_E_INVALID";
    case RA_E_UNSUPPORTED: return "RA_E_UNSUPPORTED";
    case RA_E_ALIGN: return "RA_E_ALIGN";
    case RA_E_HIP: return "RA_E_HIP";
    case RA_E_WORKSPACE: return "RA_E_WORKSPACE";
    default: return "RA_E_UNKNOWN";
  }
}

const char *ra_last_error(void) { return g_err.c_str(); }

size_t ra_block_attn_workspace_bytes(const ra_tensor *q, const ra_tensor *k) {
  if (!q || !k || q->h <= 0 || k->h <= 0 || q->h % k->h) return 0;
  const int G = (int)(q->h / k->h);
  const Geometry geo = geometry(q->dtype);
  const int GP = choose_gp(q->s, G, geo.QT);
  return single_item_ws(q->dtype, q->b, q->h, GP, q->s, k->s, q->d);
}

}  // extern "C"

namespace {

// Host-side checks of a block call (no HIP call).
ra_status check_block(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v, int mask, const ra_tensor *out,
                      const ra_tensor *lse) {
  ra_status st;
  if ((st = check_qkv(q, k, v)) || (st = check_out(q, out, lse, "out", "lse"))) return st;
  if (mask < RA_MASK_NONE || mask > RA_MASK_CAUSAL_BOTTOM_RIGHT) return fail(RA_E_INVALID, "unknown mask kind %d", mask);
  if (mask == RA_MASK_CAUSAL_BOTTOM_RIGHT && q->s > k->s)
    return fail(RA_E_INVALID, "bottom-right causal mask needs Sq <= Sk");
  return RA_OK;
}

// One query block against one K/V block (arguments already checked).
ra_status block_attn(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v, int mask, ra_tensor *out,
                     ra_tensor *lse, void *workspace, size_t workspace_bytes, void *stream) {
  AttnArgs a{};
  fill_strides(a, q, k, v);
  set_dest(a, (float *)out->data, out->sb, out->ss, out->sh, (float *)lse->data, lse->sb, lse->ss, lse->sh);
  const Geometry geo = geometry(q->dtype);
  a.GP = choose_gp(q->s, a.G, geo.QT);
  a.mode = kWrite;
  a.nitems = 1;
  KItem &it = a.items[0];
  it.q_start = 0;
  it.q_len = (int32_t)q->s;
  it.qpos0 = mask == RA_MASK_CAUSAL_BOTTOM_RIGHT ? (int32_t)(k->s - q->s) : 0;
  it.o_row0 = 0;
  it.nsplit = 1;
  it.nseg = 1;
  it.first = 1;
  it.seg[0].kv_start = 0;
  it.seg[0].kv_len = (int32_t)k->s;
  it.seg[0].kpos0 = 0;
  it.seg[0].causal = mask != RA_MASK_NONE;
  return run_single_item(a, q->dtype, (int)q->d, (char *)workspace, workspace_bytes, stream);
}

}  // namespace

extern "C" {

ra_status ra_block_attn_fwd(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v, int mask,
                            ra_tensor *out, ra_tensor *lse, void *workspace, size_t workspace_bytes,
                            void *stream) {
  ra_status st;
  if ((st = check_block(q, k, v, mask, out, lse))) return st;
  if (q->s == 0 || q->b == 0) return RA_OK;
  return block_attn(q, k, v, mask, out, lse, workspace, workspace_bytes, stream);
}

ra_status ra_block_attn_fwd_noalloc(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v, int mask,
                                    ra_tensor *out, ra_tensor *lse, void *stream) {
  ra_status st;
  if ((st = check_block(q, k, v, mask, out, lse))) return st;
  // The split partials this block would use (0 when the keys are not split).
  const size_t need = ra_block_attn_workspace_bytes(q, k);
  if (need > RA_NOALLOC_SCRATCH_BYTES)
    return fail(RA_E_UNSUPPORTED, "split-K partials of %zu bytes exceed the static scratch of %zu bytes", need,
                (size_t)RA_NOALLOC_SCRATCH_BYTES);
  if (q->s == 0 || q->b == 0) return RA_OK;
  void *ws = nullptr;
  size_t ws_bytes = 0;
  const int rc = noalloc_scratch(&ws, &ws_bytes);
  if (rc) return hip_fail(rc, "static scratch address");
  return block_attn(q, k, v, mask, out, lse, ws, ws_bytes, stream);
}

ra_status ra_merge(ra_tensor *out, ra_tensor *lse, const ra_tensor *bout, const ra_tensor *blse, void *stream) {
  ra_status st;
  if ((st = check_tensor(out, "out", false)) || (st = check_tensor(lse, "lse", true)) ||
      (st = check_tensor(bout, "block_out", false)) || (st = check_tensor(blse, "block_lse", true)))
    return st;
  if (out->dtype != RA_F32 || bout->dtype != RA_F32) return fail(RA_E_UNSUPPORTED, "merge operands must be fp32");
  // One thread per 4 dims; the thread of dims 0..3 writes the new lse after
  // every thread of its row has read the old one.  That order holds only when
  // a row's threads sit in one wave, i.e. when d/4 divides the wave size.
  if (out->d % 4 || 64 % (out->d / 4))
    return fail(RA_E_UNSUPPORTED, "merge head_dim %lld not supported (4, 8, 16, 32, 64, 128 or 256)",
                (long long)out->d);
  if (bout->b != out->b || bout->s != out->s || bout->h != out->h || bout->d != out->d)
    return fail(RA_E_INVALID, "block_out shape differs from out");
  if (lse->b != out->b || lse->s != out->s || lse->h != out->h || blse->b != out->b || blse->s != out->s ||
      blse->h != out->h)
    return fail(RA_E_INVALID, "lse shapes must be [B, S, H] of out");
  if (out->b == 0 || out->s == 0) return RA_OK;  // nothing to merge (empty tensors may share a null pointer)
  if (out->data == bout->data) return fail(RA_E_INVALID, "out must not alias block_out");
  MergeArgs m{};
  m.out = (float *)out->data, m.lse = (float *)lse->data;
  m.bout = (const float *)bout->data, m.blse = (const float *)blse->data;
  m.o_sb = out->sb, m.o_ss = out->ss, m.o_sh = (int32_t)out->sh;
  m.l_sb = lse->sb, m.l_ss = lse->ss, m.l_sh = (int32_t)lse->sh;
  m.bo_sb = bout->sb, m.bo_ss = bout->ss, m.bo_sh = (int32_t)bout->sh;
  m.bl_sb = blse->sb, m.bl_ss = blse->ss, m.bl_sh = (int32_t)blse->sh;
  m.B = (int32_t)out->b, m.H = (int32_t)out->h, m.D = (int32_t)out->d;
  m.total_rows = (int32_t)out->s;
  m.nranges = 1;
  m.ranges[0] = MRange{0, 0, (int32_t)out->s, 0};
  ProfScope ps(RA_KERNEL_MERGE, stream);
  const int rc = launch_merge(m, stream);
  return rc ? hip_fail(rc, "merge launch") : RA_OK;
}

}  // extern "C"

namespace {

struct RingShape {
  int64_t ws_rows;            // rows of the block-result workspace
  std::vector<ra_plan_item> items;
};

// Layouts whose queries have one owner and whose K/V blocks are the ranks'
// shards (decode, chunked prefill).
bool kv_sharded(int kind) { return kind == RA_LAYOUT_KV_SHARDED || kind == RA_LAYOUT_KV_SHARDED_CAUSAL; }

// Row of the block-result workspace for the first query row of an item.
int64_t ws_row_of(const ra_layout *L, int P, int64_t S, const ra_plan_item &it) {
  if (L->rank < 0 || kv_sharded(L->kind)) return it.q_start;
  if (L->kind == RA_LAYOUT_ZIGZAG_CAUSAL) {
    const int64_t c = S / (2 * P);
    return it.q_start == (int64_t)L->rank * c ? 0 : c + (it.q_start - (int64_t)(2 * P - 1 - L->rank) * c);
  }
  return it.q_start - (int64_t)L->rank * (S / P);
}

ra_status ring_setup(const ra_tensor *q, const ra_tensor *k, int P, const ra_layout *L, RingShape &rs) {
  const int n = ra_ring_plan(q->s, k->s, P, L, nullptr, 0);
  if (n < 0) return fail(RA_E_INVALID, "no ring plan for Sq=%lld Sk=%lld P=%d layout=%d rank=%d", (long long)q->s,
                         (long long)k->s, P, L->kind, L->rank);
  rs.items.resize(n);
  ra_ring_plan(q->s, k->s, P, L, rs.items.data(), n);
  if (kv_sharded(L->kind) || L->rank < 0)
    rs.ws_rows = q->s;
  else
    rs.ws_rows = q->s / P;
  return RA_OK;
}

size_t ring_ws_bytes(const ra_tensor *q, const ra_tensor *k, int P, const ra_layout *L, const RingShape &rs) {
  size_t bytes = 0;
  if (!L->fuse_merge) bytes += (size_t)q->b * rs.ws_rows * q->h * (q->d + 1) * sizeof(float);
  if (kv_sharded(L->kind)) {
    const Geometry geo = geometry(q->dtype);
    const int G = (int)(q->h / k->h);
    const int GP = choose_gp(q->s, G, geo.QT);
    const Split g = L->fuse_merge ? choose_gather(kv_sharded_wgs(q->dtype, q->b, q->h, GP, q->s), k->s / P, P, geo.KT)
                                  : Split{1, 0};
    if (g.nsplit > 0 && L->fuse_merge)
      bytes += gather_ws(g, P, q->b, q->h, q->s, q->d);
    else
      bytes += single_item_ws(q->dtype, q->b, q->h, GP, q->s, k->s / P, q->d);
  }
  return (bytes + 255) / 256 * 256;
}

}  // namespace

extern "C" {

size_t ra_ring_workspace_bytes(const ra_tensor *q, const ra_tensor *k, int P, const ra_layout *layout) {
  if (!q || !k || !layout || q->h <= 0 || k->h <= 0 || q->h % k->h) return 0;
  RingShape rs;
  if (ring_setup(q, k, P, layout, rs)) return 0;
  return ring_ws_bytes(q, k, P, layout, rs);
}

ra_status ra_ring_forward(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v, int P, const ra_layout *L,
                          ra_tensor *out, ra_tensor *lse, void *stream) {
  ra_status st;
  if ((st = check_qkv(q, k, v)) || (st = check_out(q, out, lse, "out", "lse"))) return st;
  if (!L) return fail(RA_E_INVALID, "null layout");
  if (P < 1 || P > 16) return fail(RA_E_UNSUPPORTED, "P must be in [1, 16]");
  if (L->kind < RA_LAYOUT_CONTIG || L->kind > RA_LAYOUT_KV_SHARDED_CAUSAL) return fail(RA_E_INVALID, "unknown layout kind");
  if (!kv_sharded(L->kind) && q->s != k->s) return fail(RA_E_INVALID, "ring layouts need Sq == Sk");
  if (L->kind == RA_LAYOUT_KV_SHARDED_CAUSAL && q->s > k->s)
    return fail(RA_E_INVALID, "KV_SHARDED_CAUSAL needs Sq <= Sk (queries are the last Sq tokens)");
  RingShape rs;
  if ((st = ring_setup(q, k, P, L, rs))) return st;
  const size_t need = ring_ws_bytes(q, k, P, L, rs);
  if (need > 0 && (L->workspace == nullptr || L->workspace_bytes < need))
    return fail(RA_E_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, L->workspace_bytes);
  if (L->workspace && reinterpret_cast<uintptr_t>(L->workspace) % 256)
    return fail(RA_E_ALIGN, "workspace must be 256-byte aligned");
  if (q->b == 0 || q->s == 0) return RA_OK;

  const int D = (int)q->d;
  const int dtype = q->dtype;
  char *ws = (char *)L->workspace;
  // Block-result workspace (unfused): bout [B][ws_rows][Hq][D], blse [B][Hq][ws_rows].
  float *ws_out = nullptr, *ws_lse = nullptr;
  char *ws_split = ws;
  size_t ws_split_bytes = L->workspace_bytes;
  const int64_t wr = rs.ws_rows;
  if (!L->fuse_merge) {
    ws_out = reinterpret_cast<float *>(ws);
    ws_lse = ws_out + (size_t)q->b * wr * q->h * D;
    const size_t blk = ((size_t)q->b * wr * q->h * (D + 1) * sizeof(float) + 255) / 256 * 256;
    ws_split = ws + blk;
    ws_split_bytes = L->workspace_bytes - blk;
  }

  AttnArgs base{};
  fill_strides(base, q, k, v);
  int64_t qlen_max = 0;
  for (auto &p : rs.items) qlen_max = std::max(qlen_max, p.q_len);
  base.GP = choose_gp(qlen_max, base.G, geometry(dtype).QT);
  const Geometry geo = geometry(dtype);

  if (kv_sharded(L->kind) && L->fuse_merge) {
    const Split g = choose_gather(kv_sharded_wgs(dtype, q->b, q->h, base.GP, q->s), k->s / P, P, geo.KT);
    if (g.nsplit > 0) {
      AttnArgs a = base;
      set_dest(a, (float *)out->data, out->sb, out->ss, out->sh, (float *)lse->data, lse->sb, lse->ss, lse->sh);
      return run_gather(a, rs.items, g, dtype, D, ws, stream);
    }
  }

  for (int t = 0; t < P; ++t) {
    std::vector<ra_plan_item> step;
    for (auto &p : rs.items)
      if (p.step == t) step.push_back(p);
    if (step.empty()) continue;
    if ((int)step.size() > kMaxItems) return fail(RA_E_UNSUPPORTED, "too many items in one step");
    // Heaviest items first: their tiles start earliest on every XCD.
    std::stable_sort(step.begin(), step.end(), [](const ra_plan_item &x, const ra_plan_item &y) {
      auto w = [](const ra_plan_item &p) {
        int64_t s = 0;
        for (int i = 0; i < p.nseg; ++i) s += p.seg[i].causal ? p.seg[i].kv_len / 2 : p.seg[i].kv_len;
        return s;
      };
      return w(x) > w(y);
    });

    // Group: first items always write straight into (out, lse); the others
    // merge in the epilogue (fused) or go through the workspace (unfused).
    for (int pass = 0; pass < 2; ++pass) {
      AttnArgs a = base;
      std::vector<MRange> ranges;
      int32_t prefix = 0;
      for (auto &p : step) {
        if ((pass == 0) != (p.first != 0)) continue;
        const bool to_ws = pass == 1 && !L->fuse_merge;
        const int64_t orow = to_ws ? ws_row_of(L, P, q->s, p) : p.q_start;
        a.items[a.nitems++] = to_kitem(p, orow);
        if (to_ws) {
          ranges.push_back(MRange{(int32_t)p.q_start, (int32_t)orow, (int32_t)p.q_len, prefix});
          prefix += (int32_t)p.q_len;
        }
      }
      if (a.nitems == 0) continue;
      const bool to_ws = pass == 1 && !L->fuse_merge;
      if (to_ws)
        set_dest(a, ws_out, wr * q->h * D, (int64_t)q->h * D, D, ws_lse, (int64_t)q->h * wr, 1, wr);
      else
        set_dest(a, (float *)out->data, out->sb, out->ss, out->sh, (float *)lse->data, lse->sb, lse->ss, lse->sh);
      a.mode = (pass == 1 && L->fuse_merge) ? kMerge : kWrite;

      if (a.nitems == 1 && kv_sharded(L->kind)) {
        if ((st = run_single_item(a, dtype, D, ws_split, ws_split_bytes, stream))) return st;
      } else {
        finish_tiles(a, geo.QT);
        if (a.n_work > 0) {
          ProfScope ps(RA_KERNEL_ATTN, stream);
          const int rc = launch_attn(a, dtype, D, stream);
          if (rc) return hip_fail(rc, "attention launch");
        }
      }
      if (to_ws) {
        MergeArgs m{};
        m.out = (float *)out->data, m.lse = (float *)lse->data;
        m.bout = ws_out, m.blse = ws_lse;
        m.o_sb = out->sb, m.o_ss = out->ss, m.o_sh = (int32_t)out->sh;
        m.l_sb = lse->sb, m.l_ss = lse->ss, m.l_sh = (int32_t)lse->sh;
        m.bo_sb = wr * q->h * D, m.bo_ss = (int64_t)q->h * D, m.bo_sh = D;
        m.bl_sb = (int64_t)q->h * wr, m.bl_ss = 1, m.bl_sh = (int32_t)wr;
        m.B = (int32_t)q->b, m.H = (int32_t)q->h, m.D = D;
        m.total_rows = prefix;
        m.nranges = (int32_t)ranges.size();
        for (size_t i = 0; i < ranges.size(); ++i) m.ranges[i] = ranges[i];
        ProfScope ps(RA_KERNEL_MERGE, stream);
        const int rc = launch_merge(m, stream);
        if (rc) return hip_fail(rc, "merge launch");
      }
    }
  }
  return RA_OK;
}

ra_status ra_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.on = on != 0;
  g_prof.recs.clear();
  g_prof.next = 0;
  return RA_OK;
}

ra_status ra_profile_read(int64_t *launches, double *total_ms, int n_kinds) {
  if (!launches || !total_ms || n_kinds < 1) return fail(RA_E_INVALID, "null output arrays");
  std::lock_guard<std::mutex> lk(g_prof.mu);
  for (int i = 0; i < n_kinds; ++i) launches[i] = 0, total_ms[i] = 0.0;
  for (auto &r : g_prof.recs) {
    if (hipEventSynchronize(r.b) != hipSuccess) return fail(RA_E_HIP, "event synchronize failed");
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return fail(RA_E_HIP, "event elapsed time failed");
    if (r.kind < n_kinds) launches[r.kind] += 1, total_ms[r.kind] += ms;
  }
  g_prof.recs.clear();
  g_prof.next = 0;
  return RA_OK;
}

}  // extern "C"
