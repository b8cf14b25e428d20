// Internal structures shared by the host dispatcher (ra_api.cpp) and the HIP
// kernels (ra_kernels.hip).  Everything here is plain data passed by value as
// kernel arguments: a launch carries its whole work table, so no device-side
// plan buffer is ever allocated.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace ra {

constexpr int kMaxItems = 32;   // work items per launch (2 per rank, P <= 16)
constexpr int kMaxRanges = 32;  // row ranges per merge launch

// Output modes of the attention / split-reduce kernels.
enum OutMode : int32_t {
  kWrite = 0,   // overwrite (out, lse) with the block result
  kMerge = 1,   // fold the block result into the running (out, lse) in place
  kSplit = 2,   // write split-K partials to the workspace
};

struct KSeg {
  int32_t kv_start;   // first key row (index into k/v)
  int32_t kv_len;     // number of key rows
  int32_t kpos0;      // global position of key row kv_start
  int32_t causal;     // 1: key visible iff kpos <= qpos
};

struct KItem {
  int32_t q_start;    // first query token row (index into q)
  int32_t q_len;      // query tokens
  int32_t qpos0;      // global position of token row q_start
  int32_t o_row0;     // first output row (index into out/lse) for q_start
  int32_t tile0;      // first work tile of this item (prefix sum)
  int32_t nqt;        // query tiles (of packed rows)
  int32_t nsplit;     // key splits (1 = none)
  int32_t split_len;  // keys per split (multiple of the key tile)
  int32_t nseg;       // 1 or 2
  int32_t first;      // 1: overwrite even in kMerge mode
  int32_t work;       // relative work estimate (host side ordering only)
  int32_t split0;     // partial index of this item's split 0 (kSplit mode)
  KSeg seg[2];
};

struct AttnArgs {
  const void *q, *k, *v;
  float *out, *lse;               // destination (final, running or block)
  float *part_out, *part_lse;     // split-K partials (kSplit)
  int64_t q_sb, q_ss, k_sb, k_ss, v_sb, v_ss, o_sb, o_ss, l_sb, l_ss;
  int32_t q_sh, k_sh, v_sh, o_sh, l_sh;
  int32_t B, Hq, Hkv, G;          // G = Hq / Hkv
  int32_t GP;                     // query heads packed into one tile's rows
  int32_t nhb;                    // head blocks = Hq / GP
  int32_t ntiles;                 // work tiles per (batch, head block)
  int32_t n_work;                 // B * nhb * ntiles
  int32_t per_xcd;                // work-groups per XCD (grid = 8 * per_xcd)
  int32_t per_xcd_pairs;          // B * nhb / 8 when that divides evenly, else 0
  int32_t mode;                   // OutMode
  int32_t part_rows;              // rows per split in the partial buffers (q_len of item 0)
  int32_t nitems;
  float scale_log2;               // softmax scale * log2(e)
  KItem items[kMaxItems];
};

// Row ranges for the merge kernel: dst rows [dst0, dst0+len) of (out, lse)
// absorb src rows [src0, src0+len) of (block_out, block_lse).
struct MRange {
  int32_t dst0, src0, len, prefix;  // prefix: rows before this range
};

struct MergeArgs {
  float *out, *lse;
  const float *bout, *blse;
  int64_t o_sb, o_ss, l_sb, l_ss, bo_sb, bo_ss, bl_sb, bl_ss;
  int32_t o_sh, l_sh, bo_sh, bl_sh;
  int32_t B, H, D;
  int32_t total_rows;             // sum of range lengths
  int32_t nranges;
  int32_t pad;
  MRange ranges[kMaxRanges];
};

// Split-K reduction: fold nsplit partials of rows (b, h, t) and write or merge
// into (out, lse).
struct SplitArgs {
  float *out, *lse;
  const float *part_out, *part_lse;
  int64_t o_sb, o_ss, l_sb, l_ss;
  int32_t o_sh, l_sh;
  int32_t B, H, D, rows, nsplit;  // rows = query tokens of the item
  int32_t o_row0;                 // output row of token 0
  int32_t mode;                   // kWrite or kMerge
  int32_t first;
};

// Launchers (defined in ra_kernels.hip).  Return a hipError_t as int.
int launch_attn(const AttnArgs &a, int dtype, int head_dim, void *stream);
int launch_merge(const MergeArgs &a, void *stream);
int launch_split_reduce(const SplitArgs &a, void *stream);

// Device address of the static scratch array on the current device (looked
// up once per device) and its size in bytes.  Returns a hipError_t as int.
int noalloc_scratch(void **ptr, size_t *bytes);

// Tile geometry the host needs for planning.
constexpr int kQTileF32 = 128;   // packed query rows per work-group (fp32 kernel)
constexpr int kQTileBF16 = 128;  // packed query rows per work-group (bf16 kernel: 4 waves x 32)
constexpr int kKTileBF16 = 32;   // keys per LDS tile (bf16)
constexpr int kKTileF32 = 32;    // keys per LDS tile (fp32)

}  // namespace ra
