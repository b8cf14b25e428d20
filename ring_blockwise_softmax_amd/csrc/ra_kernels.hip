// HIP kernels for exact blockwise attention on gfx950 (MI355X).
//
// What is computed (TokenRing review, pith.science, "What carries the
// argument"; Ring Attention record, anthology-of-the-sota): attention of a
// block of query rows against one or two key/value segments, returning the
// normalised partial output and its natural-log row log-sum-exp, optionally
// folded straight into a running (out, lse) pair with the sigma rule
//     out <- out - sigmoid(blse - lse) * (out - bout)
//     lse <- lse - ln sigmoid(lse - blse)
// evaluated in its overflow-free form max(lse, blse) + log1p(exp(-|diff|)).
//
// Kernel shape (bf16 path; one work-group = 4 waves = 128 packed query rows,
// three work-groups per CU for d = 128):
//  * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    the key index runs down the MFMA M dimension and the query index across
//    N, so each lane owns one query column and the softmax row reductions are
//    register-local plus one v_permlane32_swap between the lane halves.
//  * The P*V product is likewise out^T = V^T P^T: the exponentiated score
//    registers are already laid out as the B operand, so P never touches LDS.
//    The V^T A operand comes from the row-major V tile through
//    ds_read_b64_tr_b16 (16-lane transpose reads), so V is staged as loaded.
//  * K/V tiles of 32 keys go global -> LDS directly (global_load_lds_dwordx4)
//    into a 3-deep ring, two tiles ahead of use, one barrier per tile.  Each
//    stage runs S, softmax and P*V of its tile in order; the three resident
//    work-groups per CU overlap one another's phases instead.
//  * Online softmax in the exp2 domain against a running reference: a tile
//    is exponentiated against the row's current reference without taking its
//    maximum first, and redone against its exact maximum only when some row
//    lacks a reference or its probabilities sum past 2^8.  The final
//    normalisation uses the same reference, so the result is unchanged.
//  * Work tiles are assigned XCD-contiguously: consecutive tiles of one
//    (batch, head) land on the same XCD and share its L2 copy of K/V.
//
// The fp32 path computes the same thing on v_mfma_f32_32x32x2_f32 with K/V
// staged through registers, with no rounding of inputs or probabilities.

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "ra.h"
#include "ra_internal.h"

namespace ra {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kThreads = 256;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescaleThreshold = 8.0f;  // log2 units (fp32 kernel's lazy rescale)
constexpr float kProbSumLimit = 256.0f;    // 2^kRescaleThreshold: bf16 fast-path bound

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// Work-group barrier without a memory fence.  __syncthreads() adds a release
// fence, which waits for every outstanding global access, including LDS
// copies still in flight for later tiles.  The pipelines below order their
// LDS traffic themselves (explicit vmcnt waits for the tile being published;
// every read of a recycled buffer is consumed before the barrier); the
// memory clobber keeps the compiler from moving accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

// 16 bytes per lane from global memory straight into LDS: lane i reads
// sbase + voff (a wave-uniform 64-bit base in an SGPR pair plus a 32-bit
// lane offset, so no per-lane 64-bit address arithmetic) and its bytes land
// at lds_addr + 16*i.  Written as inline asm so that the compiler does not
// track these copies and wait for them before unrelated LDS reads; the
// kernels wait for them explicitly (s_waitcnt vmcnt) before publishing a
// tile.  No register outputs; the addresses are consumed at issue.  The LDS
// destination is read from M0, which is bound as an input operand ("{m0}"),
// so the compiler itself loads M0 and knows it is live up to the copy; the
// s_nop is the one wait state an M0 write needs before an LDS DMA reads it.
template <bool NT>
__device__ __forceinline__ void copy16_to_lds(const void *sbase, uint32_t voff, uint32_t lds_addr) {
  if constexpr (NT)
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :
                 : "v"(voff), "s"(sbase), "{m0}"(lds_addr)
                 : "memory");
  else
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "{m0}"(lds_addr)
                 : "memory");
}

// max / sum of a value with its partner lane in the other half of the wave.
__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

// ---------------------------------------------------------------------------
// Work decoding shared by both attention kernels.
// ---------------------------------------------------------------------------
struct Tile {
  int b, hb, item, qt, split;
};

__device__ __forceinline__ bool decode_tile(const AttnArgs &a, Tile &t) {
  // When the (batch, head block) pairs divide evenly over the 8 XCDs they
  // are cut into 8 contiguous chunks, one per XCD (blockIdx % 8), so every
  // XCD gets the same mix of items and its L2 holds the K/V of its own heads.  Within an XCD the order is item-major
  // (items come heaviest first), then pair, then query tile (last tile first:
  // under a causal mask it sees the most keys) and split.
  const int L = blockIdx.x;
  const int x = L & 7, l = L >> 3;
  if (a.per_xcd_pairs == 0) {
    // fewer pairs than XCDs (or not a multiple of 8): consecutive work
    // indices, head-major, split evenly over the XCDs
    const int idx = x * a.per_xcd + l;
    if (idx >= a.n_work) return false;
    const int tt = idx % a.ntiles;
    const int rest = idx / a.ntiles;
    t.hb = rest % a.nhb;
    t.b = rest / a.nhb;
    int it = 0;
    while (it + 1 < a.nitems && tt >= a.items[it + 1].tile0) ++it;
    t.item = it;
    const int e = tt - a.items[it].tile0;
    t.qt = a.items[it].nqt - 1 - e / a.items[it].nsplit;
    t.split = e % a.items[it].nsplit;
    return true;
  }
  const int np = a.per_xcd_pairs;
  const int p0 = x * np;
  if (l >= np * a.ntiles) return false;
  int it = 0;
  while (it + 1 < a.nitems && l >= np * a.items[it + 1].tile0) ++it;
  t.item = it;
  const KItem &item = a.items[it];
  const int per_pair = item.nqt * item.nsplit;
  const int e = l - np * item.tile0;
  const int pair = p0 + e / per_pair;
  const int tt = e % per_pair;
  t.hb = pair % a.nhb;
  t.b = pair / a.nhb;
  t.qt = item.nqt - 1 - tt / item.nsplit;
  t.split = tt % item.nsplit;
  return true;
}

// Key range [lo, hi) of segment s for this tile (split and causal limits).
struct SegRange {
  int kv_start, kpos0, causal, lo, hi;
};

__device__ __forceinline__ SegRange seg_range(const KItem &it, int s, int split, int qpos_max) {
  SegRange r;
  r.kv_start = it.seg[s].kv_start;
  r.kpos0 = it.seg[s].kpos0;
  r.causal = it.seg[s].causal;
  r.lo = 0;
  r.hi = it.seg[s].kv_len;
  if (it.nsplit > 1) {
    r.lo = split * it.split_len;
    r.hi = min(r.hi, r.lo + it.split_len);
  }
  if (r.causal) r.hi = min(r.hi, qpos_max - r.kpos0 + 1);
  if (r.hi < r.lo) r.hi = r.lo;
  return r;
}

// ---------------------------------------------------------------------------
// Epilogue: normalise, then write, merge or store a split partial.
// acc holds out^T for this lane's query column: element r of block mb is
// d = 32*mb + 8*(r/4) + 4*g + (r%4).
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void epilogue(const AttnArgs &a, const KItem &it, const Tile &t, int prow,
                                         bool row_ok, f32x16 (&acc)[D / 32], float m_run,
                                         float l_part, int g) {
  const float l_tot = sum_halves(l_part);
  if (!row_ok) return;
  const int tok = prow / a.GP;
  const int h = t.hb * a.GP + prow % a.GP;
  const bool empty = !(l_tot > 0.0f);
  const float inv = empty ? 0.0f : 1.0f / l_tot;
  const float blse = empty ? neg_inf() : (m_run + __log2f(l_tot)) * kLn2;

  if (a.mode == kSplit) {
    const int64_t prow_idx = ((int64_t)((it.split0 + t.split) * a.B + t.b) * a.Hq + h) * a.part_rows + tok;
    float *po = a.part_out + prow_idx * D;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d0 = 32 * mb + 8 * i4 + 4 * g;
        f32x4 v = {acc[mb][4 * i4] * inv, acc[mb][4 * i4 + 1] * inv, acc[mb][4 * i4 + 2] * inv,
                   acc[mb][4 * i4 + 3] * inv};
        *(f32x4 *)(po + d0) = v;
      }
    if (g == 0) a.part_lse[prow_idx] = blse;
    return;
  }

  const int orow = it.o_row0 + tok;
  float *op = a.out + (int64_t)t.b * a.o_sb + (int64_t)orow * a.o_ss + (int64_t)h * a.o_sh;
  float *lp = a.lse + (int64_t)t.b * a.l_sb + (int64_t)orow * a.l_ss + (int64_t)h * a.l_sh;

  if (a.mode == kMerge && !it.first) {
    const float lse_run = *lp;
    if (empty) return;  // an empty partial is the identity
    if (lse_run == neg_inf()) {
#pragma unroll
      for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d0 = 32 * mb + 8 * i4 + 4 * g;
          f32x4 v = {acc[mb][4 * i4] * inv, acc[mb][4 * i4 + 1] * inv, acc[mb][4 * i4 + 2] * inv,
                     acc[mb][4 * i4 + 3] * inv};
          *(f32x4 *)(op + d0) = v;
        }
      if (g == 0) *lp = blse;
      return;
    }
    const float diff = blse - lse_run;
    const float w = 1.0f / (1.0f + __expf(-diff));
    const float new_lse = fmaxf(lse_run, blse) + log1pf(__expf(-fabsf(diff)));
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d0 = 32 * mb + 8 * i4 + 4 * g;
        f32x4 o = *(const f32x4 *)(op + d0);
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = o[j] - w * (o[j] - acc[mb][4 * i4 + j] * inv);
        *(f32x4 *)(op + d0) = o;
      }
    if (g == 0) *lp = new_lse;
    return;
  }

#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d0 = 32 * mb + 8 * i4 + 4 * g;
      f32x4 v = {acc[mb][4 * i4] * inv, acc[mb][4 * i4 + 1] * inv, acc[mb][4 * i4 + 2] * inv,
                 acc[mb][4 * i4 + 3] * inv};
      *(f32x4 *)(op + d0) = v;
    }
  if (g == 0) *lp = blse;
}

// ---------------------------------------------------------------------------
// bf16 kernel
// ---------------------------------------------------------------------------
// One work-group = 4 waves, each owning 32 packed query rows (QT = 128).
// Keys advance in 32-key tiles held in a ring of three LDS buffers (K then V
// in each).  Tiles are copied straight from global memory into LDS with
// global_load_lds_dwordx4 (no staging registers), two tiles ahead of use,
// with one barrier per tile.  The copies are inline asm, invisible to the
// compiler's wait insertion, so LDS reads of one buffer never wait for
// copies in flight into another; each stage waits for its own tile
// (s_waitcnt vmcnt) before the barrier that publishes it.
//
// There is no software pipeline inside a wave: a stage computes S, the
// softmax and P*V of its tile in order.  Instead the kernel is sized for
// three work-groups per CU (<= 168 VGPRs, 48 KB LDS each for d = 128), so
// each SIMD runs three waves of three independent work-groups whose phases
// drift apart: one wave's exponentials overlap another's matrix products.
//
// LDS rows are unpadded (2*D bytes) with the 16-byte chunks of each row
// permuted by an XOR swizzle, chosen so that both the K operand reads (16
// rows x 16 B per group of 16 lanes) and the V transpose reads (4 rows x
// 64 B per half-wave) hit 64 distinct banks.
template <int D>
struct Bf16Cfg {
  static constexpr int NW = 4;                        // waves per work-group
  static constexpr int THREADS = 64 * NW;
  static constexpr int KT = kKTileBF16;               // keys per LDS tile (32)
  static constexpr int QT = 32 * NW;                  // packed rows per work-group
  static constexpr int NBUF = 3;                      // ring of LDS buffers
  static constexpr int PF = NBUF - 1;                 // tiles copied ahead of use
  static constexpr int OCC = D == 128 ? 3 : 4;        // work-groups per CU
  static constexpr int ROWB = 2 * D;                  // bytes per LDS row
  static constexpr int TILE_BYTES = KT * ROWB;        // one tensor, one tile
  static constexpr int BUF_BYTES = 2 * TILE_BYTES;    // K then V
  static constexpr size_t LDS_BYTES = (size_t)NBUF * BUF_BYTES;
  static constexpr int BLOCKS = TILE_BYTES / 1024;    // 1 KB direct-load blocks per tensor tile
  static constexpr int CPW = 2 * BLOCKS / NW;         // blocks (K and V) copied per wave
  static constexpr int RPB = 1024 / ROWB;             // rows per block
  static constexpr int CH = D / 8;                    // 16-byte chunks per row
  static_assert(BLOCKS % NW == 0, "K and V blocks must split evenly over the waves");
  static_assert(OCC * LDS_BYTES <= 160 * 1024, "LDS of the resident work-groups");
  __device__ static int swz(int r) {
    if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  }
  // Byte offset of element e (a multiple of 4 inside one chunk) of row r.
  __device__ static int off(int r, int e) { return r * ROWB + ((((e >> 3) ^ swz(r)) << 4) | ((e & 7) << 1)); }
};

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;

// NT: K/V are streamed once (no other work-group reads them), so their
// copies carry the non-temporal hint.
// ROT: for launches of a few rounds of work-groups.  The work-groups that
// start together on a CU would otherwise finish far apart (the oldest wave
// issues first) with nothing left to fill the CU; here they take turns at
// the highest wave priority, one ring period of tiles at a time, from a
// phase hashed from the work-group index, so they progress evenly.
template <int D, bool NT, bool ROT = false>
__global__ __launch_bounds__(Bf16Cfg<D>::THREADS, Bf16Cfg<D>::OCC) void attn_fwd_bf16(const AttnArgs a) {
  using C = Bf16Cfg<D>;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[];
  // Buffer b of the ring (b is a compile-time constant after unrolling).
  auto bufp = [&](int b) -> lds_u8 * { return (lds_u8 *)smem_raw + b * C::BUF_BYTES; };

  Tile t;
  if (!decode_tile(a, t)) return;
  const KItem &it = a.items[t.item];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int n = lane & 31;  // query column of this lane
  const int g = lane >> 5;  // lane half
  const int i16 = lane & 15, G16 = lane >> 4;

  const int rows_total = it.q_len * a.GP;
  const int tile_row0 = t.qt * C::QT;
  const int wave_row0 = tile_row0 + wave * 32;
  const int prow = wave_row0 + n;
  const bool row_ok = prow < rows_total;
  const int hkv = (t.hb * a.GP) / a.G;
  const int qpos = it.qpos0 + (row_ok ? prow : rows_total - 1) / a.GP;
  const int wave_qpos_min = it.qpos0 + min(wave_row0, rows_total - 1) / a.GP;
  const int tile_qpos_max = it.qpos0 + (min(tile_row0 + C::QT, rows_total) - 1) / a.GP;
  const int wave_qpos_max = it.qpos0 + min(wave_row0 + 31, rows_total - 1) / a.GP;

  // Q fragment (B operand of S^T = K Q^T): d = 16*kc + 8*g + 0..7.
  bf16x8 qf[D / 16];
  {
    const int pr = row_ok ? prow : 0;
    const int tok = pr / a.GP;
    const int h = t.hb * a.GP + pr % a.GP;
    const bf16 *qp = reinterpret_cast<const bf16 *>(a.q) + (int64_t)t.b * a.q_sb +
                     (int64_t)(it.q_start + tok) * a.q_ss + (int64_t)h * a.q_sh + 8 * g;
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
      qf[kc] = *(const bf16x8 *)(qp + 16 * kc);
      if (!row_ok) qf[kc] = bf16x8{};
    }
  }

  f32x16 acc[D / 32];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb) acc[mb] = f32x16{};
  float m_run = neg_inf();
  float l_part = 0.0f;
  bool ref_ok = false;  // wave-uniform: every lane's m_run is finite

  // Key tiles of the (up to two) segments, flattened.
  const SegRange sr0 = seg_range(it, 0, t.split, tile_qpos_max);
  const SegRange sr1 = it.nseg > 1 ? seg_range(it, 1, t.split, tile_qpos_max) : sr0;
  const int nt0 = (sr0.hi - sr0.lo + C::KT - 1) / C::KT;
  const int nt1 = it.nseg > 1 ? (sr1.hi - sr1.lo + C::KT - 1) / C::KT : 0;
  const int ntiles = nt0 + nt1;

  const bf16 *kbase = reinterpret_cast<const bf16 *>(a.k) + (int64_t)t.b * a.k_sb + (int64_t)hkv * a.k_sh;
  const bf16 *vbase = reinterpret_cast<const bf16 *>(a.v) + (int64_t)t.b * a.v_sb + (int64_t)hkv * a.v_sh;

  // Direct-load geometry: this wave copies blocks bi = wave + NW*u of the
  // tile (K blocks for u < CPW/2, then V).  Block b covers tile rows b*RPB ..;
  // lane writes physical chunk lane%CH of row b*RPB + lane/CH, which holds
  // logical chunk (lane%CH) ^ swz(row).  Byte offsets are from the tile's
  // first row, for full tiles (clamped rows are recomputed on partial ones).
  auto is_v = [](int u) { return u >= C::CPW / 2; };
  int ld_row[C::CPW], ld_col[C::CPW], ld_lds[C::CPW];
  uint32_t ld_off[C::CPW];
#pragma unroll
  for (int u = 0; u < C::CPW; ++u) {
    const int blk = wave + C::NW * (is_v(u) ? u - C::CPW / 2 : u);
    ld_row[u] = blk * C::RPB + lane / C::CH;
    ld_col[u] = (((lane % C::CH) ^ C::swz(ld_row[u])) * 8);
    ld_lds[u] = (is_v(u) ? C::TILE_BYTES : 0) + blk * 1024;
    ld_off[u] = (uint32_t)(ld_row[u] * (int)(is_v(u) ? a.v_ss : a.k_ss) + ld_col[u]) * 2u;
  }

  // LDS read offsets (bytes, relative to a buffer): K operand for each kc,
  // V transpose operand for each (mb, second 8-row half).
  int koff[D / 16], voff[D / 32][2];
#pragma unroll
  for (int kc = 0; kc < D / 16; ++kc) koff[kc] = C::off(n, 16 * kc + 8 * g);
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
      voff[mb][s2] = C::TILE_BYTES +
                     C::off(4 * g + (i16 >> 2) + 8 * s2, 32 * mb + 16 * (G16 & 1) + 4 * (i16 & 3));

  // Copy cursor: cpk/cpv point at the first K/V row of the next tile to copy
  // and advance one tile per copy (switching segment once), so the steady
  // state needs no 64-bit address arithmetic.
  const int64_t kstep = (int64_t)C::KT * a.k_ss * 2, vstep = (int64_t)C::KT * a.v_ss * 2;
  const char *kseg1 = reinterpret_cast<const char *>(kbase + (int64_t)(sr1.kv_start + sr1.lo) * a.k_ss);
  const char *vseg1 = reinterpret_cast<const char *>(vbase + (int64_t)(sr1.kv_start + sr1.lo) * a.v_ss);
  const char *cpk = reinterpret_cast<const char *>(kbase + (int64_t)(sr0.kv_start + sr0.lo) * a.k_ss);
  const char *cpv = reinterpret_cast<const char *>(vbase + (int64_t)(sr0.kv_start + sr0.lo) * a.v_ss);
  if (nt0 == 0) {  // first segment empty in this split
    cpk = kseg1;
    cpv = vseg1;
  }
  bool cp_seg0 = nt0 > 0;               // cursor in the first segment
  int cp_left = cp_seg0 ? nt0 : nt1;     // tiles left in the cursor's segment

  // Copy the next tile (K and V) into LDS buffer `buf` and advance the
  // cursor.  Only a segment's last tile can be ragged: its rows past the
  // valid range are clamped to the last valid row (finite data, masked in
  // the softmax).
  auto issue_next = [&](int buf) {
    if (--cp_left != 0) {
#pragma unroll
      for (int u = 0; u < C::CPW; ++u)
        copy16_to_lds<NT>(is_v(u) ? cpv : cpk, ld_off[u], (uint32_t)(uintptr_t)(bufp(buf) + ld_lds[u]));
      cpk += kstep;
      cpv += vstep;
    } else {
      const SegRange &sr = cp_seg0 ? sr0 : sr1;
      const int nvalid = (sr.hi - sr.lo) - ((cp_seg0 ? nt0 : nt1) - 1) * C::KT;
#pragma unroll
      for (int u = 0; u < C::CPW; ++u) {
        const int row = min(ld_row[u], nvalid - 1);
        const uint32_t o = (uint32_t)(row * (int)(is_v(u) ? a.v_ss : a.k_ss) + ld_col[u]) * 2u;
        copy16_to_lds<NT>(is_v(u) ? cpv : cpk, o, (uint32_t)(uintptr_t)(bufp(buf) + ld_lds[u]));
      }
      cpk = kseg1;
      cpv = vseg1;
      cp_seg0 = false;
      cp_left = nt1;
    }
  };

  // Tiles whose segment-local first key kb is at or past these limits need
  // the per-element mask for this wave (ragged segment end, or keys after
  // some of this wave's queries under the causal mask).
  auto first_masked = [&](const SegRange &sr) {
    int lim = sr.hi - C::KT + 1;
    if (sr.causal) lim = min(lim, wave_qpos_min - sr.kpos0 - C::KT + 2);
    return lim;
  };
  const int fm0 = first_masked(sr0), fm1 = first_masked(sr1);

  // One stage: tile ti sits in buffer bc.  After the S products the next
  // copy (tile ti+PF into buffer bl, which every wave finished reading before
  // this stage's barrier) is issued, so its address work overlaps the
  // matrix cores.
  auto step = [&](int ti, int bc, bool copy, int bl) {
    f32x16 s = f32x16{};
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
      const bf16x8 ka = *(const lds_bf16x8 *)(bufp(bc) + koff[kc]);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[kc], s, 0, 0, 0);
    }
    if (copy) issue_next(bl);
    const bool seg1 = ti >= nt0;
    const int kb = (seg1 ? sr1.lo + (ti - nt0) * C::KT : sr0.lo + ti * C::KT);
    if (kb >= (seg1 ? fm1 : fm0)) {
      const SegRange &sr = seg1 ? sr1 : sr0;
      // key (segment-local) visible iff key < lim
      const int lim = sr.causal ? min(sr.hi, qpos - sr.kpos0 + 1) : sr.hi;
      const int kl = kb + 4 * g;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kl + 8 * (r >> 2) + (r & 3);
        s[r] = key < lim ? s[r] : neg_inf();
      }
    }
    // P = exp2(s * scale_log2 - m): fp32 for the row sum, bf16 (RNE) for P*V.
    // Returns this lane's sum of the tile's 16 probabilities.
    bf16x8 pb[2];
    auto exps = [&](float moff) {
      float t = 0.0f;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * c + e], a.scale_log2, -moff));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * c + e + 1], a.scale_log2, -moff));
          const bf16x2 pp = {(bf16)p0, (bf16)p1};
          pb[c][e] = pp[0];
          pb[c][e + 1] = pp[1];
          t += p0 + p1;
        }
      }
      return t;
    };
    // Fast path: exponentiate against the running reference m_run without
    // this tile's maximum.  It stands when every lane has a finite reference
    // and no lane's probabilities sum past 2^8 (so none exceeds 2^8: no
    // overflow, and the reference stays within 8 of the row maximum).
    // Otherwise the tile is redone against its exact maximum, rescaling the
    // lanes whose maximum grew.
    float tsum = 0.0f;
    bool redo = !ref_ok;
    if (ref_ok) {
      tsum = exps(m_run);
      redo = __builtin_amdgcn_ballot_w64(!(tsum <= kProbSumLimit)) != 0;
    }
    if (__builtin_expect(redo, 0)) {
      float mx = __builtin_fmaxf(__builtin_fmaxf(s[0], s[1]), s[2]);
#pragma unroll
      for (int r = 3; r < 15; r += 2) mx = __builtin_fmaxf(__builtin_fmaxf(mx, s[r]), s[r + 1]);
      mx = __builtin_fmaxf(mx, s[15]);
      mx = max_halves(mx) * a.scale_log2;
      const float m_new = fmaxf(m_run, mx);
      const bool need = m_new > m_run;
      if (__builtin_amdgcn_ballot_w64(need) != 0) {
        const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
        m_run = need ? m_new : m_run;
        l_part *= alpha;
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[mb][r] *= alpha;
      }
      tsum = exps(m_run == neg_inf() ? 0.0f : m_run);
      ref_ok = __builtin_amdgcn_ballot_w64(m_run == neg_inf()) == 0;
    }
    l_part += tsum;
    // out^T += V^T P^T over two 16-key chunks (chunk c is 16 rows further).
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int mb = 0; mb < D / 32; ++mb) {
        const lds_u8 *vb = bufp(bc) + 16 * c * C::ROWB;
        const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(vb + voff[mb][0]));
        const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(vb + voff[mb][1]));
        const s16x8 vv = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv), pb[c], acc[mb], 0, 0, 0);
      }
    }
  };

  // Tiles are copied PF tiles ahead of use.  Copies complete in order, so
  // "tile ti has landed" is "at most the copies issued after it are still
  // outstanding": (PF - 1) tiles of CPW instructions each.
  static_assert((C::PF - 1) * C::CPW == 4 || (C::PF - 1) * C::CPW == 2, "wait immediates below");
  auto wait_tile = [&](int ti) {
    if (ti + C::PF - 1 < ntiles) {
      if constexpr ((C::PF - 1) * C::CPW == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    } else {  // the last tiles: nothing was issued after them
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
  };

  // Tiles this wave computes: none if its 32 rows are all past the item (a
  // ragged last query tile, or fewer packed rows than the work-group); under
  // a causal last segment, only up to the key of its last row, rounded up to
  // a whole group of NBUF stages (the extra tiles are fully masked and add
  // exact zeros).  Past them the wave only does its share of the copies,
  // with the same waits and barriers, in a second loop; the stage body is not
  // duplicated and the steady-state loop carries no test.
  int nt_live = ntiles;
  if (wave_row0 >= rows_total) {
    nt_live = 0;
  } else {
    const SegRange &sl = it.nseg > 1 ? sr1 : sr0;
    if (sl.causal) {
      const int lim = min(sl.hi, wave_qpos_max - sl.kpos0 + 1);
      const int need = lim <= sl.lo ? 0 : (lim - sl.lo + C::KT - 1) / C::KT;
      nt_live = (it.nseg > 1 ? nt0 : 0) + min(it.nseg > 1 ? nt1 : nt0, need);
    }
  }

  const int nt_main = min(ntiles, (nt_live + C::NBUF - 1) / C::NBUF * C::NBUF);

  const int npro = min(ntiles, C::PF);
  for (int j = 0; j < npro; ++j) issue_next(j);
  int ti = 0;
  const int rot0 = (int)((blockIdx.x * 2654435761u) >> 30) % 3;
  for (; ti < nt_main; ti += C::NBUF) {
    if constexpr (ROT) {
      const int p = (ti / C::NBUF + rot0) % 3;
      if (p == 0) __builtin_amdgcn_s_setprio(2);
      else if (p == 1) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
    }
#pragma unroll
    for (int k = 0; k < C::NBUF; ++k) {
      if (ti + k >= ntiles) break;
      wait_tile(ti + k);
      lds_barrier();
      step(ti + k, k, ti + k + C::PF < ntiles, (k + C::PF) % C::NBUF);
    }
  }
  if constexpr (ROT) __builtin_amdgcn_s_setprio(0);
  for (; ti < ntiles; ti += C::NBUF) {  // copies only
#pragma unroll
    for (int k = 0; k < C::NBUF; ++k) {
      if (ti + k >= ntiles) break;
      wait_tile(ti + k);
      lds_barrier();
      if (ti + k + C::PF < ntiles) issue_next((k + C::PF) % C::NBUF);
    }
  }

  epilogue<D>(a, it, t, prow, row_ok, acc, m_run, l_part, g);
}

// ---------------------------------------------------------------------------
// fp32 kernel (exact path): v_mfma_f32_32x32x2_f32, no rounding.  Bounded
// for two work-groups per CU (<= 256 registers per lane, two double-buffered
// padded K/V tiles of 67.6 KB at d = 128), so each SIMD runs two waves and
// one wave's softmax and tile copy overlap the other's products.
// ---------------------------------------------------------------------------
template <int D>
struct F32Cfg {
  static constexpr int KT = kKTileF32;
  static constexpr int QT = kQTileF32;
  static constexpr int LD = D + 4;
  static constexpr int CHUNKS = KT * D / 4;
  static constexpr int CPT = CHUNKS / kThreads;
  static constexpr int TILE_ELEMS = KT * LD;
  static constexpr size_t LDS_BYTES = 2 * 2 * TILE_ELEMS * sizeof(float);
  static_assert(2 * LDS_BYTES <= 160 * 1024, "LDS of two resident work-groups");
};

template <int D>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_f32(const AttnArgs a) {
  using C = F32Cfg<D>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  float *smem = reinterpret_cast<float *>(smem_raw);

  Tile t;
  if (!decode_tile(a, t)) return;
  const KItem &it = a.items[t.item];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;
  const int g = lane >> 5;

  const int rows_total = it.q_len * a.GP;
  const int tile_row0 = t.qt * C::QT;
  const int wave_row0 = tile_row0 + wave * 32;
  const int prow = wave_row0 + n;
  const bool row_ok = prow < rows_total;
  const int hkv = (t.hb * a.GP) / a.G;
  const int qpos = it.qpos0 + (row_ok ? prow : rows_total - 1) / a.GP;
  const int wave_last = min(wave_row0 + 31, rows_total - 1);
  const int wave_qpos_min = it.qpos0 + min(wave_row0, rows_total - 1) / a.GP;
  const int wave_qpos_max = it.qpos0 + wave_last / a.GP;
  const bool wave_active = wave_row0 < rows_total;
  const int tile_qpos_max = it.qpos0 + (min(tile_row0 + C::QT, rows_total) - 1) / a.GP;

  // Q fragment: lane half g holds d = (D/2)*g + kc, kc = 0 .. D/2-1.
  float qf[D / 2];
  {
    const int tok = (row_ok ? prow : 0) / a.GP;
    const int h = t.hb * a.GP + (row_ok ? prow : 0) % a.GP;
    const float *qp = reinterpret_cast<const float *>(a.q) + (int64_t)t.b * a.q_sb +
                      (int64_t)(it.q_start + tok) * a.q_ss + (int64_t)h * a.q_sh + (D / 2) * g;
#pragma unroll
    for (int j = 0; j < D / 8; ++j) {
      f32x4 v = row_ok ? *(const f32x4 *)(qp + 4 * j) : f32x4{};
      qf[4 * j] = v[0];
      qf[4 * j + 1] = v[1];
      qf[4 * j + 2] = v[2];
      qf[4 * j + 3] = v[3];
    }
  }

  f32x16 acc[D / 32];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb) acc[mb] = f32x16{};
  float m_run = neg_inf();
  float l_part = 0.0f;

  SegRange sr0 = seg_range(it, 0, t.split, tile_qpos_max);
  SegRange sr1 = sr0;
  int nt0 = (sr0.hi - sr0.lo + C::KT - 1) / C::KT;
  int nt1 = 0;
  if (it.nseg > 1) {
    sr1 = seg_range(it, 1, t.split, tile_qpos_max);
    nt1 = (sr1.hi - sr1.lo + C::KT - 1) / C::KT;
  }
  const int ntiles = nt0 + nt1;

  const float *kbase = reinterpret_cast<const float *>(a.k) + (int64_t)t.b * a.k_sb + (int64_t)hkv * a.k_sh;
  const float *vbase = reinterpret_cast<const float *>(a.v) + (int64_t)t.b * a.v_sb + (int64_t)hkv * a.v_sh;

  f32x4 kreg[C::CPT], vreg[C::CPT];

  auto tile_info = [&](int ti, SegRange &sr, int &key0) {
    if (ti < nt0) {
      sr = sr0;
      key0 = sr0.lo + ti * C::KT;
    } else {
      sr = sr1;
      key0 = sr1.lo + (ti - nt0) * C::KT;
    }
  };
  auto gload = [&](int ti) {
    SegRange sr;
    int key0;
    tile_info(ti, sr, key0);
    const int nvalid = sr.hi - key0;
#pragma unroll
    for (int u = 0; u < C::CPT; ++u) {
      const int c = tid + kThreads * u;
      const int key = c / (D / 4);
      const int col = (c % (D / 4)) * 4;
      if (key < nvalid) {
        const int64_t row = sr.kv_start + key0 + key;
        kreg[u] = *(const f32x4 *)(kbase + row * a.k_ss + col);
        vreg[u] = *(const f32x4 *)(vbase + row * a.v_ss + col);
      } else {
        kreg[u] = f32x4{};
        vreg[u] = f32x4{};
      }
    }
  };
  auto lstore = [&](int buf) {
    float *Ks = smem + buf * 2 * C::TILE_ELEMS;
    float *Vs = Ks + C::TILE_ELEMS;
#pragma unroll
    for (int u = 0; u < C::CPT; ++u) {
      const int c = tid + kThreads * u;
      const int key = c / (D / 4);
      const int col = (c % (D / 4)) * 4;
      *(f32x4 *)(Ks + key * C::LD + col) = kreg[u];
      *(f32x4 *)(Vs + key * C::LD + col) = vreg[u];
    }
  };

  if (ntiles > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();

  for (int ti = 0; ti < ntiles; ++ti) {
    const int buf = ti & 1;
    if (ti + 1 < ntiles) gload(ti + 1);
    SegRange sr;
    int kb;
    tile_info(ti, sr, kb);
    const float *Ks = smem + buf * 2 * C::TILE_ELEMS;
    const float *Vs = Ks + C::TILE_ELEMS;

    const bool skip = !wave_active || kb >= sr.hi || (sr.causal && sr.kpos0 + kb > wave_qpos_max);
    if (!skip) {
      const bool need_mask = (kb + 32 > sr.hi) || (sr.causal && sr.kpos0 + kb + 31 > wave_qpos_min);
      f32x16 s = f32x16{};
#pragma unroll
      for (int j = 0; j < D / 8; ++j) {
        const f32x4 ka = *(const f32x4 *)(Ks + n * C::LD + (D / 2) * g + 4 * j);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          s = __builtin_amdgcn_mfma_f32_32x32x2f32(ka[e], qf[4 * j + e], s, 0, 0, 0);
      }
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb + 8 * (r >> 2) + 4 * g + (r & 3);
          const bool vis = key < sr.hi && (!sr.causal || sr.kpos0 + key <= qpos);
          if (!vis) s[r] = neg_inf();
        }
      }
      float mx = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
      mx = max_halves(mx) * a.scale_log2;
      const float m_new = fmaxf(m_run, mx);
      const bool need = m_new > m_run + kRescaleThreshold;
      if (__builtin_amdgcn_ballot_w64(need)) {
        const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
        m_run = need ? m_new : m_run;
        l_part *= alpha;
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[mb][r] *= alpha;
      }
      const float moff = (m_run == neg_inf()) ? 0.0f : m_run;
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], a.scale_log2, -moff));
        l_part += p[r];
      }
      // out^T += V^T P^T: register r of P pairs key 8*(r/4) + 4*g + r%4.
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int krow = 8 * (r >> 2) + 4 * g + (r & 3);
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
          acc[mb] = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[krow * C::LD + 32 * mb + n], p[r], acc[mb], 0, 0, 0);
      }
    }

    if (ti + 1 < ntiles) lstore(buf ^ 1);
    __syncthreads();
  }

  epilogue<D>(a, it, t, prow, row_ok, acc, m_run, l_part, g);
}

// ---------------------------------------------------------------------------
// Standalone merge: one float4 of one (row, head) per thread.  Both outputs
// and the partial are streamed once, so the float4 traffic is non-temporal.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void merge_kernel(const MergeArgs a) {
  const int per_row = a.D / 4;
  const int64_t f = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)a.B * a.total_rows * a.H * per_row;
  if (f >= total) return;
  int d4, h, row, b;
  if (total < ((int64_t)1 << 31)) {  // 32-bit index arithmetic
    const uint32_t f32 = (uint32_t)f;
    d4 = (int)(f32 % (uint32_t)per_row);
    uint32_t rest = f32 / (uint32_t)per_row;
    h = (int)(rest % (uint32_t)a.H);
    rest /= (uint32_t)a.H;
    row = (int)(rest % (uint32_t)a.total_rows);
    b = (int)(rest / (uint32_t)a.total_rows);
  } else {
    d4 = (int)(f % per_row);
    int64_t rest = f / per_row;
    h = (int)(rest % a.H);
    rest /= a.H;
    row = (int)(rest % a.total_rows);
    b = (int)(rest / a.total_rows);
  }
  int k = 0;
  while (k + 1 < a.nranges && row >= a.ranges[k + 1].prefix) ++k;
  const int off = row - a.ranges[k].prefix;
  const int dr = a.ranges[k].dst0 + off;
  const int sr = a.ranges[k].src0 + off;

  float *op = a.out + (int64_t)b * a.o_sb + (int64_t)dr * a.o_ss + (int64_t)h * a.o_sh + 4 * d4;
  float *lp = a.lse + (int64_t)b * a.l_sb + (int64_t)dr * a.l_ss + (int64_t)h * a.l_sh;
  const float *bop = a.bout + (int64_t)b * a.bo_sb + (int64_t)sr * a.bo_ss + (int64_t)h * a.bo_sh + 4 * d4;
  const float *blp = a.blse + (int64_t)b * a.bl_sb + (int64_t)sr * a.bl_ss + (int64_t)h * a.bl_sh;

  // All four loads are issued before any test, so each thread pays one
  // memory round trip; the -inf identity cases are resolved with selects.
  const float blse = *blp;
  const float lse = *lp;
  const f32x4 bo = __builtin_nontemporal_load((const f32x4 *)bop);
  const f32x4 o = __builtin_nontemporal_load((const f32x4 *)op);
  const bool block_empty = blse == neg_inf();
  const bool run_empty = lse == neg_inf();
  const float diff = blse - lse;  // used only when both are finite
  const float w = 1.0f / (1.0f + __expf(-diff));
  f32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) r[j] = block_empty ? o[j] : (run_empty ? bo[j] : o[j] - w * (o[j] - bo[j]));
  __builtin_nontemporal_store(r, (f32x4 *)op);
  if (d4 == 0)
    *lp = block_empty ? lse : (run_empty ? blse : fmaxf(lse, blse) + log1pf(__expf(-fabsf(diff))));
}

// ---------------------------------------------------------------------------
// Split-K reduction.  The nsplit partials of a row are softmax results over
// disjoint key ranges; their combination is the log-sum-exp weighted mean
//   lse = m + ln sum_s exp(lse_s - m),  out = sum_s exp(lse_s - lse) out_s
// (m = max_s lse_s), the closed form of folding them with the merge rule.
// One work-group per (batch, head, row): kSplitGroups groups of D/4 threads
// (one float4 of the row each) take every kSplitGroups-th split, so each
// thread issues few independent loads; the groups' sums meet in LDS.  Then
// write, or merge into the running pair with the merge rule.
// ---------------------------------------------------------------------------
constexpr int kSplitGroups = 8;

template <int D>
__global__ __launch_bounds__(kSplitGroups * D / 4) void split_reduce_kernel(const SplitArgs a) {
  constexpr int per_row = D / 4;
  __shared__ float s_max[kSplitGroups], s_wsum[kSplitGroups];
  __shared__ f32x4 s_out[kSplitGroups][per_row];
  const int d4 = threadIdx.x % per_row;
  const int sg = threadIdx.x / per_row;
  int64_t rest = blockIdx.x;
  const int tok = (int)(rest % a.rows);
  rest /= a.rows;
  const int h = (int)(rest % a.H);
  const int b = (int)(rest / a.H);

  const int64_t split_stride = (int64_t)a.B * a.H * a.rows;
  const int64_t pr0 = ((int64_t)b * a.H + h) * a.rows + tok;
  constexpr int kU = 4;  // splits per thread per round of loads
  float m = neg_inf();
  for (int s0 = sg; s0 < a.nsplit; s0 += kU * kSplitGroups) {
    float lv[kU];
#pragma unroll
    for (int j = 0; j < kU; ++j) lv[j] = a.part_lse[pr0 + min(s0 + j * kSplitGroups, a.nsplit - 1) * split_stride];
#pragma unroll
    for (int j = 0; j < kU; ++j) m = fmaxf(m, lv[j]);
  }
  if (d4 == 0) s_max[sg] = m;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kSplitGroups; ++j) m = fmaxf(m, s_max[j]);

  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.0f;
  if (m != neg_inf()) {
    for (int s0 = sg; s0 < a.nsplit; s0 += kU * kSplitGroups) {
      float lv[kU];
      f32x4 po[kU];
#pragma unroll
      for (int j = 0; j < kU; ++j) {
        const int64_t pr = pr0 + min(s0 + j * kSplitGroups, a.nsplit - 1) * split_stride;
        lv[j] = a.part_lse[pr];
        po[j] = *(const f32x4 *)(a.part_out + pr * D + 4 * d4);
      }
#pragma unroll
      for (int j = 0; j < kU; ++j) {
        const float w = (s0 + j * kSplitGroups < a.nsplit) ? __expf(lv[j] - m) : 0.0f;  // 0 for an empty split
        wsum += w;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = __builtin_fmaf(w, po[j][e], o[e]);
      }
    }
  }
  s_out[sg][d4] = o;
  if (d4 == 0) s_wsum[sg] = wsum;
  __syncthreads();
  if (sg != 0) return;
  float l = neg_inf();
  if (m != neg_inf()) {
    wsum = 0.0f;
    o = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kSplitGroups; ++j) {
      wsum += s_wsum[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] += s_out[j][d4][e];
    }
    const float inv = 1.0f / wsum;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] *= inv;
    l = m + __logf(wsum);
  }

  const int orow = a.o_row0 + tok;
  float *op = a.out + (int64_t)b * a.o_sb + (int64_t)orow * a.o_ss + (int64_t)h * a.o_sh + 4 * d4;
  float *lp = a.lse + (int64_t)b * a.l_sb + (int64_t)orow * a.l_ss + (int64_t)h * a.l_sh;
  if (a.mode == kMerge && !a.first) {
    if (l == neg_inf()) return;
    const float lr = *lp;
    if (lr != neg_inf()) {
      const float diff = l - lr;
      const float w = 1.0f / (1.0f + __expf(-diff));
      f32x4 r = *(const f32x4 *)op;
#pragma unroll
      for (int j = 0; j < 4; ++j) r[j] = r[j] - w * (r[j] - o[j]);
      o = r;
      l = fmaxf(lr, l) + log1pf(__expf(-fabsf(diff)));
    }
  }
  *(f32x4 *)op = o;
  if (d4 == 0) *lp = l;
}

// Row-parallel form for many rows and few partials (a prefill chunk gathered
// over the K/V shards): one thread per (row, 4 dims), every partial of its
// row loaded up front, no cross-thread reduction.  Same combination and
// same partial order as split_reduce_kernel.
constexpr int kRowsMaxSplits = 16;
constexpr int kRowsThreads = 256;

template <int D>
__global__ __launch_bounds__(kRowsThreads) void split_reduce_rows_kernel(const SplitArgs a) {
  constexpr int per_row = D / 4;
  const int64_t nrows = (int64_t)a.B * a.H * a.rows;
  const int64_t r = (int64_t)blockIdx.x * (kRowsThreads / per_row) + threadIdx.x / per_row;
  if (r >= nrows) return;
  const int d4 = threadIdx.x % per_row;
  const int tok = (int)(r % a.rows);
  const int h = (int)((r / a.rows) % a.H);
  const int b = (int)(r / ((int64_t)a.rows * a.H));
  const int64_t split_stride = nrows;

  float lv[kRowsMaxSplits];
  f32x4 po[kRowsMaxSplits];
#pragma unroll
  for (int s = 0; s < kRowsMaxSplits; ++s) {
    if (s < a.nsplit) {
      lv[s] = a.part_lse[r + s * split_stride];
      po[s] = *(const f32x4 *)(a.part_out + (r + s * split_stride) * D + 4 * d4);
    }
  }
  float m = neg_inf();
#pragma unroll
  for (int s = 0; s < kRowsMaxSplits; ++s)
    if (s < a.nsplit) m = fmaxf(m, lv[s]);
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  float l = neg_inf();
  if (m != neg_inf()) {
    float wsum = 0.0f;
#pragma unroll
    for (int s = 0; s < kRowsMaxSplits; ++s) {
      if (s < a.nsplit) {
        const float w = __expf(lv[s] - m);  // 0 for an empty partial
        wsum += w;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = __builtin_fmaf(w, po[s][e], o[e]);
      }
    }
    const float inv = 1.0f / wsum;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] *= inv;
    l = m + __logf(wsum);
  }

  const int orow = a.o_row0 + tok;
  float *op = a.out + (int64_t)b * a.o_sb + (int64_t)orow * a.o_ss + (int64_t)h * a.o_sh + 4 * d4;
  float *lp = a.lse + (int64_t)b * a.l_sb + (int64_t)orow * a.l_ss + (int64_t)h * a.l_sh;
  if (a.mode == kMerge && !a.first) {
    if (l == neg_inf()) return;
    const float lr = *lp;
    if (lr != neg_inf()) {
      const float diff = l - lr;
      const float w = 1.0f / (1.0f + __expf(-diff));
      f32x4 rr = *(const f32x4 *)op;
#pragma unroll
      for (int j = 0; j < 4; ++j) rr[j] = rr[j] - w * (rr[j] - o[j]);
      o = rr;
      l = fmaxf(lr, l) + log1pf(__expf(-fabsf(diff)));
    }
  }
  *(f32x4 *)op = o;
  if (d4 == 0) *lp = l;
}

// ---------------------------------------------------------------------------
// Static scratch of the entry point that allocates nothing.  Each GPU holds
// its own copy from code-object load to process end.  Host code never uses
// the array's name as an address (on the host it is only a stand-in symbol):
// the device address is looked up once per device and passed to kernels.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[RA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

int noalloc_scratch(void **ptr, size_t *bytes) {
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t rc = hipGetDevice(&dev);
  if (rc != hipSuccess) return (int)rc;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (addr[dev] == nullptr) {
    void *p = nullptr;
    rc = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (rc != hipSuccess) return (int)rc;
    if (p == nullptr) return (int)hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  *bytes = sizeof(scratch);
  return 0;
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
// Dynamic LDS above the default limit must be allowed once per kernel.  The
// attribute is set by the initialiser of a function-local static, which C++
// runs exactly once even when several host threads launch concurrently.
template <typename K>
static int allow_lds(K kernel, size_t bytes) {
  return (int)hipFuncSetAttribute((const void *)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <int D, bool NT, bool ROT>
static int launch_bf16(const AttnArgs &a, dim3 grid, hipStream_t s) {
  static const int attr = allow_lds(attn_fwd_bf16<D, NT, ROT>, Bf16Cfg<D>::LDS_BYTES);
  if (attr) return attr;
  attn_fwd_bf16<D, NT, ROT><<<grid, dim3(Bf16Cfg<D>::THREADS), Bf16Cfg<D>::LDS_BYTES, s>>>(a);
  return 0;
}

// Compute units of the current device, read once per device.
static int cu_count() {
  static std::atomic<int> cache[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Rotating priorities pay in launches of up to about four rounds of resident
// work-groups (one rank's ring step, one block); in long launches the usual
// oldest-first order keeps the copy pipelines steadier.
template <int D>
static bool few_rounds(dim3 grid) {
  return (int64_t)grid.x <= (int64_t)4 * cu_count() * Bf16Cfg<D>::OCC;
}

template <int D>
static int launch_f32(const AttnArgs &a, dim3 grid, dim3 block, hipStream_t s) {
  static const int attr = allow_lds(attn_fwd_f32<D>, F32Cfg<D>::LDS_BYTES);
  if (attr) return attr;
  attn_fwd_f32<D><<<grid, block, F32Cfg<D>::LDS_BYTES, s>>>(a);
  return 0;
}

int launch_attn(const AttnArgs &a, int dtype, int head_dim, void *stream) {
  const dim3 grid(a.per_xcd * 8), block(kThreads);
  hipStream_t s = (hipStream_t)stream;
  int rc;
  if (dtype == 0) {
    // K/V read by exactly one work-group (one query tile per item, all the
    // query heads of a K/V head packed into it, e.g. decode): stream them.
    bool streamed = a.GP == a.G;
    for (int i = 0; i < a.nitems; ++i) streamed = streamed && a.items[i].nqt == 1;
    if (streamed)
      rc = head_dim == 128 ? launch_bf16<128, true, false>(a, grid, s) : launch_bf16<64, true, false>(a, grid, s);
    else if (head_dim == 128)
      rc = few_rounds<128>(grid) ? launch_bf16<128, false, true>(a, grid, s) : launch_bf16<128, false, false>(a, grid, s);
    else
      rc = few_rounds<64>(grid) ? launch_bf16<64, false, true>(a, grid, s) : launch_bf16<64, false, false>(a, grid, s);
  } else {
    rc = head_dim == 128 ? launch_f32<128>(a, grid, block, s) : launch_f32<64>(a, grid, block, s);
  }
  if (rc) return rc;
  return (int)hipGetLastError();
}

int launch_merge(const MergeArgs &a, void *stream) {
  const int64_t total = (int64_t)a.B * a.total_rows * a.H * (a.D / 4);
  if (total == 0) return 0;
  const dim3 grid((unsigned)((total + 255) / 256)), block(256);
  hipLaunchKernelGGL(merge_kernel, grid, block, 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

int launch_split_reduce(const SplitArgs &a, void *stream) {
  const int64_t rows = (int64_t)a.B * a.H * a.rows;
  if (rows == 0) return 0;
  if (a.nsplit <= kRowsMaxSplits && rows >= 4096) {  // many rows, few partials
    const int rows_per_wg = kRowsThreads / (a.D / 4);
    const dim3 g((unsigned)((rows + rows_per_wg - 1) / rows_per_wg));
    if (a.D == 128)
      split_reduce_rows_kernel<128><<<g, dim3(kRowsThreads), 0, (hipStream_t)stream>>>(a);
    else
      split_reduce_rows_kernel<64><<<g, dim3(kRowsThreads), 0, (hipStream_t)stream>>>(a);
    return (int)hipGetLastError();
  }
  const dim3 grid((unsigned)rows);
  if (a.D == 128)
    split_reduce_kernel<128><<<grid, dim3(kSplitGroups * 32), 0, (hipStream_t)stream>>>(a);
  else
    split_reduce_kernel<64><<<grid, dim3(kSplitGroups * 16), 0, (hipStream_t)stream>>>(a);
  return (int)hipGetLastError();
}

}  // namespace ra
