// fd_plan.cpp -- host planner: how many chunks, how long, which kernel.
//
// "Flash-Decoding for long-context inference" (Stanford CRFM), section
// "Multi-head attention for decoding": with one query per head the only
// parallelism a plain attention kernel has is batch x heads, so at small
// batch it occupies a sliver of the GPU; the Flash-Decoding section adds
// the key/value sequence as a further parallel dimension, paid for by a
// small merge step.  The shipped libraries pick between the split and the
// unsplit kernel by problem size.  This planner makes that choice for the
// compute-unit count of the device at hand (256 on MI355X):
//
//   * kernel: the matrix cores for bf16, and for fp32 from groups of 3
//     query heads (at D = 64 also smaller groups from 4096 keys) and for
//     every paged or several-token call; the vector ALU for the other fp32
//     shapes (planned for two workgroups per CU, below);
//   * work units U = B * Hkv: one workgroup streams one KV-head slab range
//     and serves all Hq / Hkv query heads of that group, so K/V are read
//     from HBM exactly once;
//   * aim for kBlocksPerCU workgroups per CU; split each sequence into
//     S = ceil(target / U) chunks, each a multiple of the 32-key tile and at
//     least kMinChunk keys -- or a single tile on the matrix cores, when
//     one-tile chunks of every sequence still fit one round of workgroups
//     and leave a row at most kMaxTileChunks partials.  Short chunks pay: at
//     batch 1 a workgroup's time is mostly the latency of its tile chain,
//     so 64-key chunks over all CUs beat 256-key chunks over a quarter of
//     them (1024 keys: 7.8 against 10.3 us), and 32-key ones beat 64-key
//     ones (7.5 against 7.9 us);
//   * S == 1 means no partials and no merge pass at all; it is taken when a
//     split would not take more than kSplitGain keys of 256 bytes (one
//     D = 128 bf16 row) off each workgroup's share, about what the merge
//     pass costs; the matrix-core pass counts it in bytes, so rows of
//     D = 64 give twice the keys;
//   * with per-sequence lengths the mix is unknown on the host (the library
//     never reads device memory synchronously), so chunks are also capped
//     at kVarlenChunk keys, so that no single long sequence sets the finish
//     time, and the grid is cut to max(half the chunk count's upper bound,
//     kGridPerCU per CU): the matrix-core kernel lets a workgroup take a
//     second chunk, and most of the bound is usually empty.  A paged cache
//     always comes with per-sequence lengths; its Lmax is the block table's
//     capacity, max_pages * page_size.
//
// The constants are this library's own (the pages give none) and the
// result of any plan is the same attention; only speed depends on them.
#include <algorithm>
#include <cmath>

#include "fd_internal.h"

namespace fd {

namespace {

// Tunables (measured on MI355X; overridable at build time for sweeps).
#ifndef FD_BLOCKS_PER_CU
#define FD_BLOCKS_PER_CU 1
#endif
#ifndef FD_MIN_CHUNK
#define FD_MIN_CHUNK 64
#endif
#ifndef FD_SPLIT_GAIN
#define FD_SPLIT_GAIN 256
#endif
#ifndef FD_VARLEN_CHUNK
#define FD_VARLEN_CHUNK 2048
#endif
#ifndef FD_MFMA_WAVES
#define FD_MFMA_WAVES 4
#endif
// Partial layout: -1 by the rounds of workgroups (the rule below), 0 always
// row-major, 1 always chunk-major (for measuring one against the other).
#ifndef FD_PARTIAL_LAYOUT
#define FD_PARTIAL_LAYOUT -1
#endif
constexpr int kBlocksPerCU = FD_BLOCKS_PER_CU;
constexpr int kMinChunk = FD_MIN_CHUNK;
constexpr int kSplitGain = FD_SPLIT_GAIN;
constexpr int kVarlenChunk = FD_VARLEN_CHUNK;
constexpr int kGridPerCU = 8;
// One-tile chunks at most this many per sequence (the merge of more
// partials per row outweighs the shorter chunks: measured at batch 1, 2
// KV heads, 2048 keys, 64 one-tile chunks took 9.1 us against 8.5 in 32).
constexpr int kMaxTileChunks = 32;
constexpr int kMfmaWaves = FD_MFMA_WAVES;
static_assert(kMfmaWaves == 2 || kMfmaWaves == 4 || kMfmaWaves == 8,
              "the matrix-core kernel is built for 2, 4 or 8 wavefronts");
constexpr int kValuWaves = 4;
// The vector-ALU kernel is latency-bound per workgroup, so it is planned
// for two workgroups per CU, twice the matrix-core pass (short caches also
// take one-tile chunks, below).  Measured (fp32, device time of steps
// replayed from a graph) against four per CU: 16k keys, 32 query / 8 KV
// heads, D = 128: 31.1 us against 32.6; 64 / 8 heads 48.4 against 54.0;
// 64k keys 94.9 against 102.1; one sequence of 8 query heads on one KV
// head at 16k keys 23.7 against 27.7 (256 chunks against 512); at 8192 keys
// and below within 1-3% either way.
constexpr int kValuBlocksPerCU = 2;

int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }
int round_up(long a, long b) { return (int)(((a + b - 1) / b) * b); }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

int validate_shape(int B, int Hq, int Hkv, int D, int Lmax,
                   fd_dtype_t dtype) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Lmax <= 0)
    return FD_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return FD_ERR_INVALID_ARG;
  if (dtype != FD_BF16 && dtype != FD_F16 && dtype != FD_F32)
    return FD_ERR_UNSUPPORTED;
  if (D != 64 && D != 128 && D != 256) return FD_ERR_UNSUPPORTED;
  if (Hq / Hkv > kMaxHeadsPerKv) return FD_ERR_UNSUPPORTED;
  // Keys per sequence: chunk sizes, key offsets and lo + C stay in int.
  // (2^30 keys of one KV head at D = 128 are 256 GB, beyond any GPU's HBM.)
  if (Lmax > kMaxKeys) return FD_ERR_UNSUPPORTED;
  // Index arithmetic below uses int for per-slab row counts and size_t for
  // element offsets; guard the products that are computed in int.
  if ((long)B * Hkv > (1L << 30) || (long)B * Hq > (1L << 30))
    return FD_ERR_UNSUPPORTED;
  return FD_OK;
}

WorkspaceLayout workspace_layout(const Plan &p) {
  WorkspaceLayout w{0, 0, 0, 0};
  if (!p.combine) return w;
  size_t rows = (size_t)p.B * p.Tq * p.Hq * p.splits;
  w.ticket_bytes = p.fused ? align256((size_t)p.B * p.Hkv * sizeof(int)) : 0;
  w.o_part_off = w.ticket_bytes;
  w.lse_part_off = w.o_part_off + align256(rows * p.D * sizeof(float));
  w.total = w.lse_part_off + align256(rows * sizeof(float));
  return w;
}

int make_plan(int B, int Hq, int Hkv, int D, int Lmax, fd_dtype_t dtype,
              bool varlen, int requested_splits, int requested_variant,
              int flags, int num_cus, Plan *p, Extra extra) {
  int rc = validate_shape(B, Hq, Hkv, D, Lmax, dtype);
  if (rc != FD_OK) return rc;
  if (extra.Tq < 1) return FD_ERR_INVALID_ARG;
  // Several new tokens or a paged cache: the matrix-core kernels only (bf16
  // or fp32), whose 16-column q-tile holds the G * Tq query rows of a KV
  // head (or of a virtual one, below).
  const bool general = extra.Tq > 1 || extra.paged;
  if (general) {
    if (requested_variant == FD_VARIANT_VALU) return FD_ERR_UNSUPPORTED;
    if (extra.Tq > kMaxGroup) return FD_ERR_UNSUPPORTED;
    if ((long)B * Hq * extra.Tq > (1L << 30)) return FD_ERR_UNSUPPORTED;
  }
  if (num_cus <= 0) return FD_ERR_INVALID_ARG;
  if (requested_splits < 0) return FD_ERR_INVALID_ARG;
  if (requested_variant < FD_VARIANT_AUTO ||
      requested_variant > FD_VARIANT_VALU)
    return FD_ERR_INVALID_ARG;
  if (flags & ~kKnownFlags) return FD_ERR_INVALID_ARG;
  // The unified maximum (FlashDecoding++) is built for the 16-bit (bf16 or
  // fp16) matrix-core pass over a contiguous cache, one token per sequence.
  const bool unified = flags & FD_FLAG_UNIFIED_MAX;
  if (unified && (dtype == FD_F32 || general ||
                  requested_variant == FD_VARIANT_VALU))
    return FD_ERR_UNSUPPORTED;

  Plan q{};
  q.B = B;
  q.Hq = Hq;
  q.Hkv = Hkv;
  q.G = Hq / Hkv;
  q.D = D;
  q.Lmax = Lmax;
  q.Tq = extra.Tq;
  q.dtype = dtype;
  q.varlen = varlen;
  q.paged = extra.paged;
  q.unified = unified;
  q.num_cus = num_cus;

  // Kernel variant: bf16 and fp16 on the matrix cores.  fp32 on the matrix
  // cores too
  // from groups of 3 query heads (and, at D = 64, for smaller groups from
  // 4096 keys on); below that on the vector ALU, whose cost per key grows
  // with G while the fp32 MFMA pass pays for 16 columns at any G.  Measured
  // (fp32, device time of steps replayed from a graph, vector ALU against
  // matrix cores at each one's planned split count), one sequence on 8 KV
  // heads: D = 128, 16k keys, G = 1 26.0 / 28.6 us, G = 2 26.7 / 28.6,
  // G = 3 30.5 / 28.7, G = 4 30.5 / 28.7, G = 8 47.8 / 29.4; 64k keys G = 2
  // 83.5 / 85.8, G = 4 91.7 / 85.8; D = 64, G = 1: 1024 keys 6.6 / 7.2,
  // 4096 keys 8.8 / 8.7, 16k keys 15.9 / 15.6; G = 3 at 1024 keys 8.1 / 7.4.
  // Paged caches and several tokens run on the matrix cores only.
  // Head dimension 256: the matrix cores only.
  if (requested_variant != FD_VARIANT_AUTO)
    q.variant = requested_variant;
  else
    q.variant = dtype != FD_F32 || general || q.G >= 3 || D > 128 ||
                        (D == 64 && Lmax >= 4096)
                    ? FD_VARIANT_MFMA
                    : FD_VARIANT_VALU;
  if (q.variant == FD_VARIANT_VALU && D > 128) return FD_ERR_UNSUPPORTED;
  // The 16-bit vector-ALU kernel keeps G query rows of 8 values per lane in
  // registers; beyond 4 rows the matrix-core kernel is the one to use.  The
  // fp32 one serves up to 16.
  if (q.variant == FD_VARIANT_VALU && dtype != FD_F32 && q.G > 4)
    return FD_ERR_UNSUPPORTED;
  if (q.variant == FD_VARIANT_VALU && q.G > kMaxGroup)
    return FD_ERR_UNSUPPORTED;
  // The vector-ALU kernel computes G dot products per key, each finished by
  // a butterfly across the lanes of a row; past 8 query heads (16 rows in
  // registers, two wavefronts) it ran at 0.27 TB/s.  Even groups of 10-16
  // heads run as two half-groups instead, each its own virtual KV head on
  // the same slab: K/V are read twice, at the rate of the 8-row kernel.
  q.kv_rep = 1;
  if (q.variant == FD_VARIANT_VALU && q.G > 8 && q.G % 2 == 0) {
    q.kv_rep = 2;
    q.Hkv *= 2;
    q.G /= 2;
  }
  // Matrix cores: more than 16 query rows per KV head (G * Tq) run as the
  // fewest equal virtual groups that fit the q-tile, each a virtual KV head
  // reading the same slab, so K/V are read kv_rep times (multi-query models
  // with many query heads per KV head; several tokens of a large group).
  if (q.variant == FD_VARIANT_MFMA && (long)q.G * q.Tq > kMaxGroup) {
    int r = (q.G * q.Tq + kMaxGroup - 1) / kMaxGroup;
    while (q.G % r != 0 || (q.G / r) * q.Tq > kMaxGroup) ++r;
    q.kv_rep = r;
    q.Hkv *= r;
    q.G /= r;
  }
  if (q.variant == FD_VARIANT_MFMA)
    q.waves = kMfmaWaves;
  else
    q.waves = q.G > 8 ? 2 : kValuWaves;  // keeps LDS of the merge <= 33 KB

  const int blocks_per_cu =
      q.variant == FD_VARIANT_VALU ? kValuBlocksPerCU : kBlocksPerCU;
  const int max_splits = ceil_div(Lmax, kKeyTile);
  const int full_chunk = round_up(Lmax, kKeyTile);
  int chunk;
  if (requested_splits > 0) {
    int s = std::min(requested_splits, max_splits);
    chunk = round_up(ceil_div(Lmax, s), kKeyTile);
  } else {
    const long units = (long)B * q.Hkv;
    const long target = (long)num_cus * blocks_per_cu;
    int s = (int)std::max(1L, (target + units - 1) / units);
    chunk = round_up(ceil_div(Lmax, s), kKeyTile);
    // Matrix cores, short caches: one-tile chunks when they all run in one
    // round and a row merges at most kMaxTileChunks partials.  Measured
    // (device time of steps replayed from a graph), 64 query / 8 KV heads,
    // D = 128, batch 1: 384 keys 7.44 -> 6.91 us, 640 keys 7.93 -> 7.33,
    // 1024 keys 7.86 -> 7.54; batch 2 at 512 keys 7.94 -> 7.44; with 8 KV
    // heads at 1280 keys (40 tiles, 320 workgroups) they were slower.
    const int tiles = ceil_div(Lmax, kKeyTile);
    const bool mfma = q.variant == FD_VARIANT_MFMA;
    // The vector-ALU kernel does G dot products per key, so its chunks pay
    // for themselves sooner as G grows: from G = 4 on, one-tile chunks up to
    // twice as many per sequence (measured, fp32, one sequence, 4 query
    // heads on each of 4 KV heads, D = 128, 2048 keys: 12.6 -> 10.6 us; at
    // 16k keys 128-key chunks were fastest).
    const bool tile_chunks =
        (tiles <= kMaxTileChunks ||
         (!mfma && q.G >= 4 && tiles <= 2 * kMaxTileChunks)) &&
        units * tiles <= target;
    const int chunk64 = std::max(chunk, std::min(kMinChunk, full_chunk));
    chunk = mfma && tile_chunks
                ? std::max(chunk, std::min(kKeyTile, full_chunk))
                : chunk64;
    // Short caches: one launch beats two.  The merge pass (a second kernel)
    // costs about as much as a workgroup streaming kSplitGain more keys, so
    // a split must take more than that off each workgroup's share.
    // Measured on MI355X (device time of steps replayed from a graph):
    // batch 1, 64 query / 8 KV heads, 256 keys: 6.4 us unsplit, 7.0 in
    // 8 chunks; 512 keys: 10.1 unsplit, 7.4 in 16 chunks; 16 sequences
    // at 512 keys: 12.4 unsplit, 13.3 in two chunks.  D = 64 rows are half
    // as long: 384 keys, 5.8 unsplit against 6.9 in six chunks.
    // Counted in bytes of 256-byte rows (one D = 128 bf16 row), and on the
    // vector ALU per query row of the group, whose work per key is G dot
    // products (measured, fp32, 256 keys: 16 query heads on one KV head,
    // D = 64, 53 us unsplit against 17 in 8 chunks; 8 heads, D = 128,
    // 2 sequences, 11.2 against 7.1).
    const int elem = dtype == FD_F32 ? 4 : 2;
    const int gain =
        kSplitGain * 256 / (D * elem) / (mfma ? 1 : q.G);
    if (Lmax - chunk <= gain) {
      chunk = full_chunk;
    } else if (!mfma && tile_chunks) {
      // fp32: decided on 64-key chunks, split into one-tile ones
      // (measured, 8 heads, D = 64, one sequence, 1024 keys: 7.0 -> 6.8 us;
      // four sequences, 512 keys: 7.6 -> 7.4)
      chunk = std::max(round_up(ceil_div(Lmax, s), kKeyTile), kKeyTile);
    }
    // Unknown lengths: no chunk longer than kVarlenChunk, and no longer
    // than the even split would make it were every sequence full.
    if (varlen) chunk = std::min(chunk, kVarlenChunk);
  }
  q.chunk = chunk;
  q.splits = ceil_div(Lmax, chunk);
  q.combine = q.splits > 1 || (flags & FD_FLAG_PARTIALS);
  q.fused = q.combine && (flags & FD_FLAG_FUSED_MERGE);
  long grid = (long)B * q.Hkv * q.splits;
  if (grid > 0x7FFFFFFFL) return FD_ERR_UNSUPPORTED;
  // Per-sequence lengths: the chunk count is only an upper bound (every
  // sequence at Lmax), and each workgroup of the matrix-core kernel can take
  // two chunks, so launch max(half the bound, kGridPerCU per CU): enough for
  // the hardware to deal typical batches one chunk per workgroup, with
  // fewer empty workgroups at the end of the dispatch.
  // When every chunk id any lengths could need fits in one round of
  // workgroups, the matrix-core kernel maps ids straight to (b, s, g) and
  // reads only its own sequence's length: no work list to build, and no
  // order to keep, since all chunks run at once.
  q.direct = varlen && q.variant == FD_VARIANT_MFMA &&
             grid <= (long)num_cus * kBlocksPerCU;
  if (varlen && q.variant == FD_VARIANT_MFMA)
    grid = std::min(grid, std::max((grid + 1) / 2, (long)num_cus * kGridPerCU));
  q.grid = (int)grid;
  // Partial layout.  When the workgroups run in several rounds, chunks that
  // finish store their partials while the others still stream K/V, and on
  // MI355X those stores slow the read stream far beyond their bytes; one
  // contiguous block per chunk (chunk-major) costs less there than G rows
  // S partials apart.  When every chunk runs in the same round, the stores
  // come together at the end, and the merge's contiguous reads of each
  // row's partials (row-major) are the cheaper side.
  q.chunk_major = q.combine && (FD_PARTIAL_LAYOUT >= 0
                                    ? FD_PARTIAL_LAYOUT == 1
                                    : grid > (long)num_cus * blocks_per_cu);
  q.ws_bytes = workspace_layout(q).total;
  *p = q;
  return FD_OK;
}

}  // namespace fd
