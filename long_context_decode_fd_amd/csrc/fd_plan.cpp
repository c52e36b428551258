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
//   * work units U = B * Hkv: one workgroup streams one KV-head slab range
//     and serves all Hq / Hkv query heads of that group, so K/V are read
//     from HBM exactly once;
//   * aim for kBlocksPerCU workgroups per CU; split each sequence into
//     S = ceil(target / U) chunks, each a multiple of the 32-key tile and at
//     least kMinChunk keys (the per-workgroup prologue and the partial
//     write, 2 * G * 4 bytes per key-row pair, must stay small next to the
//     2 * C * D * elem bytes of K/V a chunk streams);
//   * S == 1 means no partials and no merge pass at all; caches of up to
//     2 * kMinChunk keys always take it (one launch beats two there);
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
#define FD_MIN_CHUNK 256
#endif
#ifndef FD_VARLEN_CHUNK
#define FD_VARLEN_CHUNK 2048
#endif
#ifndef FD_MFMA_WAVES
#define FD_MFMA_WAVES 4
#endif
constexpr int kBlocksPerCU = FD_BLOCKS_PER_CU;
constexpr int kMinChunk = FD_MIN_CHUNK;
constexpr int kVarlenChunk = FD_VARLEN_CHUNK;
constexpr int kGridPerCU = 8;
constexpr int kMfmaWaves = FD_MFMA_WAVES;
static_assert(kMfmaWaves == 2 || kMfmaWaves == 4 || kMfmaWaves == 8,
              "the matrix-core kernel is built for 2, 4 or 8 wavefronts");
constexpr int kValuWaves = 4;

int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }
int round_up(long a, long b) { return (int)(((a + b - 1) / b) * b); }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

int validate_shape(int B, int Hq, int Hkv, int D, int Lmax,
                   fd_dtype_t dtype) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Lmax <= 0)
    return FD_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return FD_ERR_INVALID_ARG;
  if (dtype != FD_BF16 && dtype != FD_F32) return FD_ERR_UNSUPPORTED;
  if (D != 64 && D != 128) return FD_ERR_UNSUPPORTED;
  if (Hq / Hkv > kMaxGroup) return FD_ERR_UNSUPPORTED;
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
  // Several new tokens or a paged cache: the matrix-core kernel only, with
  // all G * Tq query rows of a KV head in its 16-column q-tile.
  const bool general = extra.Tq > 1 || extra.paged;
  if (general) {
    if (dtype != FD_BF16 || requested_variant == FD_VARIANT_VALU)
      return FD_ERR_UNSUPPORTED;
    if ((long)(Hq / Hkv) * extra.Tq > kMaxGroup) return FD_ERR_UNSUPPORTED;
    if ((long)B * Hq * extra.Tq > (1L << 30)) return FD_ERR_UNSUPPORTED;
  }
  if (num_cus <= 0) return FD_ERR_INVALID_ARG;
  if (requested_splits < 0) return FD_ERR_INVALID_ARG;
  if (requested_variant < FD_VARIANT_AUTO ||
      requested_variant > FD_VARIANT_VALU)
    return FD_ERR_INVALID_ARG;
  if (flags & ~kKnownFlags) return FD_ERR_INVALID_ARG;
  // The unified maximum (FlashDecoding++) is built for the bf16
  // matrix-core pass over a contiguous cache, one token per sequence.
  const bool unified = flags & FD_FLAG_UNIFIED_MAX;
  if (unified && (dtype != FD_BF16 || general ||
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

  // Kernel variant: matrix cores need bf16; fp32 runs on the vector ALU.
  if (requested_variant == FD_VARIANT_MFMA && dtype != FD_BF16)
    return FD_ERR_UNSUPPORTED;
  if (requested_variant != FD_VARIANT_AUTO)
    q.variant = requested_variant;
  else
    q.variant = dtype == FD_BF16 ? FD_VARIANT_MFMA : FD_VARIANT_VALU;
  // The bf16 vector-ALU kernel keeps G query rows of 8 values per lane in
  // registers; beyond 4 rows the matrix-core kernel is the one to use.
  if (q.variant == FD_VARIANT_VALU && dtype == FD_BF16 && q.G > 4)
    return FD_ERR_UNSUPPORTED;
  if (q.variant == FD_VARIANT_MFMA)
    q.waves = kMfmaWaves;
  else
    q.waves = q.G > 8 ? 2 : kValuWaves;  // keeps LDS of the merge <= 33 KB

  const int max_splits = ceil_div(Lmax, kKeyTile);
  const int full_chunk = round_up(Lmax, kKeyTile);
  int chunk;
  if (requested_splits > 0) {
    int s = std::min(requested_splits, max_splits);
    chunk = round_up(ceil_div(Lmax, s), kKeyTile);
  } else {
    const long units = (long)B * Hkv;
    const long target = (long)num_cus * kBlocksPerCU;
    int s = (int)std::max(1L, (target + units - 1) / units);
    chunk = round_up(ceil_div(Lmax, s), kKeyTile);
    chunk = std::max(chunk, std::min(kMinChunk, full_chunk));
    // Short caches: one launch beats two.  Up to 2 * kMinChunk keys the
    // merge pass (a second kernel) costs more than streaming the whole
    // sequence in one workgroup per (sequence, KV head): measured, batch 1
    // at 512 keys took 9.8 us unsplit against 12.8 us in two chunks; from
    // 768 keys on the split is ahead.
    if (Lmax <= 2 * kMinChunk) chunk = full_chunk;
    // Unknown lengths: no chunk longer than kVarlenChunk, and no longer
    // than the even split would make it were every sequence full.
    if (varlen) chunk = std::min(chunk, kVarlenChunk);
  }
  q.chunk = chunk;
  q.splits = ceil_div(Lmax, chunk);
  q.combine = q.splits > 1 || (flags & FD_FLAG_PARTIALS);
  q.fused = q.combine && (flags & FD_FLAG_FUSED_MERGE);
  long grid = (long)B * Hkv * q.splits;
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
  q.ws_bytes = workspace_layout(q).total;
  *p = q;
  return FD_OK;
}

}  // namespace fd
