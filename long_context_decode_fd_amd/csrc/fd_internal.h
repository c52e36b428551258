// fd_internal.h -- declarations shared by the planner, the C ABI layer and
// the kernels of libfd.so.  Not installed; the public contract is fd.h.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "fd.h"

namespace fd {

// Keys per MFMA tile step of one wavefront, and the granularity of chunks.
constexpr int kKeyTile = 32;
// Largest query group (Hq / Hkv) one workgroup handles: the MFMA q-tile
// has 16 columns.  Larger groups run as several virtual KV heads.
constexpr int kMaxGroup = 16;
// Largest Hq / Hkv the library takes.
constexpr int kMaxHeadsPerKv = 128;
// Largest Lmax (keys per sequence) the library plans for.
constexpr int kMaxKeys = 1 << 30;

// Everything a launch needs, decided on the host.
struct Plan {
  int B, Hq, Hkv, G, D, Lmax;  // paged cache: Lmax = max_pages * page_size
  int Tq;                       // new query tokens per sequence (1: decode)
  fd_dtype_t dtype;
  bool varlen;
  bool paged;
  bool unified;     // unified-maximum softmax (FD_FLAG_UNIFIED_MAX)
  int num_cus;
  int variant;      // FD_VARIANT_MFMA or FD_VARIANT_VALU
  int waves;        // wavefronts per workgroup of the per-chunk pass
  int chunk;        // keys per chunk (multiple of kKeyTile)
  int splits;       // ceil(Lmax / chunk)
  int grid;         // workgroups of the per-chunk pass (upper bound)
  bool direct;      // with seqlens: chunk ids map straight to (b, s, g)
  bool combine;     // chunks leave partials to be merged (splits > 1)
  bool fused;       // merged by the last workgroup of each group
  bool chunk_major; // partial layout: chunk-major (several rounds of
                    // workgroups) or row-major (one round)
  int kv_rep;       // a group runs as kv_rep virtual KV heads on the same
                    // K/V slab (matrix cores: G * Tq > 16 query rows;
                    // vector ALU: half-groups past 8 heads): Hkv and G above
                    // are the virtual ones (Hkv * kv_rep, G / kv_rep)
  size_t ws_bytes;  // tickets + partial outputs + partial lse
};

// Host-side checks of sizes/dtype shared by fd_plan and the decode calls.
int validate_shape(int B, int Hq, int Hkv, int D, int Lmax, fd_dtype_t dtype);

// Cache layout and query count beyond the plain decode call.
struct Extra {
  int Tq = 1;          // query tokens per sequence
  bool paged = false;  // K/V in pages behind a block table
};

// Flags the planner accepts (the public ones of fd.h).
constexpr int kKnownFlags =
    FD_FLAG_FUSED_MERGE | FD_FLAG_PARTIALS | FD_FLAG_UNIFIED_MAX;

// Fills *p for a validated shape; requested_splits 0 = heuristic.
int make_plan(int B, int Hq, int Hkv, int D, int Lmax, fd_dtype_t dtype,
              bool varlen, int requested_splits, int requested_variant,
              int flags, int num_cus, Plan *p, Extra extra = Extra());

// Byte offsets inside a workspace: the fused merge's per-group tickets
// (int32 [B * Hkv], must be zero when a call starts; the kernels leave
// them zero) come first, then the partial outputs and partial lse.
struct WorkspaceLayout {
  size_t ticket_bytes, o_part_off, lse_part_off, total;
};
WorkspaceLayout workspace_layout(const Plan &p);

// Paged K/V: token j of sequence b sits in page block_table[b][j /
// page_size], at t = j % page_size; pools [num_pages][page_size][Hkv][D]
// (token-major) or [num_pages][Hkv][page_size][D] (head_major).
struct PagedKV {
  const int32_t *block_table;
  int max_pages, page_size, num_pages;
  int head_major;
};

// Kernel launches (fd_kernels.hip).  Return hipError_t as int.
struct LaunchArgs {
  const void *q, *k, *v;
  const int32_t *seqlens;
  PagedKV paged;  // used when the plan is paged
  void *out;
  float *lse;
  float *o_part;
  float *lse_part;
  int *tickets;
  float scale;
  float unified_max;  // phi (natural-log units of the scaled score)
  void *stream;
  int phases;  // kPhaseChunks | kPhaseMerge
};
constexpr int kPhaseChunks = 1;
constexpr int kPhaseMerge = 2;
int launch_decode(const Plan &p, const LaunchArgs &a);

}  // namespace fd
