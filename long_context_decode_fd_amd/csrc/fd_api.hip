// fd_api.hip -- the C ABI of libfd.so (declared and documented in fd.h).
//
// Argument checks run on the host before any HIP call, so a bad call
// returns an FD_ERR_* code without touching the device.  Then the planner
// (fd_plan.cpp) decides chunking and kernel variant for the device's
// compute-unit count, and the kernels are queued on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <mutex>
#include <vector>

#include "fd_internal.h"

namespace {

constexpr int kVersion = 20200;  // 2.2.0

bool aligned(const void *p, size_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

// Per-device compute-unit count, queried once.  The per-device tables
// below grow with std::vector and are guarded by a std::mutex; both can
// throw, and no exception may leave an extern "C" function, so each table
// access runs in a try block that turns one into a status code.
int device_cus_locked(int dev, int *out);

int device_cus(int *out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FD_ERR_HIP;
  try {
    return device_cus_locked(dev, out);
  } catch (...) {
    return FD_ERR_HIP;
  }
}

int device_cus_locked(int dev, int *out) {
  static std::mutex mu;
  static std::vector<int> cache;
  std::lock_guard<std::mutex> lk(mu);
  if ((int)cache.size() <= dev) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount,
                              dev) != hipSuccess ||
        n <= 0)
      return FD_ERR_HIP;
    cache[dev] = n;
  }
  *out = cache[dev];
  return FD_OK;
}

// Library-owned workspace, one per device, grown on demand.  Layout:
// [ticket region][partials].  The ticket region, reserved in every layout
// and zeroed once when the buffer is allocated, holds the fused merge's
// per-group tickets; fused calls leave their tickets zero again and no
// other call writes there, so steady-state calls queue kernels only.  The
// partials of every plan start right after it.  Growing frees the old
// buffer (hipFree waits for the device, so work still queued on it
// completes first); a larger buffer is queued for zeroing on the caller's
// stream before that call's kernels.  The buffer may be freed and replaced
// by any later call, so a call that needs it is refused under stream
// capture: a graph must not hold its address.
struct OwnedWorkspace {
  void *ptr = nullptr;
  size_t bytes = 0;
  size_t ticket_cap = 0;  // bytes of the ticket region (256-aligned)
};

// Smallest ticket region: room for 16384 (b, KV head) groups.
constexpr size_t kMinTicketBytes = 16384 * sizeof(int);

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int owned_workspace_locked(int dev, size_t ticket_bytes, size_t part_bytes,
                           hipStream_t stream, void **tickets, void **parts);

int owned_workspace(size_t ticket_bytes, size_t part_bytes,
                    hipStream_t stream, void **tickets, void **parts) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FD_ERR_HIP;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return FD_ERR_HIP;
  if (cs != hipStreamCaptureStatusNone) return FD_ERR_CAPTURE;
  try {
    return owned_workspace_locked(dev, ticket_bytes, part_bytes, stream,
                                  tickets, parts);
  } catch (...) {
    return FD_ERR_WORKSPACE;
  }
}

int owned_workspace_locked(int dev, size_t ticket_bytes, size_t part_bytes,
                           hipStream_t stream, void **tickets, void **parts) {
  static std::mutex mu;
  static std::vector<OwnedWorkspace> ws;
  std::lock_guard<std::mutex> lk(mu);
  if ((int)ws.size() <= dev) ws.resize(dev + 1);
  OwnedWorkspace &w = ws[dev];
  if (w.ticket_cap < ticket_bytes || w.bytes - w.ticket_cap < part_bytes) {
    const size_t tcap = round_up(
        std::max({w.ticket_cap, ticket_bytes, kMinTicketBytes}), 256);
    // Round the partials up so that slowly growing problems do not
    // reallocate often.
    size_t pcap = std::max(w.bytes - w.ticket_cap, part_bytes);
    pcap = round_up(pcap + pcap / 4, (size_t)1 << 20);
    if (w.ptr) {
      if (hipFree(w.ptr) != hipSuccess) return FD_ERR_HIP;
      w.ptr = nullptr;
      w.bytes = w.ticket_cap = 0;
    }
    void *p = nullptr;
    if (hipMalloc(&p, tcap + pcap) != hipSuccess) return FD_ERR_WORKSPACE;
    if (hipMemsetAsync(p, 0, tcap, stream) != hipSuccess) {
      (void)hipFree(p);
      return FD_ERR_HIP;
    }
    w.ptr = p;
    w.bytes = tcap + pcap;
    w.ticket_cap = tcap;
  }
  *tickets = w.ptr;
  *parts = static_cast<char *>(w.ptr) + w.ticket_cap;
  return FD_OK;
}


// Fixed scratch of fd_decode_noalloc: partials of callers that cannot
// allocate.  Each device holds its own copy of this array for the life of
// the process.  On the host, `scratch` only names the array; its device
// address is looked up once per device (hipGetSymbolAddress, with that
// device current) and only that address is ever passed to a kernel.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
static_assert(kScratchBytes == FD_NOALLOC_SCRATCH_BYTES,
              "fd.h states the scratch size");

int scratch_address_locked(int dev, void **out);

int scratch_address(void **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FD_ERR_HIP;
  try {
    return scratch_address_locked(dev, out);
  } catch (...) {
    return FD_ERR_HIP;
  }
}

int scratch_address_locked(int dev, void **out) {
  static std::mutex mu;
  static std::vector<void *> addr;
  std::lock_guard<std::mutex> lk(mu);
  if ((int)addr.size() <= dev) addr.resize(dev + 1, nullptr);
  if (addr[dev] == nullptr) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess ||
        p == nullptr)
      return FD_ERR_HIP;
    addr[dev] = p;
  }
  *out = addr[dev];
  return FD_OK;
}

// Checks of the paged-cache arguments; returns the block table's capacity
// in tokens (max_pages * page_size) through *cap.
int check_paged(const fd::PagedKV &pk, const int32_t *seqlens, int Hkv,
                int *cap) {
  if (!pk.block_table || !seqlens) return FD_ERR_INVALID_ARG;
  if (!aligned(pk.block_table, 4)) return FD_ERR_INVALID_ARG;
  if (Hkv <= 0) return FD_ERR_INVALID_ARG;
  if (pk.max_pages <= 0 || pk.page_size <= 0 || pk.num_pages <= 0)
    return FD_ERR_INVALID_ARG;
  if (pk.head_major != FD_PAGES_TOKEN_MAJOR &&
      pk.head_major != FD_PAGES_HEAD_MAJOR)
    return FD_ERR_INVALID_ARG;
  // A 16-key half tile must lie inside one page.
  if (pk.page_size % 16 != 0) return FD_ERR_UNSUPPORTED;
  // Token counts and D-element pool rows are computed in int: checked by
  // division, so that no product can overflow.
  if (pk.max_pages > INT_MAX / pk.page_size ||
      pk.num_pages > INT_MAX / pk.page_size / Hkv)
    return FD_ERR_UNSUPPORTED;
  *cap = pk.max_pages * pk.page_size;
  return FD_OK;
}

// Shared body of every decode entry point.  q/k/v may be null only when
// the chunk phase is not requested; out/lse only when the merge phase is
// not requested.  ex selects several query tokens and/or a paged cache
// (pk; then Lmax is the block table's capacity).
int run(const void *q, const void *k_cache, const void *v_cache,
        const int32_t *seqlens, int B, int Hq, int Hkv, int D, int Lmax,
        float scale, fd_dtype_t dtype, void *out, float *lse, int num_splits,
        int variant, int flags, void *workspace, size_t workspace_bytes,
        void *stream, int phases, fd::Extra ex = fd::Extra(),
        fd::PagedKV pk = fd::PagedKV{nullptr, 0, 0, 0, 0},
        float unified_max = 0.f, bool use_scratch = false) {
  const bool chunks = phases & fd::kPhaseChunks;
  const bool merge = phases & fd::kPhaseMerge;
  if (chunks) {
    if (!q || !k_cache || !v_cache) return FD_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
      return FD_ERR_INVALID_ARG;
    if (!std::isfinite(scale)) return FD_ERR_INVALID_ARG;
  }
  if (merge) {
    if (!out || !lse) return FD_ERR_INVALID_ARG;
    if (!aligned(out, 16) || !aligned(lse, 4)) return FD_ERR_INVALID_ARG;
  }
  if (seqlens && !aligned(seqlens, 4)) return FD_ERR_INVALID_ARG;
  int rc = fd::validate_shape(B, Hq, Hkv, D, Lmax, dtype);
  if (rc != FD_OK) return rc;
  if (num_splits < 0 || variant < FD_VARIANT_AUTO ||
      variant > FD_VARIANT_VALU || (flags & ~fd::kKnownFlags))
    return FD_ERR_INVALID_ARG;
  if ((flags & FD_FLAG_UNIFIED_MAX) && !std::isfinite(unified_max))
    return FD_ERR_INVALID_ARG;
  if (workspace == nullptr && workspace_bytes != 0) return FD_ERR_INVALID_ARG;
  if (workspace && !aligned(workspace, 256)) return FD_ERR_INVALID_ARG;
  // The phase calls exchange partials through the caller's workspace.
  if (phases != (fd::kPhaseChunks | fd::kPhaseMerge) && !workspace)
    return FD_ERR_INVALID_ARG;

  // Every remaining check is the planner's: run it once for them before
  // the first HIP call, then for the device's compute-unit count.
  fd::Plan p;
  rc = fd::make_plan(B, Hq, Hkv, D, Lmax, dtype, seqlens != nullptr,
                     num_splits, variant, flags, 1, &p, ex);
  if (rc != FD_OK) return rc;
  int ncu = 0;
  rc = device_cus(&ncu);
  if (rc != FD_OK) return rc;
  rc = fd::make_plan(B, Hq, Hkv, D, Lmax, dtype, seqlens != nullptr,
                     num_splits, variant, flags, ncu, &p, ex);
  if (rc != FD_OK) return rc;
  if (phases != (fd::kPhaseChunks | fd::kPhaseMerge) && p.fused)
    return FD_ERR_INVALID_ARG;  // the fused merge has no separate phase

  fd::LaunchArgs a{};
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.seqlens = seqlens;
  a.paged = pk;
  a.out = out;
  a.lse = lse;
  a.scale = scale;
  a.unified_max = unified_max;
  a.stream = stream;
  a.phases = phases;
  if (p.combine) {
    const fd::WorkspaceLayout lay = fd::workspace_layout(p);
    char *tickets = static_cast<char *>(workspace);
    char *parts = tickets + lay.o_part_off;
    if (use_scratch) {
      if (p.ws_bytes > kScratchBytes) return FD_ERR_TOO_LARGE;
      void *sp = nullptr;
      rc = scratch_address(&sp);
      if (rc != FD_OK) return rc;
      tickets = static_cast<char *>(sp);
      parts = tickets + lay.o_part_off;
    } else if (workspace) {
      if (workspace_bytes < p.ws_bytes) return FD_ERR_WORKSPACE;
    } else {
      void *t = nullptr, *pp = nullptr;
      rc = owned_workspace(lay.ticket_bytes, lay.total - lay.o_part_off,
                           static_cast<hipStream_t>(stream), &t, &pp);
      if (rc != FD_OK) return rc;
      tickets = static_cast<char *>(t);
      parts = static_cast<char *>(pp);
    }
    a.tickets = lay.ticket_bytes ? reinterpret_cast<int *>(tickets) : nullptr;
    a.o_part = reinterpret_cast<float *>(parts);
    a.lse_part = reinterpret_cast<float *>(parts + (lay.lse_part_off -
                                                    lay.o_part_off));
  }
  return fd::launch_decode(p, a) == 0 ? FD_OK : FD_ERR_HIP;
}

}  // namespace

extern "C" {

int fd_decode_ex(const void *q, const void *k_cache, const void *v_cache,
                 const int32_t *seqlens, int B, int Hq, int Hkv, int D,
                 int Lmax, float scale, fd_dtype_t dtype, void *out,
                 float *lse, int num_splits, int variant, int flags,
                 void *workspace, size_t workspace_bytes, void *stream) {
  if (flags & FD_FLAG_UNIFIED_MAX) return FD_ERR_INVALID_ARG;  // needs phi
  return run(q, k_cache, v_cache, seqlens, B, Hq, Hkv, D, Lmax, scale, dtype,
             out, lse, num_splits, variant, flags, workspace, workspace_bytes,
             stream, fd::kPhaseChunks | fd::kPhaseMerge);
}

int fd_decode(const void *q, const void *k_cache, const void *v_cache,
              const int32_t *seqlens, int B, int Hq, int Hkv, int D,
              int Lmax, float scale, fd_dtype_t dtype, void *out, float *lse,
              void *stream) {
  return fd_decode_ex(q, k_cache, v_cache, seqlens, B, Hq, Hkv, D, Lmax,
                      scale, dtype, out, lse, 0, FD_VARIANT_AUTO, 0, nullptr,
                      0, stream);
}

int fd_decode_noalloc(const void *q, const void *k_cache,
                      const void *v_cache, const int32_t *seqlens, int B,
                      int Hq, int Hkv, int D, int Lmax, float scale,
                      fd_dtype_t dtype, void *out, float *lse, int num_splits,
                      int variant, int flags, void *stream) {
  if (flags & (FD_FLAG_UNIFIED_MAX | FD_FLAG_FUSED_MERGE))
    return (flags & FD_FLAG_UNIFIED_MAX) ? FD_ERR_INVALID_ARG
                                         : FD_ERR_UNSUPPORTED;
  return run(q, k_cache, v_cache, seqlens, B, Hq, Hkv, D, Lmax, scale, dtype,
             out, lse, num_splits, variant, flags, nullptr, 0, stream,
             fd::kPhaseChunks | fd::kPhaseMerge, fd::Extra(),
             fd::PagedKV{nullptr, 0, 0, 0, 0}, 0.f, true);
}

int fd_decode_partials(const void *q, const void *k_cache,
                       const void *v_cache, const int32_t *seqlens, int B,
                       int Hq, int Hkv, int D, int Lmax, float scale,
                       fd_dtype_t dtype, int num_splits, int variant,
                       int flags, void *workspace, size_t workspace_bytes,
                       void *stream) {
  if (flags & FD_FLAG_UNIFIED_MAX) return FD_ERR_INVALID_ARG;
  return run(q, k_cache, v_cache, seqlens, B, Hq, Hkv, D, Lmax, scale, dtype,
             nullptr, nullptr, num_splits, variant, flags | FD_FLAG_PARTIALS,
             workspace, workspace_bytes, stream, fd::kPhaseChunks);
}

int fd_merge_partials(const int32_t *seqlens, int B, int Hq, int Hkv, int D,
                      int Lmax, fd_dtype_t dtype, int num_splits, int variant,
                      int flags, const void *workspace,
                      size_t workspace_bytes, void *out, float *lse,
                      void *stream) {
  if (flags & FD_FLAG_UNIFIED_MAX) return FD_ERR_INVALID_ARG;
  return run(nullptr, nullptr, nullptr, seqlens, B, Hq, Hkv, D, Lmax, 0.f,
             dtype, out, lse, num_splits, variant, flags | FD_FLAG_PARTIALS,
             const_cast<void *>(workspace), workspace_bytes, stream,
             fd::kPhaseMerge);
}

int fd_decode_paged(const void *q, const void *k_pages, const void *v_pages,
                    const int32_t *block_table, int max_pages, int page_size,
                    int num_pages, int layout, const int32_t *seqlens, int B,
                    int Tq, int Hq, int Hkv, int D, float scale,
                    fd_dtype_t dtype, void *out, float *lse, int num_splits,
                    int flags, void *workspace, size_t workspace_bytes,
                    void *stream) {
  if (Tq <= 0 || (flags & FD_FLAG_UNIFIED_MAX)) return FD_ERR_INVALID_ARG;
  const fd::PagedKV pk{block_table, max_pages, page_size, num_pages, layout};
  int cap = 0;
  const int rc = check_paged(pk, seqlens, Hkv, &cap);
  if (rc != FD_OK) return rc;
  fd::Extra ex;
  ex.paged = true;
  ex.Tq = Tq;
  return run(q, k_pages, v_pages, seqlens, B, Hq, Hkv, D, cap, scale, dtype,
             out, lse, num_splits, FD_VARIANT_AUTO, flags, workspace,
             workspace_bytes, stream, fd::kPhaseChunks | fd::kPhaseMerge, ex,
             pk);
}

int fd_decode_multiquery(const void *q, const void *k_cache,
                         const void *v_cache, const int32_t *seqlens, int B,
                         int Tq, int Hq, int Hkv, int D, int Lmax, float scale,
                         fd_dtype_t dtype, void *out, float *lse,
                         int num_splits, int flags, void *workspace,
                         size_t workspace_bytes, void *stream) {
  if (Tq <= 0 || (flags & FD_FLAG_UNIFIED_MAX)) return FD_ERR_INVALID_ARG;
  fd::Extra ex;
  ex.Tq = Tq;
  return run(q, k_cache, v_cache, seqlens, B, Hq, Hkv, D, Lmax, scale, dtype,
             out, lse, num_splits, FD_VARIANT_AUTO, flags, workspace,
             workspace_bytes, stream, fd::kPhaseChunks | fd::kPhaseMerge, ex);
}

int fd_decode_unified_max(const void *q, const void *k_cache,
                          const void *v_cache, const int32_t *seqlens, int B,
                          int Hq, int Hkv, int D, int Lmax, float scale,
                          fd_dtype_t dtype, void *out, float *lse, float phi,
                          int num_splits, int flags, void *workspace,
                          size_t workspace_bytes, void *stream) {
  return run(q, k_cache, v_cache, seqlens, B, Hq, Hkv, D, Lmax, scale, dtype,
             out, lse, num_splits, FD_VARIANT_AUTO,
             flags | FD_FLAG_UNIFIED_MAX, workspace, workspace_bytes, stream,
             fd::kPhaseChunks | fd::kPhaseMerge, fd::Extra(),
             fd::PagedKV{nullptr, 0, 0, 0, 0}, phi);
}

int fd_plan_ex(int B, int Tq, int Hq, int Hkv, int D, int Lmax,
               fd_dtype_t dtype, int varlen, int paged, int num_splits,
               int variant, int flags, int num_cus, fd_plan_t *plan) {
  if (!plan) return FD_ERR_INVALID_ARG;
  if (num_cus < 0 || Tq <= 0) return FD_ERR_INVALID_ARG;
  fd::Extra ex;
  ex.Tq = Tq;
  ex.paged = paged != 0;
  const bool vl = varlen != 0 || ex.paged;
  fd::Plan p;
  int rc = fd::make_plan(B, Hq, Hkv, D, Lmax, dtype, vl, num_splits, variant,
                         flags, 1, &p, ex);
  if (rc != FD_OK) return rc;
  if (num_cus == 0) {
    rc = device_cus(&num_cus);
    if (rc != FD_OK) return rc;
  }
  rc = fd::make_plan(B, Hq, Hkv, D, Lmax, dtype, vl, num_splits, variant,
                     flags, num_cus, &p, ex);
  if (rc != FD_OK) return rc;
  const fd::WorkspaceLayout lay = fd::workspace_layout(p);
  plan->num_splits = p.splits;
  plan->chunk = p.chunk;
  plan->variant = p.variant;
  plan->waves_per_block = p.waves;
  plan->grid = p.grid;
  plan->combine = p.combine ? 1 : 0;
  plan->merge = !p.combine ? FD_MERGE_NONE
                           : (p.fused ? FD_MERGE_FUSED : FD_MERGE_SEPARATE);
  plan->num_cus = p.num_cus;
  plan->workspace_bytes = p.ws_bytes;
  plan->ticket_bytes = lay.ticket_bytes;
  plan->o_part_offset = p.combine ? lay.o_part_off : 0;
  plan->lse_part_offset = p.combine ? lay.lse_part_off : 0;
  plan->partial_layout =
      p.chunk_major ? FD_PARTIALS_CHUNK_MAJOR : FD_PARTIALS_ROW_MAJOR;
  plan->partial_group = p.G;
  return FD_OK;
}

int fd_plan(int B, int Hq, int Hkv, int D, int Lmax, fd_dtype_t dtype,
            int varlen, int num_splits, int variant, int flags, int num_cus,
            fd_plan_t *plan) {
  return fd_plan_ex(B, 1, Hq, Hkv, D, Lmax, dtype, varlen, 0, num_splits,
                    variant, flags, num_cus, plan);
}

size_t fd_workspace_bytes(int B, int Hq, int Hkv, int D, int Lmax,
                          fd_dtype_t dtype, int varlen, int num_splits,
                          int variant, int flags) {
  fd_plan_t p;
  if (fd_plan(B, Hq, Hkv, D, Lmax, dtype, varlen, num_splits, variant, flags,
              0, &p) != FD_OK)
    return 0;
  return p.workspace_bytes;
}

const char *fd_status_string(int status) {
  switch (status) {
    case FD_OK:
      return "ok";
    case FD_ERR_INVALID_ARG:
      return "invalid argument (null or misaligned pointer, non-positive "
             "size, Hq not a multiple of Hkv, or non-finite scale)";
    case FD_ERR_UNSUPPORTED:
      return "unsupported configuration (head dim, dtype, group size or "
             "variant)";
    case FD_ERR_WORKSPACE:
      return "workspace too small or could not be allocated";
    case FD_ERR_HIP:
      return "HIP runtime error";
    case FD_ERR_CAPTURE:
      return "the library-owned workspace cannot be used under stream "
             "capture; pass a caller workspace";
    case FD_ERR_TOO_LARGE:
      return "the plan's partials exceed fd_decode_noalloc's fixed 64 MiB "
             "scratch array";
    default:
      return "unknown status";
  }
}

int fd_version(void) { return kVersion; }

}  // extern "C"
