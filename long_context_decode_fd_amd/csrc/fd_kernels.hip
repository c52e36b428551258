// fd_kernels.hip -- split-KV decode attention kernels for gfx950 (MI355X).
//
// Method: "Flash-Decoding for long-context inference" (Dao, Haziza, Massa,
// Sizov; Stanford CRFM), section "A faster attention for decoding:
// Flash-Decoding".  The keys/values of every sequence are cut into chunks;
// each chunk is attended to on its own, in parallel, and leaves its
// normalised output plus one log-sum-exp per query row; a last pass
// rescales the chunks by their log-sum-exp and sums them.  Inside a chunk
// the softmax is built up tile by tile with a running maximum and a
// rescaled running sum, the iterative form the page says makes the split
// possible.
//
// MI355X mapping (our own design; the page's kernel targets A100):
//   * one workgroup per (sequence b, KV head g, chunk s) -- with
//     per-sequence lengths a workgroup may take a second chunk, and the
//     chunk list puts each sequence's short last chunk after every full
//     one; a workgroup serves all G = Hq / Hkv query heads of KV head g,
//     so each K/V byte leaves HBM once;
//   * bf16: each 64-lane wavefront streams 32-key tiles straight from HBM
//     into registers in the operand layout of v_mfma_f32_16x16x32_bf16,
//     the next tile's K in flight while the current tile computes, and
//     computes S^T = K Q^T (16 keys x 16 padded heads per MFMA) and
//     O^T += V^T P^T; the accumulator's column is the query head, so each
//     lane rescales only its own head's accumulators;
//   * the per-head running max is shared across the four 16-lane groups of
//     a wavefront with two cross-lane shuffles per tile; exponentials run
//     as exp2 with log2(e) folded into the scale;
//   * the wavefronts of a workgroup take interleaved tiles and merge their
//     (max, sum, accumulator) states through LDS at the end, so a chunk
//     writes one partial per query row;
//   * when every KV slab starts at the same offset modulo 32 MB, each
//     chunk walks its tiles from a start point taken from (b, g) and wraps
//     (TileOrder): slabs streamed in lockstep at such a stride run far
//     below the usual rate on MI355X;
//   * the same kernel, by template switches, reads the tiles from a paged
//     pool through a block table (K staged through LDS as whole 256-byte
//     rows at D = 128), serves several causal new tokens per sequence
//     (their query rows share the 16-column q-tile), or takes the
//     unified-maximum softmax of FlashDecoding++ with an exact fallback;
//   * fp32 runs a matrix-core kernel on v_mfma_f32_16x16x4_f32 (16-key
//     halves, the next half in flight) from groups of 3 query heads, and
//     for every paged or several-token call; the smallest fp32 groups (and
//     bf16 tiny groups, on request) a vector-ALU kernel with 16-byte loads
//     per lane and shuffle reductions of the dot products;
//   * a second, small kernel merges the chunk partials of every query row
//     (or, opt-in, the last workgroup of each group merges them).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fd_internal.h"

namespace fd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// K/V are streamed exactly once per call: nontemporal loads keep them from
// displacing lines that are reused (q, partials) and measurably raise the
// sustained read rate on MI355X.
__device__ __forceinline__ uint4 load_stream(const uint4 *p) {
  const u32x4 t =
      __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ uint2 load_stream(const uint2 *p) {
  const u32x2 t =
      __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
  return make_uint2(t.x, t.y);
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
#define FD_NEG_INF (-__builtin_huge_valf())

__device__ __forceinline__ float exp2_f(float x) {
  return __builtin_amdgcn_exp2f(x);
}
__device__ __forceinline__ float log2_f(float x) {
  return __builtin_amdgcn_logf(x);
}
__device__ __forceinline__ int clamp_len(int L, int Lmax) {
  return L < 0 ? 0 : (L > Lmax ? Lmax : L);
}

// What a per-chunk workgroup does with its result.
constexpr int kModeDirect = 0;    // one chunk per sequence: write out/lse
constexpr int kModePartial = 1;   // write the chunk partial (merge kernel)
constexpr int kModeFused = 2;     // partial, then the last one merges

// ---------------------------------------------------------------------------
// Work decomposition shared by the per-chunk kernels and the merge kernel.

struct Work {
  int b, g, s;
  int lo, hi;  // keys [lo, hi) of slab (b, g); lo == hi only when L_b == 0
  int L;       // clamped length of sequence b
  int nb;      // chunks of sequence b
  int items;   // length of the whole work list when the scan knows it
               // (at most 64 sequences), else INT_MAX
  bool valid;
};

// Chunks of sequence b: n_b = max(1, ceil(L_b / C)); a sequence of length 0
// keeps one empty chunk so that its output row is still written.
__device__ __forceinline__ int chunks_of(int L, int C) {
  return max(1, (L + C - 1) / C);
}

// Work id -> (b, g, s).  Equal lengths, or a grid that covers every chunk
// id any lengths could need (direct): ids run over the chunks sequence by
// sequence, chunk-major, KV head fastest: id = (b * S + s) * Hkv + g, and
// only seqlens[b] is read (one load with a workgroup-uniform address; ids
// past the sequence's chunks do nothing).
// Otherwise (per-sequence lengths, smaller grid): first every full chunk
// (C keys) in that order, then
// each sequence's short last chunk, longest first (ties by sequence), so
// that the chunks dispatched last are the shortest; the prefix over the
// sequences is a wavefront scan of the seqlens (a few dozen instructions
// per wavefront), and the ranking of the last chunks a loop over the
// wavefront's 64 lanes (sequences beyond 64 keep their natural order).
__device__ Work find_work(int bid, const int32_t *__restrict__ seqlens, int B,
                          int Hkv, int Lmax, int C, bool direct) {
  Work w;
  w.valid = false;
  w.b = w.g = w.s = w.lo = w.hi = w.L = w.nb = 0;
  w.items = INT_MAX;
  if (seqlens == nullptr || direct) {
    const int S = (Lmax + C - 1) / C;
    const int per_b = S * Hkv;
    const int b = bid / per_b;
    if (b >= B) return w;
    const int r = bid - b * per_b;
    const int L = seqlens ? clamp_len(seqlens[b], Lmax) : Lmax;
    w.b = b;
    w.s = r / Hkv;
    w.g = r - w.s * Hkv;
    w.lo = w.s * C;
    w.hi = max(w.lo, min(w.lo + C, L));
    w.L = L;
    w.nb = chunks_of(L, C);
    w.valid = w.s < w.nb;
    return w;
  }
  const int lane = threadIdx.x & 63;
  // Pass 1: the full chunks (C keys), sequence by sequence.
  int base = 0;
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int b = b0 + lane;
    int L = 0, blocks = 0;
    if (b < B) {
      L = clamp_len(seqlens[b], Lmax);
      blocks = (L / C) * Hkv;
    }
    int incl = blocks;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(incl, off, 64);
      if (lane >= off) incl += t;
    }
    const int total = __shfl(incl, 63, 64);
    if (B <= 64) {
      // the whole list: every full chunk, then one last chunk per
      // sequence whose length is not a multiple of C (or is 0)
      const bool has_last = b < B && (L % C != 0 || L == 0);
      w.items = total + __popcll(__ballot(has_last)) * Hkv;
    }
    if (bid < base + total) {
      const unsigned long long hit = __ballot(base + incl > bid);
      const int src = __ffsll((unsigned long long)hit) - 1;
      const int excl = __shfl(incl - blocks, src, 64);
      const int Lb = __shfl(L, src, 64);
      const int r = bid - base - excl;
      w.b = b0 + src;
      w.s = r / Hkv;
      w.g = r - w.s * Hkv;
      w.lo = w.s * C;
      w.hi = w.lo + C;
      w.L = Lb;
      w.nb = chunks_of(Lb, C);
      w.valid = true;
      return w;
    }
    base += total;
  }
  // Pass 2: each sequence's last chunk when it is short (or the empty chunk
  // of a length-0 sequence), longest first, so the work dispatched last is
  // the shortest.
  const int r = bid - base;
  const int j = r / Hkv;
  for (int b0 = 0, done = 0; b0 < B; b0 += 64) {
    const int b = b0 + lane;
    int L = 0, rem = 0;
    bool has = false;
    if (b < B) {
      L = clamp_len(seqlens[b], Lmax);
      rem = L % C;
      has = rem != 0 || L == 0;
    }
    const unsigned long long hv = __ballot(has);
    const int cnt = __popcll(hv);
    if (j < done + cnt) {
      int rank = 0;  // among this batch's last chunks: longer first, then b
      if (B <= 64) {
#pragma unroll 8
        for (int o = 0; o < 64; ++o) {
          const int ro = __shfl(rem, o, 64);
          const bool ho = (hv >> o) & 1ull;
          rank += (ho && (ro > rem || (ro == rem && o < lane))) ? 1 : 0;
        }
      } else {
        rank = __popcll(hv & ((1ull << lane) - 1ull));
      }
      const unsigned long long hit = __ballot(has && rank == j - done);
      const int src = __ffsll((unsigned long long)hit) - 1;
      const int Lb = __shfl(L, src, 64);
      w.b = b0 + src;
      w.s = Lb / C;
      w.g = r - j * Hkv;
      w.lo = w.s * C;
      w.hi = Lb;
      w.L = Lb;
      w.nb = chunks_of(Lb, C);
      w.valid = true;
      return w;
    }
    done += cnt;
  }
  return w;
}

// Query rows served by the workgroup of (b, g): column c < G * Tq of the
// q-tile is new token t = c / G and query head g * G + c % G.  q, out and
// the partials are laid out [B][Tq][Hq] (Tq = 1: [B][Hq]).
__device__ __forceinline__ size_t row_of(const Work &w, int G, int Hq, int Tq,
                                         int c) {
  const int t = c / G, h = c - t * G;
  return ((size_t)w.b * Tq + t) * Hq + (size_t)w.g * G + h;
}

// Where the chunk partials live (the plan picks the layout).  Partial i is
// lse_part[i] and o_part[i * D ..].
//   row-major    (one round of workgroups): the S partials of a query row
//                r = (b, t, head) are consecutive, i = r * S + s;
//   chunk-major  (several rounds): the G * Tq rows of one chunk of (b, g)
//                are consecutive, i = ((b * Hkv + g) * S + s) * G * Tq + c
//                with c = t * G + h the q-tile column, so a chunk stores
//                one contiguous block of G * Tq * D floats.
// Either way the partials of one query row are base + s * stride.
struct PartLayout {
  int G, Tq, Hq, Hkv, S;
  bool chunk_major;
  struct Row {
    size_t base;
    int stride;
  };
  // q-tile column c of the group (b, g)
  __device__ __forceinline__ Row row(int b, int g, int c) const {
    if (chunk_major)
      return {((size_t)b * Hkv + g) * S * (size_t)(G * Tq) + c, G * Tq};
    const int t = c / G, h = c - t * G;
    return {(((size_t)b * Tq + t) * Hq + (size_t)g * G + h) * S, 1};
  }
  // query row r = (b * Tq + t) * Hq + head of the outputs
  __device__ __forceinline__ Row row_of_out(size_t r) const {
    const int b = (int)(r / ((size_t)Tq * Hq));
    const int th = (int)(r - (size_t)b * Tq * Hq);
    const int t = th / Hq, hq = th - t * Hq;
    const int g = hq / G;
    return row(b, g, t * G + (hq - g * G));
  }
  // partial of chunk w.s, column c
  __device__ __forceinline__ size_t at(const Work &w, int c) const {
    const Row r = row(w.b, w.g, c);
    return r.base + (size_t)w.s * r.stride;
  }
};

// ---------------------------------------------------------------------------
// Element helpers.

__device__ __forceinline__ uint16_t to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);  // round to nearest even
}

template <typename T>
__device__ __forceinline__ void store_out(T *p, float x);
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t *p, float x) {
  *p = to_bf16_bits(x);
}
template <>
__device__ __forceinline__ void store_out<float>(float *p, float x) {
  *p = x;
}
template <>
__device__ __forceinline__ void store_out<_Float16>(_Float16 *p, float x) {
  *p = (_Float16)x;  // round to nearest even
}

// Bit pattern of a 16-bit output element: bf16 bits (uint16_t) or fp16.
template <typename T>
__device__ __forceinline__ uint32_t bits16(float x);
template <>
__device__ __forceinline__ uint32_t bits16<uint16_t>(float x) {
  return to_bf16_bits(x);
}
template <>
__device__ __forceinline__ uint32_t bits16<_Float16>(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}

// The 16-bit element types of the matrix-core pass, E = __bf16 or
// _Float16 (IEEE binary16): the 8-element operand vector of one
// v_mfma_f32_16x16x32 lane and the output element (bf16 outputs are kept
// as their bit patterns).
template <typename E>
struct E16;
template <>
struct E16<__bf16> {
  typedef bf16x8 vec;
  typedef uint16_t out;
};
template <>
struct E16<_Float16> {
  typedef f16x8 vec;
  typedef _Float16 out;
};
__device__ __forceinline__ floatx4 mfma32(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma32(f16x8 a, f16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Merge of the workgroup's softmax states and the chunk's store (the
// vector-ALU kernel).
//
// Slot sl holds, for query row h of the group: running max m (log2 units of
// the scaled score), running sum l, and the unnormalised accumulator
// O[h][0..D).  The merged row is M = max m, weight 2^(m - M) per slot; the
// chunk's output is sum(w O) / sum(w l) and its log-sum-exp (natural log)
// is ln2 * (M + log2 sum(w l)).  With no keys at all: out 0, lse -inf.
template <int D, typename OutT>
__device__ void merge_and_store(const float *sm_m, const float *sm_l,
                                const float *sm_o, int nslot, int rows,
                                const PartLayout &pl, const Work &w,
                                int mode, OutT *__restrict__ out,
                                float *__restrict__ lse,
                                float *__restrict__ o_part,
                                float *__restrict__ lse_part) {
  const int G = pl.G, Tq = pl.Tq, Hq = pl.Hq;
  for (int idx = threadIdx.x; idx < G * Tq * D; idx += blockDim.x) {
    const int h = idx / D, d = idx - h * D;
    float M = FD_NEG_INF;
    for (int sl = 0; sl < nslot; ++sl) M = fmaxf(M, sm_m[sl * rows + h]);
    float o, ls;
    if (M == FD_NEG_INF) {
      o = 0.f;
      ls = FD_NEG_INF;
    } else {
      float O = 0.f, Ls = 0.f;
      for (int sl = 0; sl < nslot; ++sl) {
        const float wt = exp2_f(sm_m[sl * rows + h] - M);
        O += wt * sm_o[(sl * rows + h) * (D + 1) + d];
        Ls += wt * sm_l[sl * rows + h];
      }
      o = O / Ls;
      ls = (M + log2_f(Ls)) * kLn2;
    }
    const size_t hq = row_of(w, G, Hq, Tq, h);
    if (mode == kModeDirect) {
      store_out<OutT>(out + hq * D + d, o);
      if (d == 0) lse[hq] = ls;
    } else if (mode == kModePartial) {
      const size_t row = pl.at(w, h);
      o_part[row * D + d] = o;
      if (d == 0) lse_part[row] = ls;
    } else {
      // Read by another workgroup of this launch, possibly on another XCD:
      // device-coherent stores (written through the local L2).
      const size_t row = pl.at(w, h);
      __hip_atomic_store(o_part + row * D + d, o, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      if (d == 0)
        __hip_atomic_store(lse_part + row, ls, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ---------------------------------------------------------------------------
// Fused merge: the last workgroup of a (b, g) group merges its chunks.
//
// Every workgroup that wrote a chunk partial takes a ticket from its
// group's counter.  The one that takes ticket nb - 1 knows that all nb
// partials of the group are written; it merges them into out/lse exactly
// as the separate merge pass would and puts the counter back to zero for
// the next call.  No workgroup ever waits for another, so there is no
// co-residency requirement.
//
// Ordering across MI355X's eight XCDs, whose L2 caches are not coherent
// with each other:
//   writers  every partial is stored with the cache policy of an
//            agent-scope atomic store (sc1), which gfx950 writes through
//            its XCD's L2 to the device coherence point: 16-byte stores
//            (store_through) from the matrix-core kernels, agent-scope
//            atomic stores of 4 bytes from the vector-ALU kernel.  Each
//            thread then waits for all of its memory operations to
//            complete (s_waitcnt 0) before the workgroup barrier, and only
//            then does one thread take the ticket (an agent-scope atomic).
//            This is the part of an agent-scope release that concerns
//            written-through stores; the other part, an L2 write-back of
//            ordinary stores, is left out on purpose: there are none to
//            publish, and it would write back the XCD's whole L2 once per
//            workgroup (measured: far slower than a second launch).
//   reader   the last workgroup issues an agent-scope acquire fence after
//            its ticket came back (one L1/L2 invalidate per group, not per
//            workgroup); its ordinary 16-byte loads of the partials then
//            miss the invalidated caches and read the coherence point.
//
// The merge spreads the group's G x D outputs over the workgroup as
// (row, 4 columns) items; when there are fewer items than threads, each
// item's chunks are split over `slices` threads whose states meet in LDS.
constexpr int kTailBatch = 16;

// 16 bytes written through the XCD's L2 to the device coherence point
// (sc1: the cache policy of an agent-scope atomic store), for a partial
// that another workgroup of the same launch reads.
__device__ __forceinline__ void store_through(float *p, float4 v) {
  const floatx4 t = {v.x, v.y, v.z, v.w};
  asm volatile("global_store_dwordx4 %0, %1, off sc1" ::"v"(p), "v"(t)
               : "memory");
}

struct TailState {
  float M, W;   // running max (natural-log units) and rescaled weight sum
  float4 acc;   // rescaled weighted sum of 4 output columns
};

// Folds chunks s = s_first, s_first + s_step, ... of item `it` (q-tile
// column it / (D/4), output columns 4 (it % (D/4)) ..) into a TailState,
// kTailBatch chunks per step with all of a step's loads issued first.
template <int D>
__device__ TailState merge_item(const Work &w, const PartLayout &pl, int it,
                                int s_first, int s_step,
                                const float *__restrict__ o_part,
                                const float *__restrict__ lse_part) {
  constexpr int V4 = D / 4;
  const int h = it / V4, d4 = it - h * V4;
  const PartLayout::Row pr = pl.row(w.b, w.g, h);
  const float *lp = lse_part + pr.base;
  const float *op = o_part + pr.base * D + d4 * 4;
  const int ls_step = pr.stride;
  const size_t o_step = (size_t)pr.stride * D;
  TailState st{FD_NEG_INF, 0.f, make_float4(0.f, 0.f, 0.f, 0.f)};
  for (int s0 = s_first; s0 < w.nb; s0 += s_step * kTailBatch) {
    float ls[kTailBatch];
    float4 ov[kTailBatch];
#pragma unroll
    for (int j = 0; j < kTailBatch; ++j) {
      const int s = s0 + j * s_step;
      const int sc = s < w.nb ? s : s0;
      const float *l1 = lp + (size_t)sc * ls_step;
      const float *o4 = op + (size_t)sc * o_step;
      ls[j] = s < w.nb ? *l1 : FD_NEG_INF;
      ov[j] = *reinterpret_cast<const float4 *>(o4);
    }
    float mb = ls[0];
#pragma unroll
    for (int j = 1; j < kTailBatch; ++j) mb = fmaxf(mb, ls[j]);
    const float Mn = fmaxf(st.M, mb);
    if (Mn == FD_NEG_INF) continue;
    const float r = exp2_f((st.M - Mn) * kLog2e);
    st.W *= r;
    st.acc.x *= r;
    st.acc.y *= r;
    st.acc.z *= r;
    st.acc.w *= r;
#pragma unroll
    for (int j = 0; j < kTailBatch; ++j) {
      const float wt = exp2_f((ls[j] - Mn) * kLog2e);
      st.W += wt;
      st.acc.x += wt * ov[j].x;
      st.acc.y += wt * ov[j].y;
      st.acc.z += wt * ov[j].z;
      st.acc.w += wt * ov[j].w;
    }
    st.M = Mn;
  }
  return st;
}

// Writes 4 output columns of one row (and the row's lse with the first 4).
template <int D, typename OutT>
__device__ void store_item(const Work &w, int G, int Tq, int Hq, int it,
                           float M, float W, float4 a, OutT *__restrict__ out,
                           float *__restrict__ lse) {
  constexpr int V4 = D / 4;
  const int h = it / V4, d4 = it - h * V4;
  const size_t row = row_of(w, G, Hq, Tq, h);
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  float ls = FD_NEG_INF;
  if (M != FD_NEG_INF) {
    o = make_float4(a.x / W, a.y / W, a.z / W, a.w / W);
    ls = M + log2_f(W) * kLn2;
  }
  OutT *dst = out + row * D + d4 * 4;
  store_out<OutT>(dst + 0, o.x);
  store_out<OutT>(dst + 1, o.y);
  store_out<OutT>(dst + 2, o.z);
  store_out<OutT>(dst + 3, o.w);
  if (d4 == 0) lse[row] = ls;
}

// Merges the nb chunk partials of group (w.b, w.g) into out/lse: items
// [it0, it1) of the group's G * Tq * D / 4 (row, 4 columns) items, with
// the whole workgroup (the fused path's last workgroup takes all items;
// the merge pass splits a group's items over several workgroups).
template <int D, typename OutT>
__device__ void group_merge(const Work &w, const PartLayout &pl, int it0,
                            int it1, const float *__restrict__ o_part,
                            const float *__restrict__ lse_part,
                            OutT *__restrict__ out, float *__restrict__ lse,
                            float *scratch) {
  const int G = pl.G, Tq = pl.Tq, Hq = pl.Hq;
  const int T = blockDim.x, tid = threadIdx.x;
  const int items = it1 - it0;
  // More items than threads: each thread merges whole items on its own.
  // Otherwise each item's chunks are split over `slices` threads.
  const int slices = max(1, T / items);
  if (slices == 1) {
    for (int it = it0 + tid; it < it1; it += T) {
      const TailState st = merge_item<D>(w, pl, it, 0, 1, o_part,
                                                   lse_part);
      store_item<D, OutT>(w, G, Tq, Hq, it, st.M, st.W, st.acc, out, lse);
    }
    return;
  }
  float *sM = scratch, *sW = scratch + T;
  float4 *sA = reinterpret_cast<float4 *>(scratch + 2 * T);
  TailState st{FD_NEG_INF, 0.f, make_float4(0.f, 0.f, 0.f, 0.f)};
  if (tid < items * slices)
    st = merge_item<D>(w, pl, it0 + tid % items, tid / items,
                                 slices, o_part, lse_part);
  sM[tid] = st.M;
  sW[tid] = st.W;
  sA[tid] = st.acc;
  __syncthreads();
  if (tid < items) {
    float Mt = FD_NEG_INF;
    for (int sl = 0; sl < slices; ++sl) Mt = fmaxf(Mt, sM[sl * items + tid]);
    float Wt = 0.f;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    if (Mt != FD_NEG_INF) {
      for (int sl = 0; sl < slices; ++sl) {
        const int k = sl * items + tid;
        const float r = exp2_f((sM[k] - Mt) * kLog2e);
        Wt += r * sW[k];
        a.x += r * sA[k].x;
        a.y += r * sA[k].y;
        a.z += r * sA[k].z;
        a.w += r * sA[k].w;
      }
    }
    store_item<D, OutT>(w, G, Tq, Hq, it0 + tid, Mt, Wt, a, out, lse);
  }
}

template <int D, typename OutT>
__device__ void merge_group_if_last(const Work &w, const PartLayout &pl,
                                    const float *__restrict__ o_part,
                                    const float *__restrict__ lse_part,
                                    int *__restrict__ tickets,
                                    OutT *__restrict__ out,
                                    float *__restrict__ lse, float *scratch,
                                    int *sm_flag) {
  // Writer side: every memory operation of this thread, the agent-scope
  // partial stores included, has completed before the barrier, so the
  // relaxed ticket below cannot overtake any partial of the workgroup.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    int *t = tickets + (size_t)w.b * pl.Hkv + w.g;
    const int prev = __hip_atomic_fetch_add(t, 1, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
    const int last = prev == w.nb - 1;
    if (last)
      __hip_atomic_store(t, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *sm_flag = last;
  }
  __syncthreads();
  if (!*sm_flag) return;
  // Reader side: acquire at agent scope after the ticket, then read the
  // partials with agent-scope atomic loads.
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  group_merge<D, OutT>(w, pl, 0, pl.G * pl.Tq * (D / 4), o_part, lse_part,
                       out, lse, scratch);
}

// ---------------------------------------------------------------------------
// bf16 matrix-core kernel.
//
// Operand layouts of v_mfma_f32_16x16x32_bf16 (lane l, n = l % 16,
// q4 = l / 16): A supplies row n, k = 8 q4 .. 8 q4 + 7; B supplies column n,
// the same k; the 16x16 fp32 result sits in lane l as rows 4 q4 .. 4 q4 + 3
// of column n.
//
//   scores  S^T[key][head] = sum_d K[key][d] Q[head][d]
//           A = K rows of the 16-key subtile, B = Q^T (heads >= G are 0),
//           D/32 MFMAs per 16 keys.  Lane l ends with keys 4 q4 + j of
//           head n for both subtiles: 8 keys of one head.
//   output  O^T[d][head] += sum_key V[key][d] P[head][key]
//           k-slot 8 q4 + i <-> key 16 (i / 4) + 4 q4 + i % 4, i.e. exactly
//           the 8 keys whose scores lane l holds, so P^T needs no shuffle.
//           A = V^T: lane l loads, for those 8 keys, the D/16 consecutive
//           columns n * D/16 .. of V (one 16-byte or 8-byte load per key,
//           16 lanes cover a whole 256-byte row) and v_perm_b32 regroups
//           them into D/16 operands of 8 keys each; MFMA e produces
//           O^T rows d = (D/16) m + e.
template <int VW>
struct VecOf;
template <>
struct VecOf<8> {
  typedef uint4 type;
};
template <>
struct VecOf<4> {
  typedef uint2 type;
};
// D = 256: a lane's 16 columns are two 16-byte pieces 256 bytes apart (row
// pieces of 128 columns, so that each load instruction reads whole
// 256-byte stretches of the rows).
struct U32x8 {
  uint4 lo, hi;
};
template <>
struct VecOf<16> {
  typedef U32x8 type;
};

template <int VW>
__device__ __forceinline__ uint32_t dword_of(const typename VecOf<VW>::type &v,
                                             int i);
template <>
__device__ __forceinline__ uint32_t dword_of<8>(const uint4 &v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}
template <>
__device__ __forceinline__ uint32_t dword_of<4>(const uint2 &v, int i) {
  return i == 0 ? v.x : v.y;
}
template <>
__device__ __forceinline__ uint32_t dword_of<16>(const U32x8 &v, int i) {
  return i < 4 ? dword_of<8>(v.lo, i) : dword_of<8>(v.hi, i - 4);
}

// The accumulator layout: element j of block e of lane (n16, q4) holds
// query column n16 and head-dimension column acc_col(e, 4 q4 + j).
// ROWS = 0: d = i * VW + e (a lane's V columns contiguous); ROWS = R > 0:
// the lane's V columns come in pieces of R from row pieces of 16 R
// columns, d = (e / R) * 16 R + R i + e % R.
template <int VW, int ROWS>
__device__ __forceinline__ constexpr int acc_col(int e, int i) {
  return ROWS == 0 ? i * VW + e : (e / ROWS) * 16 * ROWS + ROWS * i + e % ROWS;
}
// bf16 V pieces: natural up to D = 128, 128-column row pieces at D = 256.
template <int D>
constexpr int kBf16Rows = D > 128 ? 8 : 0;

// Where the key rows of a tile live.  Contiguous cache: row r of the tile
// starting at key k0 is k[(k0 + r) * D].  Paged cache: the tile's two
// 16-key halves each lie inside one page, at h0 / h1, rows rs elements
// apart (Hkv * D token-major, D head-major).
template <int D, bool PAGED>
struct TileRows;
template <int D>
struct TileRows<D, false> {
  static constexpr bool kPaged = false;
  const uint16_t *k, *v;  // slab (b, g)
  int k0;
  __device__ const uint16_t *krow(int r) const {
    return k + (size_t)(k0 + r) * D;
  }
  __device__ const uint16_t *vrow(int r) const {
    return v + (size_t)(k0 + r) * D;
  }
};
template <int D>
struct TileRows<D, true> {
  static constexpr bool kPaged = true;
  const uint16_t *k0h, *k1h, *v0h, *v1h;
  size_t rs;
  __device__ const uint16_t *krow(int r) const {
    return (r < 16 ? k0h : k1h) + (size_t)(r & 15) * rs;
  }
  __device__ const uint16_t *vrow(int r) const {
    return (r < 16 ? v0h : v1h) + (size_t)(r & 15) * rs;
  }
};

// One 32-key tile of one wavefront, in three parts: the K loads, the V
// loads, and the math on both (the tile loop issues the next tile's K
// between this tile's V loads and its math).
// TAIL tiles load only their first `valid` rows (others re-read the last
// valid one and the V rows are zeroed) and give keys at or beyond the
// lane's `lim` a score of -inf; full tiles need neither.
//
// UNI (unified maximum): the exponentials are taken against the fixed
// phi2 instead of the column's running maximum, so there is no
// cross-lane maximum, no rescale of l and acc, and m only records the
// lane's largest x = score - phi2 for the range check that follows the
// chunk.
template <int D, bool TAIL, typename Rows>
__device__ __forceinline__ void tile_load_k(const Rows &rows, int valid,
                                            int n16, int q4,
                                            uint4 (&kr)[2][D / 32]) {
  constexpr int KK = D / 32;
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    int r = sub * 16 + n16;
    if (TAIL) r = min(r, valid - 1);
    const uint16_t *p = rows.krow(r) + q4 * 8;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      kr[sub][kk] = load_stream(reinterpret_cast<const uint4 *>(p + kk * 32));
  }
}

template <int D, bool TAIL, typename Rows>
__device__ __forceinline__ void tile_load_v(
    const Rows &rows, int valid, int n16, int q4,
    typename VecOf<D / 16>::type (&vr)[8]) {
  constexpr int VW = D / 16;
  typedef typename VecOf<VW>::type VT;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int r = (i >> 2) * 16 + q4 * 4 + (i & 3);
    if (TAIL) r = min(r, valid - 1);
    if constexpr (VW == 16) {
      const uint16_t *p = rows.vrow(r) + n16 * 8;
      vr[i].lo = load_stream(reinterpret_cast<const uint4 *>(p));
      vr[i].hi = load_stream(reinterpret_cast<const uint4 *>(p + 128));
    } else {
      vr[i] = load_stream(
          reinterpret_cast<const VT *>(rows.vrow(r) + n16 * VW));
    }
  }
}

template <int D, bool TAIL, bool UNI, bool PAGED_ROWS, typename E>
__device__ __forceinline__ void tile_compute(
    const uint4 (&kr)[2][D / 32], typename VecOf<D / 16>::type (&vr)[8],
    int valid, int lim, int n16, int q4,
    const typename E16<E>::vec (&qop)[D / 32],
    float scale_log2, float phi2, floatx4 (&acc)[D / 16], float &m,
    float &l) {
  constexpr int KK = D / 32;
  constexpr int VW = D / 16;
  typedef typename VecOf<VW>::type VT;
  typedef typename E16<E>::vec EV;
  floatx4 sc[2];
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    sc[sub] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      sc[sub] = mfma32(__builtin_bit_cast(EV, kr[sub][kk]), qop[kk], sc[sub]);
  }

  float s[8];
#pragma unroll
  for (int sub = 0; sub < 2; ++sub)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float x = UNI ? sc[sub][j] * scale_log2 - phi2 : sc[sub][j] * scale_log2;
      if (TAIL && sub * 16 + q4 * 4 + j >= lim) x = FD_NEG_INF;
      s[sub * 4 + j] = x;
    }
  float mt = s[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) mt = fmaxf(mt, s[i]);
  float mref = 0.f, alpha = 1.f, mn;
  if (UNI) {
    mn = fmaxf(m, mt);
  } else {
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    mn = fmaxf(m, mt);
    mref = mn == FD_NEG_INF ? 0.f : mn;
    alpha = exp2_f(m - mref);
  }

  // P enters the matrix cores as a pair of operands of the cache's 16-bit
  // type (hi = E(p), lo = E(p - hi); exact to 2^-17 in bf16); the running
  // sum uses fp32 p.
  EV p_hi, p_lo;
  float psum = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float p = exp2_f(s[i] - mref);
    const E hi = (E)p;
    p_hi[i] = hi;
    p_lo[i] = (E)(p - (float)hi);
    psum += p;
  }
  m = mn;
  if (UNI) {
    l += psum;
  } else {
    l = l * alpha + psum;
#pragma unroll
    for (int e = 0; e < VW; ++e) acc[e] *= alpha;
  }

  if (TAIL) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if ((i >> 2) * 16 + q4 * 4 + (i & 3) >= valid) vr[i] = VT{};
  }
  // Paged and unified-maximum tiles: left alone, the scheduler hoists the V
  // regrouping (which waits for every V load) above the softmax; keeping it
  // here lets the exponentials overlap the V loads, as the contiguous loop
  // does by itself.
  if constexpr (PAGED_ROWS || UNI) __builtin_amdgcn_sched_barrier(0);
  EV vt[VW];
#pragma unroll
  for (int e = 0; e < VW; ++e) {
    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
    uint4 t;
    t.x = __builtin_amdgcn_perm(dword_of<VW>(vr[1], e >> 1),
                                dword_of<VW>(vr[0], e >> 1), sel);
    t.y = __builtin_amdgcn_perm(dword_of<VW>(vr[3], e >> 1),
                                dword_of<VW>(vr[2], e >> 1), sel);
    t.z = __builtin_amdgcn_perm(dword_of<VW>(vr[5], e >> 1),
                                dword_of<VW>(vr[4], e >> 1), sel);
    t.w = __builtin_amdgcn_perm(dword_of<VW>(vr[7], e >> 1),
                                dword_of<VW>(vr[6], e >> 1), sel);
    vt[e] = __builtin_bit_cast(EV, t);
  }
#pragma unroll
  for (int e = 0; e < VW; ++e) acc[e] = mfma32(vt[e], p_hi, acc[e]);
#pragma unroll
  for (int e = 0; e < VW; ++e) acc[e] = mfma32(vt[e], p_lo, acc[e]);
}

// Order of a chunk's tiles.  When every KV slab starts at the same offset
// modulo 32 MB (a cache padded to 128k keys of 256 bytes puts each KV head
// exactly 32 MB after the previous one), chunks of different heads that
// stream the same offsets in lockstep run far below the usual rate on
// MI355X: measured, batch 1 at 64k keys took 61.5 us on such a cache
// against 44.5 us with 16 MB between heads, and a var-len batch lost up
// to 10% depending on which sequence sat where.  With that stride each
// chunk walks its first nrot = ntiles - 2 tiles from a start point taken
// from its (b, g), wrapping around: KV head g starts g / Hkv of the way in,
// sequence b adds a fraction of one head's share (the fractional part of b
// times the golden ratio).  The last two tiles -- the only ones that can be
// short, or cut by a causal limit -- stay last.  Other strides keep the
// plain order: they were not slow (48 MB included), and rotating there was
// neutral at 16 MB and cost 2.5% at 1 MB and 1.5% at 48 MB.
// The rule reads only the stride Lmax * D * 2 (for a paged cache, its
// table capacity) and the order only (b, g) and the chunk, so every entry
// point visits a chunk's keys in the same order.
constexpr size_t kRotateStride = size_t(32) << 20;

struct TileOrder {
  int nrot, rot;
  __device__ __forceinline__ int key0(const Work &w, int t) const {
    int u = t;
    if (t < nrot) {
      u = t + rot;
      if (u >= nrot) u -= nrot;
    }
    return w.lo + u * kKeyTile;
  }
};

__device__ __forceinline__ TileOrder tile_order(const Work &w, int Hkv,
                                                int ntiles, bool rotate) {
  TileOrder o;
  o.nrot = max(ntiles - 2, 0);
  o.rot = 0;
  if (rotate && o.nrot > 1) {
    const float xb = (float)w.b * 0.61803398875f;
    const float x = ((float)w.g + (xb - floorf(xb))) / (float)Hkv;
    o.rot = min((int)(x * (float)o.nrot), o.nrot - 1);
  }
  return o;
}

// Paged cache: for the first key of each 16-key half of this wavefront's
// tiles it0 .. it0 + 31 (lane 2 j + h: half h of tile it0 + j), the index
// of its D-element row of KV head g (of the pool's Hkv) in the pool:
// (page * page_size + t) * Hkv + g token-major, (page * Hkv + g) *
// page_size + t head-major, with t the key's place in its page.  Halves
// at or beyond the chunk end read nothing and give 0; page indices are
// clamped into the pool, so no entry of the table can make a load leave
// the K/V buffers.
__device__ __forceinline__ int page_rows(const PagedKV &pk, const Work &w,
                                         const TileOrder &ord, int Hkv, int g,
                                         int wave, int nw, int it0, int lane) {
  const int t = wave + (it0 + (lane >> 1)) * nw;
  const int key = ord.key0(w, t) + (lane & 1) * 16;
  if (key >= w.hi) return 0;
  const int j = key / pk.page_size;
  int pg = pk.block_table[(size_t)w.b * pk.max_pages + j];
  pg = min(max(pg, 0), pk.num_pages - 1);
  const int off = key - j * pk.page_size;
  return pk.head_major ? (pg * Hkv + g) * pk.page_size + off
                       : (pg * pk.page_size + off) * Hkv + g;
}

// Paged caches (D = 128): K of a tile goes through LDS.  With a head's rows
// apart in memory (2 KB apart token-major), K loads in the matrix-core
// operand layout -- each instruction reading 64 bytes of 16 rows -- stream
// markedly slower than loads of whole rows, so the paged loop loads K as
// whole rows (every 16 lanes one 256-byte row, 4 rows per instruction),
// writes them to the wavefront's LDS buffer and reads the operand layout
// back.  A contiguous cache streams either way at the same rate, and the
// extra LDS round trip makes it slower, so it keeps the direct loads.
template <int D, bool PAGED>
constexpr bool kStageK = PAGED && D == 128;

// K of a 32-key tile as whole rows: register i of lane l holds 16 bytes,
// chunk l % 16, of row 4 i + l / 16.  Rows at or beyond `valid` re-read the
// last valid row.
template <typename Rows>
__device__ __forceinline__ void load_k_rows(const Rows &rows, int valid,
                                            int lane, uint4 (&kn)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = min(4 * i + (lane >> 4), valid - 1);
    kn[i] = load_stream(
        reinterpret_cast<const uint4 *>(rows.krow(r) + (lane & 15) * 8));
  }
}

// The rows into the wavefront's LDS buffer (32 rows x 256 bytes), 16-byte
// chunks XOR-swizzled by row (slot = chunk ^ (row % 16)) so that the operand
// reads below hit distinct banks.
__device__ __forceinline__ void store_k_lds(const uint4 (&kn)[8], int lane,
                                            uint16_t *kbuf) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 4 * i + (lane >> 4);
    const int slot = (lane & 15) ^ (r & 15);
    *reinterpret_cast<uint4 *>(kbuf + i * 512 + ((r & 3) * 16 + slot) * 8) =
        kn[i];
  }
}

// The operand layout from the LDS buffer: lane (n16, q4) takes row
// sub * 16 + n16, chunk kk * 4 + q4.
__device__ __forceinline__ void load_k_operand(const uint16_t *kbuf, int n16,
                                               int q4, uint4 (&kr)[2][4]) {
#pragma unroll
  for (int sub = 0; sub < 2; ++sub)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int r = sub * 16 + n16;
      const int slot = (kk * 4 + q4) ^ n16;
      kr[sub][kk] = *reinterpret_cast<const uint4 *>(
          kbuf + (r >> 2) * 512 + ((r & 3) * 16 + slot) * 8);
    }
}

// Rows of the tile starting at key k0, wavefront iteration `it`: a slab
// offset, or two page-resident halves read from the staged page rows
// (restaged every 32 iterations).
template <int D, int NW, bool PAGED>
__device__ __forceinline__ TileRows<D, PAGED> tile_rows(
    const PagedKV &pk, const Work &w, const TileOrder &ord,
    const uint16_t *__restrict__ kc, const uint16_t *__restrict__ vc,
    size_t slab, size_t prs, int hkv_kv, int g_kv, int wave, int lane,
    int k0, int it, int &prow) {
  TileRows<D, PAGED> rows;
  if constexpr (PAGED) {
    const int slot = it & 31;
    if (slot == 0)
      prow = page_rows(pk, w, ord, hkv_kv, g_kv, wave, NW, it, lane);
    const int r0 = __builtin_amdgcn_readlane(prow, 2 * slot);
    const int r1 = __builtin_amdgcn_readlane(prow, 2 * slot + 1);
    rows.rs = prs;
    rows.k0h = kc + (size_t)r0 * D;
    rows.k1h = kc + (size_t)r1 * D;
    rows.v0h = vc + (size_t)r0 * D;
    rows.v1h = vc + (size_t)r1 * D;
  } else {
    rows.k = kc + slab;
    rows.v = vc + slab;
    rows.k0 = k0;
  }
  return rows;
}

// The per-chunk kernel is held to two workgroups per CU (one of eight
// wavefronts): left free, the compiler spends the registers of the K tile
// loaded ahead until only one wavefront fits per SIMD.  At D = 256 a
// wavefront's tiles and accumulators need more than 256 registers: one
// workgroup per CU, with the accumulation registers in use.
template <int NW, int D = 128>
constexpr int kBlocksPerCU = NW >= 8 || D > 128 ? 1 : 2;

// The tiles of a chunk, wavefront `wave` taking tiles wave, wave + NW, ...
// K of the next tile is loaded while this tile computes: per tile, V of
// this tile, then K of the next, then the math on this tile's K.  Every
// tile but a wavefront's last is full: only the chunk's last tile can be
// short, and the causal limits of several new tokens (at most 15 keys
// apart) cut into the chunk's last two tiles only, which with two or more
// wavefronts are both some wavefront's last.  Loads clamp rows to the valid
// count without branching.
template <int D, int NW, bool PAGED, bool CAUSAL, bool UNI, typename E>
__device__ __forceinline__ void chunk_tiles(
    const Work &w, const PagedKV &pk, const uint16_t *__restrict__ kc,
    const uint16_t *__restrict__ vc, size_t slab, size_t prs, int Hkv,
    int hkv_kv, int g_kv, int hi_all, int hi_col, int wave, int lane,
    int n16, int q4, const typename E16<E>::vec (&qop)[D / 32],
    float scale_log2,
    float phi2, floatx4 (&acc)[D / 16], float &m, float &l, uint16_t *kbuf,
    bool rotate) {
  static_assert(NW >= 2, "the loop relies on two or more wavefronts");
  const int ntiles = (w.hi - w.lo + kKeyTile - 1) / kKeyTile;
  int t = wave;
  if (t >= ntiles) return;
  const TileOrder ord = tile_order(w, Hkv, ntiles, rotate);
  if constexpr (kStageK<D, PAGED>) {
    // The same loop with K staged through LDS: the rows of the next tile
    // are in flight while this tile is staged, read back and computed.
    int prow = 0;
    const int kf0 = ord.key0(w, t);
    TileRows<D, PAGED> cur = tile_rows<D, NW, PAGED>(
        pk, w, ord, kc, vc, slab, prs, hkv_kv, g_kv, wave, lane, kf0, 0,
        prow);
    uint4 kn[8];
    load_k_rows(cur, min(kKeyTile, w.hi - kf0), lane, kn);
    uint4 kr[2][4];
    int it = 0;
    for (; t + NW < ntiles; t += NW, ++it) {
      store_k_lds(kn, lane, kbuf);
      typename VecOf<D / 16>::type vr[8];
      tile_load_v<D, false>(cur, kKeyTile, n16, q4, vr);
      const int kn0 = ord.key0(w, t + NW);
      TileRows<D, PAGED> nxt = tile_rows<D, NW, PAGED>(
          pk, w, ord, kc, vc, slab, prs, hkv_kv, g_kv, wave, lane, kn0,
          it + 1, prow);
      load_k_rows(nxt, min(kKeyTile, w.hi - kn0), lane, kn);
      __builtin_amdgcn_sched_barrier(0);
      load_k_operand(kbuf, n16, q4, kr);
      tile_compute<D, false, UNI, PAGED, E>(kr, vr, kKeyTile, kKeyTile, n16, q4,
                                         qop, scale_log2, phi2, acc, m, l);
      cur = nxt;
    }
    const int k0 = ord.key0(w, t);
    const int valid = min(kKeyTile, w.hi - k0);
    const bool full = CAUSAL ? k0 + kKeyTile <= hi_all : valid == kKeyTile;
    store_k_lds(kn, lane, kbuf);
    typename VecOf<D / 16>::type vr[8];
    tile_load_v<D, true>(cur, valid, n16, q4, vr);
    load_k_operand(kbuf, n16, q4, kr);
    if (full)
      tile_compute<D, false, UNI, PAGED, E>(kr, vr, kKeyTile, kKeyTile, n16, q4,
                                         qop, scale_log2, phi2, acc, m, l);
    else
      tile_compute<D, true, UNI, PAGED, E>(kr, vr, valid,
                                        CAUSAL ? hi_col - k0 : valid, n16, q4,
                                        qop, scale_log2, phi2, acc, m, l);
    return;
  }
  int prow = 0;
  const int kf0 = ord.key0(w, t);
  TileRows<D, PAGED> cur = tile_rows<D, NW, PAGED>(
      pk, w, ord, kc, vc, slab, prs, hkv_kv, g_kv, wave, lane, kf0, 0,
      prow);
  uint4 kr[2][D / 32];
  tile_load_k<D, true>(cur, min(kKeyTile, w.hi - kf0), n16, q4, kr);
  int it = 0;
  for (; t + NW < ntiles; t += NW, ++it) {
    typename VecOf<D / 16>::type vr[8];
    tile_load_v<D, false>(cur, kKeyTile, n16, q4, vr);
    __builtin_amdgcn_sched_barrier(0);
    const int kn0 = ord.key0(w, t + NW);
    TileRows<D, PAGED> nxt = tile_rows<D, NW, PAGED>(
        pk, w, ord, kc, vc, slab, prs, hkv_kv, g_kv, wave, lane, kn0,
        it + 1, prow);
    uint4 kn[2][D / 32];
    tile_load_k<D, true>(nxt, min(kKeyTile, w.hi - kn0), n16, q4, kn);
    __builtin_amdgcn_sched_barrier(0);
    tile_compute<D, false, UNI, PAGED, E>(kr, vr, kKeyTile, kKeyTile, n16, q4,
                                       qop, scale_log2, phi2, acc, m, l);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) kr[sub][kk] = kn[sub][kk];
    cur = nxt;
  }
  const int k0 = ord.key0(w, t);
  const int valid = min(kKeyTile, w.hi - k0);
  const bool full = CAUSAL ? k0 + kKeyTile <= hi_all : valid == kKeyTile;
  typename VecOf<D / 16>::type vr[8];
  tile_load_v<D, true>(cur, valid, n16, q4, vr);
  if (full)
    tile_compute<D, false, UNI, PAGED, E>(kr, vr, kKeyTile, kKeyTile, n16, q4,
                                       qop, scale_log2, phi2, acc, m, l);
  else
    tile_compute<D, true, UNI, PAGED, E>(kr, vr, valid,
                                      CAUSAL ? hi_col - k0 : valid, n16, q4,
                                      qop, scale_log2, phi2, acc, m, l);
}

// Unified maximum: a chunk column whose largest x = score - phi (log2
// units) lies outside [kUniLo<E>, kUniHi<E>] is recomputed exactly.
// Inside it, 2^x neither overflows nor loses the terms that matter.  bf16
// (fp32's exponent range): sums of up to 2^31 terms of at most 2^64, and
// the largest term at least 2^-64.  fp16, whose P operands stop at 65504
// and flush below 2^-24: the largest term lies in [1, 2^14], so the
// weights lost to the flush are as small against the row's sum as in the
// running-maximum pass, whose largest term is 1.
template <typename E>
constexpr float kUniLo = -64.f;
template <typename E>
constexpr float kUniHi = 64.f;
template <>
constexpr float kUniLo<_Float16> = 0.f;
template <>
constexpr float kUniHi<_Float16> = 14.f;

// End of a chunk in the matrix-core kernels: the wavefronts' states are
// merged with one weight per (wavefront, column).
// Every wavefront publishes its column maxima m and sums l, and wavefronts
// 1.. park their accumulators in LDS as 16-byte vectors; after one barrier
// wavefront 0 alone forms M = max m, W = sum 2^(m - M) l and the weights
// 2^(m - M) / W, adds the weighted accumulators in wavefront order and
// stores its lane's runs of four consecutive output columns,
// acc_col(4 e4, 4 q4 + j), with vector stores.  A column that saw no key
// gets out 0 and lse -inf.  OutT: uint16_t (bf16 bits), _Float16 (both
// rounded to nearest even) or float.  ROWS: the accumulator layout
// (acc_col); with any of them a lane's blocks 4 e4 .. 4 e4 + 3 of one j
// are four consecutive columns.  FUSED: the partial is read by another
// workgroup of the same launch (the fused merge), so it is written through
// to the device coherence point; a separate instantiation keeps the
// two-launch path's code as it is.
template <int D, int NW, typename OutT = uint16_t, int ROWS = 0,
          bool FUSED = false>
__device__ __forceinline__ void wave_merge_store(
    float *sm_m, float *sm_l, float *sm_o, int wave, int lane, int n16,
    int q4, int ncol, float m, float l, const floatx4 (&acc)[D / 16],
    const Work &w, const PartLayout &pl, int mode,
    OutT *__restrict__ out, float *__restrict__ lse,
    float *__restrict__ o_part, float *__restrict__ lse_part) {
  constexpr int VW = D / 16;
  constexpr int V4 = VW / 4;  // float4 per (lane, j)
  if (q4 == 0) {
    sm_m[wave * 16 + n16] = m;
    sm_l[wave * 16 + n16] = l;
  }
  float4 *park = reinterpret_cast<float4 *>(sm_o);
  if (NW > 1 && wave > 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e4 = 0; e4 < V4; ++e4)
        park[(((wave - 1) * 4 + j) * V4 + e4) * 64 + lane] = make_float4(
            acc[4 * e4][j], acc[4 * e4 + 1][j], acc[4 * e4 + 2][j],
            acc[4 * e4 + 3][j]);
  }
  __syncthreads();
  if (wave != 0 || n16 >= ncol) return;
  float ms[NW], wt[NW];
  float M = FD_NEG_INF;
#pragma unroll
  for (int sl = 0; sl < NW; ++sl) {
    ms[sl] = sm_m[sl * 16 + n16];
    M = fmaxf(M, ms[sl]);
  }
  float W = 0.f;
#pragma unroll
  for (int sl = 0; sl < NW; ++sl) {
    wt[sl] = M == FD_NEG_INF ? 0.f : exp2_f(ms[sl] - M);
    W += wt[sl] * sm_l[sl * 16 + n16];
  }
  const float inv = M == FD_NEG_INF ? 0.f : 1.f / W;
#pragma unroll
  for (int sl = 0; sl < NW; ++sl) wt[sl] *= inv;
  // out/lse row (direct) or partial index (partial mode) of this column
  const size_t row = mode == kModeDirect ? row_of(w, pl.G, pl.Hq, pl.Tq, n16)
                                         : pl.at(w, n16);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int e4 = 0; e4 < V4; ++e4) {
      float4 o = make_float4(acc[4 * e4][j] * wt[0], acc[4 * e4 + 1][j] * wt[0],
                             acc[4 * e4 + 2][j] * wt[0],
                             acc[4 * e4 + 3][j] * wt[0]);
#pragma unroll
      for (int sl = 1; sl < NW; ++sl) {
        const float4 p = park[(((sl - 1) * 4 + j) * V4 + e4) * 64 + lane];
        o.x += p.x * wt[sl];
        o.y += p.y * wt[sl];
        o.z += p.z * wt[sl];
        o.w += p.w * wt[sl];
      }
      const int d0 = acc_col<VW, ROWS>(4 * e4, q4 * 4 + j);
      if (mode == kModeDirect) {
        if constexpr (sizeof(OutT) == 2) {
          uint2 bits;
          bits.x = bits16<OutT>(o.x) | (bits16<OutT>(o.y) << 16);
          bits.y = bits16<OutT>(o.z) | (bits16<OutT>(o.w) << 16);
          *reinterpret_cast<uint2 *>(out + row * D + d0) = bits;
        } else {
          *reinterpret_cast<float4 *>(out + row * D + d0) = o;
        }
      } else if constexpr (FUSED) {
        store_through(o_part + row * D + d0, o);
      } else {
        *reinterpret_cast<float4 *>(o_part + row * D + d0) = o;
      }
    }
  }
  if (q4 == 0) {
    const float ls = M == FD_NEG_INF ? FD_NEG_INF : (M + log2_f(W)) * kLn2;
    if (mode == kModeDirect)
      lse[row] = ls;
    else if constexpr (FUSED)
      __hip_atomic_store(lse_part + row, ls, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    else
      lse_part[row] = ls;
  }
}

// One chunk of the matrix-core per-chunk pass (the kernel below runs one or
// two).  PAGED: K/V in a page pool behind a block table.  CAUSAL:
// Tq > 1 new tokens per sequence, each column with its own key limit (a
// separate instantiation keeps the single-token loop exactly as simple as
// before).
// UNI: unified-maximum softmax against phi2 (log2 units of the scaled
// score) with an exact fallback.
template <int D, int NW, bool PAGED, bool CAUSAL, bool UNI, typename E,
          bool FUSED>
__device__ __forceinline__ void chunk_pass(
    const Work &w, const uint16_t *__restrict__ q, const uint16_t *__restrict__ kc,
    const uint16_t *__restrict__ vc, const int32_t *__restrict__ seqlens,
    PagedKV pk, int B, int Hq, int Hkv, int kv_rep, int G, int Tq, int Lmax,
    int C, int S, float scale_log2, float phi2, int mode, bool chunk_major,
    typename E16<E>::out *__restrict__ out, float *__restrict__ lse,
    float *__restrict__ o_part, float *__restrict__ lse_part,
    int *__restrict__ tickets) {
  constexpr int KK = D / 32;
  constexpr int VW = D / 16;
  static_assert(16 * (D + 1) >= 6 * 64, "LDS reused by the fused merge");
  const PartLayout pl{G, Tq, Hq, Hkv, S, chunk_major};
  __shared__ float sm_m[NW * 16];
  __shared__ float sm_l[NW * 16];
  __shared__ __align__(16) float sm_o[NW * 16 * (D + 1)];
  __shared__ int sm_flag;
  constexpr int kStageElems = kStageK<D, PAGED> ? 32 * D : 8;
  __shared__ __align__(16) uint16_t sm_k[NW * kStageElems];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint16_t *kbuf = sm_k + wave * kStageElems;
  const int n16 = lane & 15, q4 = lane >> 4;
  const int ncol = G * Tq;

  typedef typename E16<E>::out OutT;
  typename E16<E>::vec qop[KK];
  {
    const bool live = n16 < ncol;
    const uint16_t *qr = q + row_of(w, G, Hq, Tq, live ? n16 : 0) * D + q4 * 8;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      uint4 t = live ? *reinterpret_cast<const uint4 *>(qr + kk * 32)
                     : make_uint4(0, 0, 0, 0);
      qop[kk] = __builtin_bit_cast(typename E16<E>::vec, t);
    }
  }
  // Causal limit among the Tq new tokens (the newest Tq keys of the
  // sequence): column c, token t = c / G, sees keys below L - (Tq - 1 - t).
  // Tiles wholly below the first token's limit need no mask.
  const int hi_col = min(w.hi, w.L - (Tq - 1 - n16 / G));
  const int hi_all = min(w.hi, w.L - (Tq - 1));

  // Groups of more than 16 query rows run as kv_rep virtual KV heads of
  // G rows each (Hkv counts them): virtual head w.g reads the cache of KV
  // head w.g / kv_rep, one of Hkv / kv_rep.
  const int hkv_kv = Hkv / kv_rep, g_kv = w.g / kv_rep;
  const size_t slab = ((size_t)w.b * hkv_kv + g_kv) * (size_t)Lmax * D;
  const size_t prs = pk.head_major ? (size_t)D : (size_t)hkv_kv * D;
  const bool rotate =
      (size_t)Lmax * D * sizeof(uint16_t) % kRotateStride == 0;

  floatx4 acc[VW];
#pragma unroll
  for (int e = 0; e < VW; ++e) acc[e] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m = FD_NEG_INF, l = 0.f;

  if constexpr (UNI) {
    // Unified maximum (FlashDecoding++): one pass against phi2.  If a
    // column's largest x = score - phi2 leaves [kUniLo, kUniHi] the
    // fixed reference risks overflow or lost precision, and the whole
    // workgroup recomputes the chunk with the running maximum.
    chunk_tiles<D, NW, PAGED, CAUSAL, true, E>(
        w, pk, kc, vc, slab, prs, Hkv, hkv_kv, g_kv, hi_all, hi_col, wave,
        lane, n16, q4, qop, scale_log2, phi2, acc, m, l, kbuf, rotate);
    float xm = fmaxf(m, __shfl_xor(m, 16, 64));
    xm = fmaxf(xm, __shfl_xor(xm, 32, 64));
    const bool bad = xm != FD_NEG_INF &&
                     !(xm >= kUniLo<E> && xm <= kUniHi<E>);
    if (__syncthreads_or(bad)) {
#pragma unroll
      for (int e = 0; e < VW; ++e) acc[e] = floatx4{0.f, 0.f, 0.f, 0.f};
      m = FD_NEG_INF;
      l = 0.f;
      chunk_tiles<D, NW, PAGED, CAUSAL, false, E>(
          w, pk, kc, vc, slab, prs, Hkv, hkv_kv, g_kv, hi_all, hi_col, wave,
          lane, n16, q4, qop, scale_log2, 0.f, acc, m, l, kbuf, rotate);
    } else {
      m = xm == FD_NEG_INF ? FD_NEG_INF : phi2;
    }
  } else {
    chunk_tiles<D, NW, PAGED, CAUSAL, false, E>(
        w, pk, kc, vc, slab, prs, Hkv, hkv_kv, g_kv, hi_all, hi_col, wave,
        lane, n16, q4, qop, scale_log2, 0.f, acc, m, l, kbuf, rotate);
  }

  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  // FUSED (mode kModeFused) is its own instantiation, so that the
  // two-launch kernels carry no code of the single-launch merge.
  wave_merge_store<D, NW, OutT, kBf16Rows<D>, FUSED>(
      sm_m, sm_l, sm_o, wave, lane, n16, q4, ncol, m, l, acc, w, pl, mode,
      out, lse, o_part, lse_part);
  if constexpr (FUSED)
    merge_group_if_last<D, OutT>(w, pl, o_part, lse_part, tickets, out, lse,
                                 sm_o, &sm_flag);
}

template <int D, int NW, bool PAGED, bool CAUSAL, bool UNI, typename E,
          bool FUSED>
__global__ __launch_bounds__(NW * 64, (kBlocksPerCU<NW, D>))
void split_mfma_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kc,
    const uint16_t *__restrict__ vc, const int32_t *__restrict__ seqlens,
    PagedKV pk, int B, int Hq, int Hkv, int kv_rep, int G, int Tq, int Lmax,
    int C, int S, float scale_log2, float phi2, int mode, bool direct,
    bool chunk_major,
    typename E16<E>::out *__restrict__ out,
    float *__restrict__ lse, float *__restrict__ o_part,
    float *__restrict__ lse_part, int *__restrict__ tickets) {
  // With per-sequence lengths the grid can be as small as half the work
  // list's upper bound: workgroup i takes chunk i and then, if it exists,
  // chunk i + gridDim.x.  (Written out twice rather than as a loop: around
  // a loop the compiler keeps lane offsets live through the tile loop and
  // spills.)
  const Work w0 = find_work(blockIdx.x, seqlens, B, Hkv, Lmax, C, direct);
  if (!w0.valid) return;
  chunk_pass<D, NW, PAGED, CAUSAL, UNI, E, FUSED>(w0, q, kc, vc, seqlens, pk, B, Hq,
                                        Hkv, kv_rep, G, Tq, Lmax, C, S,
                                        scale_log2, phi2, mode, chunk_major,
                                        out, lse, o_part, lse_part, tickets);
  // Equal lengths, a grid that covers the upper bound, or a work list that
  // ends before i + grid (its length is known from the scan for up to 64
  // sequences): one chunk each, and no second look-up.
  const long id1 = (long)blockIdx.x + gridDim.x;
  if (seqlens == nullptr || id1 >= (long)B * Hkv * S || id1 >= w0.items)
    return;
  const Work w1 = find_work((int)id1, seqlens, B, Hkv, Lmax, C, false);
  if (!w1.valid) return;
  __syncthreads();  // the second chunk reuses the LDS
  chunk_pass<D, NW, PAGED, CAUSAL, UNI, E, FUSED>(w1, q, kc, vc, seqlens, pk, B, Hq,
                                        Hkv, kv_rep, G, Tq, Lmax, C, S,
                                        scale_log2, phi2, mode, chunk_major,
                                        out, lse, o_part, lse_part, tickets);
}

// ---------------------------------------------------------------------------
// Matrix-core kernel for fp32 caches (contiguous or paged, one or several
// new tokens).
//
// v_mfma_f32_16x16x4_f32 takes one fp32 value of each operand per lane.  For
// the scores S^T = K Q^T lane (n16, q4) loads 16 bytes of key row n16 per
// register j, elements d = 16 j + 4 q4 + e (e = 0..3), and the q-tile holds
// the same d of query column n16, so one register serves four MFMAs: the
// dot product only runs over d in another order.  The scores then sit in
// the bf16 kernel's layout (lane (n16, q4), element r: key 4 q4 + r of the
// 16-key half, column n16) and the softmax is the same.  For O^T += V^T P^T
// the four keys 4 q4 + r (r fixed) form one MFMA's k-slice: its B operand
// is the lane's own p of element r, its A operand V[key][d] with
// d = 64 (e / 4) + 4 n16 + e % 4: each V load instruction reads whole
// 256-byte row pieces (16 lanes x 16 bytes), which at D = 128 streamed ~9%
// faster than 32 contiguous bytes per lane.  Element j of accumulator block
// e is then column n16, d = 64 (e / 4) + 4 (4 q4 + j) + e % 4, and the
// bf16 kernel's end-of-chunk merge is shared with that column order
// (acc_col with ROWS = 4).  P stays fp32 (no hi/lo split).  A wavefront works
// through its tiles in 16-key halves (one MFMA k-slice of scores each) and
// keeps the next half's K and V in flight while the current half computes:
// 16 KB of K/V per half at D = 128, two halves of registers, where a whole
// second 32-key tile would not fit (D = 256 keeps one half of registers).
__device__ __forceinline__ floatx4 load_stream_f4(const float *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const floatx4 *>(p));
}

template <int D>
struct F32Half {
  floatx4 k[D / 16];     // K row n16, d = 16 j + 4 q4 + e
  floatx4 v[4][D / 64];  // V row 4 q4 + r, d = 64 c + 4 n16 + e
};

// The 16 keys of a half: key r at kb + r * rs (K) and vb + r * rs (V),
// rows at or beyond `valid` re-reading the last valid one.  rs = D for a
// contiguous slab; in a page pool the half lies inside one page, rows
// Hkv * D (token-major) or D (head-major) apart.
template <int D>
__device__ __forceinline__ void f32_half_load(const float *__restrict__ kb,
                                              const float *__restrict__ vb,
                                              size_t rs, int valid, int n16,
                                              int q4, F32Half<D> &h) {
  const float *pk = kb + (size_t)min(n16, valid - 1) * rs + q4 * 4;
#pragma unroll
  for (int j = 0; j < D / 16; ++j) h.k[j] = load_stream_f4(pk + 16 * j);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float *pv = vb + (size_t)min(q4 * 4 + r, valid - 1) * rs + n16 * 4;
#pragma unroll
    for (int c = 0; c < D / 64; ++c) h.v[r][c] = load_stream_f4(pv + 64 * c);
  }
}

// MASK: keys at or beyond `lim` (this lane's column; the half's own valid
// count, or a causal limit) score -inf, and V rows at or beyond `valid`
// are zeroed.
template <int D, bool MASK>
__device__ __forceinline__ void f32_half_compute(
    F32Half<D> &h, int valid, int lim, int q4, const floatx4 (&qf)[D / 16],
    float scale_log2, floatx4 (&acc)[D / 16], float &m, float &l) {
  constexpr int VW = D / 16;
  floatx4 sc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < D / 16; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      sc = __builtin_amdgcn_mfma_f32_16x16x4f32(h.k[j][e], qf[j][e], sc, 0, 0,
                                                0);
  float s[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float x = sc[r] * scale_log2;
    if (MASK && q4 * 4 + r >= lim) x = FD_NEG_INF;
    s[r] = x;
  }
  float mt = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
  mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
  mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
  const float mn = fmaxf(m, mt);
  const float mref = mn == FD_NEG_INF ? 0.f : mn;
  const float alpha = exp2_f(m - mref);
  float p[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) p[r] = exp2_f(s[r] - mref);
  m = mn;
  l = l * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
#pragma unroll
  for (int e = 0; e < VW; ++e) acc[e] *= alpha;
  if (MASK) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (q4 * 4 + r >= valid)
#pragma unroll
        for (int c = 0; c < D / 64; ++c)
          h.v[r][c] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int e = 0; e < VW; ++e)
      acc[e] = __builtin_amdgcn_mfma_f32_16x16x4f32(h.v[r][e >> 2][e & 3],
                                                    p[r], acc[e], 0, 0, 0);
}

// One chunk of the fp32 matrix-core pass: wavefront `wave` takes tiles
// wave, wave + NW, ... in the chunk's tile order, as a list of 16-key
// halves.  Only the chunk's last tile can be short, so only the last half of
// the list can be partial (a last tile of at most 16 keys gives one half);
// the causal limits of several new tokens (at most 15 keys apart) cut only
// into the chunk's last two tiles, each some wavefront's last, so only a
// wavefront's last two halves can need masks.  PAGED: the halves' pool
// rows are staged 64 at a time (page_rows, one table entry per lane).
template <int D, int NW, bool PAGED, bool CAUSAL, bool FUSED>
__device__ __forceinline__ void f32_chunk_pass(
    const Work &w, const float *__restrict__ q, const float *__restrict__ kc,
    const float *__restrict__ vc, const PagedKV &pk, int Hq, int Hkv,
    int kv_rep, int G, int Tq, int Lmax, int S, float scale_log2, int mode,
    bool chunk_major,
    float *__restrict__ out, float *__restrict__ lse,
    float *__restrict__ o_part, float *__restrict__ lse_part,
    int *__restrict__ tickets) {
  constexpr int VW = D / 16;
  const PartLayout pl{G, Tq, Hq, Hkv, S, chunk_major};
  __shared__ float sm_m[NW * 16];
  __shared__ float sm_l[NW * 16];
  __shared__ __align__(16) float sm_o[NW * 16 * (D + 1)];
  __shared__ int sm_flag;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n16 = lane & 15, q4 = lane >> 4;
  const int ncol = G * Tq;

  floatx4 qf[D / 16];
  {
    const bool live = n16 < ncol;
    const float *qr = q + row_of(w, G, Hq, Tq, live ? n16 : 0) * D + q4 * 4;
#pragma unroll
    for (int j = 0; j < D / 16; ++j)
      qf[j] = live ? *reinterpret_cast<const floatx4 *>(qr + 16 * j)
                   : floatx4{0.f, 0.f, 0.f, 0.f};
  }
  // Causal limit of this lane's column (token t = c / G of the Tq newest)
  // and the smallest over the columns.
  const int hi_col = min(w.hi, w.L - (Tq - 1 - n16 / G));
  const int hi_all = min(w.hi, w.L - (Tq - 1));
  // virtual KV heads as in the bf16 pass
  const int hkv_kv = Hkv / kv_rep, g_kv = w.g / kv_rep;
  const size_t slab = ((size_t)w.b * hkv_kv + g_kv) * (size_t)Lmax * D;
  const size_t rs = !PAGED ? (size_t)D
                           : (pk.head_major ? (size_t)D : (size_t)hkv_kv * D);
  const bool rotate = (size_t)Lmax * D * sizeof(float) % kRotateStride == 0;

  floatx4 acc[VW];
#pragma unroll
  for (int e = 0; e < VW; ++e) acc[e] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m = FD_NEG_INF, l = 0.f;

  const int ntiles = (w.hi - w.lo + kKeyTile - 1) / kKeyTile;
  if (wave < ntiles) {
    const TileOrder ord = tile_order(w, Hkv, ntiles, rotate);
    const int nt = (ntiles - wave + NW - 1) / NW;
    const int last0 = ord.key0(w, wave + (nt - 1) * NW);
    const int nh = 2 * nt - (w.hi - last0 <= 16 ? 1 : 0);
    int prow = 0;
    auto key_of = [&](int i) {
      return ord.key0(w, wave + (i >> 1) * NW) + (i & 1) * 16;
    };
    auto load = [&](int i, F32Half<D> &h) {
      const int k0 = key_of(i);
      const float *kb, *vb;
      if constexpr (PAGED) {
        if ((i & 63) == 0)
          prow = page_rows(pk, w, ord, hkv_kv, g_kv, wave, NW, i >> 1, lane);
        const int r0 = __builtin_amdgcn_readlane(prow, i & 63);
        kb = kc + (size_t)r0 * D;
        vb = vc + (size_t)r0 * D;
      } else {
        kb = kc + slab + (size_t)k0 * D;
        vb = vc + slab + (size_t)k0 * D;
      }
      f32_half_load<D>(kb, vb, rs, min(16, w.hi - k0), n16, q4, h);
    };
    // masks only where the half is short or a causal limit cuts into it
    auto compute = [&](int i, F32Half<D> &h) {
      const int k0 = key_of(i);
      const int valid = min(16, w.hi - k0);
      if (CAUSAL ? k0 + 16 <= hi_all : valid == 16)
        f32_half_compute<D, false>(h, 16, 16, q4, qf, scale_log2, acc, m, l);
      else
        f32_half_compute<D, true>(h, valid, CAUSAL ? hi_col - k0 : valid, q4,
                                  qf, scale_log2, acc, m, l);
    };
    auto compute_full = [&](F32Half<D> &h) {
      f32_half_compute<D, false>(h, 16, 16, q4, qf, scale_log2, acc, m, l);
    };
    F32Half<D> h0, h1;
    if constexpr (D > 128) {
      // D = 256: one register set (a half is 32 KB of K/V); two spilled,
      // and measured 21-27% slower than this loop
      for (int i = 0; i < nh; ++i) {
        load(i, h0);
        compute(i, h0);
      }
    } else {
      // two register sets taken in turn (a copy between them would wait for
      // the loads in flight)
      load(0, h0);
      int i = 0;
      if constexpr (!CAUSAL) {
        for (; i + 2 < nh; i += 2) {
          load(i + 1, h1);
          __builtin_amdgcn_sched_barrier(0);
          compute_full(h0);
          load(i + 2, h0);
          __builtin_amdgcn_sched_barrier(0);
          compute_full(h1);
        }
        if (i + 2 == nh) {
          load(i + 1, h1);
          __builtin_amdgcn_sched_barrier(0);
          compute_full(h0);
          compute(i + 1, h1);
        } else {
          compute(i, h0);
        }
      } else {
        // halves before the last three are never cut
        for (; i + 3 < nh; i += 2) {
          load(i + 1, h1);
          __builtin_amdgcn_sched_barrier(0);
          compute_full(h0);
          load(i + 2, h0);
          __builtin_amdgcn_sched_barrier(0);
          compute_full(h1);
        }
        if (i + 3 == nh) {
          load(i + 1, h1);
          __builtin_amdgcn_sched_barrier(0);
          compute_full(h0);
          load(i + 2, h0);
          __builtin_amdgcn_sched_barrier(0);
          compute(i + 1, h1);
          compute(i + 2, h0);
        } else if (i + 2 == nh) {
          load(i + 1, h1);
          __builtin_amdgcn_sched_barrier(0);
          compute(i, h0);
          compute(i + 1, h1);
        } else {
          compute(i, h0);
        }
      }
    }
  }

  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  wave_merge_store<D, NW, float, 4, FUSED>(sm_m, sm_l, sm_o, wave, lane, n16,
                                           q4, ncol, m, l, acc, w, pl, mode,
                                           out, lse, o_part, lse_part);
  if constexpr (FUSED)
    merge_group_if_last<D, float>(w, pl, o_part, lse_part, tickets, out, lse,
                                  sm_o, &sm_flag);
}

// Launched exactly like split_mfma_kernel (the same plan, grid and work
// list; a workgroup may take a second chunk).
template <int D, int NW, bool PAGED, bool CAUSAL, bool FUSED>
__global__ __launch_bounds__(NW * 64, (kBlocksPerCU<NW, D>))
void split_mfma_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ kc,
    const float *__restrict__ vc, const int32_t *__restrict__ seqlens,
    PagedKV pk, int B, int Hq, int Hkv, int kv_rep, int G, int Tq, int Lmax,
    int C, int S, float scale_log2, int mode, bool direct, bool chunk_major,
    float *__restrict__ out, float *__restrict__ lse,
    float *__restrict__ o_part, float *__restrict__ lse_part,
    int *__restrict__ tickets) {
  const Work w0 = find_work(blockIdx.x, seqlens, B, Hkv, Lmax, C, direct);
  if (!w0.valid) return;
  f32_chunk_pass<D, NW, PAGED, CAUSAL, FUSED>(w0, q, kc, vc, pk, Hq, Hkv, kv_rep, G,
                                       Tq, Lmax, S, scale_log2, mode,
                                       chunk_major, out, lse, o_part,
                                       lse_part, tickets);
  const long id1 = (long)blockIdx.x + gridDim.x;
  if (seqlens == nullptr || id1 >= (long)B * Hkv * S || id1 >= w0.items)
    return;
  const Work w1 = find_work((int)id1, seqlens, B, Hkv, Lmax, C, false);
  if (!w1.valid) return;
  __syncthreads();  // the second chunk reuses the LDS
  f32_chunk_pass<D, NW, PAGED, CAUSAL, FUSED>(w1, q, kc, vc, pk, Hq, Hkv, kv_rep, G,
                                       Tq, Lmax, S, scale_log2, mode,
                                       chunk_major, out, lse, o_part,
                                       lse_part, tickets);
}

// ---------------------------------------------------------------------------
// Vector-ALU kernel (fp32; bf16 with small groups).
//
// A key row of D elements is read by LPR lanes, 16 bytes each; a wavefront
// covers RPW = 64 / LPR rows per load and U = 4 loads per tile.  Each lane
// forms partial dot products for the GT query rows it serves and a xor
// butterfly over its LPR lanes completes them.  Every row group keeps its
// own running max/sum; the groups and wavefronts meet in LDS at the end.

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int kPerLane = 4;
  __device__ static void load(const float *p, float (&x)[4]) {
    const uint4 t = load_stream(reinterpret_cast<const uint4 *>(p));
    x[0] = __builtin_bit_cast(float, t.x);
    x[1] = __builtin_bit_cast(float, t.y);
    x[2] = __builtin_bit_cast(float, t.z);
    x[3] = __builtin_bit_cast(float, t.w);
  }
};
template <>
struct Elem<uint16_t> {
  static constexpr int kPerLane = 8;
  __device__ static void load(const uint16_t *p, float (&x)[8]) {
    const uint4 t = load_stream(reinterpret_cast<const uint4 *>(p));
    const uint32_t d[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __builtin_bit_cast(float, d[i] << 16);
      x[2 * i + 1] = __builtin_bit_cast(float, d[i] & 0xFFFF0000u);
    }
  }
};
template <>
struct Elem<_Float16> {
  static constexpr int kPerLane = 8;
  __device__ static void load(const _Float16 *p, float (&x)[8]) {
    const f16x8 t = __builtin_bit_cast(
        f16x8, load_stream(reinterpret_cast<const uint4 *>(p)));
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (float)t[i];
  }
};

template <typename T, int D, int NW, int GT>
__global__ __launch_bounds__(NW * 64) void split_valu_kernel(
    const T *__restrict__ q, const T *__restrict__ kc, const T *__restrict__ vc,
    const int32_t *__restrict__ seqlens, int B, int Hq, int Hkv, int G,
    int kv_rep, int Lmax, int C, int S, float scale_log2, int mode,
    bool chunk_major, T *__restrict__ out, float *__restrict__ lse,
    float *__restrict__ o_part, float *__restrict__ lse_part,
    int *__restrict__ tickets) {
  constexpr int EPL = Elem<T>::kPerLane;
  constexpr int LPR = D / EPL;
  constexpr int RPW = 64 / LPR;
  constexpr int U = 4;
  constexpr int TK = U * RPW;
  constexpr int NSLOT = NW * RPW;
  constexpr int kMergeFloats = NSLOT * GT * (D + 1);
  constexpr int kTailFloats = 6 * NW * 64;
  __shared__ float sm_m[NSLOT * GT];
  __shared__ float sm_l[NSLOT * GT];
  __shared__ __align__(16) float
      sm_o[kMergeFloats > kTailFloats ? kMergeFloats : kTailFloats];
  __shared__ int sm_flag;

  const Work w = find_work(blockIdx.x, seqlens, B, Hkv, Lmax, C, false);
  if (!w.valid) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane % LPR, rg = lane / LPR;

  float qf[GT][EPL];
#pragma unroll
  for (int gi = 0; gi < GT; ++gi) {
    if (gi < G) {
      Elem<T>::load(q + ((size_t)w.b * Hq + (size_t)w.g * G + gi) * D +
                        col * EPL,
                    qf[gi]);
#pragma unroll
      for (int e = 0; e < EPL; ++e) qf[gi][e] *= scale_log2;
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) qf[gi][e] = 0.f;
    }
  }
  // Hkv and G may be virtual: kv_rep groups of G query heads share each
  // KV slab (query head w.g * G + gi either way).
  const size_t slab =
      ((size_t)w.b * Hkv + w.g) / kv_rep * (size_t)Lmax * D;
  const T *kslab = kc + slab + col * EPL;
  const T *vslab = vc + slab + col * EPL;

  float acc[GT][EPL], m[GT], l[GT];
#pragma unroll
  for (int gi = 0; gi < GT; ++gi) {
    m[gi] = FD_NEG_INF;
    l[gi] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[gi][e] = 0.f;
  }

  const int ntiles = (w.hi - w.lo + TK - 1) / TK;
  for (int t = wave; t < ntiles; t += NW) {
    const int k0 = w.lo + t * TK;
    float kx[U][EPL], vx[U][EPL];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = k0 + u * RPW + rg;
      ok[u] = row < w.hi;
      const int rr = ok[u] ? row : w.hi - 1;
      Elem<T>::load(kslab + (size_t)rr * D, kx[u]);
      Elem<T>::load(vslab + (size_t)rr * D, vx[u]);
      if (!ok[u]) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) vx[u][e] = 0.f;
      }
    }
#pragma unroll
    for (int gi = 0; gi < GT; ++gi) {
      float s[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) part += qf[gi][e] * kx[u][e];
#pragma unroll
        for (int off = 1; off < LPR; off <<= 1)
          part += __shfl_xor(part, off, 64);
        s[u] = ok[u] ? part : FD_NEG_INF;
      }
      float mt = s[0];
#pragma unroll
      for (int u = 1; u < U; ++u) mt = fmaxf(mt, s[u]);
      const float mn = fmaxf(m[gi], mt);
      const float mref = mn == FD_NEG_INF ? 0.f : mn;
      const float alpha = exp2_f(m[gi] - mref);
      float p[U], psum = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        p[u] = exp2_f(s[u] - mref);
        psum += p[u];
      }
      l[gi] = l[gi] * alpha + psum;
      m[gi] = mn;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        float a = acc[gi][e] * alpha;
#pragma unroll
        for (int u = 0; u < U; ++u) a += p[u] * vx[u][e];
        acc[gi][e] = a;
      }
    }
  }

  const int slot = wave * RPW + rg;
#pragma unroll
  for (int gi = 0; gi < GT; ++gi) {
    if (gi < G) {
      if (col == 0) {
        sm_m[slot * GT + gi] = m[gi];
        sm_l[slot * GT + gi] = l[gi];
      }
      float *o = sm_o + (slot * GT + gi) * (D + 1) + col * EPL;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = acc[gi][e];
    }
  }
  __syncthreads();
  const PartLayout pl{G, 1, Hq, Hkv, S, chunk_major};
  merge_and_store<D, T>(sm_m, sm_l, sm_o, NSLOT, GT, pl, w, mode, out, lse,
                        o_part, lse_part);
  if (mode == kModeFused)
    merge_group_if_last<D, T>(w, pl, o_part, lse_part, tickets, out, lse,
                              sm_o, &sm_flag);
}

// ---------------------------------------------------------------------------
// Merge pass (the default): for every query row (b, token, head),
// workgroups of MW wavefronts, one per block of 64 * CPL output columns;
// wavefront w folds chunks w, w + MW, ... into a running (M, W, acc), MB
// chunks at a time, all of a batch's loads issued before any is used (the
// pass is latency-bound: a few MB).
// Per batch: M' = max(M, max_s lse_s), r = e^(M - M'),
//   W = r W + sum_s e^(lse_s - M'),  acc = r acc + sum_s e^(lse_s - M') o_s.
// The wavefronts then meet in LDS the same way; out = acc / W and
// lse = M + ln W.  Fixed order everywhere: same chunking, same bits.
// Shapes (launch_combine): fewer rows than CUs (batch 1: 64 rows) get D / 64
// workgroups per row, one column per lane and eight chunks in flight per
// wavefront -- four wavefronts for up to 32 chunks, eight beyond; many rows
// get one workgroup of four wavefronts per row, D / 64 columns per lane,
// sixteen chunks in flight.

// Workgroups are dealt to MI355X's eight XCDs round robin (id % 8).  When
// Hkv is a multiple of 8, every chunk of kv-head g ran on XCD g % 8 (the
// chunk pass's ids are ... * Hkv + g), so the merge of a query row of that
// head is given an id on the same XCD: workgroup 8 k + x takes the k-th
// row, in row order, among the rows of kv-heads g with g % 8 == x.
// Otherwise ids are rows.  Either way it is a permutation of the rows.
__device__ __forceinline__ int merge_row(int id, int G, int Hkv) {
  if (Hkv % 8 != 0) return id;
  const int x = id % 8, k = id / 8, per = Hkv / 8;
  const int hh = k % G, g1 = (k / G) % per, bt = k / G / per;
  return (bt * Hkv + 8 * g1 + x) * G + hh;
}

template <int D, typename OutT, int CPL, int MW, int MB>
__global__ __launch_bounds__(MW * 64) void combine_kernel(
    const float *__restrict__ o_part, const float *__restrict__ lse_part,
    const int32_t *__restrict__ seqlens, PartLayout pl, int Lmax, int C,
    OutT *__restrict__ out, float *__restrict__ lse) {
  constexpr int COLS = 64 * CPL;  // output columns of this workgroup
  static_assert(D % COLS == 0, "column blocks tile the head dimension");
  __shared__ float sm_M[MW], sm_W[MW];
  __shared__ float sm_acc[MW][COLS];
  const int row = merge_row(blockIdx.x, pl.G, pl.Hkv);
  const int c0 = blockIdx.y * COLS;
  const int b = row / (pl.Tq * pl.Hq);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int L = seqlens ? clamp_len(seqlens[b], Lmax) : Lmax;
  const int nb = min(pl.S, chunks_of(L, C));
  const PartLayout::Row pr = pl.row_of_out(row);
  const float *lp = lse_part + pr.base;
  const float *op = o_part + pr.base * D + c0 + lane * CPL;
  const size_t o_step = (size_t)pr.stride * D;

  float M = FD_NEG_INF, W = 0.f, acc[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) acc[i] = 0.f;
  for (int s0 = wave; s0 < nb; s0 += MW * MB) {
    float ls[MB], ov[MB][CPL];
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      const int s = s0 + j * MW;
      const int sc = s < nb ? s : s0;
      ls[j] = s < nb ? lp[(size_t)sc * pr.stride] : FD_NEG_INF;
#pragma unroll
      for (int i = 0; i < CPL; ++i) ov[j][i] = op[(size_t)sc * o_step + i];
    }
    float mb = ls[0];
#pragma unroll
    for (int j = 1; j < MB; ++j) mb = fmaxf(mb, ls[j]);
    const float Mn = fmaxf(M, mb);
    if (Mn == FD_NEG_INF) continue;
    const float r = exp2_f((M - Mn) * kLog2e);
    W *= r;
#pragma unroll
    for (int i = 0; i < CPL; ++i) acc[i] *= r;
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      const float wt = exp2_f((ls[j] - Mn) * kLog2e);
      W += wt;
#pragma unroll
      for (int i = 0; i < CPL; ++i) acc[i] += wt * ov[j][i];
    }
    M = Mn;
  }
  if (lane == 0) {
    sm_M[wave] = M;
    sm_W[wave] = W;
  }
#pragma unroll
  for (int i = 0; i < CPL; ++i) sm_acc[wave][lane * CPL + i] = acc[i];
  __syncthreads();
  for (int d = threadIdx.x; d < COLS; d += blockDim.x) {
    float Mt = FD_NEG_INF;
#pragma unroll
    for (int w = 0; w < MW; ++w) Mt = fmaxf(Mt, sm_M[w]);
    float o = 0.f, ls_out = FD_NEG_INF;
    if (Mt != FD_NEG_INF) {
      float Wt = 0.f, a = 0.f;
#pragma unroll
      for (int w = 0; w < MW; ++w) {
        const float r = exp2_f((sm_M[w] - Mt) * kLog2e);
        Wt += r * sm_W[w];
        a += r * sm_acc[w][d];
      }
      o = a / Wt;
      ls_out = Mt + log2_f(Wt) * kLn2;
    }
    store_out<OutT>(out + (size_t)row * D + c0 + d, o);
    if (c0 + d == 0) lse[row] = ls_out;
  }
}

// Merge pass for chunk-major partials: per (sequence, KV head) group,
// gridDim.y workgroups of kGroupMergeThreads threads, each taking an equal
// share of the group's (row, 4 columns) items.  Each chunk's G * Tq rows
// are one contiguous block, so a workgroup reads its share of every block
// (a wavefront's load covers 1 KB of it, two rows' outputs at D = 128)
// where the row-wise pass reads each row's piece of every block; the
// group's chunks are split over as many thread slices as the threads
// allow, which meet in LDS (group_merge).  Spreading a group over several
// workgroups spreads a long sequence's partials over several CUs, whose
// loads then all fit in flight at once.  Group b * Hkv + g runs on the
// XCD that wrote it when B * Hkv and Hkv are multiples of 8, as in
// merge_row.
constexpr int kGroupMergeThreads = 256;
// Items per merge workgroup: one per thread of a quarter of it, so that
// each thread folds a quarter of the group's chunks.
constexpr int kGroupMergeItems = kGroupMergeThreads / 4;

template <int D, typename OutT>
__global__ __launch_bounds__(kGroupMergeThreads) void group_combine_kernel(
    const float *__restrict__ o_part, const float *__restrict__ lse_part,
    const int32_t *__restrict__ seqlens, PartLayout pl, int Lmax, int C,
    OutT *__restrict__ out, float *__restrict__ lse) {
  __shared__ __align__(16) float sm[6 * kGroupMergeThreads];
  Work w{};
  w.b = blockIdx.x / pl.Hkv;
  w.g = blockIdx.x - w.b * pl.Hkv;
  const int L = seqlens ? clamp_len(seqlens[w.b], Lmax) : Lmax;
  w.nb = min(pl.S, chunks_of(L, C));
  const int items = pl.G * pl.Tq * (D / 4);
  const int share = (items + gridDim.y - 1) / gridDim.y;
  const int it0 = blockIdx.y * share;
  const int it1 = min(items, it0 + share);
  if (it0 >= it1) return;
  group_merge<D, OutT>(w, pl, it0, it1, o_part, lse_part, out, lse, sm);
}

// ---------------------------------------------------------------------------
// Host-side dispatch.

// Chunk-major partials merged group-wise (1) or row-wise (0); a switch
// for measuring one against the other.
#ifndef FD_GROUP_MERGE
#define FD_GROUP_MERGE 1
#endif
constexpr bool kGroupMerge = FD_GROUP_MERGE != 0;

int mode_of(const Plan &p) {
  return !p.combine ? kModeDirect : (p.fused ? kModeFused : kModePartial);
}

template <typename T, int D, int NW>
hipError_t launch_valu(const Plan &p, const LaunchArgs &a, float sl2,
                       hipStream_t st) {
  const dim3 grid(p.grid), block(NW * 64);
  const T *q = static_cast<const T *>(a.q);
  const T *k = static_cast<const T *>(a.k);
  const T *v = static_cast<const T *>(a.v);
  T *out = static_cast<T *>(a.out);
  const int part = mode_of(p);
  int gt = 1;
  while (gt < p.G) gt <<= 1;
#define FD_VALU_CASE(GTV)                                                    \
  case GTV:                                                                  \
    hipLaunchKernelGGL((split_valu_kernel<T, D, NW, GTV>), grid, block, 0,   \
                       st, q, k, v, a.seqlens, p.B, p.Hq, p.Hkv, p.G,        \
                       p.kv_rep, p.Lmax, p.chunk, p.splits, sl2, part,       \
                       p.chunk_major, out, a.lse, a.o_part, a.lse_part,      \
                       a.tickets);                                           \
    break;
  switch (gt) {
    FD_VALU_CASE(1)
    FD_VALU_CASE(2)
    FD_VALU_CASE(4)
    default:
      if constexpr (sizeof(T) == 4) {
        if (gt == 8) {
          hipLaunchKernelGGL((split_valu_kernel<T, D, NW, 8>), grid, block, 0,
                             st, q, k, v, a.seqlens, p.B, p.Hq, p.Hkv, p.G,
                             p.kv_rep, p.Lmax, p.chunk, p.splits, sl2, part,
                             p.chunk_major, out, a.lse, a.o_part, a.lse_part,
                             a.tickets);
          break;
        }
        if (gt == 16) {
          hipLaunchKernelGGL((split_valu_kernel<T, D, 2, 16>), grid,
                             dim3(2 * 64), 0, st, q, k, v, a.seqlens, p.B,
                             p.Hq, p.Hkv, p.G, p.kv_rep, p.Lmax, p.chunk,
                             p.splits, sl2, part, p.chunk_major, out, a.lse,
                             a.o_part, a.lse_part, a.tickets);
          break;
        }
      }
      return hipErrorInvalidValue;
  }
#undef FD_VALU_CASE
  return hipSuccess;
}

template <int D, bool PAGED, bool CAUSAL, bool UNI, typename E>
hipError_t launch_mfma(const Plan &p, const LaunchArgs &a, float sl2,
                       hipStream_t st) {
  typedef typename E16<E>::out OutT;
  const float phi2 = a.unified_max * kLog2e;
  const dim3 grid(p.grid);
  const int part = mode_of(p);
  const uint16_t *q = static_cast<const uint16_t *>(a.q);
  const uint16_t *k = static_cast<const uint16_t *>(a.k);
  const uint16_t *v = static_cast<const uint16_t *>(a.v);
  OutT *out = static_cast<OutT *>(a.out);
#define FD_MFMA_CASE(NWV)                                                    \
  case NWV:                                                                  \
    if (p.fused)                                                             \
      hipLaunchKernelGGL(                                                    \
          (split_mfma_kernel<D, NWV, PAGED, CAUSAL, UNI, E, true>), grid,    \
          dim3(NWV * 64), 0, st, q, k, v, a.seqlens, a.paged, p.B, p.Hq,     \
          p.Hkv, p.kv_rep, p.G, p.Tq, p.Lmax, p.chunk, p.splits, sl2, phi2,  \
          part, p.direct, p.chunk_major, out, a.lse, a.o_part, a.lse_part,   \
          a.tickets);                                                        \
    else                                                                     \
      hipLaunchKernelGGL(                                                    \
          (split_mfma_kernel<D, NWV, PAGED, CAUSAL, UNI, E, false>), grid,   \
          dim3(NWV * 64), 0, st, q, k, v, a.seqlens, a.paged, p.B, p.Hq,     \
          p.Hkv, p.kv_rep, p.G, p.Tq, p.Lmax, p.chunk, p.splits, sl2, phi2,  \
          part, p.direct, p.chunk_major, out, a.lse, a.o_part, a.lse_part,   \
          a.tickets);                                                        \
    break;
  switch (p.waves) {
    FD_MFMA_CASE(2)
    FD_MFMA_CASE(4)
    FD_MFMA_CASE(8)
    default:
      return hipErrorInvalidValue;
  }
#undef FD_MFMA_CASE
  return hipSuccess;
}

template <int D, bool PAGED, bool CAUSAL>
hipError_t launch_mfma_f32(const Plan &p, const LaunchArgs &a, float sl2,
                           hipStream_t st) {
  if (p.waves != 4) return hipErrorInvalidValue;
  const float *q = static_cast<const float *>(a.q);
  const float *k = static_cast<const float *>(a.k);
  const float *v = static_cast<const float *>(a.v);
  float *out = static_cast<float *>(a.out);
  if (p.fused)
    hipLaunchKernelGGL((split_mfma_f32_kernel<D, 4, PAGED, CAUSAL, true>),
                       dim3(p.grid), dim3(4 * 64), 0, st, q, k, v, a.seqlens,
                       a.paged, p.B, p.Hq, p.Hkv, p.kv_rep, p.G, p.Tq, p.Lmax,
                       p.chunk, p.splits, sl2, mode_of(p), p.direct,
                       p.chunk_major, out, a.lse, a.o_part, a.lse_part,
                       a.tickets);
  else
    hipLaunchKernelGGL((split_mfma_f32_kernel<D, 4, PAGED, CAUSAL, false>),
                       dim3(p.grid), dim3(4 * 64), 0, st, q, k, v, a.seqlens,
                       a.paged, p.B, p.Hq, p.Hkv, p.kv_rep, p.G, p.Tq, p.Lmax,
                       p.chunk, p.splits, sl2, mode_of(p), p.direct,
                       p.chunk_major, out, a.lse, a.o_part, a.lse_part,
                       a.tickets);
  return hipSuccess;
}

template <int D>
hipError_t launch_mfma_f32_any(const Plan &p, const LaunchArgs &a, float sl2,
                               hipStream_t st) {
  const bool causal = p.Tq > 1;
  return p.paged ? (causal ? launch_mfma_f32<D, true, true>(p, a, sl2, st)
                           : launch_mfma_f32<D, true, false>(p, a, sl2, st))
                 : (causal ? launch_mfma_f32<D, false, true>(p, a, sl2, st)
                           : launch_mfma_f32<D, false, false>(p, a, sl2, st));
}

template <int D, typename E>
hipError_t launch_mfma_any(const Plan &p, const LaunchArgs &a, float sl2,
                           hipStream_t st) {
  const bool causal = p.Tq > 1;
  if (p.unified)  // the planner allows it for contiguous single-token calls
    return p.paged || causal
               ? hipErrorInvalidValue
               : launch_mfma<D, false, false, true, E>(p, a, sl2, st);
  return p.paged
             ? (causal ? launch_mfma<D, true, true, false, E>(p, a, sl2, st)
                       : launch_mfma<D, true, false, false, E>(p, a, sl2, st))
             : (causal
                    ? launch_mfma<D, false, true, false, E>(p, a, sl2, st)
                    : launch_mfma<D, false, false, false, E>(p, a, sl2, st));
}

template <typename E>
hipError_t launch_mfma_16(const Plan &p, const LaunchArgs &a, float sl2,
                          hipStream_t st) {
  return p.D == 256   ? launch_mfma_any<256, E>(p, a, sl2, st)
         : p.D == 128 ? launch_mfma_any<128, E>(p, a, sl2, st)
                      : launch_mfma_any<64, E>(p, a, sl2, st);
}

template <int D, typename OutT>
void launch_combine(const Plan &p, const LaunchArgs &a, hipStream_t st) {
  const int rows = p.B * p.Tq * p.Hq;
  const PartLayout pl{p.G, p.Tq, p.Hq, p.Hkv, p.splits, p.chunk_major};
  if (p.chunk_major && kGroupMerge) {
    const int items = p.G * p.Tq * (D / 4);
    const int split = (items + kGroupMergeItems - 1) / kGroupMergeItems;
    hipLaunchKernelGGL((group_combine_kernel<D, OutT>),
                       dim3(p.B * p.Hkv, split), dim3(kGroupMergeThreads), 0,
                       st, a.o_part, a.lse_part, a.seqlens, pl, p.Lmax,
                       p.chunk, static_cast<OutT *>(a.out), a.lse);
  }
  else if (rows < p.num_cus && p.splits <= 32)
    hipLaunchKernelGGL((combine_kernel<D, OutT, 1, 4, 8>), dim3(rows, D / 64),
                       dim3(4 * 64), 0, st, a.o_part, a.lse_part, a.seqlens,
                       pl, p.Lmax, p.chunk, static_cast<OutT *>(a.out),
                       a.lse);
  else if (rows < p.num_cus)
    hipLaunchKernelGGL((combine_kernel<D, OutT, 1, 8, 8>), dim3(rows, D / 64),
                       dim3(8 * 64), 0, st, a.o_part, a.lse_part, a.seqlens,
                       pl, p.Lmax, p.chunk, static_cast<OutT *>(a.out),
                       a.lse);
  else
    hipLaunchKernelGGL((combine_kernel<D, OutT, D / 64, 4, 16>), dim3(rows),
                       dim3(4 * 64), 0, st, a.o_part, a.lse_part, a.seqlens,
                       pl, p.Lmax, p.chunk, static_cast<OutT *>(a.out),
                       a.lse);
}

}  // namespace

int launch_decode(const Plan &p, const LaunchArgs &a) {
  hipStream_t st = static_cast<hipStream_t>(a.stream);
  const float sl2 = a.scale * kLog2e;
  hipError_t e = hipSuccess;
  if (!(a.phases & kPhaseChunks)) {
    // merge only
  } else if (p.variant == FD_VARIANT_MFMA && p.dtype == FD_F32) {
    // the planner keeps the unified maximum to bf16
    e = p.unified        ? hipErrorInvalidValue
        : p.D == 256 ? launch_mfma_f32_any<256>(p, a, sl2, st)
        : p.D == 128 ? launch_mfma_f32_any<128>(p, a, sl2, st)
                     : launch_mfma_f32_any<64>(p, a, sl2, st);
  } else if (p.variant == FD_VARIANT_MFMA) {
    e = p.dtype == FD_F16 ? launch_mfma_16<_Float16>(p, a, sl2, st)
                          : launch_mfma_16<__bf16>(p, a, sl2, st);
  } else if (p.paged || p.Tq != 1 || p.D > 128) {
    e = hipErrorInvalidValue;  // the planner sends these to the MFMA kernel
  } else if (p.dtype == FD_BF16) {
    e = p.D == 128 ? launch_valu<uint16_t, 128, 4>(p, a, sl2, st)
                   : launch_valu<uint16_t, 64, 4>(p, a, sl2, st);
  } else if (p.dtype == FD_F16) {
    e = p.D == 128 ? launch_valu<_Float16, 128, 4>(p, a, sl2, st)
                   : launch_valu<_Float16, 64, 4>(p, a, sl2, st);
  } else {
    e = p.D == 128 ? launch_valu<float, 128, 4>(p, a, sl2, st)
                   : launch_valu<float, 64, 4>(p, a, sl2, st);
  }
  if (e != hipSuccess) return (int)e;
  e = hipGetLastError();
  if (e != hipSuccess) return (int)e;
  if ((a.phases & kPhaseMerge) && p.combine && !p.fused) {
    if (p.dtype == FD_BF16) {
      if (p.D == 256)
        launch_combine<256, uint16_t>(p, a, st);
      else if (p.D == 128)
        launch_combine<128, uint16_t>(p, a, st);
      else
        launch_combine<64, uint16_t>(p, a, st);
    } else if (p.dtype == FD_F16) {
      if (p.D == 256)
        launch_combine<256, _Float16>(p, a, st);
      else if (p.D == 128)
        launch_combine<128, _Float16>(p, a, st);
      else
        launch_combine<64, _Float16>(p, a, st);
    } else {
      if (p.D == 256)
        launch_combine<256, float>(p, a, st);
      else if (p.D == 128)
        launch_combine<128, float>(p, a, st);
      else
        launch_combine<64, float>(p, a, st);
    }
    e = hipGetLastError();
  }
  return (int)e;
}

}  // namespace fd
