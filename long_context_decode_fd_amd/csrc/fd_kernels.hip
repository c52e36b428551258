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
//   * one workgroup per (sequence b, KV head g, chunk s); it serves all
//     G = Hq / Hkv query heads of KV head g, so each K/V byte leaves HBM
//     once;
//   * bf16: each 64-lane wavefront streams 32-key tiles straight from HBM
//     into registers in the operand layout of v_mfma_f32_16x16x32_bf16 and
//     computes S^T = K Q^T (16 keys x 16 padded heads per MFMA) and
//     O^T += V^T P^T; the accumulator's column is the query head, so each
//     lane rescales only its own head's accumulators;
//   * the per-head running max is shared across the four 16-lane groups of
//     a wavefront with two cross-lane shuffles per tile; exponentials run
//     as exp2 with log2(e) folded into the scale;
//   * the wavefronts of a workgroup take interleaved tiles and merge their
//     (max, sum, accumulator) states through LDS at the end, so a chunk
//     writes one partial per query row;
//   * fp32 (and bf16 tiny groups) run a vector-ALU kernel with 16-byte
//     loads per lane and shuffle reductions of the dot products.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fd_internal.h"

namespace fd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

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

// ---------------------------------------------------------------------------
// Work decomposition shared by the per-chunk kernels and the merge kernel.

struct Work {
  int b, g, s;
  int lo, hi;  // keys [lo, hi) of slab (b, g); lo == hi only when L_b == 0
  bool valid;
};

// Chunks of sequence b: n_b = max(1, ceil(L_b / C)); a sequence of length 0
// keeps one empty chunk so that its output row is still written.
__device__ __forceinline__ int chunks_of(int L, int C) {
  return max(1, (L + C - 1) / C);
}

// Workgroup id -> (b, g, s).  Ids run over the chunks that exist, sequence
// by sequence, chunk-major, KV head fastest: id = (prefix_b + s) * Hkv + g.
// With per-sequence lengths the prefix over sequences is a wavefront scan
// of the seqlens (every wavefront does it; it is a few dozen instructions).
__device__ Work find_work(int bid, const int32_t *__restrict__ seqlens, int B,
                          int Hkv, int Lmax, int C) {
  Work w;
  w.valid = false;
  w.b = w.g = w.s = w.lo = w.hi = 0;
  if (seqlens == nullptr) {
    const int S = (Lmax + C - 1) / C;
    const int per_b = S * Hkv;
    const int b = bid / per_b;
    if (b >= B) return w;
    const int r = bid - b * per_b;
    w.b = b;
    w.s = r / Hkv;
    w.g = r - w.s * Hkv;
    w.lo = w.s * C;
    w.hi = min(w.lo + C, Lmax);
    w.valid = true;
    return w;
  }
  const int lane = threadIdx.x & 63;
  int base = 0;
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int b = b0 + lane;
    int L = 0, blocks = 0;
    if (b < B) {
      L = clamp_len(seqlens[b], Lmax);
      blocks = chunks_of(L, C) * Hkv;
    }
    int incl = blocks;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(incl, off, 64);
      if (lane >= off) incl += t;
    }
    const int total = __shfl(incl, 63, 64);
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
      w.hi = max(w.lo, min(w.lo + C, Lb));
      w.valid = true;
      return w;
    }
    base += total;
  }
  return w;
}

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

// ---------------------------------------------------------------------------
// Merge of the workgroup's softmax states and the chunk's store.
//
// Slot sl holds, for query row h of the group: running max m (log2 units of
// the scaled score), running sum l, and the unnormalised accumulator
// O[h][0..D).  The merged row is M = max m, weight 2^(m - M) per slot; the
// chunk's output is sum(w O) / sum(w l) and its log-sum-exp (natural log)
// is ln2 * (M + log2 sum(w l)).  With no keys at all: out 0, lse -inf.
template <int D, typename OutT>
__device__ void merge_and_store(const float *sm_m, const float *sm_l,
                                const float *sm_o, int nslot, int rows,
                                int G, const Work &w, int Hq, int S,
                                bool partial, OutT *__restrict__ out,
                                float *__restrict__ lse,
                                float *__restrict__ o_part,
                                float *__restrict__ lse_part) {
  for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
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
    const size_t hq = (size_t)w.b * Hq + (size_t)w.g * G + h;
    if (!partial) {
      store_out<OutT>(out + hq * D + d, o);
      if (d == 0) lse[hq] = ls;
    } else {
      const size_t row = hq * S + w.s;
      o_part[row * D + d] = o;
      if (d == 0) lse_part[row] = ls;
    }
  }
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

template <int D, bool TAIL>
__device__ __forceinline__ void mfma_tile(
    const uint16_t *__restrict__ kslab, const uint16_t *__restrict__ vslab,
    int k0, int valid, int n16, int q4, const bf16x8 (&qop)[D / 32],
    float scale_log2, floatx4 (&acc)[D / 16], float &m, float &l) {
  constexpr int KK = D / 32;
  constexpr int VW = D / 16;
  typedef typename VecOf<VW>::type VT;

  uint4 kr[2][KK];
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    int r = sub * 16 + n16;
    if (TAIL) r = min(r, valid - 1);
    const uint16_t *p = kslab + (size_t)(k0 + r) * D + q4 * 8;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      kr[sub][kk] = *reinterpret_cast<const uint4 *>(p + kk * 32);
  }
  VT vr[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int r = (i >> 2) * 16 + q4 * 4 + (i & 3);
    if (TAIL) r = min(r, valid - 1);
    vr[i] = *reinterpret_cast<const VT *>(vslab + (size_t)(k0 + r) * D +
                                          n16 * VW);
  }

  floatx4 sc[2];
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    sc[sub] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      sc[sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8, kr[sub][kk]), qop[kk], sc[sub], 0, 0, 0);
  }

  float s[8];
#pragma unroll
  for (int sub = 0; sub < 2; ++sub)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float x = sc[sub][j] * scale_log2;
      if (TAIL && sub * 16 + q4 * 4 + j >= valid) x = FD_NEG_INF;
      s[sub * 4 + j] = x;
    }
  float mt = s[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) mt = fmaxf(mt, s[i]);
  mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
  mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
  const float mn = fmaxf(m, mt);
  const float mref = mn == FD_NEG_INF ? 0.f : mn;
  const float alpha = exp2_f(m - mref);

  // P enters the matrix cores as an exact-to-2^-17 pair of bf16 operands
  // (hi = bf16(p), lo = bf16(p - hi)); the running sum uses fp32 p.
  bf16x8 p_hi, p_lo;
  float psum = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float p = exp2_f(s[i] - mref);
    const __bf16 hi = (__bf16)p;
    p_hi[i] = hi;
    p_lo[i] = (__bf16)(p - (float)hi);
    psum += p;
  }
  l = l * alpha + psum;
  m = mn;
#pragma unroll
  for (int e = 0; e < VW; ++e) acc[e] *= alpha;

  if (TAIL) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if ((i >> 2) * 16 + q4 * 4 + (i & 3) >= valid) vr[i] = VT{};
  }
  bf16x8 vt[VW];
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
    vt[e] = __builtin_bit_cast(bf16x8, t);
  }
#pragma unroll
  for (int e = 0; e < VW; ++e)
    acc[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt[e], p_hi, acc[e], 0,
                                                     0, 0);
#pragma unroll
  for (int e = 0; e < VW; ++e)
    acc[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt[e], p_lo, acc[e], 0,
                                                     0, 0);
}

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void split_mfma_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kc,
    const uint16_t *__restrict__ vc, const int32_t *__restrict__ seqlens,
    int B, int Hq, int Hkv, int G, int Lmax, int C, int S, float scale_log2,
    int partial, uint16_t *__restrict__ out, float *__restrict__ lse,
    float *__restrict__ o_part, float *__restrict__ lse_part) {
  constexpr int KK = D / 32;
  constexpr int VW = D / 16;
  __shared__ float sm_m[NW * 16];
  __shared__ float sm_l[NW * 16];
  __shared__ float sm_o[NW * 16 * (D + 1)];

  const Work w = find_work(blockIdx.x, seqlens, B, Hkv, Lmax, C);
  if (!w.valid) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n16 = lane & 15, q4 = lane >> 4;

  bf16x8 qop[KK];
  {
    const bool live = n16 < G;
    const uint16_t *qr = q + ((size_t)w.b * Hq + (size_t)w.g * G +
                              (live ? n16 : 0)) * D + q4 * 8;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      uint4 t = live ? *reinterpret_cast<const uint4 *>(qr + kk * 32)
                     : make_uint4(0, 0, 0, 0);
      qop[kk] = __builtin_bit_cast(bf16x8, t);
    }
  }
  const size_t slab = ((size_t)w.b * Hkv + w.g) * (size_t)Lmax * D;
  const uint16_t *kslab = kc + slab;
  const uint16_t *vslab = vc + slab;

  floatx4 acc[VW];
#pragma unroll
  for (int e = 0; e < VW; ++e) acc[e] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m = FD_NEG_INF, l = 0.f;

  const int ntiles = (w.hi - w.lo + kKeyTile - 1) / kKeyTile;
  for (int t = wave; t < ntiles; t += NW) {
    const int k0 = w.lo + t * kKeyTile;
    const int valid = min(kKeyTile, w.hi - k0);
    if (valid == kKeyTile)
      mfma_tile<D, false>(kslab, vslab, k0, valid, n16, q4, qop, scale_log2,
                          acc, m, l);
    else
      mfma_tile<D, true>(kslab, vslab, k0, valid, n16, q4, qop, scale_log2,
                         acc, m, l);
  }

  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (n16 < G) {
    if (q4 == 0) {
      sm_m[wave * 16 + n16] = m;
      sm_l[wave * 16 + n16] = l;
    }
    float *o = sm_o + (wave * 16 + n16) * (D + 1);
#pragma unroll
    for (int e = 0; e < VW; ++e)
#pragma unroll
      for (int j = 0; j < 4; ++j) o[(q4 * 4 + j) * VW + e] = acc[e][j];
  }
  __syncthreads();
  merge_and_store<D, uint16_t>(sm_m, sm_l, sm_o, NW, 16, G, w, Hq, S,
                               partial != 0, out, lse, o_part, lse_part);
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
    const float4 t = *reinterpret_cast<const float4 *>(p);
    x[0] = t.x;
    x[1] = t.y;
    x[2] = t.z;
    x[3] = t.w;
  }
};
template <>
struct Elem<uint16_t> {
  static constexpr int kPerLane = 8;
  __device__ static void load(const uint16_t *p, float (&x)[8]) {
    const uint4 t = *reinterpret_cast<const uint4 *>(p);
    const uint32_t d[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __builtin_bit_cast(float, d[i] << 16);
      x[2 * i + 1] = __builtin_bit_cast(float, d[i] & 0xFFFF0000u);
    }
  }
};

template <typename T, int D, int NW, int GT>
__global__ __launch_bounds__(NW * 64) void split_valu_kernel(
    const T *__restrict__ q, const T *__restrict__ kc, const T *__restrict__ vc,
    const int32_t *__restrict__ seqlens, int B, int Hq, int Hkv, int G,
    int Lmax, int C, int S, float scale_log2, int partial,
    T *__restrict__ out, float *__restrict__ lse, float *__restrict__ o_part,
    float *__restrict__ lse_part) {
  constexpr int EPL = Elem<T>::kPerLane;
  constexpr int LPR = D / EPL;
  constexpr int RPW = 64 / LPR;
  constexpr int U = 4;
  constexpr int TK = U * RPW;
  constexpr int NSLOT = NW * RPW;
  __shared__ float sm_m[NSLOT * GT];
  __shared__ float sm_l[NSLOT * GT];
  __shared__ float sm_o[NSLOT * GT * (D + 1)];

  const Work w = find_work(blockIdx.x, seqlens, B, Hkv, Lmax, C);
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
  const size_t slab = ((size_t)w.b * Hkv + w.g) * (size_t)Lmax * D;
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
  merge_and_store<D, T>(sm_m, sm_l, sm_o, NSLOT, GT, G, w, Hq, S,
                        partial != 0, out, lse, o_part, lse_part);
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of the chunks: one wavefront per (b, query head).
// M = max_s lse_s, w_s = exp(lse_s - M), out = sum w_s o_s / sum w_s,
// lse = M + ln sum w_s.  Summation order is fixed (s ascending), so a given
// chunking always gives the same bits.
template <int D, typename OutT>
__global__ __launch_bounds__(64) void combine_kernel(
    const float *__restrict__ o_part, const float *__restrict__ lse_part,
    const int32_t *__restrict__ seqlens, int Hq, int Lmax, int C, int S,
    OutT *__restrict__ out, float *__restrict__ lse) {
  constexpr int DPL = D / 64;
  const int row = blockIdx.x;
  const int b = row / Hq;
  const int lane = threadIdx.x;
  const int L = seqlens ? clamp_len(seqlens[b], Lmax) : Lmax;
  const int nb = min(S, chunks_of(L, C));
  const float *lp = lse_part + (size_t)row * S;
  const float *op = o_part + (size_t)row * S * D + lane * DPL;

  float M = FD_NEG_INF;
  for (int s = lane; s < nb; s += 64) M = fmaxf(M, lp[s]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));

  float acc[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc[i] = 0.f;
  float W = 0.f;
  if (M != FD_NEG_INF) {
    const float Ml2 = M * kLog2e;
#pragma unroll 4
    for (int s = 0; s < nb; ++s) {
      const float wt = exp2_f(lp[s] * kLog2e - Ml2);
      W += wt;
#pragma unroll
      for (int i = 0; i < DPL; ++i) acc[i] += wt * op[(size_t)s * D + i];
    }
  }
  OutT *o = out + (size_t)row * D + lane * DPL;
  if (M == FD_NEG_INF) {
#pragma unroll
    for (int i = 0; i < DPL; ++i) store_out<OutT>(o + i, 0.f);
    if (lane == 0) lse[row] = FD_NEG_INF;
  } else {
#pragma unroll
    for (int i = 0; i < DPL; ++i) store_out<OutT>(o + i, acc[i] / W);
    if (lane == 0) lse[row] = M + log2_f(W) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// Host-side dispatch.

template <typename T, int D, int NW>
hipError_t launch_valu(const Plan &p, const LaunchArgs &a, float sl2,
                       hipStream_t st) {
  const dim3 grid(p.grid), block(NW * 64);
  const T *q = static_cast<const T *>(a.q);
  const T *k = static_cast<const T *>(a.k);
  const T *v = static_cast<const T *>(a.v);
  T *out = static_cast<T *>(a.out);
  const int part = p.combine ? 1 : 0;
  int gt = 1;
  while (gt < p.G) gt <<= 1;
#define FD_VALU_CASE(GTV)                                                    \
  case GTV:                                                                  \
    hipLaunchKernelGGL((split_valu_kernel<T, D, NW, GTV>), grid, block, 0,   \
                       st, q, k, v, a.seqlens, p.B, p.Hq, p.Hkv, p.G, p.Lmax, \
                       p.chunk, p.splits, sl2, part, out, a.lse, a.o_part,    \
                       a.lse_part);                                          \
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
                             p.Lmax, p.chunk, p.splits, sl2, part, out, a.lse,
                             a.o_part, a.lse_part);
          break;
        }
        if (gt == 16) {
          hipLaunchKernelGGL((split_valu_kernel<T, D, 2, 16>), grid,
                             dim3(2 * 64), 0, st, q, k, v, a.seqlens, p.B,
                             p.Hq, p.Hkv, p.G, p.Lmax, p.chunk, p.splits, sl2,
                             part, out, a.lse, a.o_part, a.lse_part);
          break;
        }
      }
      return hipErrorInvalidValue;
  }
#undef FD_VALU_CASE
  return hipSuccess;
}

template <int D>
hipError_t launch_mfma(const Plan &p, const LaunchArgs &a, float sl2,
                       hipStream_t st) {
  const dim3 grid(p.grid);
  const int part = p.combine ? 1 : 0;
  const uint16_t *q = static_cast<const uint16_t *>(a.q);
  const uint16_t *k = static_cast<const uint16_t *>(a.k);
  const uint16_t *v = static_cast<const uint16_t *>(a.v);
  uint16_t *out = static_cast<uint16_t *>(a.out);
#define FD_MFMA_CASE(NWV)                                                    \
  case NWV:                                                                  \
    hipLaunchKernelGGL((split_mfma_kernel<D, NWV>), grid, dim3(NWV * 64), 0, \
                       st, q, k, v, a.seqlens, p.B, p.Hq, p.Hkv, p.G, p.Lmax, \
                       p.chunk, p.splits, sl2, part, out, a.lse, a.o_part,    \
                       a.lse_part);                                          \
    break;
  switch (p.waves) {
    FD_MFMA_CASE(1)
    FD_MFMA_CASE(2)
    FD_MFMA_CASE(4)
    FD_MFMA_CASE(8)
    default:
      return hipErrorInvalidValue;
  }
#undef FD_MFMA_CASE
  return hipSuccess;
}

template <int D, typename OutT>
void launch_combine(const Plan &p, const LaunchArgs &a, hipStream_t st) {
  hipLaunchKernelGGL((combine_kernel<D, OutT>), dim3(p.B * p.Hq), dim3(64), 0,
                     st, a.o_part, a.lse_part, a.seqlens, p.Hq, p.Lmax,
                     p.chunk, p.splits, static_cast<OutT *>(a.out), a.lse);
}

}  // namespace

int launch_decode(const Plan &p, const LaunchArgs &a) {
  hipStream_t st = static_cast<hipStream_t>(a.stream);
  const float sl2 = a.scale * kLog2e;
  hipError_t e;
  if (p.variant == FD_VARIANT_MFMA) {
    e = p.D == 128 ? launch_mfma<128>(p, a, sl2, st)
                   : launch_mfma<64>(p, a, sl2, st);
  } else if (p.dtype == FD_BF16) {
    e = p.D == 128 ? launch_valu<uint16_t, 128, 4>(p, a, sl2, st)
                   : launch_valu<uint16_t, 64, 4>(p, a, sl2, st);
  } else {
    e = p.D == 128 ? launch_valu<float, 128, 4>(p, a, sl2, st)
                   : launch_valu<float, 64, 4>(p, a, sl2, st);
  }
  if (e != hipSuccess) return (int)e;
  e = hipGetLastError();
  if (e != hipSuccess) return (int)e;
  if (p.combine) {
    if (p.dtype == FD_BF16) {
      if (p.D == 128)
        launch_combine<128, uint16_t>(p, a, st);
      else
        launch_combine<64, uint16_t>(p, a, st);
    } else {
      if (p.D == 128)
        launch_combine<128, float>(p, a, st);
      else
        launch_combine<64, float>(p, a, st);
    }
    e = hipGetLastError();
  }
  return (int)e;
}

}  // namespace fd
