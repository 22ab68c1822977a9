// Grouped-query single-token decode attention over a KV cache, for gfx950 (MI355X).
//
// What it computes ("Add Pallas GPU decode attention in Maxtext inference", PR 1066,
// Description and Tests): for every sequence b and query head h (KV head g = h / G), the
// newest token's query attends to cache entries 0 .. len_b - 1 of KV head g:
// O = softmax(scale * q . k_j) v_j, LSE = ln sum_j exp(scale * q . k_j).
//
// The work is bandwidth bound (every cached byte is read once and used for G heads), so it
// runs on the vector ALUs, not MFMA:
//  * Split-K: workgroup (split s, kv head g, sequence b) owns keys [s*L_s, (s+1)*L_s) clipped
//    to len_b and all G query heads of g; it writes (max, sum, unnormalised output) partials.
//    Splits past len_b exit at once, so nothing beyond the valid length is ever loaded.
//  * Second pass: the partials of each (b, h) are merged with log-sum-exp weights.
//  * bf16, D = 128 or 64, G <= 8 (the fast path): every K and V load of the split is issued
//    before any arithmetic, so a workgroup keeps its whole split (2 x 64 KB at D = 128) in
//    flight; scores use v_dot2 on bf16 pairs with 4 lanes per key row and a DPP reduction.
//  * bf16, D = 128, G > 8: the products are a dense contraction (each byte feeds G heads) and run
//    on the matrix cores, in workgroups of up to 16 query heads.
//  * Other cases (fp32 caches, D = 64 with G > 8) use a simpler split kernel with the same
//    partial layout.
//  * The merge is a separate launch: merging inside the split kernel (last workgroup to
//    arrive) needs a device-scope release per workgroup, which on this part writes back the
//    whole L2 and costs far more than the second launch.
#include <mutex>

#include "common.h"

namespace cpattn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxG = 8;  // query heads processed together per pass over a split
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct DecParams {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* lengths;
  void* o;
  float* lse;
  float* ws;
  int B, Hq, Hkv, G, max_len, nsplit, split_len;
  float scale_log2;
};

template <typename T>
struct Vec16;  // 16 bytes of T, widened to float
template <>
struct Vec16<__bf16> {
  static constexpr int N = 8;
  __device__ static void load(const __bf16* p, float* out) {
    u32x4 raw = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(raw[i] << 16);
      out[2 * i + 1] = __uint_as_float(raw[i] & 0xffff0000u);
    }
  }
};
template <>
struct Vec16<float> {
  static constexpr int N = 4;
  __device__ static void load(const float* p, float* out) {
    f32x4 raw = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = raw[i];
  }
};

__device__ __forceinline__ float to_float(float x) { return x; }
__device__ __forceinline__ float to_float(__bf16 x) { return (float)x; }

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecParams p) {
  constexpr int DPL = Vec16<T>::N;   // dims per lane
  constexpr int LPR = D / DPL;       // lanes per key row
  constexpr int RPW = 64 / LPR;      // rows per wave step
  constexpr int SLOTS = kThreads / LPR;  // key slots in the workgroup
  static_assert(64 % LPR == 0, "row must fit a wavefront");

  __shared__ float s_score[kMaxG][kDecodeSplitLen];
  __shared__ float s_stat[2][kMaxG];
  __shared__ float s_red[kWaves][kMaxG][D];

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  int len = p.lengths[b];
  len = len < 0 ? 0 : (len > p.max_len ? p.max_len : len);
  const int k0 = split * p.split_len;
  if (k0 >= len) return;
  const int nk = min(p.split_len, len - k0);

  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int dc = lane % LPR;           // which 16-byte chunk of the row
  const int slot = tid / LPR;          // key slot

  const T* qg = static_cast<const T*>(p.q);
  const T* kslab = static_cast<const T*>(p.k) + ((int64_t)b * p.Hkv + g) * p.max_len * D;
  const T* vslab = static_cast<const T*>(p.v) + ((int64_t)b * p.Hkv + g) * p.max_len * D;

  for (int h0 = 0; h0 < p.G; h0 += kMaxG) {
    const int ng = min(kMaxG, p.G - h0);
    // query chunks of the heads in this pass
    float qv[kMaxG][DPL];
#pragma unroll
    for (int hh = 0; hh < kMaxG; ++hh) {
      if (hh < ng) {
        const T* qh = qg + ((int64_t)b * p.Hq + g * p.G + h0 + hh) * D + dc * DPL;
        Vec16<T>::load(qh, qv[hh]);
      }
    }

    // ---- scores: each row is spread over LPR lanes; butterfly sum inside the lane group
    for (int r0 = 0; r0 < nk; r0 += SLOTS) {
      const int kk = r0 + slot;
      float kv[DPL];
      if (kk < nk) {
        Vec16<T>::load(kslab + (int64_t)(k0 + kk) * D + dc * DPL, kv);
      } else {
#pragma unroll
        for (int i = 0; i < DPL; ++i) kv[i] = 0.f;
      }
#pragma unroll
      for (int hh = 0; hh < kMaxG; ++hh) {
        if (hh < ng) {
          float acc = 0.f;
#pragma unroll
          for (int i = 0; i < DPL; ++i) acc = __builtin_fmaf(qv[hh][i], kv[i], acc);
#pragma unroll
          for (int off = LPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
          if (dc == 0 && kk < nk) s_score[hh][kk] = acc * p.scale_log2;
        }
      }
    }
    __syncthreads();

    // ---- per-head max and sum over the split (one wave per head)
    for (int hh = wave; hh < ng; hh += kWaves) {
      float m = -INFINITY;
      for (int i = lane; i < nk; i += 64) m = fmaxf(m, s_score[hh][i]);
      for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
      float l = 0.f;
      for (int i = lane; i < nk; i += 64) {
        float e = __builtin_amdgcn_exp2f(s_score[hh][i] - m);
        s_score[hh][i] = e;
        l += e;
      }
      for (int off = 32; off >= 1; off >>= 1) l += __shfl_xor(l, off);
      if (lane == 0) {
        s_stat[0][hh] = m;
        s_stat[1][hh] = l;
      }
    }
    __syncthreads();

    // ---- unnormalised P V: key slots accumulate their own keys, then reduce over slots
    float acc[kMaxG][DPL];
#pragma unroll
    for (int hh = 0; hh < kMaxG; ++hh)
#pragma unroll
      for (int i = 0; i < DPL; ++i) acc[hh][i] = 0.f;
    for (int kk = slot; kk < nk; kk += SLOTS) {
      float vv[DPL];
      Vec16<T>::load(vslab + (int64_t)(k0 + kk) * D + dc * DPL, vv);
#pragma unroll
      for (int hh = 0; hh < kMaxG; ++hh) {
        if (hh < ng) {
          const float pw = s_score[hh][kk];
#pragma unroll
          for (int i = 0; i < DPL; ++i) acc[hh][i] = __builtin_fmaf(pw, vv[i], acc[hh][i]);
        }
      }
    }
    // reduce the RPW slots inside the wave (lanes dc, dc+LPR, ...)
#pragma unroll
    for (int hh = 0; hh < kMaxG; ++hh) {
      if (hh < ng) {
#pragma unroll
        for (int i = 0; i < DPL; ++i) {
          float x = acc[hh][i];
          for (int off = LPR; off < 64; off <<= 1) x += __shfl_xor(x, off);
          acc[hh][i] = x;
        }
      }
    }
    if (lane < LPR) {
#pragma unroll
      for (int hh = 0; hh < kMaxG; ++hh)
        if (hh < ng)
#pragma unroll
          for (int i = 0; i < DPL; ++i) s_red[wave][hh][dc * DPL + i] = acc[hh][i];
    }
    __syncthreads();
    // final sum over waves and write the partial (o[0..D), m, l) for each head
    for (int idx = tid; idx < ng * D; idx += kThreads) {
      const int hh = idx / D, d = idx % D;
      float x = 0.f;
#pragma unroll
      for (int wv = 0; wv < kWaves; ++wv) x += s_red[wv][hh][d];
      const int h = g * p.G + h0 + hh;
      float* part = p.ws + (((int64_t)b * p.Hq + h) * p.nsplit + split) * (D + 2);
      part[d] = x;
      if (d == 0) {
        part[D] = s_stat[0][hh];
        part[D + 1] = s_stat[1][hh];
      }
    }
    __syncthreads();
  }
}

// Block -> (sequence b, query head h) of the merge, on the XCD where the split kernel ran the
// splits of (b, kv head of h) (decode_xcd_item), so the partials may still be in that XCD's L2.
__device__ __forceinline__ bool merge_item(const DecParams& p, int& b, int& h) {
  int hg, g;
  if (!decode_xcd_item(blockIdx.x, p.G, p.Hkv, p.B, hg, g, b)) return false;
  h = g * p.G + hg;
  return true;
}

// Second pass: thread d of block (b, h) merges every split's partial of that (b, h). NS is the
// workspace's split count when it is small enough to unroll (0: a runtime loop). Unrolled, the
// loads of every split's partial are issued together with the load of the sequence's length, so
// no load waits on another; splits past the length are then left out by selection, never by
// arithmetic, so whatever an unwritten slot holds cannot reach the result.
template <typename T, int D, int NS>
__global__ __launch_bounds__(D) void decode_merge_kernel(DecParams p) {
  int b, h;
  if (!merge_item(p, b, h)) return;
  const int bh = b * p.Hq + h;
  const int d = threadIdx.x;
  const float* part = p.ws + (int64_t)bh * p.nsplit * (D + 2);
  float M = -INFINITY, L = 0.f, acc = 0.f;
  if constexpr (NS > 0) {
    static_assert(NS <= 64, "one lane per split");
    // lane t of each wave loads split min(t, NS-1)'s (max, sum) pair; the pairs are broadcast
    // from those lanes with v_readlane once they have arrived
    const int lane = d % 64;
    const float2 ml = *reinterpret_cast<const float2*>(part + min(lane, NS - 1) * (D + 2) + D);
    float o[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) o[s] = part[s * (D + 2) + d];
    int len = p.lengths[b];
    // every load above is in flight before the first wait: the empty asm uses each loaded
    // register, so no load can be sunk into a branch below it
#pragma unroll
    for (int s = 0; s < NS; ++s) asm volatile("" ::"v"(o[s]));
    asm volatile("" ::"v"(ml.x), "v"(ml.y), "s"(len));
    len = len < 0 ? 0 : (len > p.max_len ? p.max_len : len);
    const int nvalid = (len + p.split_len - 1) / p.split_len;
    float m[NS], l[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      m[s] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ml.x), s));
      l[s] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ml.y), s));
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) M = s < nvalid ? fmaxf(M, m[s]) : M;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const float w = __builtin_amdgcn_exp2f(m[s] - M);
      L = s < nvalid ? __builtin_fmaf(w, l[s], L) : L;
      acc = s < nvalid ? __builtin_fmaf(w, o[s], acc) : acc;
    }
  } else {
    int len = p.lengths[b];
    len = len < 0 ? 0 : (len > p.max_len ? p.max_len : len);
    const int nvalid = (len + p.split_len - 1) / p.split_len;
    for (int s = 0; s < nvalid; ++s) M = fmaxf(M, part[s * (D + 2) + D]);
    for (int s = 0; s < nvalid; ++s) {
      const float w = __builtin_amdgcn_exp2f(part[s * (D + 2) + D] - M);
      L = __builtin_fmaf(w, part[s * (D + 2) + D + 1], L);
      acc = __builtin_fmaf(w, part[s * (D + 2) + d], acc);
    }
  }
  // a sequence of length 0 has no key: output 0 and log-sum-exp ln 0 = -inf
  const bool empty = !(L > 0.f);
  T* out = static_cast<T*>(p.o) + (int64_t)bh * D;
  out[d] = empty ? (T)0.f : (T)(acc / L);
  if (p.lse && d == 0) p.lse[bh] = empty ? -INFINITY : (M + __builtin_amdgcn_logf(L)) * kLn2;
}

template <typename T, int D, int NS>
void launch_merge_ns(const DecParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((decode_merge_kernel<T, D, NS>), dim3(decode_xcd_blocks(p.G, p.Hkv, p.B)), dim3(D), 0, stream, p);
}

// The merge pass for the workspace's split count: unrolled up to 16 splits (a 4096-key cache at
// 256 keys per split), a runtime loop beyond.
template <typename T, int D>
void launch_merge(const DecParams& p, hipStream_t stream) {
  switch (p.nsplit) {
    case 1: launch_merge_ns<T, D, 1>(p, stream); break;
    case 2: launch_merge_ns<T, D, 2>(p, stream); break;
    case 3: launch_merge_ns<T, D, 3>(p, stream); break;
    case 4: launch_merge_ns<T, D, 4>(p, stream); break;
    case 5: launch_merge_ns<T, D, 5>(p, stream); break;
    case 6: launch_merge_ns<T, D, 6>(p, stream); break;
    case 7: launch_merge_ns<T, D, 7>(p, stream); break;
    case 8: launch_merge_ns<T, D, 8>(p, stream); break;
    case 9: launch_merge_ns<T, D, 9>(p, stream); break;
    case 10: launch_merge_ns<T, D, 10>(p, stream); break;
    case 11: launch_merge_ns<T, D, 11>(p, stream); break;
    case 12: launch_merge_ns<T, D, 12>(p, stream); break;
    case 13: launch_merge_ns<T, D, 13>(p, stream); break;
    case 14: launch_merge_ns<T, D, 14>(p, stream); break;
    case 15: launch_merge_ns<T, D, 15>(p, stream); break;
    case 16: launch_merge_ns<T, D, 16>(p, stream); break;
    default: launch_merge_ns<T, D, 0>(p, stream); break;
  }
}

// Merge of decode results computed over disjoint slices of every sequence's keys (the shards of
// a cache split along its length): block (b, h); O = sum_r w_r o_r / sum_r w_r and
// LSE = M + ln sum_r w_r with w_r = exp(lse_r - M), M = max_r lse_r. A part whose log-sum-exp
// is -inf (an empty slice) has weight 0 and its output is not read into the sum.
template <typename T>
__global__ __launch_bounds__(256) void decode_lse_merge_kernel(const T* __restrict__ o_parts,
                                                               const float* __restrict__ lse_parts, T* __restrict__ out,
                                                               float* __restrict__ lse_out, int R, int64_t BH, int D) {
  const int64_t bh = blockIdx.x;
  float M = -INFINITY;
  for (int r = 0; r < R; ++r) M = fmaxf(M, lse_parts[r * BH + bh]);
  const bool empty = M == -INFINITY;
  float L = 0.f;
  if (!empty)
    for (int r = 0; r < R; ++r) L += __builtin_amdgcn_exp2f((lse_parts[r * BH + bh] - M) * kLog2e);
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float acc = 0.f;
    if (!empty) {
      for (int r = 0; r < R; ++r) {
        const float lr = lse_parts[r * BH + bh];
        if (lr != -INFINITY) acc += __builtin_amdgcn_exp2f((lr - M) * kLog2e) * to_float(o_parts[(r * BH + bh) * D + d]);
      }
    }
    out[bh * D + d] = empty ? (T)0.f : (T)(acc / L);
  }
  if (lse_out && threadIdx.x == 0) lse_out[bh] = empty ? -INFINITY : M + __builtin_amdgcn_logf(L) * kLn2;
}

// The same merge for up to 8 parts and D <= 256 with one thread per dim: every part's
// log-sum-exp and output element are loaded before any arithmetic, so the block waits on one
// round of loads instead of one per dependent step. An empty part's output (whatever it holds)
// is dropped by a select, not multiplied by its zero weight.
template <typename T, int R>
__global__ __launch_bounds__(256) void decode_lse_merge_r_kernel(const T* __restrict__ o_parts,
                                                                 const float* __restrict__ lse_parts, T* __restrict__ out,
                                                                 float* __restrict__ lse_out, int64_t BH, int D) {
  const int64_t bh = blockIdx.x;
  const int d = threadIdx.x;
  const int dd = d < D ? d : D - 1;  // threads past the last dim load it again and store nothing
  float lr[R], ov[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    lr[r] = lse_parts[r * BH + bh];
    ov[r] = to_float(o_parts[(r * BH + bh) * D + dd]);
  }
  float M = -INFINITY;
#pragma unroll
  for (int r = 0; r < R; ++r) M = fmaxf(M, lr[r]);
  const bool empty = M == -INFINITY;
  float L = 0.f, acc = 0.f;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const bool live = lr[r] != -INFINITY;
    const float wr = __builtin_amdgcn_exp2f((lr[r] - M) * kLog2e);
    L += live ? wr : 0.f;
    acc += live ? wr * ov[r] : 0.f;
  }
  if (d < D) out[bh * D + d] = empty ? (T)0.f : (T)(acc / L);
  if (lse_out && d == 0) lse_out[bh] = empty ? -INFINITY : M + __builtin_amdgcn_logf(L) * kLn2;
}

template <typename T>
void launch_lse_merge(const DecodeMergeArgs& a, int64_t bh, hipStream_t stream) {
  const T* op = static_cast<const T*>(a.o_parts);
  T* o = static_cast<T*>(a.o);
  const int threads = a.d >= 256 ? 256 : ((a.d + 63) / 64) * 64;
  if (a.d <= 256 && a.parts >= 1 && a.parts <= 8) {
    switch (a.parts) {
#define CPA_MERGE_R(R)                                                                                          \
  case R:                                                                                                      \
    hipLaunchKernelGGL((decode_lse_merge_r_kernel<T, R>), dim3((unsigned)bh), dim3(threads), 0, stream, op,   \
                       a.lse_parts, o, a.lse, bh, a.d);                                                        \
    return;
      CPA_MERGE_R(1) CPA_MERGE_R(2) CPA_MERGE_R(3) CPA_MERGE_R(4) CPA_MERGE_R(5) CPA_MERGE_R(6) CPA_MERGE_R(7)
      CPA_MERGE_R(8)
#undef CPA_MERGE_R
    }
  }
  hipLaunchKernelGGL(decode_lse_merge_kernel<T>, dim3((unsigned)bh), dim3(threads), 0, stream, op, a.lse_parts, o,
                     a.lse, a.parts, bh, a.d);
}

// ------------------------------------------------------------------------------------------
// bf16 fast path: one workgroup of 512 threads per (split of 256 keys, kv head, sequence); a
// cache of at most 1024 keys takes 128-key splits instead, so that it still spreads over the
// part (the merge reads the split length from the parameters)
// ------------------------------------------------------------------------------------------
constexpr int kFastThreads = 512;
constexpr int kFastWaves = kFastThreads / 64;

// Reinterpret one 32-bit word as a bf16 pair. The word is taken as a scalar argument: applying
// __builtin_bit_cast to an ext-vector element directly (v[i], v.y) makes this clang read
// element 0 whatever the index.
__device__ __forceinline__ bf16x2 as_bf16x2(unsigned u) { return __builtin_bit_cast(bf16x2, u); }

__device__ __forceinline__ float dot8_bf16(const u32x4& a, const u32x4& b, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const unsigned ai = a[i], bi = b[i];
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(ai), as_bf16x2(bi), acc, false);
  }
  return acc;
}

__device__ __forceinline__ float dpp_quad_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_quad_xor2(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
}
template <int D, int G, int SL>
__global__ __launch_bounds__(kFastThreads, 6) void decode_bf16_split_kernel(DecParams p) {
  constexpr int KC = D / 32;              // 16-byte K chunks per lane (4 lanes per key row)
  constexpr int KROWS = kFastThreads / 4;  // key rows per K pass
  constexpr int KP = SL / KROWS;           // K passes
  constexpr int LPRV = D / 8;              // lanes per V row (one 16-byte chunk each)
  constexpr int VS = kFastThreads / LPRV;  // V row slots
  constexpr int VR = SL / VS;              // V rows per lane (consecutive pairs share a v_dot2)
  static_assert(SL % KROWS == 0 && SL % VS == 0 && VR % 2 == 0, "split / thread layout mismatch");
  // The P V reduction buffer shares its LDS with the scores, which are dead once the
  // probabilities are formed.
  static_assert(G <= kFastWaves, "one wave per head in the softmax pass");
  constexpr int kRedFloats = kFastWaves * G * D;
  constexpr int kScoreFloats = G * SL;

  __shared__ float s_sr[kRedFloats > kScoreFloats ? kRedFloats : kScoreFloats];
  float(*s_s)[SL] = reinterpret_cast<float(*)[SL]>(s_sr);           // scores, log2 units
  float(*s_red)[G][D] = reinterpret_cast<float(*)[G][D]>(s_sr);     // per-wave P V sums
  __shared__ __attribute__((aligned(16))) __bf16 s_pb[G][VS][VR];  // bf16 probabilities by V slot
  __shared__ __attribute__((aligned(16))) __bf16 s_q[G][D];
  __shared__ float s_m[G], s_l[G];

  int split, g, b;
  if (!decode_xcd_item(blockIdx.x, p.nsplit, p.Hkv, p.B, split, g, b)) return;
  int len = p.lengths[b];
  len = len < 0 ? 0 : (len > p.max_len ? p.max_len : len);
  const int k0 = split * SL;
  if (k0 >= len) return;
  const int nk = min(SL, len - k0);
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;

  const int64_t slab = ((int64_t)b * p.Hkv + g) * p.max_len * D;
  const __bf16* kb = static_cast<const __bf16*>(p.k) + slab + (int64_t)k0 * D;
  const __bf16* vb = static_cast<const __bf16*>(p.v) + slab + (int64_t)k0 * D;

  // ---- issue the query load, then every K and V load of the split, before any arithmetic.
  // The loads are unconditional (no branch around a load, so the compiler inserts no wait
  // between them): a row past the split's last valid key re-reads that last key, whose score
  // is then replaced by -inf, so its probability is exactly 0. In that order the query is
  // waited for first, K next and V last, so the scores start while V is still in flight.
  const __bf16* qg = static_cast<const __bf16*>(p.q) + ((int64_t)b * p.Hq + (int64_t)g * p.G) * D;
  static_assert(G * (D / 8) <= kFastThreads, "one 16-byte query chunk per thread");
  const int qi = min(tid, G * (D / 8) - 1);
  const u32x4 qraw = *reinterpret_cast<const u32x4*>(qg + (int64_t)(qi / (D / 8)) * D + (qi % (D / 8)) * 8);
  // K: a lane quad owns a key row and each load instruction of the quad reads one contiguous
  // 64-byte segment of it.
  const int kq = tid % 4;
  u32x4 kr[KP][KC];
#pragma unroll
  for (int ps = 0; ps < KP; ++ps) {
    const int row = min(ps * KROWS + tid / 4, nk - 1);
#pragma unroll
    for (int cc = 0; cc < KC; ++cc)
      kr[ps][cc] = *reinterpret_cast<const u32x4*>(kb + (int64_t)row * D + (cc * 4 + kq) * 8);
  }
  const int vc = tid % LPRV;
  const int vslot = tid / LPRV;
  u32x4 vr[VR];
#pragma unroll
  for (int i = 0; i < VR; ++i) {
    const int row = min(i * VS + vslot, nk - 1);
    vr[i] = *reinterpret_cast<const u32x4*>(vb + (int64_t)row * D + vc * 8);
  }

  // every load above is issued before the query's LDS store waits for its data
  __builtin_amdgcn_sched_barrier(0);
  // ---- the group's query vectors into LDS
  // (threads past the last chunk store that chunk again: the same bytes to the same address; an
  // unconditional store keeps the compiler from sinking the query load behind the K/V loads)
  *reinterpret_cast<u32x4*>(&s_q[qi / (D / 8)][(qi % (D / 8)) * 8]) = qraw;
  __syncthreads();

  // ---- scores (log2 units): 4 lanes per key row, DPP sum inside each lane quad
#pragma unroll
  for (int ps = 0; ps < KP; ++ps) {
    const int row = ps * KROWS + tid / 4;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      {
        float acc = 0.f;
#pragma unroll
        for (int cc = 0; cc < KC; ++cc)
          acc = dot8_bf16(kr[ps][cc], *reinterpret_cast<const u32x4*>(&s_q[h][(cc * 4 + kq) * 8]), acc);
        acc += dpp_quad_xor1(acc);
        acc += dpp_quad_xor2(acc);
        if (kq == 0) s_s[h][row] = row < nk ? acc * p.scale_log2 : -INFINITY;
        // keep the scheduler from hoisting every head's query reads (register pressure)
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  __syncthreads();

  // ---- per-head max / probabilities / sum over the split: one wave per head. Probabilities
  // are rounded to bf16 once; the sum adds the rounded values, and they are stored where the
  // P V step reads them (by V row slot, consecutive rows of a slot adjacent).
  if (wave < G) {
    const int h = wave;
    float x[SL / 64];
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < SL / 64; ++j) {
      x[j] = s_s[h][lane + 64 * j];
      m = fmaxf(m, x[j]);
    }
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    float l = 0.f;
#pragma unroll
    for (int j = 0; j < SL / 64; ++j) {
      const int row = lane + 64 * j;
      const __bf16 e = (__bf16)__builtin_amdgcn_exp2f(x[j] - m);
      s_pb[h][row % VS][row / VS] = e;
      l += (float)e;
    }
    for (int off = 32; off >= 1; off >>= 1) l += __shfl_xor(l, off);
    if (lane == 0) {
      s_m[h] = m;
      s_l[h] = l;
    }
  }
  __syncthreads();

  // ---- unnormalised P V: v_dot2 over pairs of this lane's rows (p pair . v pair per dim).
  // The (row a, row b) bf16 pairs of every dim are formed once; heads are then done one at a
  // time so only 8 accumulators are live.
  static_assert(LPRV == 16 || LPRV == 8, "the slot reduction below takes 16 or 8 lanes per V row");
  unsigned vp[VR / 2][8];
#pragma unroll
  for (int pi = 0; pi < VR / 2; ++pi) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const unsigned a = vr[2 * pi][j], c = vr[2 * pi + 1][j];
      vp[pi][2 * j] = __builtin_amdgcn_perm(c, a, 0x05040100u);      // dim 2j of rows (a, b)
      vp[pi][2 * j + 1] = __builtin_amdgcn_perm(c, a, 0x07060302u);  // dim 2j+1 of rows (a, b)
    }
  }
  // Sum over the row slots of the wave (4 of 16 lanes at D = 128, 8 of 8 lanes at D = 64) with
  // lane-swap "transpose" steps, each reducing two accumulators: after the 32-lane step the
  // lower half of register i holds dim 2i and the upper half dim 2i+1 (H = lane bit 5); after
  // the 16-lane step row R (lane bit 4) of register j holds dim 4j + 2R + H; at D = 64 a third
  // step between lanes 8 apart (S = lane bit 3) leaves dim 4S + 2R + H of the lane's chunk.
  const int hsel = ((lane >> 4) & 1) * 2 + (lane >> 5);  // 2R + H
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float a8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) a8[e] = 0.f;
#pragma unroll
    for (int pi = 0; pi < VR / 2; ++pi) {
      const unsigned pw = reinterpret_cast<const unsigned*>(&s_pb[h][vslot][0])[pi];
#pragma unroll
      for (int e = 0; e < 8; ++e) a8[e] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pw), as_bf16x2(vp[pi][e]), a8[e], false);
    }
    float hv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(a8[2 * i]), __float_as_uint(a8[2 * i + 1]), false,
                                                 false);
      hv[i] = __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
    }
    float h2[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      auto pr = __builtin_amdgcn_permlane16_swap(__float_as_uint(hv[2 * j]), __float_as_uint(hv[2 * j + 1]), false,
                                                 false);
      h2[j] = __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
    }
    if constexpr (LPRV == 16) {
#pragma unroll
      for (int j = 0; j < 2; ++j) s_red[wave][h][vc * 8 + 4 * j + hsel] = h2[j];
    } else {
      // lanes l and l ^ 8 (a 16-lane row rotated by 8): each keeps h2[S] and adds the other's
      const bool s_hi = (lane >> 3) & 1;
      const float send = s_hi ? h2[0] : h2[1], keep = s_hi ? h2[1] : h2[0];
      const float got = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(send), 0x128, 0xF, 0xF, true));
      s_red[wave][h][vc * 8 + 4 * (int)s_hi + hsel] = keep + got;
    }
  }
  __syncthreads();

  // ---- this split's partial: (o[0..D), max, sum) per head
  for (int idx = tid; idx < G * D; idx += kFastThreads) {
    const int h = idx / D, d = idx % D;
    float x = 0.f;
#pragma unroll
    for (int wv = 0; wv < kFastWaves; ++wv) x += s_red[wv][h][d];
    float* part = p.ws + (((int64_t)b * p.Hq + g * p.G + h) * p.nsplit + split) * (D + 2);
    part[d] = x;
    if (d == 0) {
      part[D] = s_m[h];
      part[D + 1] = s_l[h];
    }
  }
}

// ---- bf16, D = 128, G > 8: both products on the matrix cores ----
// With more than 8 query heads per kv head every cached byte feeds that many heads, and the
// products are a dense contraction the v_dot2 kernel can no longer hide under the reads (taking
// the heads in groups of at most 8 over the same registers, it ran 56 us at G = 12 and 64 us at
// G = 16 on the 24 x 8 x 2048 cache, against 39 us at G = 6 and 40 and 41 us here). There the
// two products run on v_mfma_f32_16x16x32_bf16, as in the int8 decode: workgroup = (block of up to 16 query heads, 256-key split, kv head, sequence), 4 waves
// of 64 keys. The head blocks of one split are dispatched next to each other on one XCD, so the
// second reads the split's K and V from that XCD's L2.
//  * S^T = K Q^T per 16-key block: lane (key col, group gq) holds dims 32 gq + 8 i .. + 7 of its
//    key row for k-step i (the same permutation in Q), 64 contiguous bytes per lane and block.
//  * O^T = V^T P^T per 32-key block and 16-dim block, P in registers as the B operand. The
//    wave's V rows reach LDS by direct-to-LDS copies with XOR-swizzled 16-byte chunks and come
//    back through the transposing read ds_read_b64_tr_b16 (a 16-lane group reads 4 rows x 16
//    dims; output lane j holds dim j of the 4 rows), two reads per MFMA.
//  * The max is taken over the whole workgroup, so the waves' partials add without rescaling;
//    the partial layout is the other split kernels', and the same merge finishes the call.
constexpr int kMfThreads = 256;
constexpr int kMfWaves = kMfThreads / 64;
constexpr int kMfHeads = 16;                                  // query heads per workgroup (MFMA N)
constexpr int kMfD = 128;
constexpr int kMfRowBytes = kMfD * 2;
constexpr int kMfOStride = kMfD + 4;                           // fp32 stride of the wave outputs
constexpr int kMfVBytes = kDecodeSplitLen * kMfRowBytes;       // 64 KB V tile
constexpr int kMfOBytes = kMfWaves * kMfHeads * kMfOStride * 4;
constexpr int kMfLdsBytes = kMfVBytes > kMfOBytes ? kMfVBytes : kMfOBytes;
static_assert(kDecodeSplitLen == kMfWaves * 64, "a wave owns 64 keys of the split");

// Slot of the V tile's 16-byte chunk c of row r: c ^ mf_swz(r). The 4 rows one 16-lane group
// reads in a transposed load (r & 3 = 0..3) land in 4 distinct 32-byte slots.
__device__ __forceinline__ int mf_swz(int r) { return (2 * (r & 3)) ^ (8 * ((r >> 2) & 1)); }

__global__ __launch_bounds__(kMfThreads) void decode_bf16_mfma_split_kernel(DecParams p, int nhb) {
  constexpr int SL = kDecodeSplitLen;
  constexpr int D = kMfD;
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  __shared__ __attribute__((aligned(16))) char s_v[kMfLdsBytes];  // V tile, then the wave outputs
  __shared__ float s_max[kMfWaves][kMfHeads];
  __shared__ float s_sum[kMfWaves][kMfHeads];

  int inner, g, b;  // the (b, g) pair's XCD, as in the merge that reads the partials
  if (!decode_xcd_item(blockIdx.x, p.nsplit * nhb, p.Hkv, p.B, inner, g, b)) return;
  const int hb = inner % nhb, split = inner / nhb;
  int len = p.lengths[b];
  len = len < 0 ? 0 : (len > p.max_len ? p.max_len : len);
  const int k0 = split * SL;
  if (k0 >= len) return;
  const int nk = min(SL, len - k0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, gq = lane >> 4;

  const int64_t row0 = ((int64_t)b * p.Hkv + g) * p.max_len + k0;  // cache row of the split's key 0
  const char* kt = reinterpret_cast<const char*>(static_cast<const __bf16*>(p.k) + row0 * D);
  const char* vt = reinterpret_cast<const char*>(static_cast<const __bf16*>(p.v) + row0 * D);

  // Every load of the split is issued before the first wait, V first (the V copies go straight
  // to LDS through inline asm, which the compiler does not count; loads return in order, so
  // each wait the compiler places for its own loads also covers them). No load sits in a
  // branch; rows past the valid length re-read the last valid row (finite, masked).
  // ---- V rows of this wave into LDS: copy u moves rows 64 wave + 4 u .. + 3 (1 KB); lane l
  // fills slot l & 15 of row l >> 4 with the chunk the swizzle puts there.
  const unsigned lds_v = (unsigned)(uintptr_t)s_v;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int r = wave * 64 + u * 4 + (lane >> 4);
    const int c = (lane & 15) ^ mf_swz(r);
    dma16_sv(vt, (unsigned)(min(r, nk - 1) * kMfRowBytes + c * 16), lds_v + (wave * 64 + u * 4) * kMfRowBytes);
  }
  // ---- K: key block kb of this wave, row col, bytes [64 gq, 64 gq + 64)
  u32x4 kr[4][4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const int row = min(wave * 64 + kb * 16 + col, nk - 1);
    const u32x4* src = reinterpret_cast<const u32x4*>(kt + (int64_t)row * kMfRowBytes + 64 * gq);
#pragma unroll
    for (int i = 0; i < 4; ++i) kr[kb][i] = src[i];
  }
  // ---- queries (B operand): head col of the block, dims 32 gq + 8 i .. + 7 for k-step i; a
  // column past the group's last head reads that head and is then zeroed
  const int hg = hb * kMfHeads + col;  // head within the group
  const bool hvalid = hg < p.G;
  bf16x8 qf[4];
  {
    const __bf16* qh = static_cast<const __bf16*>(p.q) + ((int64_t)b * p.Hq + (int64_t)g * p.G + min(hg, p.G - 1)) * D +
                       32 * gq;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 raw = *reinterpret_cast<const u32x4*>(qh + 8 * i);
      const u32x4 z = {0u, 0u, 0u, 0u};
      qf[i] = __builtin_bit_cast(bf16x8, hvalid ? raw : z);
    }
  }

  // ---- scores (log2 units): lane holds head col, keys 64 wave + 16 kb + 4 gq + j
  float x[4][4];
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[kb][i]), qf[i], acc, 0, 0, 0);
    const int key0 = wave * 64 + kb * 16 + 4 * gq;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[kb][j] = key0 + j < nk ? acc[j] * p.scale_log2 : -INFINITY;
      mx = fmaxf(mx, x[kb][j]);
    }
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  if (lane < 16) s_max[wave][lane] = mx;
  __syncthreads();
  float M = s_max[0][col];
#pragma unroll
  for (int w = 1; w < kMfWaves; ++w) M = fmaxf(M, s_max[w][col]);  // finite: key 0 is valid

  // ---- probabilities: rounded to bf16 once; the sum adds the rounded values
  float l = 0.f;
  __bf16 pv[4][4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      pv[kb][j] = (__bf16)__builtin_amdgcn_exp2f(x[kb][j] - M);
      l += (float)pv[kb][j];
    }
  }
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);

  // ---- O^T += V^T P^T. Group gq's transposed reads for key block t: lane 4e + q of the group
  // reads row 64 wave + 32 t + 4 gq + e (lo) or that + 16 (hi), dims 16 db + 4 q .. + 3; the 8
  // keys are those of pv[2t][0..3], pv[2t + 1][0..3] in that order.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's V copies have landed
  const int e = (lane & 15) >> 2, q4 = lane & 3;
  f32x4 oacc[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const bf16x8 pb8 = {pv[2 * t][0], pv[2 * t][1], pv[2 * t][2], pv[2 * t][3],
                        pv[2 * t + 1][0], pv[2 * t + 1][1], pv[2 * t + 1][2], pv[2 * t + 1][3]};
    const int rlo = wave * 64 + 32 * t + 4 * gq + e, rhi = rlo + 16;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const int c = 2 * db + (q4 >> 1), within = 8 * (q4 & 1);
      const char* alo = s_v + rlo * kMfRowBytes + ((c ^ mf_swz(rlo)) * 16) + within;
      const char* ahi = s_v + rhi * kMfRowBytes + ((c ^ mf_swz(rhi)) * 16) + within;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(alo));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(ahi));
      const i16x8 cat = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cat), pb8, oacc[db], 0, 0, 0);
    }
  }
  __syncthreads();  // every wave's transposed reads are done: the tile memory takes the outputs

  // ---- sum of the four waves' outputs: lane holds head col, dims 16 db + 4 gq + r
  float* s_o = reinterpret_cast<float*>(s_v);
  if (hvalid) {
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
      *reinterpret_cast<f32x4*>(&s_o[(wave * kMfHeads + col) * kMfOStride + 16 * db + 4 * gq]) = oacc[db];
  }
  if (lane < 16) s_sum[wave][lane] = l;
  __syncthreads();
  const int nh = min(kMfHeads, p.G - hb * kMfHeads);
  for (int idx = tid; idx < nh * D; idx += kMfThreads) {
    const int h = idx / D, d = idx % D;
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < kMfWaves; ++w) o += s_o[(w * kMfHeads + h) * kMfOStride + d];
    float* part = p.ws + (((int64_t)b * p.Hq + (int64_t)g * p.G + hb * kMfHeads + h) * p.nsplit + split) * (D + 2);
    part[d] = o;
    if (d == 0) {
      float m = s_max[0][h], s = s_sum[0][h];
#pragma unroll
      for (int w = 1; w < kMfWaves; ++w) m = fmaxf(m, s_max[w][h]);
#pragma unroll
      for (int w = 1; w < kMfWaves; ++w) s += s_sum[w][h];
      part[D] = m;
      part[D + 1] = s;
    }
  }
}

void launch_mfma_128(const DecParams& p, hipStream_t stream) {
  const int nhb = (p.G + kMfHeads - 1) / kMfHeads;
  hipLaunchKernelGGL(decode_bf16_mfma_split_kernel, dim3(decode_xcd_blocks(p.nsplit * nhb, p.Hkv, p.B)),
                     dim3(kMfThreads), 0, stream, p, nhb);
}

template <int D, int G>
void launch_fast(const DecParams& p, hipStream_t stream) {
  if (p.split_len == kDecodeShortSplitLen)
    hipLaunchKernelGGL((decode_bf16_split_kernel<D, G, kDecodeShortSplitLen>),
                       dim3(decode_xcd_blocks(p.nsplit, p.Hkv, p.B)), dim3(kFastThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_bf16_split_kernel<D, G, kDecodeSplitLen>), dim3(decode_xcd_blocks(p.nsplit, p.Hkv, p.B)),
                       dim3(kFastThreads), 0, stream, p);
}

bool launch_fast_128(const DecParams& p, hipStream_t stream) {
  switch (p.G) {
    case 1: launch_fast<128, 1>(p, stream); return true;
    case 2: launch_fast<128, 2>(p, stream); return true;
    case 3: launch_fast<128, 3>(p, stream); return true;
    case 4: launch_fast<128, 4>(p, stream); return true;
    case 5: launch_fast<128, 5>(p, stream); return true;
    case 6: launch_fast<128, 6>(p, stream); return true;
    case 7: launch_fast<128, 7>(p, stream); return true;
    case 8: launch_fast<128, 8>(p, stream); return true;
    default: return false;
  }
}

bool launch_fast_64(const DecParams& p, hipStream_t stream) {
  switch (p.G) {
    case 1: launch_fast<64, 1>(p, stream); return true;
    case 2: launch_fast<64, 2>(p, stream); return true;
    case 3: launch_fast<64, 3>(p, stream); return true;
    case 4: launch_fast<64, 4>(p, stream); return true;
    case 5: launch_fast<64, 5>(p, stream); return true;
    case 6: launch_fast<64, 6>(p, stream); return true;
    case 7: launch_fast<64, 7>(p, stream); return true;
    case 8: launch_fast<64, 8>(p, stream); return true;
    default: return false;
  }
}

template <typename T>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
  DecParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.lengths = a.lengths;
  p.o = a.o;
  p.lse = a.lse;
  p.ws = a.ws;
  p.B = a.batch;
  p.Hq = a.hq;
  p.Hkv = a.hkv;
  p.G = a.hq / a.hkv;
  p.max_len = a.max_len;
  p.nsplit = a.nsplit;
  p.split_len = a.split_len;
  p.scale_log2 = a.scale * kLog2e;
  if (p.B == 0 || p.Hq == 0) return hipSuccess;
  if constexpr (sizeof(T) == 2) {
    // the v_dot2 kernels: 128-key splits for a short cache, else the default 256
    DecParams pf = p;
    if (decode_short_cache(p.max_len)) {
      pf.split_len = kDecodeShortSplitLen;
      pf.nsplit = (p.max_len + kDecodeShortSplitLen - 1) / kDecodeShortSplitLen;
    }
    if (a.d == 128 && launch_fast_128(pf, stream)) {
      launch_merge<T, 128>(pf, stream);
      return hipGetLastError();
    }
    if (a.d == 128) {  // G > 8
      launch_mfma_128(p, stream);
      launch_merge<T, 128>(p, stream);
      return hipGetLastError();
    }
    if (a.d == 64 && launch_fast_64(pf, stream)) {
      launch_merge<T, 64>(pf, stream);
      return hipGetLastError();
    }
  }
  dim3 g1(p.nsplit, p.Hkv, p.B);
  if (a.d == 128) {
    hipLaunchKernelGGL((decode_split_kernel<T, 128>), g1, dim3(kThreads), 0, stream, p);
    launch_merge<T, 128>(p, stream);
  } else if (a.d == 64) {
    hipLaunchKernelGGL((decode_split_kernel<T, 64>), g1, dim3(kThreads), 0, stream, p);
    launch_merge<T, 64>(p, stream);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

// ------------------------------------------------------------------------------------------
// Device scratch of the allocation-free decode call
// ------------------------------------------------------------------------------------------
// gqa_decode_attention_noalloc keeps its split partials in this file-scope array instead of a
// caller workspace. Each GPU the library runs on holds its own copy until the process ends. In
// host code the name is only a host-side stand-in, never a device address: the address on the
// current GPU comes from hipGetSymbolAddress, taken once per device and kept below, and only
// that address is handed to the kernels.
static __device__ __align__(256) char scratch[kDecodeNoAllocScratchBytes];

hipError_t decode_noalloc_scratch(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream) { return launch_typed<__bf16>(a, stream); }
hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t stream) { return launch_typed<float>(a, stream); }

hipError_t launch_decode_split_merge(const int32_t* lengths, float* ws, void* o, float* lse, int batch, int hq,
                                     int hkv, int max_len, int d, bool bf16, hipStream_t stream) {
  if (batch == 0 || hq == 0) return hipSuccess;
  if (hkv <= 0 || hq % hkv != 0) return hipErrorInvalidValue;
  DecParams p{};
  p.lengths = lengths;
  p.ws = ws;
  p.o = o;
  p.lse = lse;
  p.B = batch;
  p.Hq = hq;
  p.Hkv = hkv;
  p.G = hq / hkv;
  p.max_len = max_len;
  p.nsplit = decode_nsplit(max_len);
  p.split_len = kDecodeSplitLen;
  if (d == 128) {
    if (bf16)
      launch_merge<__bf16, 128>(p, stream);
    else
      launch_merge<float, 128>(p, stream);
  } else if (d == 64) {
    if (bf16)
      launch_merge<__bf16, 64>(p, stream);
    else
      launch_merge<float, 64>(p, stream);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_merge(const DecodeMergeArgs& a, hipStream_t stream) {
  const int64_t bh = (int64_t)a.batch * a.hq;
  if (bh == 0) return hipSuccess;
  if (a.bf16)
    launch_lse_merge<__bf16>(a, bh, stream);
  else
    launch_lse_merge<float>(a, bh, stream);
  return hipGetLastError();
}

}  // namespace cpattn
