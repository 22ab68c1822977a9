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
//  * A second kernel merges the partials of each (b, h) with log-sum-exp weights.
//  * Loads are 16 bytes per lane and a key row is spread over D*elt/16 lanes, so each
//    wavefront load instruction reads whole contiguous rows of the (b, g) cache slab.
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

template <typename T, int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(DecParams p) {
  const int bh = blockIdx.x;
  const int b = bh / p.Hq;
  const int d = threadIdx.x;
  int len = p.lengths[b];
  len = len < 0 ? 0 : (len > p.max_len ? p.max_len : len);
  const int nvalid = (len + p.split_len - 1) / p.split_len;
  const float* part = p.ws + (int64_t)bh * p.nsplit * (D + 2);
  float M = -INFINITY;
  for (int s = 0; s < nvalid; ++s) M = fmaxf(M, part[s * (D + 2) + D]);
  float L = 0.f, acc = 0.f;
  for (int s = 0; s < nvalid; ++s) {
    const float w = __builtin_amdgcn_exp2f(part[s * (D + 2) + D] - M);
    L = __builtin_fmaf(w, part[s * (D + 2) + D + 1], L);
    acc = __builtin_fmaf(w, part[s * (D + 2) + d], acc);
  }
  T* o = static_cast<T*>(p.o) + (int64_t)bh * D;
  o[d] = (T)(acc / L);
  if (p.lse && d == 0) p.lse[bh] = (M + __builtin_amdgcn_logf(L)) * kLn2;
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
  dim3 g1(p.nsplit, p.Hkv, p.B);
  if (a.d == 128) {
    hipLaunchKernelGGL((decode_split_kernel<T, 128>), g1, dim3(kThreads), 0, stream, p);
    hipLaunchKernelGGL((decode_merge_kernel<T, 128>), dim3(p.B * p.Hq), dim3(128), 0, stream, p);
  } else if (a.d == 64) {
    hipLaunchKernelGGL((decode_split_kernel<T, 64>), g1, dim3(kThreads), 0, stream, p);
    hipLaunchKernelGGL((decode_merge_kernel<T, 64>), dim3(p.B * p.Hq), dim3(64), 0, stream, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream) { return launch_typed<__bf16>(a, stream); }
hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t stream) { return launch_typed<float>(a, stream); }

}  // namespace cpattn
