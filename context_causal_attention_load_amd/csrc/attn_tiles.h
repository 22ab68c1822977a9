// Tile-walk helpers shared by the attention forward and backward kernels (gfx950): work-item
// decomposition over (batch, kv head, row block, head slice), the rows' original positions,
// the visible-key tile cursor over the load-balanced chunks, the LDS chunk swizzle, and
// wave reductions. Internal to libcpattn.so.
#pragma once

#include "common.h"

namespace cpattn {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBK = 64;          // keys per KV tile
constexpr int kRowsPerWave = 32;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;  // log2 units: probabilities stay <= 2^8

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* qpos;
  void* o;
  float* lse;
  int B, S, Sq, Hq, Hkv, G, cp, c, rank;
  int hpw, wpr, bm, nrb, nhs, n_items, per_xcd;
  float scale_log2;
};

template <int CH>
__device__ __forceinline__ int swz(int row) {
  if constexpr (CH % 16 == 0) {
    return ((row & 3) << 2) | ((row >> 2) & 3);
  } else {
    return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
  }
}

__device__ __forceinline__ float wave_max32(float x) {
  // max with the lane 32 away (both halves end with the same value)
  auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
}

__device__ __forceinline__ float wave_sum32(float x) {
  auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
}

__device__ __forceinline__ int wave_min_i(int x) {
  for (int off = 32; off >= 1; off >>= 1) x = min(x, __shfl_xor(x, off));
  return x;
}
__device__ __forceinline__ int wave_max_i(int x) {
  for (int off = 32; off >= 1; off >>= 1) x = max(x, __shfl_xor(x, off));
  return x;
}


struct WorkItem {
  int b, g, head0, row_blk;
};

__device__ __forceinline__ bool decode_item(const FwdParams& p, WorkItem& w) {
  int bid = blockIdx.x;
  int xcd = bid % kNumXcd;
  int slot = bid / kNumXcd;
  int W = xcd * p.per_xcd + slot;
  if (W >= p.n_items) return false;
  int hs = W % p.nhs;
  int t = W / p.nhs;
  int rb_desc = t % p.nrb;
  t /= p.nrb;
  w.g = t % p.Hkv;
  w.b = t / p.Hkv;
  w.row_blk = p.nrb - 1 - rb_desc;  // heavy first: later rows hold later positions
  w.head0 = w.g * p.G + hs * p.hpw;
  return true;
}

// Shared prologue: the row positions of this lane and the workgroup's [qmin, qmax].
__device__ __forceinline__ void row_positions(const FwdParams& p, const WorkItem& w, int wave, int lane,
                                              int& my_row, int& my_pos, int& qmin, int& qmax,
                                              int* s_red) {
  int row0 = w.row_blk * p.bm + (wave % p.wpr) * kRowsPerWave;
  my_row = row0 + (lane & 31);
  bool valid = my_row < p.Sq;
  int pos = -1;
  if (valid) {
    if (p.qpos) {
      pos = p.qpos[my_row];
    } else {
      pos = (int)lb_src((int64_t)p.rank * 2 * p.c + my_row, p.c, p.cp);
    }
    pos = min(pos, p.S - 1);
  }
  my_pos = pos;
  int vmin = valid ? pos : 0x7fffffff;
  int vmax = valid ? pos : -1;
  vmin = wave_min_i(vmin);
  vmax = wave_max_i(vmax);
  if (lane == 0) {
    s_red[wave] = vmin;
    s_red[kWaves + wave] = vmax;
  }
  __syncthreads();
  qmin = 0x7fffffff;
  qmax = -1;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    qmin = min(qmin, s_red[i]);
    qmax = max(qmax, s_red[kWaves + i]);
  }
}

// Tile cursor over the visible keys: chunks 0..imax in original order, 64-key tiles inside.
struct TileCursor {
  int chunk, t0;
};

template <int BK = kBK>
__device__ __forceinline__ void next_tile(TileCursor& tc, int c, int qmax) {
  tc.t0 += BK;
  if (tc.t0 >= c || tc.chunk * c + tc.t0 > qmax) {
    tc.chunk += 1;
    tc.t0 = 0;
  }
}

inline int gcd_int(int a, int b) {
  while (b) {
    int t = a % b;
    a = b;
    b = t;
  }
  return a;
}

inline FwdParams make_params(const AttnArgs& a) {
  FwdParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.qpos = a.q_pos;
  p.o = a.o;
  p.lse = a.lse;
  p.B = a.batch;
  p.S = a.seq;
  p.Sq = a.sq;
  p.Hq = a.hq;
  p.Hkv = a.hkv;
  p.G = a.hq / a.hkv;
  p.cp = a.cp;
  p.c = a.seq / (2 * a.cp);
  p.rank = a.rank;
  p.hpw = gcd_int(p.G, kWaves);
  p.wpr = kWaves / p.hpw;
  p.bm = kRowsPerWave * p.wpr;
  p.nrb = (p.Sq + p.bm - 1) / p.bm;
  p.nhs = p.G / p.hpw;
  p.n_items = p.B * p.Hkv * p.nrb * p.nhs;
  p.per_xcd = (p.n_items + kNumXcd - 1) / kNumXcd;
  p.scale_log2 = a.scale * kLog2e;
  return p;
}

}  // namespace
}  // namespace cpattn
