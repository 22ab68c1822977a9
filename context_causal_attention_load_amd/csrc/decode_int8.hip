// Grouped-query decode attention over an int8 KV cache, and the cache quantizer, for gfx950.
//
// What it computes ("rename context to context_autoregressive", PR 1453, Description: the
// decode benchmark runs with the KV cache quantized to int8; the page gives no formula, and the
// reading taken is symmetric absmax with one float32 scale per cached row, i.e. per (sequence,
// kv head, position)): the decode attention of decode.hip with K and V taken as code * scale.
// The quantizer writes such a cache from bf16 or fp32 rows: amax = max |x|, scale = amax / 127,
// code = round-half-even(x / scale), both divisions correctly rounded in float32.
//
// Design. An int8 cache halves the bytes of a bf16 one, so if the products ran on v_dot2 (as in
// the bf16 decode) the vector ALUs, not HBM, would set the time. Both products therefore run on
// the matrix cores with v_mfma_f32_16x16x32_bf16 (int8 values are exact in bf16):
//  * Workgroup = (split of 256 keys, kv head x block of up to 16 query heads, sequence); its 4
//    waves own 64 keys each. Splits past the sequence's length exit at once.
//  * S^T = K Q^T per 16-key block: the A operand is 16 key rows x 32 dims. The dims of a k-step
//    are permuted (lane group gq, k-step i -> dims 32gq + 8i .. +7, the same in Q), so each lane
//    reads one contiguous 32-byte slice of a key row for all 4 k-steps.
//  * Products times (row K scale x softmax scale x log2 e) give log2-unit scores; the max is
//    taken over the whole workgroup, so the four waves' partials add without rescaling.
//    Probabilities exp2(s - max) are rounded to bf16 once and summed; the V scale of the key is
//    folded into the probability (one more bf16 rounding) before the PV product.
//  * O^T = V^T P^T per 32-key block and 16-dim block: P stays in registers as the B operand; the
//    output layout of the S^T products already gives each lane 8 keys of one head. The wave's V
//    rows are copied to LDS by direct-to-LDS loads with XOR-swizzled 16-byte chunks and read
//    back with ds_read_tr8_b64, which hands each lane 8 rows of one column. The rows a lane
//    group reads are chosen to be exactly the 8 keys its P fragment holds.
//  * The waves' outputs are summed in LDS into one split partial (o[128], max, sum; log2 units),
//    the layout of decode.hip's split kernels, and decode.hip's second pass merges the splits.
#include "common.h"

namespace cpattn {
namespace {

constexpr int kI8Threads = 256;
constexpr int kI8Waves = kI8Threads / 64;
constexpr int kHeadBlock = 16;  // query heads per workgroup (MFMA N)
constexpr int kI8D = 128;       // head dim of the int8 path
constexpr int kOStride = kI8D + 4;  // fp32 row stride of the wave outputs in LDS (padding)
constexpr int kVTileBytes = kDecodeSplitLen * kI8D;
constexpr int kOBytes = kI8Waves * kHeadBlock * kOStride * 4;
constexpr int kLdsBytes = kVTileBytes > kOBytes ? kVTileBytes : kOBytes;
static_assert(kDecodeSplitLen == kI8Waves * 64, "a wave owns 64 keys of the split");

typedef int i32x2 __attribute__((ext_vector_type(2)));

struct I8Params {
  const __bf16* q;
  const int8_t* k;
  const int8_t* v;
  const float* ks;
  const float* vs;
  const int32_t* lengths;
  float* ws;
  int B, Hq, Hkv, G, nhb, max_len, nsplit;
  float scale_log2;
};

// 8 int8 values (two dwords, lowest byte first) to bf16; exact.
__device__ __forceinline__ bf16x8 i8x8_to_bf16(unsigned lo, unsigned hi) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = (__bf16)(float)(int)(signed char)(lo >> (8 * i));
    r[4 + i] = (__bf16)(float)(int)(signed char)(hi >> (8 * i));
  }
  return r;
}

// Slot of the V tile's 16-byte chunk c of row r is c ^ swz(r). The 8 rows one 16-lane group
// reads in a transposed load have distinct swz values, so its 16 lanes hit distinct banks.
__device__ __forceinline__ int swz(int r) { return (r & 3) | ((r >> 2) & 4); }

__global__ __launch_bounds__(kI8Threads) void decode_i8_split_kernel(I8Params p) {
  constexpr int SL = kDecodeSplitLen;
  constexpr int D = kI8D;
  __shared__ __attribute__((aligned(16))) char s_v[kLdsBytes];  // V tile, then the wave outputs
  __shared__ __attribute__((aligned(16))) float s_ks[SL];
  __shared__ __attribute__((aligned(16))) float s_vs[SL];
  __shared__ float s_max[kI8Waves][kHeadBlock];
  __shared__ float s_sum[kI8Waves][kHeadBlock];

  int inner, g, b;  // the (b, g) pair's XCD, as in the merge that reads the partials
  if (!decode_xcd_item(blockIdx.x, p.nsplit * p.nhb, p.Hkv, p.B, inner, g, b)) return;
  const int split = inner % p.nsplit, hb = inner / p.nsplit;
  int len = p.lengths[b];
  len = len < 0 ? 0 : (len > p.max_len ? p.max_len : len);
  const int k0 = split * SL;
  if (k0 >= len) return;
  const int nk = min(SL, len - k0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, gq = lane >> 4;

  const int64_t row0 = ((int64_t)b * p.Hkv + g) * p.max_len + k0;  // cache row of the split's key 0
  const int8_t* kt = p.k + row0 * D;
  const char* vt = reinterpret_cast<const char*>(p.v + row0 * D);

  // Every load of the split is issued before the first wait, V first. The V copies go straight
  // to LDS through inline asm, which the compiler does not count: issued ahead of every load it
  // does count, and with loads returning in order, each wait the compiler places for its own
  // loads also covers them. No load sits in a branch (a branch around a load lets the compiler
  // place a wait inside it).
  // ---- V rows of this wave into LDS: copy u moves rows 64 wave + 8u .. + 7 (1 KB); lane l
  // fills slot l & 7 of row l >> 3 with the chunk that the swizzle puts there.
  const unsigned lds_v = (unsigned)(uintptr_t)s_v;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int r = wave * 64 + u * 8 + (lane >> 3);
    const int c = (lane & 7) ^ swz(r);
    dma16_sv(vt, (unsigned)(min(r, nk - 1) * D + c * 16), lds_v + (wave * 64 + u * 8) * D);
  }
  // ---- K: key block kb of this wave, row col, bytes [32 gq, 32 gq + 32). Rows past the valid
  // length re-read the last valid row (finite; their scores are masked).
  u32x4 kr[4][2];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const int row = min(wave * 64 + kb * 16 + col, nk - 1);
    const u32x4* src = reinterpret_cast<const u32x4*>(kt + (int64_t)row * D + 32 * gq);
    kr[kb][0] = src[0];
    kr[kb][1] = src[1];
  }
  // ---- queries (B operand): head col of the block, dims 32 gq + 8 i .. + 7 for k-step i. A
  // column past the group's last head reads that head and is then zeroed.
  const int hg = hb * kHeadBlock + col;  // head within the group
  const bool hvalid = hg < p.G;
  bf16x8 qf[4];
  {
    const __bf16* qh = p.q + ((int64_t)b * p.Hq + (int64_t)g * p.G + min(hg, p.G - 1)) * D + 32 * gq;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 raw = *reinterpret_cast<const u32x4*>(qh + 8 * i);
      const u32x4 z = {0u, 0u, 0u, 0u};
      qf[i] = __builtin_bit_cast(bf16x8, hvalid ? raw : z);
    }
  }
  // ---- row scales of the split
  {
    const int row = min(tid, nk - 1);
    s_ks[tid] = p.ks[row0 + row];
    s_vs[tid] = p.vs[row0 + row];
  }
  __syncthreads();  // row scales visible

  // ---- scores (log2 units): lane holds head col, keys 64 wave + 16 kb + 4 gq + j
  float x[4][4];
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const unsigned lo = kr[kb][i >> 1][2 * (i & 1)], hi = kr[kb][i >> 1][2 * (i & 1) + 1];
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(i8x8_to_bf16(lo, hi), qf[i], acc, 0, 0, 0);
    }
    const int key0 = wave * 64 + kb * 16 + 4 * gq;
    const f32x4 ksc = *reinterpret_cast<const f32x4*>(&s_ks[key0]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float sv = acc[j] * (ksc[j] * p.scale_log2);
      x[kb][j] = key0 + j < nk ? sv : -INFINITY;
      mx = fmaxf(mx, x[kb][j]);
    }
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  if (lane < 16) s_max[wave][lane] = mx;
  __syncthreads();
  float M = s_max[0][col];
#pragma unroll
  for (int w = 1; w < kI8Waves; ++w) M = fmaxf(M, s_max[w][col]);  // finite: key 0 is valid

  // ---- probabilities: bf16 once, summed; V scale folded in for the PV product
  float l = 0.f;
  __bf16 pv[4][4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const f32x4 vsc = *reinterpret_cast<const f32x4*>(&s_vs[wave * 64 + kb * 16 + 4 * gq]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const __bf16 pb = (__bf16)__builtin_amdgcn_exp2f(x[kb][j] - M);
      l += (float)pb;
      pv[kb][j] = (__bf16)((float)pb * vsc[j]);
    }
  }
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);

  // ---- O^T += V^T P^T. Transposed read of lane (e = col >> 1, half = col & 1) in group gq:
  // row 64 wave + 32 t + 16 (e >> 2) + 4 gq + (e & 3), bytes 8 half .. + 7 of the 16-dim block;
  // the group's 8 rows are then the keys of pv[2t][0..3], pv[2t+1][0..3] in that order. For
  // these rows swz(row) == e.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's V copies have landed
  const int e = col >> 1;
  f32x4 oacc[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const bf16x8 pb8 = {pv[2 * t][0], pv[2 * t][1], pv[2 * t][2], pv[2 * t][3],
                        pv[2 * t + 1][0], pv[2 * t + 1][1], pv[2 * t + 1][2], pv[2 * t + 1][3]};
    const int row = wave * 64 + 32 * t + 16 * (e >> 2) + 4 * gq + (e & 3);
    const char* rb = s_v + row * D + 8 * (col & 1);
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const i32x2 raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (__attribute__((address_space(3))) i32x2*)(rb + ((db ^ e) * 16)));
      oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(i8x8_to_bf16((unsigned)raw[0], (unsigned)raw[1]), pb8,
                                                         oacc[db], 0, 0, 0);
    }
  }
  __syncthreads();  // every wave's transposed reads are done: the tile memory takes the outputs

  // ---- sum of the four waves' outputs: lane holds head col, dims 16 db + 4 gq + r
  float* s_o = reinterpret_cast<float*>(s_v);
  if (hg < p.G) {
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
      *reinterpret_cast<f32x4*>(&s_o[(wave * kHeadBlock + col) * kOStride + 16 * db + 4 * gq]) = oacc[db];
  }
  if (lane < 16) s_sum[wave][lane] = l;
  __syncthreads();
  const int nh = min(kHeadBlock, p.G - hb * kHeadBlock);
  for (int idx = tid; idx < nh * D; idx += kI8Threads) {
    const int h = idx / D, d = idx % D;
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < kI8Waves; ++w) o += s_o[(w * kHeadBlock + h) * kOStride + d];
    float* part = p.ws + (((int64_t)b * p.Hq + (int64_t)g * p.G + hb * kHeadBlock + h) * p.nsplit + split) * (D + 2);
    part[d] = o;
    if (d == 0) {
      float m = s_max[0][h], s = s_sum[0][h];
#pragma unroll
      for (int w = 1; w < kI8Waves; ++w) m = fmaxf(m, s_max[w][h]);
#pragma unroll
      for (int w = 1; w < kI8Waves; ++w) s += s_sum[w][h];
      part[D] = m;
      part[D + 1] = s;
    }
  }
}

// One wave per row: amax by a wave reduction, then codes. Plain float division (correctly
// rounded in HIP unless fast-math is asked for) and rintf (ties to even).
template <typename T>
__global__ __launch_bounds__(256) void kv_quantize_kernel(const T* __restrict__ x, int8_t* __restrict__ codes,
                                                          float* __restrict__ scales, int64_t rows, int D) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const T* xr = x + row * D;
  float amax = 0.f;
  for (int d = lane; d < D; d += 64) amax = fmaxf(amax, fabsf((float)xr[d]));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const float s = amax / 127.0f;
  int8_t* cr = codes + row * D;
  for (int d = lane; d < D; d += 64) {
    const float c = s > 0.f ? rintf((float)xr[d] / s) : 0.f;
    cr[d] = (int8_t)(int)fminf(fmaxf(c, -127.f), 127.f);
  }
  if (lane == 0) scales[row] = s;
}

}  // namespace

hipError_t launch_decode_int8(const DecodeInt8Args& a, hipStream_t stream) {
  if (a.batch == 0 || a.hq == 0) return hipSuccess;
  I8Params p;
  p.q = static_cast<const __bf16*>(a.q);
  p.k = a.k;
  p.v = a.v;
  p.ks = a.k_scale;
  p.vs = a.v_scale;
  p.lengths = a.lengths;
  p.ws = a.ws;
  p.B = a.batch;
  p.Hq = a.hq;
  p.Hkv = a.hkv;
  p.G = a.hq / a.hkv;
  p.nhb = (p.G + kHeadBlock - 1) / kHeadBlock;
  p.max_len = a.max_len;
  p.nsplit = decode_nsplit(a.max_len);
  p.scale_log2 = a.scale * 1.4426950408889634f;
  hipLaunchKernelGGL(decode_i8_split_kernel, dim3(decode_xcd_blocks(p.nsplit * p.nhb, p.Hkv, p.B)), dim3(kI8Threads), 0,
                     stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_decode_split_merge(a.lengths, a.ws, a.o, a.lse, a.batch, a.hq, a.hkv, a.max_len, kI8D, true, stream);
}

hipError_t launch_kv_quantize(const void* x, int8_t* codes, float* scales, int64_t rows, int d, bool bf16,
                              hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (bf16)
    hipLaunchKernelGGL(kv_quantize_kernel<__bf16>, grid, dim3(256), 0, stream, static_cast<const __bf16*>(x), codes,
                       scales, rows, d);
  else
    hipLaunchKernelGGL(kv_quantize_kernel<float>, grid, dim3(256), 0, stream, static_cast<const float*>(x), codes,
                       scales, rows, d);
  return hipGetLastError();
}

}  // namespace cpattn
