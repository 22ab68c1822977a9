// Load-balance permutation kernels: a row gather (permute) and the inverse row scatter
// (unpermute) along the sequence axis, moving raw bytes. This is the token reorder of
// "Add context parallelism" (PR 1445, Description), done there with an XLA gather.
//
// HBM-bound copy: each row is moved with the widest vector (16/8/4/2/1 bytes) that the row
// size and both base pointers allow; a workgroup copies whole rows, so every load and store of
// a wavefront is contiguous within a row.
#include "common.h"

namespace cpattn {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

template <typename T>
struct PermuteParams {
  const char* src;
  char* dst;
  uint32_t outer, seq, c, cp, row_begin, row_count;
  uint64_t row_bytes;
  uint32_t epr;  // elements of T per row
  uint32_t nrows;  // outer * row_count
  bool scatter;
};

template <typename T>
__device__ inline void row_ptrs(const PermuteParams<T>& p, uint32_t R, const T*& s, T*& d) {
  uint32_t o = R / p.row_count;
  uint32_t i = R - o * p.row_count;
  uint32_t j = p.row_begin + i;
  uint32_t two_c = 2 * p.c;
  uint32_t r = j / two_c;
  uint32_t w = j - r * two_c;
  uint32_t pos = w < p.c ? r * p.c + w : (2 * p.cp - 1 - r) * p.c + (w - p.c);
  uint64_t win_row = (uint64_t)o * p.row_count + i;
  uint64_t nat_row = (uint64_t)o * p.seq + pos;
  if (!p.scatter) {
    s = reinterpret_cast<const T*>(p.src + nat_row * p.row_bytes);
    d = reinterpret_cast<T*>(p.dst + win_row * p.row_bytes);
  } else {
    s = reinterpret_cast<const T*>(p.src + win_row * p.row_bytes);
    d = reinterpret_cast<T*>(p.dst + nat_row * p.row_bytes);
  }
}

// Rows of at least kThreads elements: the workgroup walks its rows one at a time.
template <typename T>
__global__ __launch_bounds__(kThreads) void permute_long_rows(PermuteParams<T> p) {
  for (uint32_t R = blockIdx.x; R < p.nrows; R += gridDim.x) {
    const T* s;
    T* d;
    row_ptrs(p, R, s, d);
    uint32_t e = threadIdx.x;
    for (; e + (kUnroll - 1) * kThreads < p.epr; e += kUnroll * kThreads) {
      T v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(s + e + u * kThreads);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) __builtin_nontemporal_store(v[u], d + e + u * kThreads);
    }
    for (; e < p.epr; e += kThreads) __builtin_nontemporal_store(__builtin_nontemporal_load(s + e), d + e);
  }
}

// Short rows: each thread owns one element slot of one row; a workgroup covers
// kThreads / epr rows per step.
template <typename T>
__global__ __launch_bounds__(kThreads) void permute_short_rows(PermuteParams<T> p) {
  uint32_t rpi = kThreads / p.epr;
  uint32_t sub = threadIdx.x / p.epr;
  uint32_t e = threadIdx.x - sub * p.epr;
  if (sub >= rpi) return;
  for (uint32_t R = blockIdx.x * rpi + sub; R < p.nrows; R += gridDim.x * rpi) {
    const T* s;
    T* d;
    row_ptrs(p, R, s, d);
    d[e] = s[e];
  }
}

template <typename T>
hipError_t launch_typed(const void* src, void* dst, int64_t outer, int64_t seq, int64_t row_bytes,
                        int64_t cp, int64_t row_begin, int64_t row_count, bool scatter,
                        hipStream_t stream) {
  PermuteParams<T> p;
  p.src = static_cast<const char*>(src);
  p.dst = static_cast<char*>(dst);
  p.outer = (uint32_t)outer;
  p.seq = (uint32_t)seq;
  p.cp = (uint32_t)cp;
  p.c = (uint32_t)(seq / (2 * cp));
  p.row_begin = (uint32_t)row_begin;
  p.row_count = (uint32_t)row_count;
  p.row_bytes = (uint64_t)row_bytes;
  p.epr = (uint32_t)(row_bytes / (int64_t)sizeof(T));
  p.nrows = (uint32_t)(outer * row_count);
  p.scatter = scatter;
  if (p.epr >= (uint32_t)kThreads) {
    uint32_t grid = p.nrows < 65536u ? p.nrows : 65536u;
    hipLaunchKernelGGL(permute_long_rows<T>, dim3(grid), dim3(kThreads), 0, stream, p);
  } else {
    uint32_t rpi = kThreads / p.epr;
    uint64_t need = (p.nrows + rpi - 1) / rpi;
    uint32_t grid = need < 65536u ? (uint32_t)need : 65536u;
    hipLaunchKernelGGL(permute_short_rows<T>, dim3(grid), dim3(kThreads), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_permute(const void* src, void* dst, int64_t outer, int64_t seq, int64_t row_bytes,
                          int64_t cp, int64_t row_begin, int64_t row_count, bool scatter,
                          hipStream_t stream) {
  uintptr_t align = (uintptr_t)src | (uintptr_t)dst | (uintptr_t)row_bytes;
  if (align % 16 == 0)
    return launch_typed<u32x4>(src, dst, outer, seq, row_bytes, cp, row_begin, row_count, scatter, stream);
  if (align % 8 == 0)
    return launch_typed<u32x2>(src, dst, outer, seq, row_bytes, cp, row_begin, row_count, scatter, stream);
  if (align % 4 == 0)
    return launch_typed<uint32_t>(src, dst, outer, seq, row_bytes, cp, row_begin, row_count, scatter, stream);
  if (align % 2 == 0)
    return launch_typed<uint16_t>(src, dst, outer, seq, row_bytes, cp, row_begin, row_count, scatter, stream);
  return launch_typed<uint8_t>(src, dst, outer, seq, row_bytes, cp, row_begin, row_count, scatter, stream);
}

}  // namespace cpattn
