// Tile-walk helpers shared by the attention forward and backward kernels (gfx950): work-item
// decomposition over (batch, kv head, row block, head slice), the rows' original positions,
// the visible-key tile cursor over the load-balanced chunks, the LDS chunk swizzle, and
// wave reductions. Internal to libcpattn.so.
#pragma once

#include <algorithm>

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

// Key-range split of heavy row blocks (small grids only; the forward and the backward's dQ): a
// plan lists, for each (batch, kv head, head slice) unit, its pieces heaviest first; a piece is a
// range of a row block's visible key tiles. Row blocks cut into several pieces write partials to
// the caller's workspace and a merge kernel combines them.
constexpr int kSplitMaxPieces = 96;
constexpr int kSplitMaxRb = 64;

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
  // split plan (n_pieces == 0: one item per row block, no partials); piece i of a cut row block
  // owns its visible tiles [i tau, min((i + 1) tau, T))
  int n_pieces, n_slots, tau;
  float* part_o;   // [unit, slot, bm rows, hpw heads, Dv] unnormalised outputs
  float* part_ml;  // [unit, slot, hpw heads, bm rows, 2] running max (log2 units) and row sum
  unsigned char piece_rb[kSplitMaxPieces];   // row block of each piece
  unsigned char piece_idx[kSplitMaxPieces];  // index of the piece within its row block
  unsigned char piece_cnt[kSplitMaxPieces];  // pieces of that row block
  signed char piece_slot[kSplitMaxPieces];   // partial slot, -1 when the row block is not split
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
  int unit;   // (b, g, head slice) index
  int piece;  // piece of the split plan, -1 without one
};

__device__ __forceinline__ bool decode_item(const FwdParams& p, WorkItem& w) {
  int bid = blockIdx.x;
  int xcd = bid % kNumXcd;
  int slot = bid / kNumXcd;
  int hs, k, bg;
  if (p.n_pieces) {
    // split plan: each XCD owns per_xcd (batch, kv head) pairs and runs their pieces heaviest
    // first across all of them (piece index outermost)
    hs = slot % p.nhs;
    int t = slot / p.nhs;
    const int pl = t % p.per_xcd;
    k = t / p.per_xcd;
    bg = xcd * p.per_xcd + pl;
    if (k >= p.n_pieces || bg >= p.B * p.Hkv) return false;
    w.piece = k;  // pieces are listed heaviest first
    w.row_blk = p.piece_rb[k];
  } else {
    int W = xcd * p.per_xcd + slot;
    if (W >= p.n_items) return false;
    hs = W % p.nhs;
    int t = W / p.nhs;
    k = t % p.nrb;
    bg = t / p.nrb;
    w.piece = -1;
    w.row_blk = p.nrb - 1 - k;  // heavy first: later rows hold later positions
  }
  w.g = bg % p.Hkv;
  w.b = bg / p.Hkv;
  w.unit = bg * p.nhs + hs;
  w.head0 = w.g * p.G + hs * p.hpw;
  return true;
}

// Key tiles a row block visits (chunks 0..imax in original order, BK-key tiles, the last chunk
// cut at the block's largest position qmax): the same count on the host and the device.
__host__ __device__ inline int visible_tiles(int qmax, int c, int cp, int bk) {
  const int imax = qmax / c < 2 * cp - 1 ? qmax / c : 2 * cp - 1;
  const int tpc = (c + bk - 1) / bk;
  const int in_last = (qmax - imax * c + 1 + bk - 1) / bk;
  return imax * tpc + (in_last < tpc ? in_last : tpc);
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
  p.n_pieces = 0;
  p.n_slots = 0;
  p.tau = 0;
  p.part_o = nullptr;
  p.part_ml = nullptr;
  return p;
}

// ---- split plan (host)
// A rank's time is that of its busiest compute unit. With at least two work items per CU the
// heavy-first order evens the CUs out; below that (the 8192-token shape at cp = 4 has one 256-row
// block per CU, and its heaviest block sees twice the keys of the average one) the heaviest row
// block sets the time. There the visible key tiles of the heavy row blocks are cut into pieces,
// each piece a work item.
constexpr int kSplitBelowItems = 512;   // plan a split only for grids with fewer work items
constexpr int kSplitTargetItems = 256;  // pieces no smaller than the grid's tiles per CU

struct SplitPlan {
  int n_pieces = 0, n_slots = 0, n_split = 0, tau = 0;
  unsigned char rb[kSplitMaxPieces], idx[kSplitMaxPieces], cnt[kSplitMaxPieces];
  signed char slot[kSplitMaxPieces];
  unsigned char srb[kSplitMaxRb], sslot[kSplitMaxRb], scnt[kSplitMaxRb];  // cut row blocks
};

// Plans the split of the rank's own shard (positions from cp and rank: the plan needs them on
// the host) for a kernel that walks bk-key tiles. tau, the tiles per CU if the rank's work were
// spread evenly (no less than min_tiles), bounds a work item: a row block of T > tau tiles is cut
// into pieces of tau tiles and a remainder, and the pieces are dispatched largest first, so the
// remainders and the small row blocks fill the CUs that free first and every CU ends near tau.
// False when the grid has enough work items, the plan would not fit its tables, or no row block
// is cut.
inline bool plan_split_tiles(const FwdParams& p, int bk, int min_tiles, SplitPlan& sp) {
  if (p.n_items >= kSplitBelowItems || p.nrb > kSplitMaxRb) return false;
  int T[kSplitMaxRb];
  int64_t total = 0;
  for (int rb = 0; rb < p.nrb; ++rb) {
    const int last_row = std::min(p.Sq, (rb + 1) * p.bm) - 1;
    const int qmax = (int)std::min<int64_t>(lb_src((int64_t)p.rank * 2 * p.c + last_row, p.c, p.cp), p.S - 1);
    T[rb] = visible_tiles(qmax, p.c, p.cp, bk);
    total += T[rb];
  }
  const int64_t units = (int64_t)p.B * p.Hkv * p.nhs;
  const int tau = (int)std::max<int64_t>(min_tiles, (total * units + kSplitTargetItems - 1) / kSplitTargetItems);
  int k = 0, slot = 0;
  for (int rb = p.nrb - 1; rb >= 0; --rb) {  // latest positions (heaviest row blocks) first
    const int n = (T[rb] + tau - 1) / tau;
    if (k + n > kSplitMaxPieces) return false;
    for (int i = 0; i < n; ++i, ++k) {
      sp.rb[k] = (unsigned char)rb;
      sp.idx[k] = (unsigned char)i;
      sp.cnt[k] = (unsigned char)n;
      sp.slot[k] = (signed char)(n > 1 ? slot + i : -1);
    }
    if (n > 1) {
      if (slot + n > 127) return false;
      sp.srb[sp.n_split] = (unsigned char)rb;
      sp.sslot[sp.n_split] = (unsigned char)slot;
      sp.scnt[sp.n_split] = (unsigned char)n;
      ++sp.n_split;
      slot += n;
    }
  }
  if (sp.n_split == 0) return false;
  sp.n_pieces = k;
  sp.n_slots = slot;
  sp.tau = tau;
  // Dispatch the pieces largest first (workgroups start in list order, each on the CU that frees
  // first). A piece keeps its slot, so the merge's order, and with it the result, does not change.
  int order[kSplitMaxPieces], size[kSplitMaxPieces];
  for (int i = 0; i < k; ++i) {
    const int j = sp.idx[i];
    size[i] = std::min(T[sp.rb[i]], (j + 1) * tau) - j * tau;
    order[i] = i;
  }
  std::stable_sort(order, order + k, [&](int a, int b) { return size[a] > size[b]; });
  unsigned char rb[kSplitMaxPieces], idx[kSplitMaxPieces], cnt[kSplitMaxPieces];
  signed char sl[kSplitMaxPieces];
  for (int i = 0; i < k; ++i) {
    rb[i] = sp.rb[order[i]];
    idx[i] = sp.idx[order[i]];
    cnt[i] = sp.cnt[order[i]];
    sl[i] = sp.slot[order[i]];
  }
  std::copy(rb, rb + k, sp.rb);
  std::copy(idx, idx + k, sp.idx);
  std::copy(cnt, cnt + k, sp.cnt);
  std::copy(sl, sl + k, sp.slot);
  return true;
}

// Partial slots of a plan: (batch, kv head, head slice) units x slots.
inline size_t split_slot_count(const FwdParams& p, const SplitPlan& sp) {
  return (size_t)p.B * p.Hkv * p.nhs * sp.n_slots;
}

// Switches the work decomposition to the plan's pieces (decode_item then walks them).
inline void apply_split(FwdParams& p, const SplitPlan& sp) {
  p.n_pieces = sp.n_pieces;
  p.n_slots = sp.n_slots;
  p.tau = sp.tau;
  for (int k = 0; k < sp.n_pieces; ++k) {
    p.piece_rb[k] = sp.rb[k];
    p.piece_idx[k] = sp.idx[k];
    p.piece_cnt[k] = sp.cnt[k];
    p.piece_slot[k] = sp.slot[k];
  }
  p.per_xcd = (p.B * p.Hkv + kNumXcd - 1) / kNumXcd;  // (batch, kv head) pairs per XCD
  p.n_items = p.per_xcd * p.nhs * sp.n_pieces;         // workgroups per XCD
}

// The range [t_beg, t_end) of a row block's T visible tiles that a work item owns (the host
// plans from the same T, so a piece's range is never empty).
__device__ __forceinline__ void piece_tiles(const FwdParams& p, const WorkItem& w, int T, int& t_beg, int& t_end) {
  t_beg = 0;
  t_end = T;
  if (w.piece >= 0 && p.piece_cnt[w.piece] > 1) {
    t_beg = p.piece_idx[w.piece] * p.tau;
    t_end = min(T, t_beg + p.tau);
  }
}

}  // namespace
}  // namespace cpattn
