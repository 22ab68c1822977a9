// Backward pass of one context-parallel rank's causal grouped-query attention, for gfx950.
//
// What it computes ("Add context parallelism", PR 1445, Description: context parallelism is
// there to train long sequences, so each rank also differentiates its shard's attention over
// the all-gathered keys and values under the same reordered causal mask). With the forward's
// O and row log-sum-exp and an upstream gradient dO, by the chain rule:
//   D_i = dO_i . O_i,  P_ij = exp(s_ij - LSE_i),  dS_ij = P_ij (dO_i . v_j - D_i),
//   dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i,  dV_j = sum_i P_ij dO_i,
// with s_ij = scale q_i . k_j over visible keys and dK, dV of a kv head summed over its query
// heads. dK and dV cover every gathered key but only this rank's queries (the part a
// reduce-scatter over ranks would sum).
//
// Three launches, bf16 inputs, fp32 accumulation, fp32 gradients:
//  * prep: -D and -LSE in log2 units (negated, so that they seed the products as they are) and
//    the rows' positions (padded to 32-row blocks) into the workspace, plus each 32-row block's
//    smallest and largest position.
//  * dq: the forward's decomposition (a wave owns one head and 32 query rows; K/V tiles of 64
//    keys stream through double-buffered LDS by direct-to-LDS copies, visited chunk by chunk
//    in original order). Per tile: S^T = K Q'^T seeded with -LSE (so the products are the
//    exponents of P), dP^T - D = V dO^T seeded with -D, dS^T = P^T (dP^T - D) rounded to bf16,
//    then dQ^T += K^T dS^T with K^T from the transposing LDS read (ds_read_b64_tr_b16).
//  * dkdv: key-stationary. A workgroup owns 32 keys per wave of one kv head (256 keys at
//    Dqk = 128, 128 at Dqk = 64); the keys' K' (scaled) and V fragments stay in registers as B
//    operands.
//    It streams (32-row query block, query head) stages of Q, dO, log2-LSE, D and positions
//    through an LDS ring of 3 slots, skipping blocks whose rows are all before the keys. (At
//    Dqk = 192 a variant with 16 keys per wave on 16x16x32 MFMAs keeps two waves per SIMD.)
//    Per stage: S = Q K'^T seeded with
//    -LSE, dP - D = dO V^T seeded with -D; P and dS come out with a lane per key, already in
//    the B-operand layout of dV^T += dO^T P and dK^T += Q^T dS, whose A operands are the
//    transposing LDS reads of the dO and Q tiles.
#include "attn_tiles.h"

namespace cpattn {
namespace {

constexpr int kBQ = 32;  // query rows per dkdv stage and per position block

struct BwdExtra {
  const __bf16* o;
  const float* lse;
  const __bf16* dout;
  float* dq;
  float* dk;
  float* dv;
  float* neg_delta;  // [B, Hq, Sqp]: -D, the seed of dP - D
  float* neg_lse2;   // [B, Hq, Sqp]: -log2(e) LSE, the seed of the exponents of P
  int32_t* pos;   // [Sqp]
  int32_t* blk;   // [2 * nqb]: min positions, then max positions
  int Sqp, nqb;
  float scale;
};

// ---- prep: rows' positions and block bounds (one thread per padded row)
__global__ __launch_bounds__(256) void bwd_positions_kernel(FwdParams p, BwdExtra e) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= e.Sqp) return;  // Sqp is a multiple of 32: whole 32-lane groups exit together
  int pos = -1;
  if (i < p.Sq) {
    pos = p.qpos ? p.qpos[i] : (int)lb_src((int64_t)p.rank * 2 * p.c + i, p.c, p.cp);
    pos = pos < 0 ? 0 : (pos > p.S - 1 ? p.S - 1 : pos);
  }
  e.pos[i] = pos;
  int mn = i < p.Sq ? pos : 0x7fffffff, mx = pos;
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) {
    mn = min(mn, __shfl_xor(mn, off, 32));
    mx = max(mx, __shfl_xor(mx, off, 32));
  }
  if ((i & 31) == 0) {
    e.blk[i / 32] = mn;
    e.blk[e.nqb + i / 32] = mx;
  }
}

// ---- prep: -D = -dO . O and -LSE * log2 e per (b, h, row), stored negated so that they seed the
// matrix products as they are; 16 lanes per row
template <int DV>
__global__ __launch_bounds__(256) void bwd_delta_kernel(FwdParams p, BwdExtra e) {
  const int64_t r = (int64_t)blockIdx.x * 16 + threadIdx.x / 16;  // (b, h, row) over padded rows
  const int64_t total = (int64_t)p.B * p.Hq * e.Sqp;
  if (r >= total) return;
  const int l16 = threadIdx.x % 16;
  const int row = (int)(r % e.Sqp);
  const int64_t bh = r / e.Sqp;
  const int h = (int)(bh % p.Hq), b = (int)(bh / p.Hq);
  float acc = 0.f;
  if (row < p.Sq) {
    const int64_t base = (((int64_t)b * p.Sq + row) * p.Hq + h) * DV;
    for (int d = l16 * 8; d < DV; d += 128) {
      const bf16x8 ov = *reinterpret_cast<const bf16x8*>(e.o + base + d);
      const bf16x8 gv = *reinterpret_cast<const bf16x8*>(e.dout + base + d);
#pragma unroll
      for (int t = 0; t < 8; ++t) acc = __builtin_fmaf((float)ov[t], (float)gv[t], acc);
    }
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 16);
  if (l16 == 0) {
    e.neg_delta[r] = -acc;
    e.neg_lse2[r] = row < p.Sq ? -e.lse[bh * p.Sq + row] * kLog2e : 0.f;
  }
}

// ------------------------------------------------------------------------------------------
// dq kernel
// ------------------------------------------------------------------------------------------
constexpr int kDqTileKeys = 64;  // keys per K/V tile of the dq kernel

// A compile-time buffer index for loops unrolled over a double buffer.
template <int V>
struct BufTag {
  static constexpr int value = V;
};

template <int DQK, int DV>
struct DqCfg {
  static constexpr int BK = kDqTileKeys;
  static constexpr int KCH = DQK / 8;
  static constexpr int VCH = DV / 8;
  static constexpr int K_BYTES = BK * KCH * 16;
  static constexpr int V_BYTES = BK * VCH * 16;
  static constexpr int STAGE = K_BYTES + V_BYTES;
  static constexpr int K_LOADS = BK * KCH / kThreads;
  static constexpr int V_LOADS = BK * VCH / kThreads;
  static_assert(BK * KCH % kThreads == 0 && BK * VCH % kThreads == 0, "tile/thread mismatch");
  static constexpr int QK_STEPS = DQK / 16;
  static constexpr int DV_STEPS = DV / 16;
  static constexpr int MQ = DQK / 32;
  static constexpr int MB = BK / 32;
  static constexpr int PKS = BK / 16;
};

template <int DQK, int DV>
__global__ __launch_bounds__(kThreads, 1) void attn_bwd_dq_kernel(FwdParams p, BwdExtra e) {
  using C = DqCfg<DQK, DV>;
  __shared__ __attribute__((aligned(16))) char lds[2 * C::STAGE];
  __shared__ int s_red[2 * kWaves];

  WorkItem w;
  if (!decode_item(p, w)) return;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64;
  const int hl = lane / 32;
  const int head = w.head0 + wave / p.wpr;

  int my_row, my_pos, qmin, qmax;
  row_positions(p, w, wave, lane, my_row, my_pos, qmin, qmax, s_red);
  if (qmax < 0) return;

  const float sl2 = p.scale_log2;
  // Q fragment (scaled, B operand of S^T = K Q'^T) and dO fragment (B operand of V dO^T):
  // lane holds row (lane & 31), dims 16 ks + 8 hl .. + 7
  bf16x8 qf[C::QK_STEPS], df[C::DV_STEPS];
  float neg_l2, neg_d;  // -log2 LSE and -D of the lane's row: the seeds of the two products
  {
    const int row = my_row < p.Sq ? my_row : p.Sq - 1;
    const bf16x8* qrow = reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(p.q) +
                                                         (((int64_t)w.b * p.Sq + row) * p.Hq + head) * DQK);
    const bf16x8* drow = reinterpret_cast<const bf16x8*>(e.dout + (((int64_t)w.b * p.Sq + row) * p.Hq + head) * DV);
#pragma unroll
    for (int ks = 0; ks < C::QK_STEPS; ++ks) {
      const bf16x8 raw = qrow[2 * ks + hl];
#pragma unroll
      for (int t = 0; t < 8; ++t) qf[ks][t] = (__bf16)((float)raw[t] * sl2);
    }
#pragma unroll
    for (int ks = 0; ks < C::DV_STEPS; ++ks) df[ks] = drow[2 * ks + hl];
    const int64_t sidx = ((int64_t)w.b * p.Hq + head) * e.Sqp + row;
    neg_l2 = e.neg_lse2[sidx];
    neg_d = e.neg_delta[sidx];
#pragma unroll
    for (int ks = 0; ks < C::QK_STEPS; ++ks) asm volatile("" ::"v"(qf[ks]));
#pragma unroll
    for (int ks = 0; ks < C::DV_STEPS; ++ks) asm volatile("" ::"v"(df[ks]));
    asm volatile("" ::"v"(neg_l2), "v"(neg_d));
  }

  const int64_t kv_row_bytes_k = (int64_t)p.Hkv * DQK * 2;
  const int64_t kv_row_bytes_v = (int64_t)p.Hkv * DV * 2;
  const char* kbase = static_cast<const char*>(p.k) + (int64_t)w.b * p.S * kv_row_bytes_k + (int64_t)w.g * DQK * 2;
  const char* vbase = static_cast<const char*>(p.v) + (int64_t)w.b * p.S * kv_row_bytes_v + (int64_t)w.g * DV * 2;
  const int c = p.c;
  // the row block's visible key tiles, or the piece of them this workgroup owns
  const int tpc = (c + C::BK - 1) / C::BK;
  int t_beg, t_end;
  piece_tiles(p, w, visible_tiles(qmax, c, p.cp, C::BK), t_beg, t_end);

  // DMA slots: wave-instruction (u, wave) fills LDS bytes [1024 (u kWaves + wave), + 1024) of a
  // tile, lane l at + 16 l, from whichever (row, chunk) the swizzle puts there. The per-lane rows
  // and columns are kept in registers, except at Dqk > 128, where they are recomputed for every
  // tile from an opaque copy of the lane index (the registers are needed elsewhere).
  constexpr int K_DMA = C::K_LOADS, V_DMA = C::V_LOADS;
  constexpr bool kKeepDmaGeometry = DQK <= 128;
  auto dma_geometry = [](int u, int wv, int ln, int ch, int& row, unsigned& col) {
    const int pos = (u * kWaves + wv) * 1024 + ln * 16;
    row = pos / (ch * 16);
    const int phys = (pos % (ch * 16)) / 16;
    col = (unsigned)((phys ^ (ch == C::KCH ? swz<C::KCH>(row) : swz<C::VCH>(row))) * 16);
  };
  int k_row[K_DMA], v_row[V_DMA];
  unsigned k_col[K_DMA], v_col[V_DMA];
  if constexpr (kKeepDmaGeometry) {
#pragma unroll
    for (int u = 0; u < K_DMA; ++u) dma_geometry(u, wave, lane, C::KCH, k_row[u], k_col[u]);
#pragma unroll
    for (int u = 0; u < V_DMA; ++u) dma_geometry(u, wave, lane, C::VCH, v_row[u], v_col[u]);
  }
  const unsigned lds0 = (unsigned)(uintptr_t)lds;
  auto dma_tile = [&](const TileCursor& tc, int b) {
    const int64_t prow0 = lb_chunk_offset(tc.chunk, c, p.cp) + tc.t0;
    const int last = min(C::BK, c - tc.t0) - 1;  // rows past a chunk's end re-read its last row
    const char* kt = kbase + prow0 * kv_row_bytes_k;
    const char* vt = vbase + prow0 * kv_row_bytes_v;
    const unsigned kl = lds0 + b * C::STAGE;
    const unsigned vl = kl + C::K_BYTES;
    int ln = lane;
    if constexpr (!kKeepDmaGeometry) asm volatile("" : "+v"(ln));
#pragma unroll
    for (int u = 0; u < K_DMA; ++u) {
      int row = 0;
      unsigned col = 0;
      if constexpr (kKeepDmaGeometry) {
        row = k_row[u];
        col = k_col[u];
      } else {
        dma_geometry(u, wave, ln, C::KCH, row, col);
      }
      dma16_sv(kt, (unsigned)(min(row, last) * kv_row_bytes_k) + col, kl + (u * kWaves + wave) * 1024);
    }
#pragma unroll
    for (int u = 0; u < V_DMA; ++u) {
      int row = 0;
      unsigned col = 0;
      if constexpr (kKeepDmaGeometry) {
        row = v_row[u];
        col = v_col[u];
      } else {
        dma_geometry(u, wave, ln, C::VCH, row, col);
      }
      dma16_sv(vt, (unsigned)(min(row, last) * kv_row_bytes_v) + col, vl + (u * kWaves + wave) * 1024);
    }
  };

  f32x16 dqacc[C::MQ];
#pragma unroll
  for (int m = 0; m < C::MQ; ++m) dqacc[m] = f32x16{};
  // The MFMA seeds as full vectors, read in place by the products (32 registers). At Dqk > 128
  // the Q fragments and dQ accumulators leave no room for them: the seeds are then written
  // into the accumulators from the two scalars for each 32-key block instead.
  constexpr bool kSeedVectors = DQK <= 128;
  f32x16 seed_l, seed_d;
  if constexpr (kSeedVectors) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      seed_l[r] = neg_l2;
      seed_d[r] = neg_d;
    }
  }

  TileCursor tc{t_beg / tpc, (t_beg % tpc) * C::BK};
  if (t_beg < t_end) dma_tile(tc, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  if constexpr (DQK > 128) {
    // Dqk = 192, Dv = 128: every LDS read is a lane-constant register plus an immediate. Rows of
    // the K tile hold 24 chunks, whose swizzle (< 8) only permutes the low three bits of a chunk
    // index; rows of the V tile are 256 bytes, so a row start has eight zero low bits and its
    // chunk offset can be flipped with one xor. With the tile loop unrolled by two, the double
    // buffer's offset is an immediate as well. (Recomputing these offsets for every read, as the
    // loop for the smaller head dims may, costs more vector instructions than the matrix
    // products take.)
    static_assert(C::KCH % 16 == 8 && C::VCH == 16, "layout of this loop");
    const int r31 = lane & 31, lgrp = lane >> 4, ltr_e = (lane & 15) >> 2, ltr_q = lane & 3;
    // S^T = K Q'^T: block mb, k-step ks reads kb + mb 32 rows + 128 (ks / 4) + kso[ks % 4]
    const int swk = swz<C::KCH>(r31);
    int kso[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) kso[j] = r31 * (C::KCH * 16) + (((2 * j + hl) ^ swk) << 4);
    // dP^T = V dO^T: k-step ks reads vb + mb 32 rows + (vso ^ 32 ks)
    const int vso = r31 * (C::VCH * 16) + (((hl ^ swz<C::VCH>(r31)) & 15) << 4);
    // dQ^T += K^T dS^T: k-step ks, dims block m read rows 16 ks + ra0 (+ 8) at
    // kb + 16 ks rows + 128 (m / 2) + tra[m % 2] (trb[m % 2])
    const int ra0 = 4 * (lgrp >> 1) + ltr_e;
    const int c0 = 2 * (lgrp & 1) + (ltr_q >> 1), within = 8 * (ltr_q & 1);
    int tra[2], trb[2];
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      tra[mm] = ra0 * (C::KCH * 16) + (((4 * mm + c0) ^ swz<C::KCH>(ra0)) << 4) + within;
      trb[mm] = (ra0 + 8) * (C::KCH * 16) + (((4 * mm + c0) ^ swz<C::KCH>(ra0 + 8)) << 4) + within;
    }

    auto tile = [&](auto tag, const TileCursor& cur, const TileCursor& nxt, bool has_next) {
      constexpr int B = decltype(tag)::value;
      if (has_next) dma_tile(nxt, B ^ 1);
      const char* kb = lds + B * C::STAGE;
      const char* vb = kb + C::K_BYTES;
      const int kpos0 = cur.chunk * c + cur.t0;
      const int nvalid = min(C::BK, c - cur.t0);
      const bool need_mask = (kpos0 + C::BK - 1 > qmin) || (nvalid < C::BK);
      // key kk of the tile is visible iff kk <= lim (kk < nvalid and kpos0 + kk <= my_pos)
      const int lim = min(nvalid - 1, my_pos - kpos0) - 4 * hl;
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) {
        f32x16 sacc, dacc;
        // opaque copies, so the fills are not hoisted out of the loop as full vectors
        float nl = neg_l2, nd = neg_d;
        asm volatile("" : "+v"(nl), "+v"(nd));
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sacc[r] = nl;
          dacc[r] = nd;
        }
        const char* kr = kb + mb * 32 * (C::KCH * 16);
#pragma unroll
        for (int ks = 0; ks < C::QK_STEPS; ++ks) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(kr + 128 * (ks / 4) + kso[ks % 4]);
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sacc, 0, 0, 0);
        }
        const char* vr = vb + mb * 32 * (C::VCH * 16);
#pragma unroll
        for (int ks = 0; ks < C::DV_STEPS; ++ks) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(vr + (vso ^ (32 * ks)));
          dacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, df[ks], dacc, 0, 0, 0);
        }
        if (need_mask) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kk = mb * 32 + 8 * (r / 4) + (r % 4);
            sacc[r] = kk <= lim ? sacc[r] : -INFINITY;
          }
        }
        bf16x8 dsb[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) dsb[r / 8][r % 8] = (__bf16)(__builtin_amdgcn_exp2f(sacc[r]) * dacc[r]);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const char* kt = kb + 16 * (2 * mb + j) * (C::KCH * 16);
#pragma unroll
          for (int m = 0; m < C::MQ; ++m) {
            const char* pa = kt + 128 * (m / 2) + tra[m % 2];
            const char* pb2 = kt + 128 * (m / 2) + trb[m % 2];
            i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(pa));
            i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(pb2));
            typedef short i16x8 __attribute__((ext_vector_type(8)));
            i16x8 cat = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            dqacc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, cat), dsb[j], dqacc[m], 0,
                                                               0, 0);
          }
        }
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    };
    for (int t = t_beg; t < t_end;) {
      TileCursor nx = tc;
      next_tile<C::BK>(nx, c, qmax);
      tile(BufTag<0>{}, tc, nx, t + 1 < t_end);
      tc = nx;
      if (++t == t_end) break;
      nx = tc;
      next_tile<C::BK>(nx, c, qmax);
      tile(BufTag<1>{}, tc, nx, t + 1 < t_end);
      tc = nx;
      ++t;
    }
  } else {
  int buf = 0;

  for (int t = t_beg; t < t_end; ++t) {
    TileCursor nx = tc;
    next_tile<C::BK>(nx, c, qmax);
    const bool has_next = t + 1 < t_end;
    if (has_next) dma_tile(nx, buf ^ 1);

    const char* kb = lds + buf * C::STAGE;
    const char* vb = kb + C::K_BYTES;

    const int kpos0 = tc.chunk * c + tc.t0;
    const int nvalid = min(C::BK, c - tc.t0);
    const bool need_mask = (kpos0 + C::BK - 1 > qmin) || (nvalid < C::BK);
    // key kk of the tile is visible iff kk <= lim (kk < nvalid and kpos0 + kk <= my_pos)
    const int lim = min(nvalid - 1, my_pos - kpos0) - 4 * hl;
    // for Dqk > 128, lane-dependent LDS offsets come from an opaque copy of the lane index and
    // are recomputed per tile: hoisted out of the loop they would cost registers that the wider
    // head dims do not have (for smaller dims hoisting is cheaper)
    int ln = lane;
    if constexpr (DQK > 128) asm volatile("" : "+v"(ln));  // only the widest head dims need it
    const int lhl = ln >> 5, lgrp = ln >> 4, ltr_e = (ln & 15) >> 2, ltr_q = ln & 3;

    // one 32-key block at a time: exponents of P (S^T = K Q'^T - LSE), dP^T - D = V dO^T - D,
    // dS^T rounded to bf16, then its two k-steps of dQ^T += K^T dS^T
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
      const int krow = mb * 32 + (ln & 31);
      f32x16 sacc, dacc;
      if constexpr (kSeedVectors) {
        sacc = seed_l;
        dacc = seed_d;
      } else {
        // opaque copies, so the fills are not hoisted out of the loop as full vectors again
        float nl = neg_l2, nd = neg_d;
        asm volatile("" : "+v"(nl), "+v"(nd));
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sacc[r] = nl;
          dacc[r] = nd;
        }
      }
      const char* kr = kb + krow * (C::KCH * 16);
      const int swk = swz<C::KCH>(krow);
#pragma unroll
      for (int ks = 0; ks < C::QK_STEPS; ++ks) {
        bf16x8 a = *reinterpret_cast<const bf16x8*>(kr + (((2 * ks + lhl) ^ swk) * 16));
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sacc, 0, 0, 0);
      }
      const char* vr = vb + krow * (C::VCH * 16);
      const int swv = swz<C::VCH>(krow);
#pragma unroll
      for (int ks = 0; ks < C::DV_STEPS; ++ks) {
        bf16x8 a = *reinterpret_cast<const bf16x8*>(vr + (((2 * ks + lhl) ^ swv) * 16));
        dacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, df[ks], dacc, 0, 0, 0);
      }
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = mb * 32 + 8 * (r / 4) + (r % 4);
          sacc[r] = kk <= lim ? sacc[r] : -INFINITY;
        }
      }
      // dS^T in the B-operand layout: k-step j of this block holds registers 8 j .. 8 j + 7
      bf16x8 dsb[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) dsb[r / 8][r % 8] = (__bf16)(__builtin_amdgcn_exp2f(sacc[r]) * dacc[r]);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int ks = 2 * mb + j;
        const int row_a = 16 * ks + 4 * (lgrp / 2) + ltr_e;
        const int row_b = row_a + 8;
#pragma unroll
        for (int m = 0; m < C::MQ; ++m) {
          const int col = 32 * m + 16 * (lgrp % 2) + 4 * ltr_q;
          const int ch = col / 8, within = (col % 8) * 2;
          const char* pa = kb + row_a * (C::KCH * 16) + ((ch ^ swz<C::KCH>(row_a)) * 16) + within;
          const char* pb2 = kb + row_b * (C::KCH * 16) + ((ch ^ swz<C::KCH>(row_b)) * 16) + within;
          i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(pa));
          i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(pb2));
          typedef short i16x8 __attribute__((ext_vector_type(8)));
          i16x8 cat = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          dqacc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, cat), dsb[j], dqacc[m], 0,
                                                             0, 0);
        }
      }
    }

    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    buf ^= 1;
    tc = nx;
  }
  }

  if (my_row < p.Sq) {
    // a piece of a cut row block writes its share of dQ to its partial slot (the merge adds
    // the slots); every other work item writes dQ itself
    float* og = e.dq + (((int64_t)w.b * p.Sq + my_row) * p.Hq + head) * DQK;
    if (w.piece >= 0 && p.piece_slot[w.piece] >= 0) {
      const int64_t slot = (int64_t)w.unit * p.n_slots + p.piece_slot[w.piece];
      og = p.part_o + ((slot * p.bm + (my_row - w.row_blk * p.bm)) * p.hpw + wave / p.wpr) * DQK;
    }
#pragma unroll
    for (int m = 0; m < C::MQ; ++m) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        f32x4 ov;
#pragma unroll
        for (int t = 0; t < 4; ++t) ov[t] = dqacc[m][a4 * 4 + t] * e.scale;
        *reinterpret_cast<f32x4*>(og + 32 * m + 8 * a4 + 4 * hl) = ov;
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// dQ of split row blocks (small grids): the dq kernel walks bk-key tiles, and its time is that of
// its heaviest row block when the grid has about one work item per CU. The shared planner cuts
// the heavy row blocks' visible tiles into pieces; each piece writes its scaled share of dQ to a
// slot of the caller's workspace, and this kernel adds a cut row block's slots in piece order
// (a fixed order, so the result does not depend on timing).
// ------------------------------------------------------------------------------------------
constexpr int kDqSplitMinTiles = 1024 / kDqTileKeys;  // no piece below 1024 keys

bool plan_dq_split(const AttnBwdArgs& a, const FwdParams& p, SplitPlan& sp) {
  if (a.q_pos) return false;
  return plan_split_tiles(p, kDqTileKeys, kDqSplitMinTiles, sp);
}

// The forward's work decomposition of the backward's shape (the dq kernel walks it).
FwdParams bwd_work_params(const AttnBwdArgs& a) {
  AttnArgs fa{};
  fa.q = a.q;
  fa.k = a.k;
  fa.v = a.v;
  fa.q_pos = a.q_pos;
  fa.batch = a.batch;
  fa.seq = a.seq;
  fa.sq = a.sq;
  fa.hq = a.hq;
  fa.hkv = a.hkv;
  fa.d_qk = a.d_qk;
  fa.d_v = a.d_v;
  fa.cp = a.cp;
  fa.rank = a.rank;
  fa.scale = a.scale;
  return make_params(fa);
}

struct DqMergeParams {
  const float* part;
  float* dq;
  int Sq, Hq, Hkv, G, hpw, bm, nhs, n_slots, n_split;
  unsigned char srb[kSplitMaxRb], sslot[kSplitMaxRb], scnt[kSplitMaxRb];
};

// Block (unit, cut row block, head of the slice, group of rows); thread (row, 4 dims).
template <int DQK>
__global__ __launch_bounds__(256) void attn_bwd_dq_merge_kernel(DqMergeParams m) {
  constexpr int TPR = DQK / 4;
  constexpr int RPB = 256 / TPR;
  int bid = blockIdx.x;
  const int rgs = (m.bm + RPB - 1) / RPB;
  const int rg = bid % rgs;
  bid /= rgs;
  const int lh = bid % m.hpw;
  bid /= m.hpw;
  const int j = bid % m.n_split;
  const int unit = bid / m.n_split;
  const int lrow = rg * RPB + threadIdx.x / TPR;
  const int dq = threadIdx.x % TPR;
  const int row = m.srb[j] * m.bm + lrow;
  if (lrow >= m.bm || row >= m.Sq) return;
  const int hs = unit % m.nhs, bg = unit / m.nhs;
  const int g = bg % m.Hkv, b = bg / m.Hkv;
  const int head = g * m.G + hs * m.hpw + lh;
  const int64_t slot0 = (int64_t)unit * m.n_slots + m.sslot[j];
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < m.scnt[j]; ++i) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(m.part + (((slot0 + i) * m.bm + lrow) * m.hpw + lh) * DQK + 4 * dq);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += x[e];
  }
  *reinterpret_cast<f32x4*>(m.dq + (((int64_t)b * m.Sq + row) * m.Hq + head) * DQK + 4 * dq) = acc;
}

// ------------------------------------------------------------------------------------------
// dkdv kernel
// ------------------------------------------------------------------------------------------
constexpr int kKvStages = 3;  // LDS ring: a stage's copy is issued two stages ahead

// Waves per workgroup of the dkdv kernel, 32 keys each. Every workgroup streams the Q and dO rows
// that see its keys, so more keys per workgroup means fewer passes over that stream: 8 waves
// (256 keys, one workgroup per CU) at Dqk = 128; 4 at Dqk = 64 (a stage is only four waves' worth
// of copies). Dqk = 192 has its own kernel (16 keys per wave, below).
template <int DQK>
struct KvShape {
  static_assert(DQK <= 128, "Dqk = 192 runs attn_bwd_dkdv16_kernel");
  static constexpr int WAVES = DQK == 128 ? 8 : 4;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int BKV = WAVES * 32;  // keys per workgroup
  static constexpr int MIN_WG_PER_CU = WAVES == 8 ? 1 : 2;
};

template <int DQK, int DV>
struct DkvCfg {
  static constexpr int WAVES = KvShape<DQK>::WAVES;
  static constexpr int BKV = KvShape<DQK>::BKV;
  static constexpr int QCH = DQK / 8;
  static constexpr int OCH = DV / 8;
  static constexpr int Q_BYTES = kBQ * QCH * 16;
  static constexpr int O_BYTES = kBQ * OCH * 16;
  static constexpr int STAT_BYTES = 3 * kBQ * 4;  // log2-LSE, D, positions
  static constexpr int STAGE = Q_BYTES + O_BYTES + STAT_BYTES;
  static constexpr int Q_DMA = Q_BYTES / (WAVES * 1024);
  static constexpr int O_DMA = O_BYTES / (WAVES * 1024);
  static_assert(Q_BYTES % (WAVES * 1024) == 0 && O_BYTES % (WAVES * 1024) == 0, "stage/wave mismatch");
  static constexpr int QK_STEPS = DQK / 16;
  static constexpr int DV_STEPS = DV / 16;
  static constexpr int MK = DQK / 32;
  static constexpr int MV = DV / 32;
};

struct DkvParams {
  int B, S, Sq, Hq, Hkv, G, cp, c, ntc, n_items, per_xcd;
  float scale_log2;
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
};

// A workgroup-uniform int from global memory through the scalar cache (a read, waited with
// lgkmcnt). A plain load here would be a vector load whose vmcnt wait also drains the LDS copies
// in flight.
__device__ __forceinline__ int load_uniform_i32(const int* ptr) {
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(ptr) : "memory");
  return v;
}

// One dkdv stage in three steps.
// Step 1: S = Q K'^T - LSE and dP - D = dO V^T - D for the stage in LDS at qt (its Q tile, then
// its dO tile, then log2-LSE, D and positions of its 32 rows). S and dP k-steps alternate and
// each row-fragment read is kept two MFMAs ahead of its use.
template <int DQK, int DV>
__device__ __forceinline__ void dkdv_scores(const char* qt, const bf16x8 (&kf)[DQK / 16], const bf16x8 (&vf)[DV / 16],
                                            f32x16& sacc, f32x16& dacc) {
  using C = DkvCfg<DQK, DV>;
  int ln = threadIdx.x % 64;
  asm volatile("" : "+v"(ln));
  const int row = ln & 31, lhl = ln >> 5;
  const char* ot = qt + C::Q_BYTES;
  const float* st_lse = reinterpret_cast<const float*>(ot + C::O_BYTES);
  const float* st_dlt = st_lse + kBQ;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x4 l4 = *reinterpret_cast<const f32x4*>(st_lse + 8 * i + 4 * lhl);
    const f32x4 d4 = *reinterpret_cast<const f32x4*>(st_dlt + 8 * i + 4 * lhl);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sacc[4 * i + j] = l4[j];
      dacc[4 * i + j] = d4[j];
    }
  }
  const char* qr = qt + row * (C::QCH * 16);
  const char* orow = ot + row * (C::OCH * 16);
  // chunk (2 ks + hl) ^ sw = 2 ks ^ (hl ^ sw): one xor per k-step on a per-lane constant
  const unsigned tq = (unsigned)(lhl ^ swz<C::QCH>(row)), to = (unsigned)(lhl ^ swz<C::OCH>(row));
#pragma unroll
  for (int ks = 0; ks < (C::QK_STEPS > C::DV_STEPS ? C::QK_STEPS : C::DV_STEPS); ++ks) {
    if (ks < C::QK_STEPS) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(qr + ((tq ^ (2u * ks)) << 4));
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[ks], sacc, 0, 0, 0);
    }
    if (ks < C::DV_STEPS) {
      // with equal row layouts the dO tile's offsets are the Q tile's plus its size
      const bf16x8 a = C::QCH == C::OCH ? *reinterpret_cast<const bf16x8*>(qr + ((tq ^ (2u * ks)) << 4) + C::Q_BYTES)
                                        : *reinterpret_cast<const bf16x8*>(orow + ((to ^ (2u * ks)) << 4));
      dacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, vf[ks], dacc, 0, 0, 0);
    }
  }
  {
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int i = 0; i < C::QK_STEPS + C::DV_STEPS - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  }
}

// Step 2: mask (when the stage's rows do not all see every key of the workgroup, or keys run
// past the valid ones), then P and dS in bf16 in the B-operand layout of step 3.
template <int DQK, int DV>
__device__ __forceinline__ void dkdv_probs(const char* qt, bool need_mask, int kk, int kpos, int nvalid, f32x16 sacc,
                                           const f32x16& dacc, bf16x8 (&pb)[2], bf16x8 (&dsb)[2]) {
  using C = DkvCfg<DQK, DV>;
  if (need_mask) {
    const int lhl = (threadIdx.x % 64) >> 5;
    const int* st_pos = reinterpret_cast<const int*>(qt + C::Q_BYTES + C::O_BYTES + 2 * kBQ * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int4 q4 = *reinterpret_cast<const int4*>(st_pos + 8 * i + 4 * lhl);
      const int qp[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) sacc[4 * i + j] = (kk < nvalid && kpos <= qp[j]) ? sacc[4 * i + j] : -INFINITY;
    }
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float pr = __builtin_amdgcn_exp2f(sacc[r]);
    pb[r / 8][r % 8] = (__bf16)pr;
    dsb[r / 8][r % 8] = (__bf16)(pr * dacc[r]);
  }
}

// Step 3: dV^T += dO^T P and dK^T += Q^T dS, A operands from transposing reads of the tiles.
template <int DQK, int DV>
__device__ __forceinline__ void dkdv_grads(const char* qt, const bf16x8 (&pb)[2], const bf16x8 (&dsb)[2],
                                           f32x16 (&dkacc)[DQK / 32], f32x16 (&dvacc)[DV / 32]) {
  using C = DkvCfg<DQK, DV>;
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  int ln = threadIdx.x % 64;
  asm volatile("" : "+v"(ln));
  const int lgrp = ln >> 4, ltr_e = (ln & 15) >> 2, ltr_q = ln & 3;
  const char* ot = qt + C::Q_BYTES;
  const unsigned cbase = 16u * (unsigned)(lgrp & 1) + 4u * (unsigned)ltr_q;
  const int row_a0 = 4 * (lgrp >> 1) + ltr_e, row_b0 = row_a0 + 8;
  const unsigned c0 = cbase >> 3, within = (cbase & 7u) * 2u;
  const unsigned ta = c0 ^ (unsigned)swz<C::OCH>(row_a0), tb = c0 ^ (unsigned)swz<C::OCH>(row_b0);
  const unsigned qa = c0 ^ (unsigned)swz<C::QCH>(row_a0), qb = c0 ^ (unsigned)swz<C::QCH>(row_b0);
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int row_a = 16 * ks + row_a0;
    const int row_b = row_a + 8;
#pragma unroll
    for (int m = 0; m < C::MV; ++m) {
      const char* pa = ot + row_a * (C::OCH * 16) + ((ta ^ (4u * m)) << 4) + within;
      const char* pb2 = ot + row_b * (C::OCH * 16) + ((tb ^ (4u * m)) << 4) + within;
      i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(pa));
      i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(pb2));
      i16x8 cat = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      dvacc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, cat), pb[ks], dvacc[m], 0, 0, 0);
    }
#pragma unroll
    for (int m = 0; m < C::MK; ++m) {
      const char* pa = qt + row_a * (C::QCH * 16) + ((qa ^ (4u * m)) << 4) + within;
      const char* pb2 = qt + row_b * (C::QCH * 16) + ((qb ^ (4u * m)) << 4) + within;
      i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(pa));
      i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(pb2));
      i16x8 cat = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      dkacc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, cat), dsb[ks], dkacc[m], 0, 0, 0);
    }
  }
  {
    // keep the transposing reads (two per MFMA) ahead of their MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 2 * (C::MV + C::MK) - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  }
}

template <int DQK, int DV>
__global__ __launch_bounds__(KvShape<DQK>::THREADS, KvShape<DQK>::MIN_WG_PER_CU) void attn_bwd_dkdv_kernel(
    DkvParams p, BwdExtra e) {
  using C = DkvCfg<DQK, DV>;
  __shared__ __attribute__((aligned(16))) char lds[kKvStages * C::STAGE];

  // work item: (b, g, chunk i, tile t). Each XCD takes a contiguous range of items, in which
  // tiles and chunks vary fastest, so an XCD holds whole kv heads (equal work) and its L2 serves
  // one head group's Q and dO; within the range the earliest positions (keys seen by the most
  // query rows) are dispatched first.
  const int bid = blockIdx.x;
  const int W = (bid % kNumXcd) * p.per_xcd + bid / kNumXcd;
  if (W >= p.n_items) return;
  int t = W;
  const int tile = t % p.ntc;
  t /= p.ntc;
  const int chunk = t % (2 * p.cp);
  t /= 2 * p.cp;
  const int g = t % p.Hkv;
  const int b = t / p.Hkv;
  const int t0 = tile * C::BKV;
  const int kpos0 = chunk * p.c + t0;
  const int nvalid = min(C::BKV, p.c - t0);
  const int64_t prow0 = lb_chunk_offset(chunk, p.c, p.cp) + t0;  // gathered slot of key 0

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64;
  const int hl = lane / 32;
  const int kk = wave * 32 + (lane & 31);  // this lane's key within the tile
  const int krow = min(kk, nvalid - 1);

  // K' (scaled) and V fragments, B operands: lane holds key kk, dims 16 ks + 8 hl .. + 7
  bf16x8 kf[C::QK_STEPS], vf[C::DV_STEPS];
  {
    const bf16x8* kr = reinterpret_cast<const bf16x8*>(p.k + (((int64_t)b * p.S + prow0 + krow) * p.Hkv + g) * DQK);
    const bf16x8* vr = reinterpret_cast<const bf16x8*>(p.v + (((int64_t)b * p.S + prow0 + krow) * p.Hkv + g) * DV);
#pragma unroll
    for (int ks = 0; ks < C::QK_STEPS; ++ks) {
      const bf16x8 raw = kr[2 * ks + hl];
#pragma unroll
      for (int u = 0; u < 8; ++u) kf[ks][u] = (__bf16)((float)raw[u] * p.scale_log2);
    }
#pragma unroll
    for (int ks = 0; ks < C::DV_STEPS; ++ks) vf[ks] = vr[2 * ks + hl];
#pragma unroll
    for (int ks = 0; ks < C::QK_STEPS; ++ks) asm volatile("" ::"v"(kf[ks]));
#pragma unroll
    for (int ks = 0; ks < C::DV_STEPS; ++ks) asm volatile("" ::"v"(vf[ks]));
  }

  f32x16 dkacc[C::MK], dvacc[C::MV];
#pragma unroll
  for (int m = 0; m < C::MK; ++m) dkacc[m] = f32x16{};
#pragma unroll
  for (int m = 0; m < C::MV; ++m) dvacc[m] = f32x16{};

  // stages: (query block qb, head h of the group), from the shard's last block down; blocks
  // whose rows all precede the keys skip. Streaming from the end puts every workgroup of a kv
  // head at the same rows when it starts (each row block is seen by all keys before it), so the
  // workgroups of an XCD read the same stages at about the same time and share its L2.
  const int* blkmin = e.blk;
  const int* blkmax = e.blk + e.nqb;
  auto prev_visible = [&](int qb) {
    while (qb >= 0 && load_uniform_i32(blkmax + qb) < kpos0) --qb;
    return qb;
  };

  const int64_t q_row_bytes = (int64_t)p.Hq * DQK * 2;
  const int64_t o_row_bytes = (int64_t)p.Hq * DV * 2;
  const char* qbase = reinterpret_cast<const char*>(p.q) + (int64_t)b * p.Sq * q_row_bytes;
  const char* obase = reinterpret_cast<const char*>(e.dout) + (int64_t)b * p.Sq * o_row_bytes;
  const unsigned lds0 = (unsigned)(uintptr_t)lds;
  // per-lane DMA geometry: wave-instruction u of a stage fills LDS bytes
  // [1024 (u * C::WAVES + wave), + 1024) of the Q (or dO) tile; lane l at + 16 l
  auto dma_stage = [&](int qb, int h, int bufi) {
    const unsigned ql = lds0 + bufi * C::STAGE;
    const unsigned ol = ql + C::Q_BYTES;
    const unsigned sl = ol + C::O_BYTES;
    const int last = p.Sq - 1 - qb * kBQ;  // rows past the shard re-read its last row
    const char* qt = qbase + (int64_t)qb * kBQ * q_row_bytes + (int64_t)h * DQK * 2;
    const char* ot = obase + (int64_t)qb * kBQ * o_row_bytes + (int64_t)h * DV * 2;
#pragma unroll
    for (int u = 0; u < C::Q_DMA; ++u) {
      const int pos = (u * C::WAVES + wave) * 1024 + lane * 16;
      const int row = pos / (C::QCH * 16), phys = (pos % (C::QCH * 16)) / 16;
      const unsigned off = (unsigned)(min(row, last) * q_row_bytes) + (unsigned)((phys ^ swz<C::QCH>(row)) * 16);
      dma16_sv(qt, off, ql + (u * C::WAVES + wave) * 1024);
    }
#pragma unroll
    for (int u = 0; u < C::O_DMA; ++u) {
      const int pos = (u * C::WAVES + wave) * 1024 + lane * 16;
      const int row = pos / (C::OCH * 16), phys = (pos % (C::OCH * 16)) / 16;
      const unsigned off = (unsigned)(min(row, last) * o_row_bytes) + (unsigned)((phys ^ swz<C::OCH>(row)) * 16);
      dma16_sv(ot, off, ol + (u * C::WAVES + wave) * 1024);
    }
    // log2-LSE, D and positions of the block's 32 rows (128 bytes each): waves 0, 1, 2 copy one
    // array each with 8 lanes
    if (wave < 3) {
      const int64_t sidx = ((int64_t)b * p.Hq + h) * e.Sqp + qb * kBQ;
      const char* src = wave == 0 ? reinterpret_cast<const char*>(e.neg_lse2 + sidx)
                                  : (wave == 1 ? reinterpret_cast<const char*>(e.neg_delta + sidx)
                                               : reinterpret_cast<const char*>(e.pos + qb * kBQ));
      if (lane < 8)
        asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src + lane * 16),
                     "s"(sl + wave * 128) : "memory", "m0");
    }
  };
  // wait until at most one stage's copies (this wave's) are still in flight
  auto wait_all_but_one_stage = [&]() {
    if (wave < 3)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(C::Q_DMA + C::O_DMA + 1) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(C::Q_DMA + C::O_DMA) : "memory");
  };

  const int kpos = kpos0 + kk;

  // stage sequence: (query block, head of the group), heads fastest; qb < 0 marks the end
  auto advance = [&](int& sqb, int& sh) {
    if (sqb < 0) return;
    if (++sh == p.G) {
      sh = 0;
      sqb = prev_visible(sqb - 1);
    }
  };
  int qb = prev_visible(e.nqb - 1), h = 0;
  int qb1 = qb, h1 = h;
  advance(qb1, h1);
  if (qb >= 0) dma_stage(qb, g * p.G + h, 0);
  if (qb1 >= 0) {
    dma_stage(qb1, g * p.G + h1, 1);
    wait_all_but_one_stage();
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __syncthreads();
  int buf = 0;
  while (qb >= 0) {
    int qb2 = qb1, h2 = h1;
    advance(qb2, h2);
    const int buf2 = buf >= kKvStages - 2 ? buf + 2 - kKvStages : buf + 2;
    if (qb2 >= 0) dma_stage(qb2, g * p.G + h2, buf2);  // that slot was last read two stages ago

    const char* qt = lds + buf * C::STAGE;

    // (the step functions recompute lane-dependent LDS offsets from an opaque copy of the lane
    // index in every stage: hoisted out of the loop they would hold ~40 registers and push the
    // kernel past the 256 that two waves per SIMD allow)
    f32x16 sacc, dacc;
    dkdv_scores<DQK, DV>(qt, kf, vf, sacc, dacc);
    // mask where a row does not see the key (or the key is past the tile's valid keys)
    const bool need_mask = load_uniform_i32(blkmin + qb) < kpos0 + C::BKV - 1 || nvalid < C::BKV || (qb + 1) * kBQ > p.Sq;
    bf16x8 pb[2], dsb[2];
    dkdv_probs<DQK, DV>(qt, need_mask, kk, kpos, nvalid, sacc, dacc, pb, dsb);
    dkdv_grads<DQK, DV>(qt, pb, dsb, dkacc, dvacc);

    // the next stage's copies must have landed; the one after may stay in flight
    if (qb2 >= 0)
      wait_all_but_one_stage();
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    buf = buf + 1 == kKvStages ? 0 : buf + 1;
    qb = qb1;
    h = h1;
    qb1 = qb2;
    h1 = h2;
  }

  // dK = scale dK^T, dV; lane holds key kk, dims 32 m + 8 a4 + 4 hl + t
  if (kk < nvalid) {
    float* dkr = e.dk + (((int64_t)b * p.S + prow0 + kk) * p.Hkv + g) * DQK;
    float* dvr = e.dv + (((int64_t)b * p.S + prow0 + kk) * p.Hkv + g) * DV;
#pragma unroll
    for (int m = 0; m < C::MK; ++m) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        f32x4 ov;
#pragma unroll
        for (int u = 0; u < 4; ++u) ov[u] = dkacc[m][a4 * 4 + u] * e.scale;
        *reinterpret_cast<f32x4*>(dkr + 32 * m + 8 * a4 + 4 * hl) = ov;
      }
    }
#pragma unroll
    for (int m = 0; m < C::MV; ++m) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        f32x4 ov;
#pragma unroll
        for (int u = 0; u < 4; ++u) ov[u] = dvacc[m][a4 * 4 + u];
        *reinterpret_cast<f32x4*>(dvr + 32 * m + 8 * a4 + 4 * hl) = ov;
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// dkdv kernel at Dqk = 192: 16 keys per wave on 16x16x32 MFMAs
// ------------------------------------------------------------------------------------------
// At 32 keys per wave a Dqk = 192 wave holds 336 registers and runs alone on its SIMD, waiting on
// its own LDS reads and MFMA results. With 16 keys per wave its K and V fragments (40 registers)
// and dK, dV accumulators (80) leave room for two waves per SIMD (two 4-wave workgroups of 64
// keys per CU) at the price of twice the LDS bytes per flop. The stage machinery (ring of 3,
// copies issued two stages ahead, last row block first) is the 32-key kernel's. Per stage, with
// lane (key col, group gq) of a wave:
//  * S = Q K'^T - LSE and dP - D = dO V^T - D per 16-row block mb: the A operands are 16-byte
//    reads of the Q and dO tiles (row 16 mb + col, dims 32 ks + 8 gq ..), the B operands the
//    lane's K' and V fragments; lane holds key col, rows 16 mb + 4 gq + r.
//  * P and dS (bf16) in that order are the B operands of dV^T += dO^T P and dK^T += Q^T dS:
//    k-slots 8 gq .. 8 gq + 7 are rows 4 gq + 0..3 and 16 + 4 gq + 0..3, and the A operands are
//    two transposing reads (ds_read_b64_tr_b16) of those rows of the dO and Q tiles per MFMA.
template <int DQK, int DV>
struct Dkv16Cfg {
  static constexpr int WAVES = 4;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int KPW = 16;  // keys per wave
  static constexpr int BKV = WAVES * KPW;
  static constexpr int QCH = DQK / 8;
  static constexpr int OCH = DV / 8;
  static constexpr int Q_BYTES = kBQ * QCH * 16;
  static constexpr int O_BYTES = kBQ * OCH * 16;
  static constexpr int STAT_BYTES = 3 * kBQ * 4;  // log2-LSE, D, positions
  static constexpr int STAGE = Q_BYTES + O_BYTES + STAT_BYTES;
  static constexpr int Q_DMA = Q_BYTES / (WAVES * 1024);
  static constexpr int O_DMA = O_BYTES / (WAVES * 1024);
  static_assert(Q_BYTES % (WAVES * 1024) == 0 && O_BYTES % (WAVES * 1024) == 0, "stage/wave mismatch");
  static constexpr int KS = DQK / 32;  // k-steps of S
  static constexpr int VK = DV / 32;   // k-steps of dP
  static constexpr int MK = DQK / 16;  // 16-dim blocks of dK
  static constexpr int MV = DV / 16;   // 16-dim blocks of dV
};

// Chunk swizzle of the 16-key kernel's tiles (a 16-byte chunk c of row r sits at c ^ swz16(r)).
// The S reads take one chunk of 16 consecutive rows, a transposing read a chunk pair
// {2 m, 2 m + 1} of rows 8 k .. 8 k + 7. The two forms were chosen by timing each read pattern
// on the part with the LDS bank-conflict counter. The 16-chunk (dO) form keeps the transposing
// reads conflict-free and leaves the S reads two-way conflicted; no form tried kept both free.
// The 24-chunk (Q, Dqk 192) form, row & 7, keeps both conflict-free: its 384-byte rows already
// spread rows apart by 128 bytes, and row & 7 spreads rows 8 apart. Both forms depend on row
// bits 0..3 only and stay below 8 on 24-chunk rows (the offsets below rely on that).
template <int CH>
__device__ __forceinline__ int swz16(int row) {
  static_assert(CH % 16 == 0 || CH % 16 == 8, "tiles of 16 or 24 chunks per row");
  if constexpr (CH % 16 == 0) {
    return ((row & 3) << 2) | (((row >> 2) & 1) << 1) | ((row >> 3) & 1);
  } else {
    return row & 7;
  }
}

template <int DQK, int DV>
__global__ __launch_bounds__(256, 2) void attn_bwd_dkdv16_kernel(DkvParams p, BwdExtra e) {
  using C = Dkv16Cfg<DQK, DV>;
  static_assert(C::THREADS == 256, "launch bounds");
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  __shared__ __attribute__((aligned(16))) char lds[kKvStages * C::STAGE];

  // work item (b, g, chunk i, tile t), placed as in the 32-key kernel
  const int bid = blockIdx.x;
  const int W = (bid % kNumXcd) * p.per_xcd + bid / kNumXcd;
  if (W >= p.n_items) return;
  int t = W;
  const int tile = t % p.ntc;
  t /= p.ntc;
  const int chunk = t % (2 * p.cp);
  t /= 2 * p.cp;
  const int g = t % p.Hkv;
  const int b = t / p.Hkv;
  const int t0 = tile * C::BKV;
  const int kpos0 = chunk * p.c + t0;
  const int nvalid = min(C::BKV, p.c - t0);
  const int64_t prow0 = lb_chunk_offset(chunk, p.c, p.cp) + t0;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64;
  const int col = lane & 15, gq = lane >> 4;
  const int kk = wave * C::KPW + col;  // this lane's key within the tile
  const int krow = min(kk, nvalid - 1);

  // K' (scaled) and V fragments, B operands: key kk, dims 32 ks + 8 gq .. + 7
  bf16x8 kf[C::KS], vf[C::VK];
  {
    const bf16x8* kr = reinterpret_cast<const bf16x8*>(p.k + (((int64_t)b * p.S + prow0 + krow) * p.Hkv + g) * DQK);
    const bf16x8* vr = reinterpret_cast<const bf16x8*>(p.v + (((int64_t)b * p.S + prow0 + krow) * p.Hkv + g) * DV);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const bf16x8 raw = kr[4 * ks + gq];
#pragma unroll
      for (int u = 0; u < 8; ++u) kf[ks][u] = (__bf16)((float)raw[u] * p.scale_log2);
    }
#pragma unroll
    for (int ks = 0; ks < C::VK; ++ks) vf[ks] = vr[4 * ks + gq];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) asm volatile("" ::"v"(kf[ks]));
#pragma unroll
    for (int ks = 0; ks < C::VK; ++ks) asm volatile("" ::"v"(vf[ks]));
  }

  f32x4 dkacc[C::MK], dvacc[C::MV];
#pragma unroll
  for (int m = 0; m < C::MK; ++m) dkacc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < C::MV; ++m) dvacc[m] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int* blkmin = e.blk;
  const int* blkmax = e.blk + e.nqb;
  auto prev_visible = [&](int qb) {
    while (qb >= 0 && load_uniform_i32(blkmax + qb) < kpos0) --qb;
    return qb;
  };
  const int64_t q_row_bytes = (int64_t)p.Hq * DQK * 2;
  const int64_t o_row_bytes = (int64_t)p.Hq * DV * 2;
  const char* qbase = reinterpret_cast<const char*>(p.q) + (int64_t)b * p.Sq * q_row_bytes;
  const char* obase = reinterpret_cast<const char*>(e.dout) + (int64_t)b * p.Sq * o_row_bytes;
  const unsigned lds0 = (unsigned)(uintptr_t)lds;
  // copies of a stage: wave-instruction u fills LDS bytes [1024 (u WAVES + wave), + 1024) of the
  // Q (or dO) tile, lane l at + 16 l; waves 0, 1, 2 copy the log2-LSE, D and positions
  auto dma_stage = [&](int qb, int h, int bufi) {
    const unsigned ql = lds0 + bufi * C::STAGE;
    const unsigned ol = ql + C::Q_BYTES;
    const unsigned sl = ol + C::O_BYTES;
    const int last = p.Sq - 1 - qb * kBQ;  // rows past the shard re-read its last row
    const char* qt = qbase + (int64_t)qb * kBQ * q_row_bytes + (int64_t)h * DQK * 2;
    const char* ot = obase + (int64_t)qb * kBQ * o_row_bytes + (int64_t)h * DV * 2;
#pragma unroll
    for (int u = 0; u < C::Q_DMA; ++u) {
      const int pos = (u * C::WAVES + wave) * 1024 + lane * 16;
      const int row = pos / (C::QCH * 16), phys = (pos % (C::QCH * 16)) / 16;
      const unsigned off = (unsigned)(min(row, last) * q_row_bytes) + (unsigned)((phys ^ swz16<C::QCH>(row)) * 16);
      dma16_sv(qt, off, ql + (u * C::WAVES + wave) * 1024);
    }
#pragma unroll
    for (int u = 0; u < C::O_DMA; ++u) {
      const int pos = (u * C::WAVES + wave) * 1024 + lane * 16;
      const int row = pos / (C::OCH * 16), phys = (pos % (C::OCH * 16)) / 16;
      const unsigned off = (unsigned)(min(row, last) * o_row_bytes) + (unsigned)((phys ^ swz16<C::OCH>(row)) * 16);
      dma16_sv(ot, off, ol + (u * C::WAVES + wave) * 1024);
    }
    if (wave < 3) {
      const int64_t sidx = ((int64_t)b * p.Hq + h) * e.Sqp + qb * kBQ;
      const char* src = wave == 0 ? reinterpret_cast<const char*>(e.neg_lse2 + sidx)
                                  : (wave == 1 ? reinterpret_cast<const char*>(e.neg_delta + sidx)
                                               : reinterpret_cast<const char*>(e.pos + qb * kBQ));
      if (lane < 8)
        asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src + lane * 16),
                     "s"(sl + wave * 128) : "memory", "m0");
    }
  };
  auto wait_all_but_one_stage = [&]() {
    if (wave < 3)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(C::Q_DMA + C::O_DMA + 1) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(C::Q_DMA + C::O_DMA) : "memory");
  };
  auto advance = [&](int& sqb, int& sh) {
    if (sqb < 0) return;
    if (++sh == p.G) {
      sh = 0;
      sqb = prev_visible(sqb - 1);
    }
  };
  const int kpos = kpos0 + kk;

  // Lane-constant LDS offsets of the reads within a slot, so that each read is one register
  // plus an immediate. swz16 of a row depends on its bits 0..3 only, so rows 16 mb + col, and
  // rows rlo and rlo + 16, share it; with 24 chunks per Q row the swizzle (< 8) only permutes the
  // low three bits of a chunk index.
  static_assert(C::QCH % 16 == 8 && C::OCH == 16, "layout of the offsets below");
  const int e4 = (lane & 15) >> 2, q4 = lane & 3;
  const int rlo = 4 * gq + e4;
  const int within = 8 * (q4 & 1), cx = q4 >> 1;
  int qso[2], oso[C::VK], tqo[4], too[C::MV];
#pragma unroll
  for (int j = 0; j < 2; ++j) qso[j] = col * (C::QCH * 16) + (((4 * j + gq) ^ swz16<C::QCH>(col)) << 4);
#pragma unroll
  for (int ks = 0; ks < C::VK; ++ks) oso[ks] = col * (C::OCH * 16) + (((4 * ks + gq) ^ swz16<C::OCH>(col)) << 4);
#pragma unroll
  for (int j = 0; j < 4; ++j) tqo[j] = rlo * (C::QCH * 16) + (((2 * j + cx) ^ swz16<C::QCH>(rlo)) << 4) + within;
#pragma unroll
  for (int m = 0; m < C::MV; ++m)
    too[m] = C::Q_BYTES + rlo * (C::OCH * 16) + (((2 * m + cx) ^ swz16<C::OCH>(rlo)) << 4) + within;

  int qb = prev_visible(e.nqb - 1), h = 0;
  int qb1 = qb, h1 = h;
  advance(qb1, h1);
  if (qb >= 0) dma_stage(qb, g * p.G + h, 0);
  if (qb1 >= 0) {
    dma_stage(qb1, g * p.G + h1, 1);
    wait_all_but_one_stage();
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __syncthreads();
  int buf = 0;
  while (qb >= 0) {
    int qb2 = qb1, h2 = h1;
    advance(qb2, h2);
    const int buf2 = buf >= kKvStages - 2 ? buf + 2 - kKvStages : buf + 2;
    if (qb2 >= 0) dma_stage(qb2, g * p.G + h2, buf2);  // that slot was last read two stages ago

    const char* qt = lds + buf * C::STAGE;
    const char* ot = qt + C::Q_BYTES;
    const float* st_lse = reinterpret_cast<const float*>(ot + C::O_BYTES);
    const float* st_dlt = st_lse + kBQ;
    const int* st_pos = reinterpret_cast<const int*>(st_dlt + kBQ);
    const bool need_mask = load_uniform_i32(blkmin + qb) < kpos0 + C::BKV - 1 || nvalid < C::BKV || (qb + 1) * kBQ > p.Sq;

    // ---- S - LSE and dP - D, then P and dS (bf16) in the B-operand order of the gradients
    bf16x8 pb, dsb;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(st_lse + 16 * mb + 4 * gq);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(st_dlt + 16 * mb + 4 * gq);
      f32x4 sacc = l4, dacc = d4;
      // Q: chunk 4 ks + gq of row 16 mb + col is at 8 (ks / 2) + ((4 (ks % 2) + gq) ^ swz16)
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(qt + 16 * mb * (C::QCH * 16) + 128 * (ks / 2) + qso[ks % 2]);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, kf[ks], sacc, 0, 0, 0);
      }
#pragma unroll
      for (int ks = 0; ks < C::VK; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(ot + 16 * mb * (C::OCH * 16) + oso[ks]);
        dacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, vf[ks], dacc, 0, 0, 0);
      }
      if (need_mask) {
        const int4 q4 = *reinterpret_cast<const int4*>(st_pos + 16 * mb + 4 * gq);
        const int qp[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) sacc[r] = (kk < nvalid && kpos <= qp[r]) ? sacc[r] : -INFINITY;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pr = __builtin_amdgcn_exp2f(sacc[r]);
        pb[4 * mb + r] = (__bf16)pr;
        dsb[4 * mb + r] = (__bf16)(pr * dacc[r]);
      }
    }

    // ---- dV^T += dO^T P and dK^T += Q^T dS: lane 4 e + q of group gq reads rows 4 gq + e and
    // 16 + 4 gq + e, dims 16 m + 4 q .. + 3 of the tile
    {
      // row rlo + 16 sits 16 rows after row rlo, at the same chunk
#pragma unroll
      for (int m = 0; m < C::MV; ++m) {
        const char* alo = qt + too[m];
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(alo));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(alo + 16 * (C::OCH * 16)));
        const i16x8 cat = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        dvacc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cat), pb, dvacc[m], 0, 0, 0);
      }
      // Q: chunk 2 m + cx of row rlo is at 8 (m / 4) + ((2 (m % 4) + cx) ^ swz16)
#pragma unroll
      for (int m = 0; m < C::MK; ++m) {
        const char* alo = qt + 128 * (m / 4) + tqo[m % 4];
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(alo));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(alo + 16 * (C::QCH * 16)));
        const i16x8 cat = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        dkacc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cat), dsb, dkacc[m], 0, 0, 0);
      }
    }

    // the next stage's copies must have landed; the one after may stay in flight
    if (qb2 >= 0)
      wait_all_but_one_stage();
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    buf = buf + 1 == kKvStages ? 0 : buf + 1;
    qb = qb1;
    h = h1;
    qb1 = qb2;
    h1 = h2;
  }

  // dK = scale dK^T, dV; lane holds key kk, dims 16 m + 4 gq + r
  if (kk < nvalid) {
    float* dkr = e.dk + (((int64_t)b * p.S + prow0 + kk) * p.Hkv + g) * DQK;
    float* dvr = e.dv + (((int64_t)b * p.S + prow0 + kk) * p.Hkv + g) * DV;
#pragma unroll
    for (int m = 0; m < C::MK; ++m) {
      f32x4 ov;
#pragma unroll
      for (int u = 0; u < 4; ++u) ov[u] = dkacc[m][u] * e.scale;
      *reinterpret_cast<f32x4*>(dkr + 16 * m + 4 * gq) = ov;
    }
#pragma unroll
    for (int m = 0; m < C::MV; ++m) *reinterpret_cast<f32x4*>(dvr + 16 * m + 4 * gq) = dvacc[m];
  }
}

// Keys per dkdv workgroup: the 16-keys-per-wave kernel at Dqk > 128, else the 32-key one.
template <int DQK, int DV>
constexpr int dkdv_keys_per_wg() {
  if constexpr (DQK > 128) {
    return Dkv16Cfg<DQK, DV>::BKV;
  } else {
    return KvShape<DQK>::BKV;
  }
}

template <int DQK, int DV>
hipError_t launch_bwd_typed(const AttnBwdArgs& a, hipStream_t stream) {
  const FwdParams p = bwd_work_params(a);

  BwdExtra e;
  e.o = static_cast<const __bf16*>(a.o);
  e.lse = a.lse;
  e.dout = static_cast<const __bf16*>(a.dout);
  e.dq = a.dq;
  e.dk = a.dk;
  e.dv = a.dv;
  const int Sqp = (a.sq + kBQ - 1) / kBQ * kBQ;
  e.Sqp = Sqp;
  e.nqb = Sqp / kBQ;
  e.scale = a.scale;
  char* ws = static_cast<char*>(a.ws);
  const size_t stat_bytes = (size_t)a.batch * a.hq * Sqp * 4;
  e.neg_delta = reinterpret_cast<float*>(ws);
  e.neg_lse2 = reinterpret_cast<float*>(ws + stat_bytes);
  e.pos = reinterpret_cast<int32_t*>(ws + 2 * stat_bytes);
  e.blk = reinterpret_cast<int32_t*>(ws + 2 * stat_bytes + (size_t)Sqp * 4);

  // dQ of heavy row blocks in pieces when the grid is small and the workspace holds the slots
  FwdParams pq = p;
  SplitPlan sp;
  const size_t base = attn_bwd_workspace_bytes(a.batch, a.sq, a.hq);
  const bool split = plan_dq_split(a, p, sp) &&
                     a.ws_bytes >= base + split_slot_count(p, sp) * (size_t)p.bm * p.hpw * DQK * sizeof(float);
  if (split) {
    apply_split(pq, sp);
    pq.part_o = reinterpret_cast<float*>(ws + base);
  }

  hipLaunchKernelGGL(bwd_positions_kernel, dim3((Sqp + 255) / 256), dim3(256), 0, stream, p, e);
  const int64_t rows = (int64_t)a.batch * a.hq * Sqp;
  hipLaunchKernelGGL((bwd_delta_kernel<DV>), dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, stream, p, e);
  hipLaunchKernelGGL((attn_bwd_dq_kernel<DQK, DV>), dim3((split ? pq.n_items : pq.per_xcd) * kNumXcd), dim3(kThreads),
                     0, stream, pq, e);
  if (split) {
    DqMergeParams m;
    m.part = pq.part_o;
    m.dq = a.dq;
    m.Sq = p.Sq;
    m.Hq = p.Hq;
    m.Hkv = p.Hkv;
    m.G = p.G;
    m.hpw = p.hpw;
    m.bm = p.bm;
    m.nhs = p.nhs;
    m.n_slots = sp.n_slots;
    m.n_split = sp.n_split;
    for (int j = 0; j < sp.n_split; ++j) {
      m.srb[j] = sp.srb[j];
      m.sslot[j] = sp.sslot[j];
      m.scnt[j] = sp.scnt[j];
    }
    const int rpb = 256 / (DQK / 4);
    const int64_t blocks = (int64_t)p.B * p.Hkv * p.nhs * sp.n_split * p.hpw * ((p.bm + rpb - 1) / rpb);
    hipLaunchKernelGGL(attn_bwd_dq_merge_kernel<DQK>, dim3((unsigned)blocks), dim3(256), 0, stream, m);
  }

  DkvParams d;
  d.B = a.batch;
  d.S = a.seq;
  d.Sq = a.sq;
  d.Hq = a.hq;
  d.Hkv = a.hkv;
  d.G = a.hq / a.hkv;
  d.cp = a.cp;
  d.c = a.seq / (2 * a.cp);
  // Dqk = 192: the 16-keys-per-wave kernel (two waves per SIMD)
  constexpr bool kKeys16 = DQK > 128;
  constexpr int kBkv = dkdv_keys_per_wg<DQK, DV>();
  d.ntc = (d.c + kBkv - 1) / kBkv;
  d.n_items = 2 * a.cp * d.B * d.Hkv * d.ntc;
  d.per_xcd = (d.n_items + kNumXcd - 1) / kNumXcd;
  d.scale_log2 = a.scale * kLog2e;
  d.q = static_cast<const __bf16*>(a.q);
  d.k = static_cast<const __bf16*>(a.k);
  d.v = static_cast<const __bf16*>(a.v);
  if constexpr (kKeys16) {
    hipLaunchKernelGGL((attn_bwd_dkdv16_kernel<DQK, DV>), dim3(d.per_xcd * kNumXcd), dim3(Dkv16Cfg<DQK, DV>::THREADS),
                       0, stream, d, e);
  } else {
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<DQK, DV>), dim3(d.per_xcd * kNumXcd), dim3(KvShape<DQK>::THREADS), 0,
                       stream, d, e);
  }
  return hipGetLastError();
}

}  // namespace

size_t attn_bwd_workspace_bytes(int batch, int sq, int hq) {
  const size_t sqp = ((size_t)sq + kBQ - 1) / kBQ * kBQ;
  const size_t bytes = 2 * (size_t)batch * hq * sqp * 4 + sqp * 4 + 2 * (sqp / kBQ) * 4;
  return (bytes + 255) / 256 * 256;  // the dQ partial slots of a split start 256-byte aligned
}

size_t attn_bwd_split_workspace_bytes(const AttnBwdArgs& a) {
  const FwdParams p = bwd_work_params(a);
  SplitPlan sp;
  const size_t base = attn_bwd_workspace_bytes(a.batch, a.sq, a.hq);
  if (p.n_items == 0 || !plan_dq_split(a, p, sp)) return base;
  return base + split_slot_count(p, sp) * (size_t)p.bm * p.hpw * a.d_qk * sizeof(float);
}

hipError_t launch_attn_bwd_bf16(const AttnBwdArgs& a, hipStream_t stream) {
  if (a.batch == 0 || a.sq == 0) return hipSuccess;
  if (a.d_qk == 128 && a.d_v == 128) return launch_bwd_typed<128, 128>(a, stream);
  if (a.d_qk == 64 && a.d_v == 64) return launch_bwd_typed<64, 64>(a, stream);
  if (a.d_qk == 192 && a.d_v == 128) return launch_bwd_typed<192, 128>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace cpattn
