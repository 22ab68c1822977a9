// Causal grouped-query attention forward over one context-parallel rank's query shard, for
// gfx950 (MI355X).
//
// What it computes ("Add context parallelism", PR 1445, Description; "Add support for EP to
// context parallelism in self-attention", PR 2023, unit test): for each query row i of the
// shard and query head h, softmax(scale * q_i . k_j) v_j over the keys j whose original
// position src(j) is <= the row's original position, with K/V given in the all-gathered
// (load-balanced) order; plus the row log-sum-exp.
//
// Design (bf16):
//  * A workgroup is 8 wavefronts. It owns `hpw` query heads of one KV group and 32*8/hpw query
//    rows; each wave owns one head and 32 rows. All waves stream the same K/V tiles (128 keys
//    where two stages fit in LDS, as at head dim 128; 64 at the MLA head dims) through LDS,
//    so one tile serves every head of the group that the workgroup holds.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: K (row-major
//    in LDS) is the A operand, the Q fragment lives in registers as the B operand. In the
//    result each lane holds 16 keys of ONE query row, so row max/sum need a single exchange
//    with the lane 32 away (v_permlane32_swap), and the probabilities already sit in the B
//    operand layout of the next product O^T += V^T P^T. V^T comes straight from the row-major
//    V tile with the gfx950 transposing LDS read (ds_read_b64_tr_b16).
//  * Online softmax in fp32 with base-2 exponentials; the running max is only raised when a
//    tile's max exceeds it by more than 8 (log2 units), so most tiles skip the O rescale.
//  * Probabilities are rounded to bf16 once; the row sum adds those rounded values
//    (v_dot2 with ones), so O is an exact convex combination of the bf16 weights.
//  * Causal structure of a balanced shard: KV tiles are visited chunk by chunk in original
//    order, chunk i sitting at permuted offset lb_chunk_offset(i). Only keys with position
//    <= the workgroup's largest query position are visited; tiles whose last key position is
//    <= its smallest query position skip the mask.
//  * K/V tiles are double-buffered in LDS and filled with direct global->LDS copies
//    (global_load_lds_dwordx4): the copy of tile t+1 is in flight while tile t is computed and
//    uses no registers. LDS rows use an XOR swizzle of 16-byte chunks that keeps both the
//    K-fragment reads and the transposing V reads free of bank conflicts.
//  * Scheduling groups keep every LDS fragment read two MFMAs ahead of its use.
//  * Workgroup order is XCD-aware and heavy-first: consecutive work items (same KV head,
//    neighbouring row blocks) go to the same XCD so they share its L2, and row blocks with the
//    latest positions (most keys) start first.
#include <algorithm>

#include "attn_tiles.h"

namespace cpattn {
namespace {

// ------------------------------------------------------------------------------------------
// bf16 kernel
// ------------------------------------------------------------------------------------------
// Keys per tile: 128 where two stages of K and V fit in 128 KB of LDS, else 96 where they fit
// in 120 KB (Dqk 192, Dv 128).
constexpr int bf16_bk(int dqk, int dv) { return 2 * 128 * (dqk + dv) * 2 <= 128 * 1024 ? 128 : 96; }
template <int DQK, int DV>
struct Bf16Cfg {
  static constexpr int BK = bf16_bk(DQK, DV);
  static constexpr int KCH = DQK / 8;  // 16-byte chunks per K row
  static constexpr int VCH = DV / 8;
  static constexpr int K_BYTES = BK * KCH * 16;
  static constexpr int V_BYTES = BK * VCH * 16;
  static constexpr int STAGE = K_BYTES + V_BYTES;
  // 1 KB wave-copies of the K tile per wave; at 96 keys x 24 chunks the last one is taken by
  // the first half of the waves only
  static constexpr int K_LOADS = (BK * KCH + kThreads - 1) / kThreads;
  static constexpr bool K_PART = BK * KCH % kThreads != 0;
  static constexpr int V_LOADS = BK * VCH / kThreads;
  static_assert(BK * KCH % (kThreads / 2) == 0 && BK * VCH % kThreads == 0, "tile/thread mismatch");
  static constexpr int QK_STEPS = DQK / 16;
  static constexpr int MV = DV / 32;
  static constexpr int MB = BK / 32;   // 32-key blocks of S^T
  static constexpr int PKS = BK / 16;  // k-steps of the P V product
};

template <int DQK, int DV>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_bf16_kernel(FwdParams p) {
  using C = Bf16Cfg<DQK, DV>;
  __shared__ __attribute__((aligned(16))) char lds[2 * C::STAGE];
  __shared__ int s_red[2 * kWaves];

  WorkItem w;
  if (!decode_item(p, w)) return;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64;
  const int hl = lane / 32;  // which half of the wave
  const int head = w.head0 + wave / p.wpr;

  int my_row, my_pos, qmin, qmax;
  row_positions(p, w, wave, lane, my_row, my_pos, qmin, qmax, s_red);
  if (qmax < 0) return;  // no valid row (cannot happen for a non-empty block)

  const __bf16* qg = static_cast<const __bf16*>(p.q);
  const char* kg = static_cast<const char*>(p.k);
  const char* vg = static_cast<const char*>(p.v);
  const float sl2 = p.scale_log2;

  // Q fragment (B operand of S^T = K Q^T): lane holds row (lane&31), dims 16ks + 8hl .. +7. The
  // softmax scale (times log2 e) is folded into Q once, in fp32, before the rounding to bf16,
  // so the products come out as log2-unit logits.
  bf16x8 qf[C::QK_STEPS];
  {
    int row = my_row < p.Sq ? my_row : p.Sq - 1;
    const bf16x8* qrow = reinterpret_cast<const bf16x8*>(
        qg + (((int64_t)w.b * p.Sq + row) * p.Hq + head) * DQK);
#pragma unroll
    for (int ks = 0; ks < C::QK_STEPS; ++ks) {
      const bf16x8 raw = qrow[2 * ks + hl];
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[ks][e] = (__bf16)((float)raw[e] * sl2);
    }
    // make the compiler wait for the Q loads here: otherwise its wait counting inside the loop
    // would also wait for the tile DMAs issued through inline asm
#pragma unroll
    for (int ks = 0; ks < C::QK_STEPS; ++ks) asm volatile("" ::"v"(qf[ks]));
  }

  const int64_t kv_row_bytes_k = (int64_t)p.Hkv * DQK * 2;
  const int64_t kv_row_bytes_v = (int64_t)p.Hkv * DV * 2;
  const char* kbase = kg + (int64_t)w.b * p.S * kv_row_bytes_k + (int64_t)w.g * DQK * 2;
  const char* vbase = vg + (int64_t)w.b * p.S * kv_row_bytes_v + (int64_t)w.g * DV * 2;

  const int c = p.c;

  // the row block's visible key tiles, or the piece of them this workgroup owns
  const int tpc = (c + C::BK - 1) / C::BK;
  int t_beg, t_end;
  piece_tiles(p, w, visible_tiles(qmax, c, p.cp, C::BK), t_beg, t_end);

  // DMA slots: wave-instruction (u, wave) fills LDS bytes [1024*(u*kWaves + wave), +1024) of a
  // tile, lane l at +16*l; the lane loads whichever (row, chunk) the swizzle puts there. For a
  // full tile the source byte offsets from the tile's first row are fixed per lane.
  constexpr int K_DMA = C::K_LOADS, V_DMA = C::V_LOADS;
  int k_row[K_DMA], v_row[V_DMA];
  unsigned k_col[K_DMA], v_col[V_DMA], k_off[K_DMA], v_off[V_DMA];
#pragma unroll
  for (int u = 0; u < K_DMA; ++u) {
    const int pos = (u * kWaves + wave) * 1024 + lane * 16;
    const int row = pos / (C::KCH * 16), phys = (pos % (C::KCH * 16)) / 16;
    k_row[u] = row;
    k_col[u] = (unsigned)((phys ^ swz<C::KCH>(row)) * 16);
    k_off[u] = (unsigned)(row * kv_row_bytes_k) + k_col[u];
  }
#pragma unroll
  for (int u = 0; u < V_DMA; ++u) {
    const int pos = (u * kWaves + wave) * 1024 + lane * 16;
    const int row = pos / (C::VCH * 16), phys = (pos % (C::VCH * 16)) / 16;
    v_row[u] = row;
    v_col[u] = (unsigned)((phys ^ swz<C::VCH>(row)) * 16);
    v_off[u] = (unsigned)(row * kv_row_bytes_v) + v_col[u];
  }
  const unsigned lds0 = (unsigned)(uintptr_t)lds;
  auto dma_tile = [&](const TileCursor& tc, int b) {
    const int64_t prow0 = lb_chunk_offset(tc.chunk, c, p.cp) + tc.t0;
    const int last = min(C::BK, c - tc.t0) - 1;
    const char* kt = kbase + prow0 * kv_row_bytes_k;
    const char* vt = vbase + prow0 * kv_row_bytes_v;
    const unsigned kl = lds0 + b * C::STAGE;
    const unsigned vl = kl + C::K_BYTES;
    if (last == C::BK - 1) {
#pragma unroll
      for (int u = 0; u < K_DMA; ++u)
        if (!C::K_PART || u + 1 < K_DMA || wave < kWaves / 2) dma16_sv(kt, k_off[u], kl + (u * kWaves + wave) * 1024);
#pragma unroll
      for (int u = 0; u < V_DMA; ++u) dma16_sv(vt, v_off[u], vl + (u * kWaves + wave) * 1024);
    } else {  // a chunk's partial last tile: rows past it re-read its last row (finite, masked)
#pragma unroll
      for (int u = 0; u < K_DMA; ++u)
        if (!C::K_PART || u + 1 < K_DMA || wave < kWaves / 2)
          dma16_sv(kt, (unsigned)(min(k_row[u], last) * kv_row_bytes_k) + k_col[u], kl + (u * kWaves + wave) * 1024);
#pragma unroll
      for (int u = 0; u < V_DMA; ++u)
        dma16_sv(vt, (unsigned)(min(v_row[u], last) * kv_row_bytes_v) + v_col[u], vl + (u * kWaves + wave) * 1024);
    }
  };

  f32x16 oacc[C::MV];
#pragma unroll
  for (int mv = 0; mv < C::MV; ++mv) oacc[mv] = f32x16{};
  // Running max of the row in log2 units (m_run) and the offset the scores are taken against
  // (m_use: m_run, or 0 before the first visible key). The QK product of a tile starts from
  // -m_use (cneg), so its outputs are already the exponents of the probabilities.
  float m_run = -INFINITY, m_use = 0.f;
  float thr = -INFINITY;    // raise the max when a tile's max exponent exceeds this
  f32x16 cneg = f32x16{};   // -m_use in every entry
  float l_part = 0.f;       // this lane's share of the row sum

  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  TileCursor tc{t_beg / tpc, (t_beg % tpc) * C::BK};
  if (t_beg < t_end) dma_tile(tc, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  int buf = 0;

  // per-lane transposed-read geometry for V (ds_read_b64_tr_b16): in each 16-lane group,
  // input lane 4e+q supplies row e, columns 4q..4q+3 of a 4x16 block; output lane j then holds
  // column j, rows 0..3.
  const int grp = lane / 16;
  const int tr_e = (lane % 16) / 4;
  const int tr_q = lane % 4;

  for (int t = t_beg; t < t_end; ++t) {
    TileCursor nx = tc;
    next_tile<C::BK>(nx, c, qmax);
    const bool has_next = t + 1 < t_end;
    if (has_next) dma_tile(nx, buf ^ 1);  // that stage was last read in the previous iteration

    const char* kb = lds + buf * C::STAGE;
    const char* vb = kb + C::K_BYTES;

    // ---- exponents x = K Q'^T - m_use for the tile's keys (32-key blocks)
    f32x16 s[C::MB];
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
      f32x16 acc = cneg;
      const int krow = mb * 32 + (lane & 31);
      const char* kr = kb + krow * (C::KCH * 16);
      const int sw = swz<C::KCH>(krow);
#pragma unroll
      for (int ks = 0; ks < C::QK_STEPS; ++ks) {
        bf16x8 a = *reinterpret_cast<const bf16x8*>(kr + (((2 * ks + hl) ^ sw) * 16));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], acc, 0, 0, 0);
      }
      s[mb] = acc;
    }
    // keep each K-fragment read two MFMAs ahead of its use
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int i = 0; i < C::MB * C::QK_STEPS - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);

    // ---- mask (only tiles that reach past the smallest query position, or partial tiles)
    const int kpos0 = tc.chunk * c + tc.t0;
    const int nvalid = min(C::BK, c - tc.t0);
    const bool need_mask = (kpos0 + C::BK - 1 > qmin) || (nvalid < C::BK);
    if (need_mask) {
      // key kk is visible iff kk <= lim (kk < nvalid and kpos0 + kk <= my_pos)
      const int lim = min(nvalid - 1, my_pos - kpos0) - 4 * hl;
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = mb * 32 + 8 * (r / 4) + (r % 4);  // minus the lane's 4*hl
          s[mb][r] = kk <= lim ? s[mb][r] : -INFINITY;
        }
      }
    }

    // ---- online softmax (row = lane & 31; this lane holds half of the row's exponents)
    float mt = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int r = 2; r < 16; ++r) mt = fmaxf(mt, s[0][r]);
#pragma unroll
    for (int mb = 1; mb < C::MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[mb][r]);
    mt = wave_max32(mt);
    if (__any(mt > thr)) {
      // new max for the row; shift this tile's exponents and rescale what came before
      const float m_new = fmaxf(m_run, m_use + mt);
      if (m_new != -INFINITY) {
        const float delta = m_new - m_use;
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb) s[mb] -= delta;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 when m_run = -inf
        l_part *= alpha;
#pragma unroll
        for (int mv = 0; mv < C::MV; ++mv) oacc[mv] *= alpha;
        m_run = m_new;
        m_use = m_new;
        thr = kRescaleSlack;
#pragma unroll
        for (int r = 0; r < 16; ++r) cneg[r] = -m_new;
      }
    }

    // probabilities -> bf16 B operands (k-step ks uses registers 8*(ks%2).. of block ks/2)
    bf16x8 pb[C::PKS];
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        float e0 = __builtin_amdgcn_exp2f(s[mb][r]);
        float e1 = __builtin_amdgcn_exp2f(s[mb][r + 1]);
        bf16x2 pr = __builtin_convertvector((float __attribute__((ext_vector_type(2)))){e0, e1}, bf16x2);
        l_part = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l_part, false);
        const int ks = mb * 2 + r / 8;
        const int t = r % 8;
        pb[ks][t] = pr[0];
        pb[ks][t + 1] = pr[1];
      }
    }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int mv = 0; mv < C::MV; ++mv) {
#pragma unroll
      for (int ks = 0; ks < C::PKS; ++ks) {
        const int row_a = 16 * ks + 4 * (grp / 2) + tr_e;
        const int col = 32 * mv + 16 * (grp % 2) + 4 * tr_q;
        const int ch = col / 8, within = (col % 8) * 2;
        const char* pa = vb + row_a * (C::VCH * 16) + ((ch ^ swz<C::VCH>(row_a)) * 16) + within;
        const int row_b = row_a + 8;
        const char* pb2 = vb + row_b * (C::VCH * 16) + ((ch ^ swz<C::VCH>(row_b)) * 16) + within;
        i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(pa));
        i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(pb2));
        typedef short i16x8 __attribute__((ext_vector_type(8)));
        i16x8 cat = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        bf16x8 a = __builtin_bit_cast(bf16x8, cat);
        oacc[mv] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[ks], oacc[mv], 0, 0, 0);
      }
    }
    // same for the transposed V reads (two per MFMA)
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < C::PKS * C::MV - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);

    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    buf ^= 1;
    tc = nx;
  }

  const float l_tot = wave_sum32(l_part);
  if (w.piece >= 0 && p.piece_slot[w.piece] >= 0) {
    // ---- one piece of a split row block: unnormalised O, running max and row sum
    if (my_row < p.Sq) {
      const int lrow = my_row - w.row_blk * p.bm;
      const int lhead = wave / p.wpr;
      const int64_t slot = (int64_t)w.unit * p.n_slots + p.piece_slot[w.piece];
      float* po = p.part_o + ((slot * p.bm + lrow) * p.hpw + lhead) * DV;
#pragma unroll
      for (int mv = 0; mv < C::MV; ++mv)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4)
          *reinterpret_cast<f32x4*>(po + 32 * mv + 8 * a4 + 4 * hl) =
              f32x4{oacc[mv][a4 * 4], oacc[mv][a4 * 4 + 1], oacc[mv][a4 * 4 + 2], oacc[mv][a4 * 4 + 3]};
      if (hl == 0) {
        float* pml = p.part_ml + ((slot * p.hpw + lhead) * p.bm + lrow) * 2;
        pml[0] = m_run;
        pml[1] = l_tot;
      }
    }
    return;
  }

  // ---- epilogue: O = O / l, LSE = (m + log2 l) * ln 2
  const float inv_l = 1.f / l_tot;
  if (my_row < p.Sq) {
    __bf16* og = static_cast<__bf16*>(p.o) + (((int64_t)w.b * p.Sq + my_row) * p.Hq + head) * DV;
#pragma unroll
    for (int mv = 0; mv < C::MV; ++mv) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        bf16x4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = (__bf16)(oacc[mv][a4 * 4 + e] * inv_l);
        *reinterpret_cast<bf16x4*>(og + 32 * mv + 8 * a4 + 4 * hl) = ov;
      }
    }
    if (p.lse && hl == 0) {
      p.lse[((int64_t)w.b * p.Hq + head) * p.Sq + my_row] = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
  }
}

// ------------------------------------------------------------------------------------------
// fp32 kernel (same schedule; v_mfma_f32_32x32x2_f32, probabilities kept in fp32)
// ------------------------------------------------------------------------------------------
template <int D>
struct F32Cfg {
  static constexpr int LD = D + 1;  // padded LDS row (floats): odd stride spreads banks
  static constexpr int TILE = kBK * LD;  // floats per K or V tile
  static constexpr int STAGE = 2 * TILE;
  static constexpr int CH = D / 4;  // 16-byte chunks per row in global memory
  static constexpr int LOADS = kBK * CH / kThreads;
  static_assert(kBK * CH % kThreads == 0, "tile/thread mismatch");
  static constexpr int QK_STEPS = D / 2;
  static constexpr int MV = D / 32;
};

template <int D>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_f32_kernel(FwdParams p) {
  using C = F32Cfg<D>;
  __shared__ float lds[2 * C::STAGE];
  __shared__ int s_red[2 * kWaves];

  WorkItem w;
  if (!decode_item(p, w)) return;
  const int tid = threadIdx.x;
  const int wave = tid / 64;
  const int lane = tid % 64;
  const int hl = lane / 32;
  const int head = w.head0 + wave / p.wpr;

  int my_row, my_pos, qmin, qmax;
  row_positions(p, w, wave, lane, my_row, my_pos, qmin, qmax, s_red);
  if (qmax < 0) return;

  const float* qg = static_cast<const float*>(p.q);
  const float* kg = static_cast<const float*>(p.k);
  const float* vg = static_cast<const float*>(p.v);

  float qf[C::QK_STEPS];
  {
    int row = my_row < p.Sq ? my_row : p.Sq - 1;
    const float* qrow = qg + (((int64_t)w.b * p.Sq + row) * p.Hq + head) * D;
#pragma unroll
    for (int ks = 0; ks < C::QK_STEPS; ++ks) qf[ks] = qrow[2 * ks + hl];
  }

  const int64_t kv_row = (int64_t)p.Hkv * D;
  const float* kbase = kg + (int64_t)w.b * p.S * kv_row + (int64_t)w.g * D;
  const float* vbase = vg + (int64_t)w.b * p.S * kv_row + (int64_t)w.g * D;
  const int c = p.c;
  const int imax = min(qmax / c, 2 * p.cp - 1);

  f32x4 kst[C::LOADS];
  f32x4 vst[C::LOADS];
  auto load_tile = [&](const TileCursor& tc) {
    const int64_t prow0 = lb_chunk_offset(tc.chunk, c, p.cp) + tc.t0;
    const int nvalid = min(kBK, c - tc.t0);
#pragma unroll
    for (int u = 0; u < C::LOADS; ++u) {
      int id = tid + u * kThreads;
      int row = id / C::CH, ch = id % C::CH;
      if (row < nvalid) {
        kst[u] = *reinterpret_cast<const f32x4*>(kbase + (prow0 + row) * kv_row + ch * 4);
        vst[u] = *reinterpret_cast<const f32x4*>(vbase + (prow0 + row) * kv_row + ch * 4);
      } else {
        kst[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        vst[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  auto store_tile = [&](int b) {
    float* kb = lds + b * C::STAGE;
    float* vb = kb + C::TILE;
#pragma unroll
    for (int u = 0; u < C::LOADS; ++u) {
      int id = tid + u * kThreads;
      int row = id / C::CH, ch = id % C::CH;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kb[row * C::LD + ch * 4 + e] = kst[u][e];
        vb[row * C::LD + ch * 4 + e] = vst[u][e];
      }
    }
  };

  f32x16 oacc[C::MV];
#pragma unroll
  for (int mv = 0; mv < C::MV; ++mv) oacc[mv] = f32x16{};
  float m_run = -INFINITY;
  float l_part = 0.f;
  const float sl2 = p.scale_log2;

  TileCursor tc{0, 0};
  load_tile(tc);
  store_tile(0);
  __syncthreads();
  int buf = 0;

  while (tc.chunk <= imax) {
    TileCursor nx = tc;
    next_tile(nx, c, qmax);
    const bool has_next = nx.chunk <= imax;
    if (has_next) load_tile(nx);
    const float* kb = lds + buf * C::STAGE;
    const float* vb = kb + C::TILE;

    f32x16 s[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      f32x16 acc = {};
      const float* kr = kb + (mb * 32 + (lane & 31)) * C::LD;
#pragma unroll
      for (int ks = 0; ks < C::QK_STEPS; ++ks) {
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(kr[2 * ks + hl], qf[ks], acc, 0, 0, 0);
      }
      s[mb] = acc;
    }

    const int kpos0 = tc.chunk * c + tc.t0;
    const int nvalid = min(kBK, c - tc.t0);
    const bool need_mask = (kpos0 + kBK - 1 > qmin) || (nvalid < kBK);
    if (need_mask) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          int kk = mb * 32 + 8 * (r / 4) + 4 * hl + (r % 4);
          bool vis = (kk < nvalid) && (kpos0 + kk <= my_pos);
          s[mb][r] = vis ? s[mb][r] : -INFINITY;
        }
      }
    }

    float mt = s[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[1][r]);
    mt = wave_max32(mt) * sl2;
    const bool raise = mt > m_run + kRescaleSlack;
    if (__any(raise)) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_part *= alpha;
#pragma unroll
      for (int mv = 0; mv < C::MV; ++mv) oacc[mv] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mb][r], sl2, -m_use));
        s[mb][r] = e;
        l_part += e;
      }
    }

    // O^T += V^T P^T: MFMA (mb, r) pairs key 32mb + 8(r/4) + 4*half + r%4 with that P register
#pragma unroll
    for (int mv = 0; mv < C::MV; ++mv) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = mb * 32 + 8 * (r / 4) + 4 * hl + (r % 4);
          float a = vb[key * C::LD + 32 * mv + (lane & 31)];
          oacc[mv] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, s[mb][r], oacc[mv], 0, 0, 0);
        }
      }
    }

    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    tc = nx;
  }

  const float l_tot = wave_sum32(l_part);
  const float inv_l = 1.f / l_tot;
  if (my_row < p.Sq) {
    float* og = static_cast<float*>(p.o) + (((int64_t)w.b * p.Sq + my_row) * p.Hq + head) * D;
#pragma unroll
    for (int mv = 0; mv < C::MV; ++mv) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        f32x4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = oacc[mv][a4 * 4 + e] * inv_l;
        *reinterpret_cast<f32x4*>(og + 32 * mv + 8 * a4 + 4 * hl) = ov;
      }
    }
    if (p.lse && hl == 0) {
      p.lse[((int64_t)w.b * p.Hq + head) * p.Sq + my_row] = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
  }
}

// ------------------------------------------------------------------------------------------
// Key-range split of heavy row blocks (planned by plan_split_tiles): pieces of a cut row block
// write unnormalised partials and a merge kernel combines them by their running maxima (as the
// decode does).
// ------------------------------------------------------------------------------------------
int bf16_tile_keys(int d_qk, int d_v) { return bf16_bk(d_qk, d_v); }

constexpr int kSplitMinTiles = 8;  // no piece below this many key tiles

bool plan_split(const AttnArgs& a, const FwdParams& p, SplitPlan& sp) {
  if (a.q_pos) return false;
  return plan_split_tiles(p, bf16_tile_keys(a.d_qk, a.d_v), kSplitMinTiles, sp);
}

size_t split_workspace_bytes(const FwdParams& p, const SplitPlan& sp, int d_v) {
  return split_slot_count(p, sp) * ((size_t)p.bm * p.hpw * d_v + (size_t)p.hpw * p.bm * 2) * sizeof(float);
}

struct SplitMergeParams {
  const float* part_o;
  const float* part_ml;
  void* o;
  float* lse;
  int Sq, Hq, Hkv, G, hpw, bm, nhs, n_slots, n_split;
  unsigned char srb[kSplitMaxRb], sslot[kSplitMaxRb], scnt[kSplitMaxRb];
};

// Block (unit, cut row block, head of the slice, group of rows); thread (row, 4 dims):
// M = max_i m_i, w_i = 2^(m_i - M), O = sum_i w_i o_i / sum_i w_i l_i, LSE = (M + log2 L) ln 2.
// A piece whose keys all follow a row's position has m = -inf, l = 0 and o = 0: weight 0.
template <int DV>
__global__ __launch_bounds__(256) void attn_fwd_split_merge_kernel(SplitMergeParams m) {
  constexpr int TPR = DV / 4;
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
  const int n = m.scnt[j];
  const int64_t slot0 = (int64_t)unit * m.n_slots + m.sslot[j];
  float M = -INFINITY;
  for (int i = 0; i < n; ++i) M = fmaxf(M, m.part_ml[(((slot0 + i) * m.hpw + lh) * m.bm + lrow) * 2]);
  float L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < n; ++i) {
    const float* ml = m.part_ml + (((slot0 + i) * m.hpw + lh) * m.bm + lrow) * 2;
    const float wgt = __builtin_amdgcn_exp2f(ml[0] - M);
    L = __builtin_fmaf(wgt, ml[1], L);
    const f32x4 o = *reinterpret_cast<const f32x4*>(m.part_o + (((slot0 + i) * m.bm + lrow) * m.hpw + lh) * DV + 4 * dq);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(wgt, o[e], acc[e]);
  }
  const float inv = 1.f / L;
  bf16x4 ov;
#pragma unroll
  for (int e = 0; e < 4; ++e) ov[e] = (__bf16)(acc[e] * inv);
  *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(m.o) + (((int64_t)b * m.Sq + row) * m.Hq + head) * DV + 4 * dq) = ov;
  if (m.lse && dq == 0) m.lse[((int64_t)b * m.Hq + head) * m.Sq + row] = (M + __builtin_amdgcn_logf(L)) * kLn2;
}

}  // namespace

size_t attn_fwd_workspace_bytes(const AttnArgs& a) {
  FwdParams p = make_params(a);
  SplitPlan sp;
  if (p.n_items == 0 || !plan_split(a, p, sp)) return 0;
  return split_workspace_bytes(p, sp, a.d_v);
}

hipError_t launch_attn_fwd_bf16(const AttnArgs& a, hipStream_t stream) {
  FwdParams p = make_params(a);
  if (p.n_items == 0) return hipSuccess;
  SplitPlan sp;
  const bool split = a.ws && plan_split(a, p, sp) && a.ws_bytes >= split_workspace_bytes(p, sp, a.d_v);
  if (split) {
    apply_split(p, sp);
    p.part_o = static_cast<float*>(a.ws);
    p.part_ml = p.part_o + split_slot_count(p, sp) * p.bm * p.hpw * a.d_v;
  }
  dim3 grid((split ? p.n_items : p.per_xcd) * kNumXcd), block(kThreads);
  if (a.d_qk == 128 && a.d_v == 128) {
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<128, 128>), grid, block, 0, stream, p);
  } else if (a.d_qk == 64 && a.d_v == 64) {
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<64, 64>), grid, block, 0, stream, p);
  } else if (a.d_qk == 192 && a.d_v == 128) {
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<192, 128>), grid, block, 0, stream, p);
  } else {
    return hipErrorInvalidValue;
  }
  if (split) {
    SplitMergeParams m;
    m.part_o = p.part_o;
    m.part_ml = p.part_ml;
    m.o = a.o;
    m.lse = a.lse;
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
    const int rpb = 256 / (a.d_v / 4);
    const int64_t blocks = (int64_t)p.B * p.Hkv * p.nhs * sp.n_split * p.hpw * ((p.bm + rpb - 1) / rpb);
    if (a.d_v == 128)
      hipLaunchKernelGGL(attn_fwd_split_merge_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, stream, m);
    else
      hipLaunchKernelGGL(attn_fwd_split_merge_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, stream, m);
  }
  return hipGetLastError();
}

hipError_t launch_attn_fwd_f32(const AttnArgs& a, hipStream_t stream) {
  FwdParams p = make_params(a);
  if (p.n_items == 0) return hipSuccess;
  dim3 grid(p.per_xcd * kNumXcd), block(kThreads);
  if (a.d_qk == 64 && a.d_v == 64) {
    hipLaunchKernelGGL((attn_fwd_f32_kernel<64>), grid, block, 0, stream, p);
  } else if (a.d_qk == 128 && a.d_v == 128) {
    hipLaunchKernelGGL((attn_fwd_f32_kernel<128>), grid, block, 0, stream, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace cpattn
