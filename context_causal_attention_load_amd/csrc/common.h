// Shared helpers of the gfx950 kernels: vector types, the load-balance index, launcher
// declarations. Internal to libcpattn.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/cpattn.h"

namespace cpattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// Load-balanced order ("Add context parallelism", PR 1445, Description): 2*cp chunks of c
// tokens; rank r holds chunk r then chunk 2cp-1-r, ranks concatenated in order. Permuted slot j
// therefore holds original position src(j).
__host__ __device__ inline int64_t lb_src(int64_t j, int64_t c, int64_t cp) {
  int64_t r = j / (2 * c);
  int64_t w = j - r * 2 * c;
  return w < c ? r * c + w : (2 * cp - 1 - r) * c + (w - c);
}

// Permuted row offset of original chunk i (the inverse map at chunk granularity): chunk i < cp
// is the first half of rank i's shard; chunk i >= cp is the second half of rank 2cp-1-i's.
__host__ __device__ inline int64_t lb_chunk_offset(int64_t i, int64_t c, int64_t cp) {
  return i < cp ? i * 2 * c : (2 * cp - 1 - i) * 2 * c + c;
}

// 16-byte global -> LDS copy per lane (gfx950 global_load_lds_dwordx4) from a wave-uniform base
// plus a per-lane 32-bit byte offset: lane l's 16 bytes land at LDS address lds_wave_addr + 16*l.
// Issued through inline asm, so the compiler neither tracks nor waits for it: the caller waits
// (s_waitcnt vmcnt) before the LDS bytes are read. The base lives in scalar registers, so a
// tile's copies need no per-lane 64-bit address arithmetic.
__device__ __forceinline__ void dma16_sv(const char* base, unsigned voff, unsigned lds_wave_addr) {
  // readfirstlane yields int: both halves go through unsigned so that the low word is
  // zero-extended (a sign-extended low word would corrupt the high word of the address)
  const uint64_t a = (uint64_t)(uintptr_t)base;
  const uint64_t hi = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
  const uint64_t lo = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)a);
  const char* sbase = reinterpret_cast<const char*>((hi << 32) | lo);
  const unsigned lds_addr = __builtin_amdgcn_readfirstlane(lds_wave_addr);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_addr)
               : "memory", "m0");
}

// Number of XCDs on MI355X: consecutive workgroup ids are dealt round-robin to them, and each
// has its own L2.
constexpr int kNumXcd = 8;

// Decode work placement: a 1-D grid of decode_xcd_blocks(n_inner, hkv, batch) workgroups in
// which block id -> (inner index, kv head g, sequence b) puts every block of the pair
// p = b * hkv + g on XCD p % kNumXcd (id % kNumXcd), the pairs dealt round-robin over the XCDs
// (with hkv a multiple of kNumXcd that is XCD g % kNumXcd). The split kernels use it with
// inner = split (and head block) and the merge with inner = query head within the group, so a
// pair's partials are written and read on one XCD, and every XCD gets work even with fewer kv
// heads than XCDs. Blocks past the last pair return false.
inline int64_t decode_xcd_blocks(int n_inner, int hkv, int batch) {
  return (int64_t)kNumXcd * n_inner * (((int64_t)batch * hkv + kNumXcd - 1) / kNumXcd);
}
__device__ __forceinline__ bool decode_xcd_item(int id, int n_inner, int hkv, int batch, int& inner, int& g, int& b) {
  const int xcd = id % kNumXcd, j = id / kNumXcd;  // j enumerates (pair / kNumXcd, inner)
  inner = j % n_inner;
  const int pair = (j / n_inner) * kNumXcd + xcd;
  b = pair / hkv;
  g = pair % hkv;
  return b < batch;
}

// ---- launchers (defined in the .hip files; return the launch status) ----
hipError_t launch_permute(const void* src, void* dst, int64_t outer, int64_t seq, int64_t row_bytes,
                          int64_t cp, int64_t row_begin, int64_t row_count, bool scatter,
                          hipStream_t stream);

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* q_pos;  // may be null: positions from (cp, rank)
  void* o;
  float* lse;            // may be null
  int batch, seq, sq, hq, hkv, d_qk, d_v, cp, rank;
  float scale;
  void* ws = nullptr;     // optional workspace for the split of heavy row blocks (bf16)
  size_t ws_bytes = 0;
};
// Workspace the bf16 forward uses to split heavy row blocks (0: no split for this shape).
size_t attn_fwd_workspace_bytes(const AttnArgs& a);
hipError_t launch_attn_fwd_bf16(const AttnArgs& a, hipStream_t stream);
hipError_t launch_attn_fwd_f32(const AttnArgs& a, hipStream_t stream);

struct AttnBwdArgs {
  const void* q;          // [B, Sq, Hq, Dqk] bf16
  const void* k;          // [B, S, Hkv, Dqk] bf16, gathered order
  const void* v;          // [B, S, Hkv, Dv] bf16
  const void* o;          // [B, Sq, Hq, Dv] bf16, forward output
  const float* lse;       // [B, Hq, Sq], forward row log-sum-exp (natural log)
  const void* dout;       // [B, Sq, Hq, Dv] bf16
  const int32_t* q_pos;   // may be null: positions from (cp, rank)
  float* dq;              // [B, Sq, Hq, Dqk]
  float* dk;              // [B, S, Hkv, Dqk]
  float* dv;              // [B, S, Hkv, Dv]
  void* ws;               // at least attn_bwd_workspace_bytes(batch, sq, hq) bytes
  size_t ws_bytes;        // with attn_bwd_split_workspace_bytes(...) or more, dQ is split
  int batch, seq, sq, hq, hkv, d_qk, d_v, cp, rank;
  float scale;
};
size_t attn_bwd_workspace_bytes(int batch, int sq, int hq);
// Workspace with which the backward also splits the dq kernel's heavy row blocks (small grids,
// the rank's own shard); attn_bwd_workspace_bytes when the shape is not split.
size_t attn_bwd_split_workspace_bytes(const AttnBwdArgs& a);
hipError_t launch_attn_bwd_bf16(const AttnBwdArgs& a, hipStream_t stream);

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* lengths;
  void* o;
  float* lse;
  float* ws;  // split partials [B, Hq, nsplit, d + 2]
  int batch, hq, hkv, d, max_len, nsplit, split_len;
  float scale;
};
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t stream);

struct DecodeMergeArgs {
  const void* o_parts;     // [parts, batch, hq, d]
  const float* lse_parts;  // [parts, batch, hq]
  void* o;                 // [batch, hq, d]
  float* lse;              // [batch, hq], may be null
  int parts, batch, hq, d;
  bool bf16;
};
hipError_t launch_decode_merge(const DecodeMergeArgs& a, hipStream_t stream);

struct DecodeInt8Args {
  const void* q;          // bf16 [batch, hq, 128]
  const int8_t* k;        // [batch, hkv, max_len, 128] codes
  const int8_t* v;
  const float* k_scale;   // [batch, hkv, max_len] one scale per cached row
  const float* v_scale;
  const int32_t* lengths;
  void* o;                // bf16 [batch, hq, 128]
  float* lse;             // may be null
  float* ws;              // split partials, as for DecodeArgs
  int batch, hq, hkv, max_len;
  float scale;
};
hipError_t launch_decode_int8(const DecodeInt8Args& a, hipStream_t stream);
hipError_t launch_kv_quantize(const void* x, int8_t* codes, float* scales, int64_t rows, int d, bool bf16,
                              hipStream_t stream);
// Second decode pass alone: merges the split partials in ws into o (bf16 or fp32) and lse.
hipError_t launch_decode_split_merge(const int32_t* lengths, float* ws, void* o, float* lse, int batch, int hq,
                                     int hkv, int max_len, int d, bool bf16, hipStream_t stream);

// Decode split geometry, shared by the workspace-size query and the launcher. The workspace
// holds the split partials [batch, hq, nsplit, d + 2] in float32: d unnormalised outputs, then
// the split's max and sum (log2 units).
constexpr int kDecodeSplitLen = 256;
inline int decode_nsplit(int max_len) { return (max_len + kDecodeSplitLen - 1) / kDecodeSplitLen; }
// A short cache (a length slice of an inference context-parallel job, say) has too few 256-key
// splits to fill the part, so the v_dot2 decode kernels take 128-key splits up to this length.
constexpr int kDecodeShortSplitLen = 128;
constexpr int kDecodeShortMaxLen = 1024;
inline bool decode_short_cache(int max_len) { return max_len <= kDecodeShortMaxLen; }
// Split partials a decode workspace must hold per (sequence, query head): the most any path takes.
inline int decode_ws_nsplit(int max_len) {
  return decode_short_cache(max_len) ? (max_len + kDecodeShortSplitLen - 1) / kDecodeShortSplitLen
                                     : decode_nsplit(max_len);
}

// Size of the file-scope device array that replaces the caller workspace in the
// allocation-free decode call (one copy per GPU, held until the process ends).
constexpr size_t kDecodeNoAllocScratchBytes = CPATTN_DECODE_NOALLOC_SCRATCH_BYTES;
// Device address of that array on the current GPU (looked up once per device).
hipError_t decode_noalloc_scratch(void** out);

}  // namespace cpattn
