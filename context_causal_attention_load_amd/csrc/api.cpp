// C ABI of libcpattn.so (declared in include/cpattn.h): host-side validation, then launches on
// the caller's stream. Every check runs before the first HIP call, so argument errors are
// reported without touching a device.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/cpattn.h"
#include "common.h"

using namespace cpattn;

namespace {

thread_local std::string g_last_error = "no error";

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(CPA_EHIP, "%s: HIP error %d (%s)", where, (int)e, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// The kernels are written for gfx950 only: refuse any other device instead of running them.
int check_device(const char* where) {
  static std::mutex mu;
  static int cached[64];  // 0 unknown, 1 ok, -1 unsupported
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, where);
  if (dev < 0 || dev >= 64) return fail(CPA_ENOTSUP, "%s: device index %d out of range", where, dev);
  std::lock_guard<std::mutex> lk(mu);
  if (cached[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e, where);
    cached[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    if (cached[dev] < 0) {
      return fail(CPA_ENOTSUP, "%s: device %d is %s; this library runs on gfx950 (MI355X) only", where,
                  dev, prop.gcnArchName);
    }
  }
  if (cached[dev] < 0) return fail(CPA_ENOTSUP, "%s: device %d is not gfx950", where, dev);
  return CPA_OK;
}

int check_lb(const char* where, int64_t seq, int32_t cp) {
  if (cp < 1) return fail(CPA_EINVAL, "%s: cp must be >= 1 (got %d)", where, cp);
  if (seq < 1) return fail(CPA_EINVAL, "%s: seq must be >= 1 (got %lld)", where, (long long)seq);
  if (seq % (2 * (int64_t)cp) != 0)
    return fail(CPA_EINVAL, "%s: seq (%lld) must be a multiple of 2*cp (%lld)", where, (long long)seq,
                (long long)(2 * (int64_t)cp));
  return CPA_OK;
}

int permute_common(const char* where, const void* src, void* dst, int64_t outer, int64_t seq,
                   int64_t row_bytes, int32_t cp, int64_t row_begin, int64_t row_count, bool scatter,
                   void* stream) {
  int rc = check_lb(where, seq, cp);
  if (rc) return rc;
  if (seq >= (int64_t(1) << 31)) return fail(CPA_EINVAL, "%s: seq must be < 2^31", where);
  if (outer < 0) return fail(CPA_EINVAL, "%s: outer must be >= 0", where);
  if (row_bytes < 1) return fail(CPA_EINVAL, "%s: row_bytes must be >= 1", where);
  if (row_begin < 0 || row_count < 0 || row_begin + row_count > seq)
    return fail(CPA_EINVAL, "%s: window [%lld, %lld) outside [0, %lld)", where, (long long)row_begin,
                (long long)(row_begin + row_count), (long long)seq);
  if (outer > 0 && outer * row_count >= (int64_t(1) << 31))
    return fail(CPA_EINVAL, "%s: outer * row_count must be < 2^31", where);
  if (outer == 0 || row_count == 0) return CPA_OK;
  if (!src || !dst) return fail(CPA_EINVAL, "%s: null tensor pointer", where);
  // the two buffers must not overlap
  const char* s0 = static_cast<const char*>(src);
  const char* d0 = static_cast<const char*>(dst);
  int64_t src_bytes = outer * (scatter ? row_count : seq) * row_bytes;
  int64_t dst_bytes = outer * (scatter ? seq : row_count) * row_bytes;
  if (s0 < d0 + dst_bytes && d0 < s0 + src_bytes) return fail(CPA_EINVAL, "%s: src and dst overlap", where);
  rc = check_device(where);
  if (rc) return rc;
  hipError_t e = launch_permute(src, dst, outer, seq, row_bytes, cp, row_begin, row_count, scatter,
                                static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, where);
  return CPA_OK;
}

}  // namespace

extern "C" {

const char* cpattn_last_error(void) { return g_last_error.c_str(); }

int64_t cp_load_balance_source_index(int64_t seq, int32_t cp, int64_t j) {
  if (cp < 1 || seq < 1 || seq % (2 * (int64_t)cp) != 0 || j < 0 || j >= seq) return -1;
  return lb_src(j, seq / (2 * (int64_t)cp), cp);
}

int cp_load_balance_positions(int64_t seq, int32_t cp, int64_t row_begin, int64_t row_count,
                              int32_t* out_host) {
  const char* where = "cp_load_balance_positions";
  int rc = check_lb(where, seq, cp);
  if (rc) return rc;
  if (seq >= (int64_t(1) << 31)) return fail(CPA_EINVAL, "%s: seq must be < 2^31", where);
  if (row_begin < 0 || row_count < 0 || row_begin + row_count > seq)
    return fail(CPA_EINVAL, "%s: window outside [0, seq)", where);
  if (row_count > 0 && !out_host) return fail(CPA_EINVAL, "%s: null output", where);
  const int64_t c = seq / (2 * (int64_t)cp);
  for (int64_t i = 0; i < row_count; ++i) out_host[i] = (int32_t)lb_src(row_begin + i, c, cp);
  return CPA_OK;
}

int cp_load_balance_permute(const void* src, void* dst, int64_t outer, int64_t seq, int64_t row_bytes,
                            int32_t cp, int64_t row_begin, int64_t row_count, void* stream) {
  return permute_common("cp_load_balance_permute", src, dst, outer, seq, row_bytes, cp, row_begin,
                        row_count, false, stream);
}

int cp_load_balance_unpermute(const void* src, void* dst, int64_t outer, int64_t seq, int64_t row_bytes,
                              int32_t cp, int64_t row_begin, int64_t row_count, void* stream) {
  return permute_common("cp_load_balance_unpermute", src, dst, outer, seq, row_bytes, cp, row_begin,
                        row_count, true, stream);
}

}  // extern "C"

namespace {

// Checks shared by the forward calls and the workspace query: CPA_OK or the failing status.
int fwd_shape_checks(const char* where, int32_t batch, int32_t seq, int32_t sq, int32_t hq, int32_t hkv,
                     int32_t d_qk, int32_t d_v, int32_t dtype, int32_t cp, int32_t rank, bool positions_given) {
  int rc = check_lb(where, seq, cp);
  if (rc) return rc;
  if (rank < 0 || rank >= cp) return fail(CPA_EINVAL, "%s: rank %d outside [0, %d)", where, rank, cp);
  if (batch < 0 || sq < 0) return fail(CPA_EINVAL, "%s: batch and sq must be >= 0", where);
  if (hq < 1 || hkv < 1 || hq % hkv != 0)
    return fail(CPA_EINVAL, "%s: hq (%d) must be a positive multiple of hkv (%d)", where, hq, hkv);
  if (!positions_given && sq != seq / cp)
    return fail(CPA_EINVAL, "%s: without q_positions, sq (%d) must equal seq/cp (%d)", where, sq, seq / cp);
  if (dtype != CPA_F32 && dtype != CPA_BF16) return fail(CPA_EINVAL, "%s: unknown dtype %d", where, dtype);
  bool supported = dtype == CPA_BF16 ? ((d_qk == 64 && d_v == 64) || (d_qk == 128 && d_v == 128) ||
                                         (d_qk == 192 && d_v == 128))
                                      : ((d_qk == 64 && d_v == 64) || (d_qk == 128 && d_v == 128));
  if (!supported)
    return fail(CPA_ENOTSUP, "%s: (dtype %d, d_qk %d, d_v %d) not supported", where, dtype, d_qk, d_v);
  const int64_t elt = dtype == CPA_BF16 ? 2 : 4;
  if ((int64_t)batch * seq * hkv * d_qk * elt >= (int64_t(1) << 40))
    return fail(CPA_EINVAL, "%s: tensor too large", where);
  return CPA_OK;
}

AttnArgs fwd_args(const void* q_shard, const void* k, const void* v, const int32_t* q_positions, void* o, float* lse,
                  int32_t batch, int32_t seq, int32_t sq, int32_t hq, int32_t hkv, int32_t d_qk, int32_t d_v,
                  float softmax_scale, int32_t cp, int32_t rank) {
  AttnArgs a;
  a.q = q_shard;
  a.k = k;
  a.v = v;
  a.q_pos = q_positions;
  a.o = o;
  a.lse = lse;
  a.batch = batch;
  a.seq = seq;
  a.sq = sq;
  a.hq = hq;
  a.hkv = hkv;
  a.d_qk = d_qk;
  a.d_v = d_v;
  a.cp = cp;
  a.rank = rank;
  a.scale = softmax_scale;
  return a;
}

int fwd_checked(const char* where, const void* q_shard, const void* k, const void* v, const int32_t* q_positions,
                void* o, float* lse, int32_t batch, int32_t seq, int32_t sq, int32_t hq, int32_t hkv, int32_t d_qk,
                int32_t d_v, int32_t dtype, float softmax_scale, int32_t cp, int32_t rank, void* workspace,
                size_t workspace_bytes, void* stream) {
  int rc = fwd_shape_checks(where, batch, seq, sq, hq, hkv, d_qk, d_v, dtype, cp, rank, q_positions != nullptr);
  if (rc) return rc;
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
    return fail(CPA_EINVAL, "%s: softmax_scale must be finite and > 0", where);
  if (batch == 0 || sq == 0) return CPA_OK;
  if (!q_shard || !k || !v || !o) return fail(CPA_EINVAL, "%s: null tensor pointer", where);
  if (!aligned16(q_shard) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(CPA_EINVAL, "%s: q, k, v and o must be 16-byte aligned", where);
  if (lse && ((uintptr_t)lse & 3u)) return fail(CPA_EINVAL, "%s: lse must be 4-byte aligned", where);
  if (q_positions && ((uintptr_t)q_positions & 3u))
    return fail(CPA_EINVAL, "%s: q_positions must be 4-byte aligned", where);
  if (workspace && !aligned16(workspace)) return fail(CPA_EINVAL, "%s: workspace must be 16-byte aligned", where);
  rc = check_device(where);
  if (rc) return rc;
  AttnArgs a = fwd_args(q_shard, k, v, q_positions, o, lse, batch, seq, sq, hq, hkv, d_qk, d_v, softmax_scale, cp,
                        rank);
  a.ws = workspace;
  a.ws_bytes = workspace ? workspace_bytes : 0;
  hipError_t e = dtype == CPA_BF16 ? launch_attn_fwd_bf16(a, static_cast<hipStream_t>(stream))
                                   : launch_attn_fwd_f32(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, where);
  return CPA_OK;
}

}  // namespace

extern "C" {

int cp_attention_fwd(const void* q_shard, const void* k, const void* v, const int32_t* q_positions, void* o,
                     float* lse, int32_t batch, int32_t seq, int32_t sq, int32_t hq, int32_t hkv, int32_t d_qk,
                     int32_t d_v, int32_t dtype, float softmax_scale, int32_t cp, int32_t rank, void* stream) {
  return fwd_checked("cp_attention_fwd", q_shard, k, v, q_positions, o, lse, batch, seq, sq, hq, hkv, d_qk, d_v,
                     dtype, softmax_scale, cp, rank, nullptr, 0, stream);
}

size_t cp_attention_fwd_workspace_bytes(int32_t batch, int32_t seq, int32_t hq, int32_t hkv, int32_t d_qk,
                                        int32_t d_v, int32_t dtype, int32_t cp, int32_t rank) {
  if (cp < 1 || seq < 1 || seq % (2 * (int64_t)cp) != 0) return 0;
  if (fwd_shape_checks("cp_attention_fwd_workspace_bytes", batch, seq, seq / cp, hq, hkv, d_qk, d_v, dtype, cp,
                       rank, false) != CPA_OK)
    return 0;
  if (dtype != CPA_BF16 || batch == 0) return 0;
  AttnArgs a = fwd_args(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, batch, seq, seq / cp, hq, hkv, d_qk,
                        d_v, 1.f, cp, rank);
  return attn_fwd_workspace_bytes(a);
}

int cp_attention_fwd_ws(const void* q_shard, const void* k, const void* v, const int32_t* q_positions, void* o,
                        float* lse, int32_t batch, int32_t seq, int32_t sq, int32_t hq, int32_t hkv, int32_t d_qk,
                        int32_t d_v, int32_t dtype, float softmax_scale, int32_t cp, int32_t rank, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return fwd_checked("cp_attention_fwd_ws", q_shard, k, v, q_positions, o, lse, batch, seq, sq, hq, hkv, d_qk, d_v,
                     dtype, softmax_scale, cp, rank, workspace, workspace_bytes, stream);
}

size_t cp_attention_bwd_workspace_bytes(int32_t batch, int32_t sq, int32_t hq) {
  if (batch <= 0 || sq <= 0 || hq <= 0) return 0;
  return attn_bwd_workspace_bytes(batch, sq, hq);
}

size_t cp_attention_bwd_split_workspace_bytes(int32_t batch, int32_t seq, int32_t hq, int32_t hkv, int32_t d_qk,
                                              int32_t d_v, int32_t dtype, int32_t cp, int32_t rank) {
  if (cp < 1 || seq < 1 || seq % (2 * (int64_t)cp) != 0) return 0;
  if (fwd_shape_checks("cp_attention_bwd_split_workspace_bytes", batch, seq, seq / cp, hq, hkv, d_qk, d_v, dtype, cp,
                       rank, false) != CPA_OK)
    return 0;
  if (dtype != CPA_BF16 || batch == 0) return 0;
  AttnBwdArgs a{};
  a.batch = batch;
  a.seq = seq;
  a.sq = seq / cp;
  a.hq = hq;
  a.hkv = hkv;
  a.d_qk = d_qk;
  a.d_v = d_v;
  a.cp = cp;
  a.rank = rank;
  a.scale = 1.f;
  return attn_bwd_split_workspace_bytes(a);
}

int cp_attention_bwd(const void* q_shard, const void* k, const void* v, const void* o, const float* lse,
                     const void* d_o, const int32_t* q_positions, float* dq, float* dk, float* dv, int32_t batch,
                     int32_t seq, int32_t sq, int32_t hq, int32_t hkv, int32_t d_qk, int32_t d_v, int32_t dtype,
                     float softmax_scale, int32_t cp, int32_t rank, void* workspace, size_t workspace_bytes,
                     void* stream) {
  const char* where = "cp_attention_bwd";
  int rc = check_lb(where, seq, cp);
  if (rc) return rc;
  if (rank < 0 || rank >= cp) return fail(CPA_EINVAL, "%s: rank %d outside [0, %d)", where, rank, cp);
  if (batch < 0 || sq < 0) return fail(CPA_EINVAL, "%s: batch and sq must be >= 0", where);
  if (hq < 1 || hkv < 1 || hq % hkv != 0)
    return fail(CPA_EINVAL, "%s: hq (%d) must be a positive multiple of hkv (%d)", where, hq, hkv);
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
    return fail(CPA_EINVAL, "%s: softmax_scale must be finite and > 0", where);
  if (!q_positions && sq != seq / cp)
    return fail(CPA_EINVAL, "%s: without q_positions, sq (%d) must equal seq/cp (%d)", where, sq, seq / cp);
  if (dtype != CPA_F32 && dtype != CPA_BF16) return fail(CPA_EINVAL, "%s: unknown dtype %d", where, dtype);
  if (dtype != CPA_BF16 || !((d_qk == 64 && d_v == 64) || (d_qk == 128 && d_v == 128) || (d_qk == 192 && d_v == 128)))
    return fail(CPA_ENOTSUP, "%s: (dtype %d, d_qk %d, d_v %d) not supported (bf16 with 64/64, 128/128, 192/128)",
                where, dtype, d_qk, d_v);
  if ((int64_t)batch * seq * hkv * d_qk * 4 >= (int64_t(1) << 40) ||
      (int64_t)batch * sq * hq * d_qk * 4 >= (int64_t(1) << 40) || (int64_t)hq * d_qk * 2 * 32 >= (int64_t(1) << 31))
    return fail(CPA_EINVAL, "%s: tensor too large", where);
  if (batch == 0 || sq == 0) return CPA_OK;
  if (!q_shard || !k || !v || !o || !lse || !d_o || !dq || !dk || !dv || !workspace)
    return fail(CPA_EINVAL, "%s: null pointer", where);
  if (!aligned16(q_shard) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(d_o) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv) || !aligned16(workspace))
    return fail(CPA_EINVAL, "%s: tensors and workspace must be 16-byte aligned", where);
  if (((uintptr_t)lse & 3u) || (q_positions && ((uintptr_t)q_positions & 3u)))
    return fail(CPA_EINVAL, "%s: lse and q_positions must be 4-byte aligned", where);
  const size_t need = cp_attention_bwd_workspace_bytes(batch, sq, hq);
  if (workspace_bytes < need)
    return fail(CPA_EINVAL, "%s: workspace of %zu bytes, need %zu", where, workspace_bytes, need);
  rc = check_device(where);
  if (rc) return rc;
  AttnBwdArgs a;
  a.q = q_shard;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = d_o;
  a.q_pos = q_positions;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.ws = workspace;
  a.ws_bytes = workspace_bytes;
  a.batch = batch;
  a.seq = seq;
  a.sq = sq;
  a.hq = hq;
  a.hkv = hkv;
  a.d_qk = d_qk;
  a.d_v = d_v;
  a.cp = cp;
  a.rank = rank;
  a.scale = softmax_scale;
  hipError_t e = launch_attn_bwd_bf16(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, where);
  return CPA_OK;
}

size_t gqa_decode_workspace_bytes(int32_t batch, int32_t hq, int32_t hkv, int32_t max_len, int32_t d) {
  if (batch <= 0 || hq <= 0 || hkv <= 0 || max_len <= 0 || d <= 0) return 0;
  return (size_t)batch * hq * decode_ws_nsplit(max_len) * (size_t)(d + 2) * sizeof(float);
}

}  // extern "C"

namespace {

// Checks and launch shared by the two bf16/fp32 decode entry points: `workspace` is the caller's
// buffer or the library's static scratch.
int decode_checked(const char* where, const void* q, const void* k_cache, const void* v_cache, const int32_t* lengths,
                   void* o, float* lse, int32_t batch, int32_t hq, int32_t hkv, int32_t d, int32_t max_len,
                   int32_t dtype, float softmax_scale, bool noalloc, void* workspace, size_t workspace_bytes,
                   void* stream) {
  if (batch < 0) return fail(CPA_EINVAL, "%s: batch must be >= 0", where);
  if (hq < 1 || hkv < 1 || hq % hkv != 0)
    return fail(CPA_EINVAL, "%s: hq (%d) must be a positive multiple of hkv (%d)", where, hq, hkv);
  if (max_len < 1) return fail(CPA_EINVAL, "%s: max_len must be >= 1", where);
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
    return fail(CPA_EINVAL, "%s: softmax_scale must be finite and > 0", where);
  if (dtype != CPA_F32 && dtype != CPA_BF16) return fail(CPA_EINVAL, "%s: unknown dtype %d", where, dtype);
  if (d != 64 && d != 128) return fail(CPA_ENOTSUP, "%s: head dim %d not supported (64, 128)", where, d);
  if (batch == 0) return CPA_OK;
  if ((int64_t)batch * hkv * max_len * d >= (int64_t(1) << 40)) return fail(CPA_EINVAL, "%s: cache too large", where);
  if (!q || !k_cache || !v_cache || !lengths || !o || (!noalloc && !workspace))
    return fail(CPA_EINVAL, "%s: null pointer", where);
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) ||
      (!noalloc && !aligned16(workspace)))
    return fail(CPA_EINVAL, "%s: q, caches, o and workspace must be 16-byte aligned", where);
  if (((uintptr_t)lengths & 3u) || (lse && ((uintptr_t)lse & 3u)))
    return fail(CPA_EINVAL, "%s: lengths and lse must be 4-byte aligned", where);
  const size_t need = gqa_decode_workspace_bytes(batch, hq, hkv, max_len, d);
  if (noalloc) {
    if (need > kDecodeNoAllocScratchBytes)
      return fail(CPA_EINVAL,
                  "%s: this call needs %zu bytes of split partials (batch %d x hq %d x %d splits x (d + 2) floats), "
                  "more than the library's static scratch of %zu bytes; use gqa_decode_attention with a workspace",
                  where, need, batch, hq, decode_ws_nsplit(max_len), (size_t)kDecodeNoAllocScratchBytes);
  } else if (workspace_bytes < need) {
    return fail(CPA_EINVAL, "%s: workspace of %zu bytes, need %zu", where, workspace_bytes, need);
  }
  int rc = check_device(where);
  if (rc) return rc;
  if (noalloc) {
    hipError_t e = decode_noalloc_scratch(&workspace);
    if (e != hipSuccess) return hip_fail(e, where);
  }
  DecodeArgs a;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.lengths = lengths;
  a.o = o;
  a.lse = lse;
  a.ws = static_cast<float*>(workspace);
  a.batch = batch;
  a.hq = hq;
  a.hkv = hkv;
  a.d = d;
  a.max_len = max_len;
  a.nsplit = decode_nsplit(max_len);
  a.split_len = kDecodeSplitLen;
  a.scale = softmax_scale;
  hipError_t e = dtype == CPA_BF16 ? launch_decode_bf16(a, static_cast<hipStream_t>(stream))
                                   : launch_decode_f32(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, where);
  return CPA_OK;
}

}  // namespace

extern "C" {

int gqa_decode_attention(const void* q, const void* k_cache, const void* v_cache, const int32_t* lengths,
                         void* o, float* lse, int32_t batch, int32_t hq, int32_t hkv, int32_t d,
                         int32_t max_len, int32_t dtype, float softmax_scale, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return decode_checked("gqa_decode_attention", q, k_cache, v_cache, lengths, o, lse, batch, hq, hkv, d, max_len,
                        dtype, softmax_scale, false, workspace, workspace_bytes, stream);
}

int gqa_decode_attention_noalloc(const void* q, const void* k_cache, const void* v_cache, const int32_t* lengths,
                                 void* o, float* lse, int32_t batch, int32_t hq, int32_t hkv, int32_t d,
                                 int32_t max_len, int32_t dtype, float softmax_scale, void* stream) {
  return decode_checked("gqa_decode_attention_noalloc", q, k_cache, v_cache, lengths, o, lse, batch, hq, hkv, d,
                        max_len, dtype, softmax_scale, true, nullptr, 0, stream);
}

int gqa_decode_attention_int8kv(const void* q, const int8_t* k_codes, const int8_t* v_codes,
                                const float* k_scales, const float* v_scales, const int32_t* lengths, void* o,
                                float* lse, int32_t batch, int32_t hq, int32_t hkv, int32_t d, int32_t max_len,
                                float softmax_scale, void* workspace, size_t workspace_bytes, void* stream) {
  const char* where = "gqa_decode_attention_int8kv";
  if (batch < 0) return fail(CPA_EINVAL, "%s: batch must be >= 0", where);
  if (hq < 1 || hkv < 1 || hq % hkv != 0)
    return fail(CPA_EINVAL, "%s: hq (%d) must be a positive multiple of hkv (%d)", where, hq, hkv);
  if (max_len < 1) return fail(CPA_EINVAL, "%s: max_len must be >= 1", where);
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
    return fail(CPA_EINVAL, "%s: softmax_scale must be finite and > 0", where);
  if (d != 128) return fail(CPA_ENOTSUP, "%s: head dim %d not supported (128)", where, d);
  if (batch == 0) return CPA_OK;
  const int64_t head_blocks = (int64_t)hkv * ((hq / hkv + 15) / 16);
  if (batch > 65535 || head_blocks > 65535)
    return fail(CPA_EINVAL, "%s: batch and hkv * ceil(G / 16) must be <= 65535", where);
  if ((int64_t)batch * hkv * max_len * d >= (int64_t(1) << 40)) return fail(CPA_EINVAL, "%s: cache too large", where);
  if (!q || !k_codes || !v_codes || !k_scales || !v_scales || !lengths || !o || !workspace)
    return fail(CPA_EINVAL, "%s: null pointer", where);
  if (!aligned16(q) || !aligned16(k_codes) || !aligned16(v_codes) || !aligned16(o) || !aligned16(workspace))
    return fail(CPA_EINVAL, "%s: q, code caches, o and workspace must be 16-byte aligned", where);
  if (((uintptr_t)k_scales & 3u) || ((uintptr_t)v_scales & 3u) || ((uintptr_t)lengths & 3u) ||
      (lse && ((uintptr_t)lse & 3u)))
    return fail(CPA_EINVAL, "%s: scales, lengths and lse must be 4-byte aligned", where);
  size_t need = gqa_decode_workspace_bytes(batch, hq, hkv, max_len, d);
  if (workspace_bytes < need)
    return fail(CPA_EINVAL, "%s: workspace of %zu bytes, need %zu", where, workspace_bytes, need);
  int rc = check_device(where);
  if (rc) return rc;
  DecodeInt8Args a;
  a.q = q;
  a.k = k_codes;
  a.v = v_codes;
  a.k_scale = k_scales;
  a.v_scale = v_scales;
  a.lengths = lengths;
  a.o = o;
  a.lse = lse;
  a.ws = static_cast<float*>(workspace);
  a.batch = batch;
  a.hq = hq;
  a.hkv = hkv;
  a.max_len = max_len;
  a.scale = softmax_scale;
  hipError_t e = launch_decode_int8(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, where);
  return CPA_OK;
}

int kv_cache_quantize_int8(const void* x, int8_t* codes, float* scales, int64_t rows, int32_t d, int32_t dtype,
                           void* stream) {
  const char* where = "kv_cache_quantize_int8";
  if (rows < 0) return fail(CPA_EINVAL, "%s: rows must be >= 0", where);
  if (d < 1) return fail(CPA_EINVAL, "%s: d must be >= 1", where);
  if (dtype != CPA_F32 && dtype != CPA_BF16) return fail(CPA_EINVAL, "%s: unknown dtype %d", where, dtype);
  if (rows == 0) return CPA_OK;
  if (rows >= (int64_t(1) << 33) || rows * d >= (int64_t(1) << 40))
    return fail(CPA_EINVAL, "%s: rows * d too large", where);
  if (!x || !codes || !scales) return fail(CPA_EINVAL, "%s: null pointer", where);
  const uintptr_t elem = dtype == CPA_BF16 ? 1u : 3u;
  if (((uintptr_t)x & elem) || ((uintptr_t)scales & 3u))
    return fail(CPA_EINVAL, "%s: x and scales must be aligned to their element size", where);
  int rc = check_device(where);
  if (rc) return rc;
  hipError_t e = launch_kv_quantize(x, codes, scales, rows, d, dtype == CPA_BF16, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, where);
  return CPA_OK;
}

int gqa_decode_merge(const void* o_parts, const float* lse_parts, void* o, float* lse, int32_t parts,
                     int32_t batch, int32_t hq, int32_t d, int32_t dtype, void* stream) {
  const char* where = "gqa_decode_merge";
  if (parts < 1) return fail(CPA_EINVAL, "%s: parts must be >= 1", where);
  if (batch < 0 || hq < 0) return fail(CPA_EINVAL, "%s: batch and hq must be >= 0", where);
  if (d < 1) return fail(CPA_EINVAL, "%s: d must be >= 1", where);
  if (dtype != CPA_F32 && dtype != CPA_BF16) return fail(CPA_EINVAL, "%s: unknown dtype %d", where, dtype);
  if (batch == 0 || hq == 0) return CPA_OK;
  if ((int64_t)batch * hq >= (int64_t(1) << 31)) return fail(CPA_EINVAL, "%s: batch * hq too large", where);
  if ((int64_t)parts * batch * hq * d >= (int64_t(1) << 40)) return fail(CPA_EINVAL, "%s: parts too large", where);
  if (!o_parts || !lse_parts || !o) return fail(CPA_EINVAL, "%s: null pointer", where);
  const uintptr_t elem = dtype == CPA_BF16 ? 1u : 3u;
  if (((uintptr_t)o_parts & elem) || ((uintptr_t)o & elem) || ((uintptr_t)lse_parts & 3u) ||
      (lse && ((uintptr_t)lse & 3u)))
    return fail(CPA_EINVAL, "%s: pointers must be aligned to their element size", where);
  int rc = check_device(where);
  if (rc) return rc;
  DecodeMergeArgs a;
  a.o_parts = o_parts;
  a.lse_parts = lse_parts;
  a.o = o;
  a.lse = lse;
  a.parts = parts;
  a.batch = batch;
  a.hq = hq;
  a.d = d;
  a.bf16 = dtype == CPA_BF16;
  hipError_t e = launch_decode_merge(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, where);
  return CPA_OK;
}

}  // extern "C"
