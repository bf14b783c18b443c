// Host side of the C ABI: argument validation, status codes, thread-local
// error text and dispatch to the kernels.  Nothing here allocates device
// memory or synchronises a stream.
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/tokengate.h"
#include "common.h"

namespace {

thread_local char g_err[512] = "";

tg_status fail(tg_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

tg_status ok() {
  g_err[0] = '\0';
  return TG_OK;
}

tg_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(TG_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

static_assert(tg::kSelScratchBytes == TG_SELECT_SCRATCH_BYTES, "scratch size");

namespace {
// the selection with its contract checks when they are on: offsets and
// budgets before, the kept count against the capacity after
hipError_t select_checked(const float* b, const uint8_t* pr, const int32_t* cu, const int32_t* k,
                          int n_seq, int64_t t_in, int64_t cap, int32_t* kept_idx,
                          int32_t* kept_pos, float* kept_b, int32_t* kept_cu, void* ws,
                          hipStream_t st) {
  const bool chk = tg::contract_checks_on();
  hipError_t e = hipSuccess;
  if (chk) {
    e = tg::contract_offsets(cu, n_seq, t_in, TG_CONTRACT_OFFSETS, st);
    if (e == hipSuccess) e = tg::contract_budgets(k, n_seq, st);
    if (e != hipSuccess) return e;
  }
  e = tg::launch_select(b, pr, cu, k, n_seq, t_in, cap, kept_idx, kept_pos, kept_b, kept_cu, ws, st);
  if (e == hipSuccess && chk) e = tg::contract_capacity(kept_cu, n_seq, cap, st);
  return e;
}
}  // namespace

hipError_t tg::device_cu_count(int* n_cu) {
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool cached = dev >= 0 && dev < kMaxDevices;
  if (cached) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *n_cu = c;
      return hipSuccess;
    }
  }
  e = hipDeviceGetAttribute(n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (*n_cu < 1) *n_cu = 1;
  if (cached) cache[dev].store(*n_cu, std::memory_order_relaxed);
  return hipSuccess;
}

extern "C" {

const char* tg_status_string(int s) {
  switch (s) {
    case TG_OK: return "TG_OK";
    case TG_ERR_INVALID_ARG: return "TG_ERR_INVALID_ARG";
    case TG_ERR_UNSUPPORTED: return "TG_ERR_UNSUPPORTED";
    case TG_ERR_WORKSPACE: return "TG_ERR_WORKSPACE";
    case TG_ERR_HIP: return "TG_ERR_HIP";
    default: return "TG_UNKNOWN_STATUS";
  }
}

const char* tg_last_error(void) { return g_err; }

int tg_version(void) { return 10600; }

// ----------------------------------------------------------------- score
size_t tg_score_workspace_size(int64_t t_in, int32_t n_seq) {
  if (t_in < 0 || n_seq < 0) return 0;
  return tg::score_ws_bytes(t_in, n_seq);
}

tg_status tg_score(const void* x, tg_dtype dt, int64_t x_row_stride, int64_t t_in, int32_t d,
                   int32_t h, const void* w1, const float* b1, const float* w2, float b2,
                   const uint8_t* prunable, const int32_t* cu_seqlens, int32_t n_seq, float eps,
                   float norm_eps, float* b_raw, float* b, void* ws, size_t ws_bytes,
                   tg_stream stream) {
  if (t_in < 0 || n_seq < 1 || d < 1 || h < 1)
    return fail(TG_ERR_INVALID_ARG, "tg_score: need t_in >= 0, n_seq >= 1, d >= 1, h >= 1");
  if (t_in > INT32_MAX - 4096) return fail(TG_ERR_UNSUPPORTED, "tg_score: t_in too large");
  if (!(eps >= 0.0f)) return fail(TG_ERR_INVALID_ARG, "tg_score: eps must be >= 0");
  if (norm_eps != norm_eps) return fail(TG_ERR_INVALID_ARG, "tg_score: norm_eps is NaN");
  if (dt != TG_F32 && dt != TG_BF16) return fail(TG_ERR_INVALID_ARG, "tg_score: bad dtype");
  if (x_row_stride < d) return fail(TG_ERR_INVALID_ARG, "tg_score: x_row_stride < d");
  if (!cu_seqlens || !w2 || !b || !ws) return fail(TG_ERR_INVALID_ARG, "tg_score: null pointer");
  if (t_in > 0 && (!x || !w1 || !prunable))
    return fail(TG_ERR_INVALID_ARG, "tg_score: null pointer");
  const size_t es = dt == TG_BF16 ? 2 : 4;
  if (dt == TG_BF16) {
    if (d % 64 != 0 || h % 32 != 0 || h > 256)
      return fail(TG_ERR_UNSUPPORTED, "tg_score: bf16 needs d %% 64 == 0, h %% 32 == 0, h <= 256");
    if (x_row_stride >= ((int64_t)1 << 22))     // 256 rows of 32-bit buffer offsets
      return fail(TG_ERR_UNSUPPORTED, "tg_score: bf16 needs x_row_stride < 2^22");
  } else if (h > 1024) {
    return fail(TG_ERR_UNSUPPORTED, "tg_score: f32 needs h <= 1024");
  }
  if ((x && !aligned(x, 16)) || (w1 && !aligned(w1, 16)) || ((x_row_stride * es) % 16) != 0 ||
      ((d * es) % 16) != 0)
    return fail(TG_ERR_UNSUPPORTED, "tg_score: x and w1 rows must be 16-byte aligned");
  if (ws_bytes < tg::score_ws_bytes(t_in, n_seq))
    return fail(TG_ERR_WORKSPACE, "tg_score: workspace %zu < %zu bytes", ws_bytes,
                tg::score_ws_bytes(t_in, n_seq));
  if (tg::contract_checks_on()) {
    const hipError_t ce = tg::contract_offsets(cu_seqlens, n_seq, t_in, TG_CONTRACT_OFFSETS,
                                               (hipStream_t)stream);
    if (ce != hipSuccess) return from_hip(ce, "tg_score contract check");
  }
  hipError_t e = tg::launch_score(x, (int)dt, x_row_stride, t_in, d, h, w1, b1, w2, b2, prunable,
                                  cu_seqlens, n_seq, eps, norm_eps, b_raw, b, ws,
                                  (hipStream_t)stream);
  return from_hip(e, "tg_score launch");
}

// ---------------------------------------------------------------- select
tg_status tg_kept_sizes(const int32_t* cu, const int32_t* n_prunable, const int32_t* k,
                        int32_t n_seq, int32_t* kept_cu, int64_t* t_kept) {
  if (n_seq < 0 || !cu || !n_prunable || !k || !kept_cu || !t_kept)
    return fail(TG_ERR_INVALID_ARG, "tg_kept_sizes: bad arguments");
  if (cu[0] != 0) return fail(TG_ERR_INVALID_ARG, "tg_kept_sizes: cu_seqlens[0] != 0");
  int64_t acc = 0;
  kept_cu[0] = 0;
  for (int s = 0; s < n_seq; ++s) {
    int64_t len = (int64_t)cu[s + 1] - cu[s];
    if (len < 0) return fail(TG_ERR_INVALID_ARG, "tg_kept_sizes: cu_seqlens decreases at %d", s);
    if (k[s] < 0) return fail(TG_ERR_INVALID_ARG, "tg_kept_sizes: K[%d] < 0", s);
    if (n_prunable[s] < 0 || n_prunable[s] > len)
      return fail(TG_ERR_INVALID_ARG, "tg_kept_sizes: n_prunable[%d] outside [0, len]", s);
    int64_t kp = k[s] < n_prunable[s] ? k[s] : n_prunable[s];
    acc += kp + (len - n_prunable[s]);
    if (acc > INT32_MAX) return fail(TG_ERR_UNSUPPORTED, "tg_kept_sizes: total too large");
    kept_cu[s + 1] = (int32_t)acc;
  }
  *t_kept = acc;
  return ok();
}

size_t tg_select_workspace_size(int64_t t_in, int32_t n_seq) {
  if (t_in < 0 || n_seq < 0) return 0;
  return tg::select_ws_bytes(t_in, n_seq);
}

tg_status tg_select_topk(const float* b, const uint8_t* prunable, const int32_t* cu_seqlens,
                         const int32_t* k, int32_t n_seq, int64_t t_in, int64_t cap,
                         int32_t* kept_idx, int32_t* kept_pos, float* kept_b,
                         int32_t* kept_cu_seqlens, void* ws, size_t ws_bytes, tg_stream stream) {
  if (n_seq < 1 || t_in < 0 || cap < 0)
    return fail(TG_ERR_INVALID_ARG, "tg_select_topk: need n_seq >= 1, t_in >= 0, capacity >= 0");
  if (t_in > INT32_MAX - 4096) return fail(TG_ERR_UNSUPPORTED, "tg_select_topk: t_in too large");
  if (!cu_seqlens || !k || !kept_cu_seqlens || !ws)
    return fail(TG_ERR_INVALID_ARG, "tg_select_topk: null pointer");
  if (t_in > 0 && (!b || !prunable)) return fail(TG_ERR_INVALID_ARG, "tg_select_topk: null pointer");
  if (cap > 0 && !kept_idx) return fail(TG_ERR_INVALID_ARG, "tg_select_topk: kept_idx is null");
  if (ws_bytes < tg::select_ws_bytes(t_in, n_seq))
    return fail(TG_ERR_WORKSPACE, "tg_select_topk: workspace %zu < %zu bytes", ws_bytes,
                tg::select_ws_bytes(t_in, n_seq));
  hipError_t e = select_checked(b, prunable, cu_seqlens, k, n_seq, t_in, cap, kept_idx, kept_pos,
                                kept_b, kept_cu_seqlens, ws, (hipStream_t)stream);
  return from_hip(e, "tg_select_topk launch");
}

tg_status tg_select_topk_noalloc(const float* b, const uint8_t* prunable,
                                 const int32_t* cu_seqlens, const int32_t* k, int32_t n_seq,
                                 int64_t t_in, int64_t cap, int32_t* kept_idx, int32_t* kept_pos,
                                 float* kept_b, int32_t* kept_cu_seqlens, tg_stream stream) {
  if (n_seq < 1 || t_in < 0 || cap < 0)
    return fail(TG_ERR_INVALID_ARG,
                "tg_select_topk_noalloc: need n_seq >= 1, t_in >= 0, capacity >= 0");
  if (t_in > INT32_MAX - 4096)
    return fail(TG_ERR_UNSUPPORTED, "tg_select_topk_noalloc: t_in too large");
  if (!cu_seqlens || !k || !kept_cu_seqlens)
    return fail(TG_ERR_INVALID_ARG, "tg_select_topk_noalloc: null pointer");
  if (t_in > 0 && (!b || !prunable))
    return fail(TG_ERR_INVALID_ARG, "tg_select_topk_noalloc: null pointer");
  if (cap > 0 && !kept_idx)
    return fail(TG_ERR_INVALID_ARG, "tg_select_topk_noalloc: kept_idx is null");
  const size_t need = tg::select_ws_bytes(t_in, n_seq);
  if (need > TG_SELECT_SCRATCH_BYTES)
    return fail(TG_ERR_WORKSPACE,
                "tg_select_topk_noalloc: t_in = %lld, n_seq = %d need %zu bytes of scratch, "
                "more than the static %zu",
                (long long)t_in, (int)n_seq, need, (size_t)TG_SELECT_SCRATCH_BYTES);
  void* ws = nullptr;
  hipError_t e = tg::select_scratch(&ws);
  if (e != hipSuccess) return from_hip(e, "tg_select_topk_noalloc: scratch address");
  e = select_checked(b, prunable, cu_seqlens, k, n_seq, t_in, cap, kept_idx, kept_pos, kept_b,
                     kept_cu_seqlens, ws, (hipStream_t)stream);
  return from_hip(e, "tg_select_topk_noalloc launch");
}

// ---------------------------------------------------------------- gather
tg_status tg_gather(const void* src, int64_t src_stride, int64_t n_src, int64_t row_bytes,
                    const int32_t* idx, int64_t n_rows, void* dst, int64_t dst_stride,
                    tg_stream stream) {
  if (n_rows < 0 || n_src < 0 || row_bytes < 0)
    return fail(TG_ERR_INVALID_ARG, "tg_gather: negative size");
  if (n_rows == 0 || row_bytes == 0) return ok();
  if (!src || !idx || !dst) return fail(TG_ERR_INVALID_ARG, "tg_gather: null pointer");
  if (src_stride < row_bytes || dst_stride < row_bytes)
    return fail(TG_ERR_INVALID_ARG, "tg_gather: row stride smaller than row_bytes");
  if (row_bytes % 4 != 0 || src_stride % 4 != 0 || dst_stride % 4 != 0 || !aligned(src, 4) ||
      !aligned(dst, 4))
    return fail(TG_ERR_UNSUPPORTED, "tg_gather: rows must be 4-byte multiples, 4-byte aligned");
  if (n_rows > INT32_MAX) return fail(TG_ERR_UNSUPPORTED, "tg_gather: too many rows");
  if (tg::contract_checks_on()) {
    const hipError_t ce = tg::contract_indices(idx, n_rows, n_src, (hipStream_t)stream);
    if (ce != hipSuccess) return from_hip(ce, "tg_gather contract check");
  }
  hipError_t e = tg::launch_gather(src, src_stride, n_src, row_bytes, idx, n_rows, dst, dst_stride,
                                   (hipStream_t)stream);
  return from_hip(e, "tg_gather launch");
}

// ------------------------------------------------------------ projection
tg_status tg_qkv_proj(const void* x, tg_dtype dt, int64_t xs, int64_t t, int32_t d, const void* w,
                      int32_t hq, int32_t hkv, int32_t dh, void* q, void* k, void* v,
                      tg_stream stream) {
  if (t < 0 || d < 1 || hq < 1 || hkv < 1 || dh < 1 || xs < d)
    return fail(TG_ERR_INVALID_ARG, "tg_qkv_proj: bad sizes");
  if (dt != TG_F32 && dt != TG_BF16) return fail(TG_ERR_INVALID_ARG, "tg_qkv_proj: bad dtype");
  if (dt != TG_BF16) return fail(TG_ERR_UNSUPPORTED, "tg_qkv_proj: only bf16 is implemented");
  const int64_t n_tot = (int64_t)(hq + 2 * (int64_t)hkv) * dh;
  if (d % 64 != 0 || dh % 32 != 0 || n_tot % 256 != 0 || n_tot > INT32_MAX)
    return fail(TG_ERR_UNSUPPORTED,
                "tg_qkv_proj: need d %% 64 == 0, dh %% 32 == 0, (hq + 2 hkv) * dh %% 256 == 0");
  if (xs % 8 != 0 || xs >= ((int64_t)1 << 22) || (int64_t)d * 256 * 2 > INT32_MAX)
    return fail(TG_ERR_UNSUPPORTED, "tg_qkv_proj: row stride must be a multiple of 8, < 2^22");
  if (t > INT32_MAX) return fail(TG_ERR_UNSUPPORTED, "tg_qkv_proj: too many rows");
  if (t == 0) return ok();
  if (!x || !w || !q || !k || !v) return fail(TG_ERR_INVALID_ARG, "tg_qkv_proj: null pointer");
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(q, 8) || !aligned(k, 8) || !aligned(v, 8))
    return fail(TG_ERR_UNSUPPORTED, "tg_qkv_proj: x, w 16-byte and q, k, v 8-byte aligned");
  hipError_t e = tg::launch_qkv_proj(x, xs, t, d, w, hq * dh, hkv * dh, q, k, v,
                                     (hipStream_t)stream);
  return from_hip(e, "tg_qkv_proj launch");
}

tg_status tg_qkv_proj_rope(const void* x, tg_dtype dt, int64_t xs, int64_t t, int32_t d,
                           const void* w, int32_t hq, int32_t hkv, int32_t dh, const int32_t* pos,
                           const float* q_norm, const float* k_norm, float norm_eps,
                           float rope_theta, void* q, void* k, void* v, tg_stream stream) {
  if (t < 0 || d < 1 || hq < 1 || hkv < 1 || dh < 1 || xs < d)
    return fail(TG_ERR_INVALID_ARG, "tg_qkv_proj_rope: bad sizes");
  if (dt != TG_F32 && dt != TG_BF16) return fail(TG_ERR_INVALID_ARG, "tg_qkv_proj_rope: bad dtype");
  if (dt != TG_BF16) return fail(TG_ERR_UNSUPPORTED, "tg_qkv_proj_rope: only bf16 is implemented");
  if (rope_theta != rope_theta || (rope_theta > 0.0f && rope_theta <= 1.0f))
    return fail(TG_ERR_INVALID_ARG, "tg_qkv_proj_rope: rope_theta must be > 1, or <= 0 for none");
  if ((q_norm || k_norm) && !(norm_eps >= 0.0f))
    return fail(TG_ERR_INVALID_ARG, "tg_qkv_proj_rope: norm_eps must be >= 0");
  if (rope_theta > 0.0f && t > 0 && !pos)
    return fail(TG_ERR_INVALID_ARG, "tg_qkv_proj_rope: positions are needed for the rotation");
  const int64_t nq = (int64_t)hq * dh, nkv = (int64_t)hkv * dh;
  if ((dh != 64 && dh != 128) || nq % 128 != 0 || nkv % 128 != 0)
    return fail(TG_ERR_UNSUPPORTED,
                "tg_qkv_proj_rope: need dh in {64, 128} and hq * dh, hkv * dh multiples of 128");
  const int64_t n_tot = nq + 2 * nkv;
  if (d % 64 != 0 || n_tot % 256 != 0 || n_tot > INT32_MAX)
    return fail(TG_ERR_UNSUPPORTED,
                "tg_qkv_proj_rope: need d %% 64 == 0, (hq + 2 hkv) * dh %% 256 == 0");
  if (xs % 8 != 0 || xs >= ((int64_t)1 << 22) || (int64_t)d * 256 * 2 > INT32_MAX)
    return fail(TG_ERR_UNSUPPORTED, "tg_qkv_proj_rope: row stride must be a multiple of 8, < 2^22");
  if (t > INT32_MAX) return fail(TG_ERR_UNSUPPORTED, "tg_qkv_proj_rope: too many rows");
  if (t == 0) return ok();
  if (!x || !w || !q || !k || !v) return fail(TG_ERR_INVALID_ARG, "tg_qkv_proj_rope: null pointer");
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(q, 8) || !aligned(k, 8) || !aligned(v, 8))
    return fail(TG_ERR_UNSUPPORTED, "tg_qkv_proj_rope: x, w 16-byte and q, k, v 8-byte aligned");
  hipError_t e = tg::launch_qkv_proj_rope(x, xs, t, d, w, (int)nq, (int)nkv, dh, pos, q_norm,
                                          k_norm, norm_eps, rope_theta, q, k, v,
                                          (hipStream_t)stream);
  return from_hip(e, "tg_qkv_proj_rope launch");
}

// ------------------------------------------------------------- attention
}  // extern "C"

namespace {
// tg_gated_attn and tg_gated_attn_split: checks and launch (ws: the split
// form's workspace, or null)
tg_status tg_gated_attn_impl(const void* q, const void* k, const void* v, tg_dtype dt, void* out,
                             int64_t t_kept, const float* kept_b, const int32_t* kept_pos,
                             const int32_t* kept_cu, int32_t n_seq, int32_t max_len, int32_t hq,
                             int32_t hkv, int32_t dh, const float* gain, const float* temp,
                             float sm_scale, float* lse2, void* ws, tg_stream stream,
                             const char* who) {
  if (t_kept < 0 || n_seq < 1 || max_len < 0 || hq < 1 || hkv < 1)
    return fail(TG_ERR_INVALID_ARG, "%s: bad sizes", who);
  if (hq % hkv != 0) return fail(TG_ERR_INVALID_ARG, "%s: hq %% hkv != 0", who);
  if (dt != TG_F32 && dt != TG_BF16) return fail(TG_ERR_INVALID_ARG, "%s: bad dtype", who);
  if (dh != 64 && dh != 128) return fail(TG_ERR_UNSUPPORTED, "%s: dh must be 64 or 128", who);
  const int g = hq / hkv;
  if (!((g <= 4 && 4 % g == 0) || (g > 4 && g % 4 == 0)))
    return fail(TG_ERR_UNSUPPORTED, "%s: hq/hkv must be 1, 2, 4 or a multiple of 4", who);
  if (t_kept > INT32_MAX - 4096) return fail(TG_ERR_UNSUPPORTED, "%s: t_kept too large", who);
  if (!kept_cu || !gain || !temp) return fail(TG_ERR_INVALID_ARG, "%s: null pointer", who);
  if (t_kept == 0) return ok();
  if (!q || !k || !v || !out || !kept_b)
    return fail(TG_ERR_INVALID_ARG, "%s: null pointer", who);
  if (max_len > t_kept) max_len = (int32_t)t_kept;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
    return fail(TG_ERR_UNSUPPORTED, "%s: tensors must be 16-byte aligned", who);
  if (lse2 && dt != TG_BF16)
    return fail(TG_ERR_UNSUPPORTED, "%s: lse2 is written by the bf16 path only", who);
  if (lse2 && !aligned(lse2, 4))
    return fail(TG_ERR_UNSUPPORTED, "%s: lse2 must be 4-byte aligned", who);
  if (tg::contract_checks_on()) {
    hipError_t ce = tg::contract_offsets(kept_cu, n_seq, t_kept, TG_CONTRACT_KEPT_OFFSETS,
                                         (hipStream_t)stream);
    if (ce == hipSuccess && kept_pos)
      ce = tg::contract_positions(kept_pos, kept_cu, n_seq, t_kept, (hipStream_t)stream);
    if (ce != hipSuccess) return from_hip(ce, who);
  }
  hipError_t e;
  if (dt == TG_BF16)
    e = tg::launch_attn_bf16(q, k, v, out, t_kept, kept_b, kept_pos, kept_cu, n_seq, max_len, hq,
                             hkv, dh, gain, temp, sm_scale, lse2, (hipStream_t)stream, ws);
  else
    e = tg::launch_attn_f32(q, k, v, out, t_kept, kept_b, kept_pos, kept_cu, n_seq, max_len, hq,
                            hkv, dh, gain, temp, sm_scale, (hipStream_t)stream);
  return from_hip(e, who);
}
}  // namespace

extern "C" {

tg_status tg_gated_attn(const void* q, const void* k, const void* v, tg_dtype dt, void* out,
                        int64_t t_kept, const float* kept_b, const int32_t* kept_pos,
                        const int32_t* kept_cu, int32_t n_seq, int32_t max_len, int32_t hq,
                        int32_t hkv, int32_t dh, const float* gain, const float* temp,
                        float sm_scale, float* lse2, tg_stream stream) {
  return tg_gated_attn_impl(q, k, v, dt, out, t_kept, kept_b, kept_pos, kept_cu, n_seq, max_len,
                            hq, hkv, dh, gain, temp, sm_scale, lse2, nullptr, stream,
                            "tg_gated_attn");
}

size_t tg_gated_attn_split_workspace_size(int64_t t_kept, int32_t n_seq, int32_t max_len,
                                          int32_t hq, int32_t hkv, int32_t dh) {
  if (t_kept < 0 || n_seq < 1 || max_len < 0 || hq < 1 || hkv < 1 || hq % hkv != 0 ||
      (dh != 64 && dh != 128))
    return 0;
  if (max_len > t_kept) max_len = (int32_t)t_kept;
  return tg::attn_split_ws_bytes(t_kept, n_seq, max_len, hq, hkv, dh);
}

tg_status tg_gated_attn_split(const void* q, const void* k, const void* v, tg_dtype dt, void* out,
                              int64_t t_kept, const float* kept_b, const int32_t* kept_pos,
                              const int32_t* kept_cu, int32_t n_seq, int32_t max_len, int32_t hq,
                              int32_t hkv, int32_t dh, const float* gain, const float* temp,
                              float sm_scale, float* lse2, void* ws, size_t ws_bytes,
                              tg_stream stream) {
  if (dt != TG_BF16 && dt != TG_F32)
    return fail(TG_ERR_INVALID_ARG, "tg_gated_attn_split: bad dtype");
  if (dt != TG_BF16) return fail(TG_ERR_UNSUPPORTED, "tg_gated_attn_split: bf16 only");
  if (t_kept < 0 || n_seq < 1 || max_len < 0 || hq < 1 || hkv < 1)
    return fail(TG_ERR_INVALID_ARG, "tg_gated_attn_split: bad sizes");
  const size_t need = tg_gated_attn_split_workspace_size(t_kept, n_seq, max_len, hq, hkv, dh);
  if (need > 0) {
    if (!ws || ws_bytes < need)
      return fail(TG_ERR_WORKSPACE, "tg_gated_attn_split: workspace %zu < %zu bytes",
                  ws ? ws_bytes : (size_t)0, need);
    if (!aligned(ws, 256))
      return fail(TG_ERR_UNSUPPORTED, "tg_gated_attn_split: ws must be 256-byte aligned");
  }
  // the remaining checks and the launch are tg_gated_attn's
  return tg_gated_attn_impl(q, k, v, dt, out, t_kept, kept_b, kept_pos, kept_cu, n_seq, max_len,
                            hq, hkv, dh, gain, temp, sm_scale, lse2, need > 0 ? ws : nullptr,
                            stream, "tg_gated_attn_split");
}

// ----------------------------------------------------------------- decode
size_t tg_gated_decode_workspace_size(int32_t n_seq, int32_t hq, int32_t hkv, int32_t dh,
                                      int64_t max_cache_len) {
  if (n_seq < 1 || hq < 1 || hkv < 1 || dh < 1 || max_cache_len < 0) return 0;
  return tg::decode_ws_bytes(n_seq, hq, hkv, dh, max_cache_len);
}

tg_status tg_gated_decode(const void* q, const void* k_cache, const void* v_cache, tg_dtype dt,
                          void* out, int64_t t_cache, const float* cache_b,
                          const int32_t* q_pos, const int32_t* cache_cu, int32_t n_seq,
                          int64_t max_cache_len, int32_t hq, int32_t hkv, int32_t dh,
                          const float* gain, const float* temp, float sm_scale, void* ws,
                          size_t ws_bytes, tg_stream stream) {
  if (t_cache < 0 || n_seq < 1 || max_cache_len < 0 || hq < 1 || hkv < 1)
    return fail(TG_ERR_INVALID_ARG, "tg_gated_decode: bad sizes");
  if (hq % hkv != 0) return fail(TG_ERR_INVALID_ARG, "tg_gated_decode: hq %% hkv != 0");
  if (dt != TG_F32 && dt != TG_BF16) return fail(TG_ERR_INVALID_ARG, "tg_gated_decode: bad dtype");
  if (dt != TG_BF16) return fail(TG_ERR_UNSUPPORTED, "tg_gated_decode: only bf16 is implemented");
  if (dh != 64 && dh != 128)
    return fail(TG_ERR_UNSUPPORTED, "tg_gated_decode: dh must be 64 or 128");
  const int g = hq / hkv;
  if (g != 1 && g != 2 && g != 4 && g != 8)
    return fail(TG_ERR_UNSUPPORTED, "tg_gated_decode: hq/hkv must be 1, 2, 4 or 8");
  if (t_cache > INT32_MAX) return fail(TG_ERR_UNSUPPORTED, "tg_gated_decode: t_cache too large");
  if (n_seq > 65535) return fail(TG_ERR_UNSUPPORTED, "tg_gated_decode: more than 65535 sequences");
  if ((int64_t)hkv * dh > (1 << 20))
    return fail(TG_ERR_UNSUPPORTED, "tg_gated_decode: hkv * dh too large");
  if (!q || !k_cache || !v_cache || !out || !cache_cu || !gain || !temp)
    return fail(TG_ERR_INVALID_ARG, "tg_gated_decode: null pointer");
  if (!ws) return fail(TG_ERR_INVALID_ARG, "tg_gated_decode: null workspace");
  const size_t need = tg::decode_ws_bytes(n_seq, hq, hkv, dh, max_cache_len);
  if (ws_bytes < need)
    return fail(TG_ERR_WORKSPACE, "tg_gated_decode: workspace %zu < %zu bytes", ws_bytes, need);
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 2) ||
      !aligned(ws, 4))
    return fail(TG_ERR_UNSUPPORTED, "tg_gated_decode: q, k_cache, v_cache must be 16-byte aligned");
  if (tg::contract_checks_on()) {
    const hipError_t ce = tg::contract_offsets(cache_cu, n_seq, t_cache, TG_CONTRACT_KEPT_OFFSETS,
                                               (hipStream_t)stream);
    if (ce != hipSuccess) return from_hip(ce, "tg_gated_decode contract check");
  }
  hipError_t e = tg::launch_decode(q, k_cache, v_cache, out, cache_b, cache_cu, q_pos, n_seq,
                                   t_cache, max_cache_len, hq, hkv, dh, gain, temp, sm_scale, ws,
                                   (hipStream_t)stream);
  return from_hip(e, "tg_gated_decode launch");
}

// ------------------------------------------------------- attention backward
size_t tg_gated_attn_bwd_workspace_size(int64_t t_kept, int32_t n_seq, int32_t hq, int32_t hkv) {
  if (t_kept < 0 || n_seq < 1 || hq < 1 || hkv < 1) return 0;
  return tg::attn_bwd_ws_bytes(t_kept, n_seq, hq, hkv);
}

tg_status tg_gated_attn_bwd(const void* q, const void* k, const void* v, const void* dout,
                            tg_dtype dt, int64_t t_kept, const float* kept_b,
                            const int32_t* kept_pos, const int32_t* kept_cu, int32_t n_seq,
                            int32_t hq, int32_t hkv, int32_t dh, const float* gain,
                            const float* temp, float sm_scale, float* dq, float* dk, float* dv,
                            float* db, float* dgain, float* dtemp, const void* fwd_out,
                            const float* fwd_lse2, void* ws, size_t ws_bytes, tg_stream stream) {
  if (t_kept < 0 || n_seq < 1 || hq < 1 || hkv < 1)
    return fail(TG_ERR_INVALID_ARG, "tg_gated_attn_bwd: bad sizes");
  if (hq % hkv != 0) return fail(TG_ERR_INVALID_ARG, "tg_gated_attn_bwd: hq %% hkv != 0");
  if (dt != TG_F32 && dt != TG_BF16)
    return fail(TG_ERR_INVALID_ARG, "tg_gated_attn_bwd: bad dtype");
  if (dh != 64 && dh != 128)
    return fail(TG_ERR_UNSUPPORTED, "tg_gated_attn_bwd: dh must be 64 or 128");
  if (hq > 65535 || t_kept > INT32_MAX - 4096)
    return fail(TG_ERR_UNSUPPORTED, "tg_gated_attn_bwd: sizes too large");
  if (!kept_cu || !gain || !temp || !dgain || !dtemp || !ws)
    return fail(TG_ERR_INVALID_ARG, "tg_gated_attn_bwd: null pointer");
  if (t_kept > 0 && (!q || !k || !v || !dout || !kept_b || !dq || !dk || !dv || !db))
    return fail(TG_ERR_INVALID_ARG, "tg_gated_attn_bwd: null pointer");
  const size_t need = tg::attn_bwd_ws_bytes(t_kept, n_seq, hq, hkv);
  if (ws_bytes < need)
    return fail(TG_ERR_WORKSPACE, "tg_gated_attn_bwd: workspace %zu < %zu bytes", ws_bytes, need);
  if ((q && !aligned(q, 16)) || (k && !aligned(k, 16)) || (v && !aligned(v, 16)) ||
      (dout && !aligned(dout, 16)) || (dq && !aligned(dq, 16)) || (dk && !aligned(dk, 16)) ||
      (dv && !aligned(dv, 16)) || !aligned(ws, 4))
    return fail(TG_ERR_UNSUPPORTED, "tg_gated_attn_bwd: tensors must be 16-byte aligned");
  if ((fwd_out == nullptr) != (fwd_lse2 == nullptr))
    return fail(TG_ERR_INVALID_ARG, "tg_gated_attn_bwd: give both fwd_out and fwd_lse2, or neither");
  if (fwd_out && dt != TG_BF16)
    return fail(TG_ERR_UNSUPPORTED, "tg_gated_attn_bwd: saved forward state is for bf16 only");
  if (fwd_out && (!aligned(fwd_out, 16) || !aligned(fwd_lse2, 4)))
    return fail(TG_ERR_UNSUPPORTED, "tg_gated_attn_bwd: fwd_out 16-byte, fwd_lse2 4-byte aligned");
  if (tg::contract_checks_on()) {
    hipError_t ce = tg::contract_offsets(kept_cu, n_seq, t_kept, TG_CONTRACT_KEPT_OFFSETS,
                                         (hipStream_t)stream);
    if (ce == hipSuccess && kept_pos)
      ce = tg::contract_positions(kept_pos, kept_cu, n_seq, t_kept, (hipStream_t)stream);
    if (ce != hipSuccess) return from_hip(ce, "tg_gated_attn_bwd contract check");
  }
  hipError_t e = tg::launch_attn_bwd(q, k, v, dout, (int)dt, t_kept, kept_b, kept_pos, kept_cu,
                                     n_seq, hq, hkv, dh, gain, temp, sm_scale, dq, dk, dv, db,
                                     dgain, dtemp, fwd_out, fwd_lse2, ws, (hipStream_t)stream);
  return from_hip(e, "tg_gated_attn_bwd launch");
}

// ---------------------------------------------------------- scorer backward
size_t tg_score_bwd_workspace_size(int64_t t_in, int32_t n_seq, int32_t d, int32_t h) {
  if (t_in < 0 || n_seq < 1 || d < 1 || h < 1) return 0;
  return tg::score_bwd_ws_bytes(t_in, n_seq, d, h);
}

tg_status tg_score_bwd(const void* x, tg_dtype dt, int64_t x_row_stride, int64_t t_in, int32_t d,
                       int32_t h, const void* w1, const float* b1, const float* w2,
                       const uint8_t* prunable, const int32_t* cu_seqlens, int32_t n_seq,
                       float eps, float norm_eps, const float* b_raw, const int32_t* kept_idx,
                       const int32_t* kept_cu, int64_t t_kept, const float* db_kept, float* dx,
                       float* dw1, float* db1, float* dw2, float* db2, void* ws, size_t ws_bytes,
                       tg_stream stream) {
  if (t_in < 0 || t_kept < 0 || n_seq < 1 || d < 1 || h < 1)
    return fail(TG_ERR_INVALID_ARG, "tg_score_bwd: bad sizes");
  if (!(eps >= 0.0f)) return fail(TG_ERR_INVALID_ARG, "tg_score_bwd: eps must be >= 0");
  if (norm_eps != norm_eps) return fail(TG_ERR_INVALID_ARG, "tg_score_bwd: norm_eps is NaN");
  if (dt != TG_F32 && dt != TG_BF16) return fail(TG_ERR_INVALID_ARG, "tg_score_bwd: bad dtype");
  if (x_row_stride < d) return fail(TG_ERR_INVALID_ARG, "tg_score_bwd: x_row_stride < d");
  if (d % 64 != 0 || h % 64 != 0)
    return fail(TG_ERR_UNSUPPORTED, "tg_score_bwd: needs d %% 64 == 0 and h %% 64 == 0");
  if (x_row_stride >= ((int64_t)1 << 22) || d >= (1 << 22))
    return fail(TG_ERR_UNSUPPORTED, "tg_score_bwd: needs x_row_stride, d < 2^22");
  if (t_in > INT32_MAX - 4096 || t_kept > t_in)
    return fail(TG_ERR_UNSUPPORTED, "tg_score_bwd: sizes too large");
  if (!cu_seqlens || !kept_cu || !w2 || !dw1 || !db1 || !dw2 || !db2 || !ws)
    return fail(TG_ERR_INVALID_ARG, "tg_score_bwd: null pointer");
  if (t_in > 0 && (!x || !w1 || !prunable || !b_raw))
    return fail(TG_ERR_INVALID_ARG, "tg_score_bwd: null pointer");
  if (t_kept > 0 && (!kept_idx || !db_kept))
    return fail(TG_ERR_INVALID_ARG, "tg_score_bwd: null pointer");
  const size_t need = tg::score_bwd_ws_bytes(t_in, n_seq, d, h);
  if (ws_bytes < need)
    return fail(TG_ERR_WORKSPACE, "tg_score_bwd: workspace %zu < %zu bytes", ws_bytes, need);
  if (!aligned(ws, 256)) return fail(TG_ERR_UNSUPPORTED, "tg_score_bwd: ws must be 256-byte aligned");
  const int64_t es = dt == TG_BF16 ? 2 : 4;
  if ((x && !aligned(x, 16)) || (w1 && !aligned(w1, 16)) || ((x_row_stride * es) % 16) != 0)
    return fail(TG_ERR_UNSUPPORTED, "tg_score_bwd: x and w1 rows must be 16-byte aligned");
  if (tg::contract_checks_on()) {
    hipError_t ce = tg::contract_offsets(cu_seqlens, n_seq, t_in, TG_CONTRACT_OFFSETS,
                                         (hipStream_t)stream);
    if (ce == hipSuccess)
      ce = tg::contract_offsets(kept_cu, n_seq, t_kept, TG_CONTRACT_KEPT_OFFSETS,
                                (hipStream_t)stream);
    if (ce == hipSuccess && t_kept > 0)
      ce = tg::contract_indices(kept_idx, t_kept, t_in, (hipStream_t)stream);
    if (ce != hipSuccess) return from_hip(ce, "tg_score_bwd contract check");
  }
  hipError_t e = tg::launch_score_bwd(x, (int)dt, x_row_stride, t_in, d, h, w1, b1, w2, prunable,
                                      cu_seqlens, n_seq, eps, norm_eps, b_raw, kept_idx,
                                      kept_cu, t_kept,
                                      db_kept, dx, dw1, db1, dw2, db2, ws, (hipStream_t)stream);
  return from_hip(e, "tg_score_bwd launch");
}

// ------------------------------------------------------ contract checks
tg_status tg_set_contract_checks(int32_t on) {
  tg::set_contract_checks(on != 0);
  return ok();
}

tg_status tg_contract_status(uint32_t* flags, tg_stream stream) {
  if (!flags) return fail(TG_ERR_INVALID_ARG, "tg_contract_status: flags is null");
  unsigned int f = 0u;
  const hipError_t e = tg::contract_read_and_clear(&f, (hipStream_t)stream);
  if (e != hipSuccess) return from_hip(e, "tg_contract_status");
  *flags = f;
  return ok();
}

}  // extern "C"
