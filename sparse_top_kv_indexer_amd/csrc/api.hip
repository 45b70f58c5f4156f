// C ABI of the sparse decode step: argument validation, workspace sizing and
// kernel launches.  Every entry point only enqueues on the caller's stream.
#include <math.h>

#include <algorithm>
#include <mutex>

#include "../../include/sparsekv.h"
#include "skv_internal.h"
#include "skv_topk.h"

namespace skv {
// validate.hip: the checks of a debug build, run first by the entry points
// (a no-op in release builds)
void debug_validate(const skv_kv* kv, skv_window win, const int32_t* idx, int k, hipStream_t st);
}  // namespace skv

using namespace skv;

namespace {

const skv_window kNoWindow = {nullptr, nullptr};

bool kv_ok(const skv_kv* kv) {
  if (!kv || !kv->k || !kv->seq_len) return false;
  if (kv->dtype != SKV_F32 && kv->dtype != SKV_BF16) return false;
  if (kv->B < 1 || kv->H < 1 || kv->L_max < 1) return false;
  if (kv->d_k < 8 || kv->d_k % 8 || kv->d_v < 1) return false;
  if (kv->block == 0) {
    if (kv->block_table || kv->token_table) return false;
  } else if (kv->block == 16) {
    if ((kv->block_table == nullptr) == (kv->token_table == nullptr)) return false;
    if (kv->L_max % 16) return false;
  } else {
    return false;
  }
  if (kv->v == nullptr && kv->d_v > kv->d_k) return false;
  if (kv->v != nullptr && kv->d_v != kv->d_k) return false;
  return true;
}

KvArgs to_args(const skv_kv* kv) {
  KvArgs a;
  a.k = kv->k;
  a.v = kv->v;
  a.bf16 = kv->dtype == SKV_BF16;
  a.B = kv->B;
  a.H = kv->H;
  a.d_k = kv->d_k;
  a.d_v = kv->d_v;
  a.block = kv->block;
  a.L_max = kv->L_max;
  a.block_table = kv->block_table;
  a.token_table = kv->token_table;
  a.seq_len = kv->seq_len;
  return a;
}

bool score_supported(const skv_kv* kv, int G) {
  if (kv->dtype == SKV_BF16) {
    if (G >= 2 && G <= 16 && kv->d_k % 32 == 0) {
      const int nc = kv->d_k / 32;
      return nc == 2 || nc == 4 || nc == 8 || nc == 18;
    }
    const int npl = (kv->d_k / 8 + 15) / 16;
    if (npl == 1) return G <= 8;
    if (npl == 2) return G <= 4;
    if (npl <= 5) return G == 1;
    return false;
  }
  const int npl = (kv->d_k / 4 + 15) / 16;
  if (npl <= 2) return G <= 8;
  if (npl <= 4) return G <= 2;
  return false;
}

skv_status launched(hipError_t e) {
  if (e == hipErrorInvalidValue) return SKV_EUNSUPPORTED;
  return e == hipSuccess ? SKV_OK : SKV_ELAUNCH;
}

// Library-owned scratch of sparsekv_select_attend_noalloc: one copy per GPU
// (a device global), held until the process ends.  Host code never passes
// `scratch` itself to a kernel -- on the host that name is only a stand-in --
// but the address hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchBytes = (size_t)16 << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's copy of scratch, resolved once per device.
hipError_t scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return e != hipSuccess ? e : hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

// GQA rows longer than one sweep in the fused calls: the slice listing, then
// the kernel that finishes each row's selection and attends over it (k <=
// 4096, at most 1024 listing slices); other shapes take the sliced top-k
// (finished by one workgroup per row), then the split attention and merge.
bool long_select_attend_supported(const KvArgs& a, int G) {
  return a.bf16 && a.v != nullptr && a.d_k == 128 && a.d_v == 128 && G >= 1 && G <= 8 &&
         topk_supported(a.L_max) && attend_supported(a, G);
}

skv_status long_select_attend(const KvArgs& a, const void* q, int G, skv_window win, int k,
                              float scale, const float* scores, int32_t* idx, int32_t* count,
                              float* out, void* ws, size_t th, size_t ws_bytes,
                              hipStream_t stream) {
  if (finish_attend_supported(a, G, k))
    return launched(launch_finish_attend(a, q, G, scores, win.lo, win.hi, k, ws, scale, idx, count,
                                         out, (float*)((char*)ws + th), stream));
  const hipError_t e = launch_topk(scores, a.B * a.H, a.H, a.L_max, win.lo, win.hi, k, idx, count,
                                   ws, true, stream);
  if (e != hipSuccess) return launched(e);
  return launched(launch_gather_attend(a, q, G, idx, k, win.lo, win.hi, scale, out,
                                       (char*)ws + th, ws_bytes - th, stream));
}

// Scratch layout of the fused step without a workspace: the rows' key
// histograms (must be zero when the scan starts), then the split partials.
size_t noalloc_hist_bytes(int rows) { return ((size_t)rows * 4096 * 4 + 255) & ~(size_t)255; }

__global__ __launch_bounds__(256) void zero_words_kernel(uint4* p, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

extern "C" {

skv_status sparsekv_score(const skv_kv* kv, const void* q, int32_t G, float* scores,
                          hipStream_t stream) {
  if (!kv_ok(kv) || !q || !scores || G < 1) return SKV_EINVAL;
  if (!score_supported(kv, G)) return SKV_EUNSUPPORTED;
  debug_validate(kv, kNoWindow, nullptr, 0, stream);
  return launched(launch_score(to_args(kv), q, G, scores, nullptr, nullptr, nullptr, stream));
}

skv_status sparsekv_topk(const float* scores, int32_t B, int32_t H, int32_t L_max,
                         skv_window win, int32_t k, int32_t* idx, int32_t* count, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
  if (!scores || !idx || !count || !win.lo || !win.hi) return SKV_EINVAL;
  if (B < 1 || H < 1 || L_max < 1 || k < 1 || k > L_max) return SKV_EINVAL;
  if (!topk_supported(L_max)) return SKV_EUNSUPPORTED;
  if (!ws || ws_bytes < topk_workspace_bytes(B * H, L_max)) return SKV_EWORKSPACE;
  return launched(launch_topk(scores, B * H, H, L_max, win.lo, win.hi, k, idx, count, ws, false,
                              stream));
}

skv_status sparsekv_score_hist(const skv_kv* kv, const void* q, int32_t G, skv_window win,
                               float* scores, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!kv_ok(kv) || !q || !scores || G < 1 || !win.lo || !win.hi) return SKV_EINVAL;
  if (!score_supported(kv, G) || !topk_supported(kv->L_max)) return SKV_EUNSUPPORTED;
  if (!ws || ws_bytes < topk_workspace_bytes(kv->B * kv->H, kv->L_max)) return SKV_EWORKSPACE;
  debug_validate(kv, win, nullptr, 0, stream);
  return launched(launch_score(to_args(kv), q, G, scores, win.lo, win.hi, (uint32_t*)ws, stream));
}

skv_status sparsekv_topk_resume(const float* scores, int32_t B, int32_t H, int32_t L_max,
                                skv_window win, int32_t k, int32_t* idx, int32_t* count,
                                void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!scores || !idx || !count || !win.lo || !win.hi) return SKV_EINVAL;
  if (B < 1 || H < 1 || L_max < 1 || k < 1 || k > L_max) return SKV_EINVAL;
  if (!topk_supported(L_max)) return SKV_EUNSUPPORTED;
  if (!ws || ws_bytes < topk_workspace_bytes(B * H, L_max)) return SKV_EWORKSPACE;
  return launched(launch_topk(scores, B * H, H, L_max, win.lo, win.hi, k, idx, count, ws, true,
                              stream));
}

skv_status sparsekv_score_prefilter(const skv_kv* kv, const void* q, int32_t G, skv_window win,
                                    const float* thr, float* scores, void* ws, size_t ws_bytes,
                                    hipStream_t stream) {
  if (!kv_ok(kv) || !q || !scores || !thr || G < 1 || !win.lo || !win.hi) return SKV_EINVAL;
  const KvArgs a = to_args(kv);
  if (!score_supported(kv, G) || !score_prefilter_supported(a, G) || !topk_supported(kv->L_max))
    return SKV_EUNSUPPORTED;
  const int rows = kv->B * kv->H;
  if (!ws || ws_bytes < topk_workspace_bytes(rows, kv->L_max)) return SKV_EWORKSPACE;
  debug_validate(kv, win, nullptr, 0, stream);
  const TopkWs w = TopkWs::carve(ws, rows, kv->L_max);
  return launched(launch_score_prefilter(a, q, G, scores, win.lo, win.hi, thr, w.lkey, w.lpos,
                                         w.ctr, kRowList, stream));
}

skv_status sparsekv_topk_prefiltered(const float* scores, int32_t B, int32_t H, int32_t L_max,
                                     skv_window win, int32_t k, float* thr, float alpha,
                                     int32_t* idx, int32_t* count, int32_t* used, void* ws,
                                     size_t ws_bytes, hipStream_t stream) {
  if (!scores || !idx || !count || !thr || !win.lo || !win.hi) return SKV_EINVAL;
  if (B < 1 || H < 1 || L_max < 1 || k < 1 || k > L_max || !(alpha >= 0.f && alpha <= 1.f))
    return SKV_EINVAL;
  if (!topk_survivors_supported(L_max)) return SKV_EUNSUPPORTED;
  if (!ws || ws_bytes < topk_workspace_bytes(B * H, L_max)) return SKV_EWORKSPACE;
  return launched(launch_topk_survivors(scores, B * H, H, L_max, win.lo, win.hi, k, idx, count,
                                        ws, thr, alpha, used, stream));
}

skv_status sparsekv_select(const skv_kv* kv, const void* q, int32_t G, skv_window win, int32_t k,
                           float* scores, int32_t* idx, int32_t* count, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
  if (!kv_ok(kv) || !q || !scores || !idx || !count || G < 1 || k < 1) return SKV_EINVAL;
  if (k > kv->L_max || !win.lo || !win.hi) return SKV_EINVAL;
  if (!score_supported(kv, G) || !topk_supported(kv->L_max)) return SKV_EUNSUPPORTED;
  const int rows = kv->B * kv->H;
  if (!ws || ws_bytes < topk_workspace_bytes(rows, kv->L_max)) return SKV_EWORKSPACE;
  debug_validate(kv, win, nullptr, 0, stream);
  hipError_t e = launch_score(to_args(kv), q, G, scores, win.lo, win.hi, (uint32_t*)ws, stream);
  if (e != hipSuccess) return launched(e);
  return launched(launch_topk(scores, rows, kv->H, kv->L_max, win.lo, win.hi, k, idx, count, ws,
                              true, stream));
}

skv_status sparsekv_gather_attend(const skv_kv* kv, const void* q, int32_t G, const int32_t* idx,
                                  int32_t k, skv_window win, float scale, float* out, void* ws,
                                  size_t ws_bytes, hipStream_t stream) {
  if (!kv_ok(kv) || !q || !out || G < 1 || k < 0 || (k > 0 && !idx)) return SKV_EINVAL;
  if (k > kv->L_max) return SKV_EINVAL;
  if (!win.lo || !win.hi || !isfinite(scale)) return SKV_EINVAL;
  const KvArgs a = to_args(kv);
  debug_validate(kv, win, idx, k, stream);
  if (kv->v == nullptr) {
    if (!mla_supported(a, G)) return SKV_EUNSUPPORTED;
    const size_t need = mla_workspace_bytes(a, G, k);
    if (need && (!ws || ws_bytes < need)) return SKV_EWORKSPACE;
    return launched(launch_mla_attend(a, q, G, idx, k, win.lo, win.hi, scale, out, ws, ws_bytes,
                                      stream));
  }
  if (!attend_supported(a, G)) return SKV_EUNSUPPORTED;
  const size_t need = attend_workspace_bytes(a, G, k);
  if (!ws || ws_bytes < need) return SKV_EWORKSPACE;
  return launched(
      launch_gather_attend(a, q, G, idx, k, win.lo, win.hi, scale, out, ws, ws_bytes, stream));
}

skv_status sparsekv_select_attend(const skv_kv* kv, const void* q, int32_t G, skv_window win,
                                  int32_t k, float scale, float* scores, int32_t* idx,
                                  int32_t* count, float* out, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  if (!kv_ok(kv) || !q || !scores || !idx || !count || !out || G < 1 || k < 1) return SKV_EINVAL;
  if (k > kv->L_max || !win.lo || !win.hi || !isfinite(scale)) return SKV_EINVAL;
  const KvArgs a = to_args(kv);
  const bool one_sweep = select_attend_supported(a, G);
  if (!score_supported(kv, G) || (!one_sweep && !long_select_attend_supported(a, G)))
    return SKV_EUNSUPPORTED;
  const size_t th = topk_workspace_bytes(kv->B * kv->H, kv->L_max);
  const size_t pb = one_sweep ? select_attend_partial_bytes(a, G) : attend_workspace_bytes(a, G, k);
  if (!ws || ws_bytes < th + pb) return SKV_EWORKSPACE;
  debug_validate(kv, win, nullptr, 0, stream);
  uint32_t* hist = (uint32_t*)ws;
  float* part = (float*)((char*)ws + th);
  // few long rows: the scan lists segment candidates instead of the
  // histogram, and the finishing kernel selects from them (no listing kernel)
  if (sparsekv_segments(kv, G, k) > 0) {
    const skv_status st =
        sparsekv_score_segments(kv, q, G, win, k, scores, ws, ws_bytes, stream);
    if (st != SKV_OK) return st;
    return sparsekv_select_attend_segments(kv, q, G, win, k, scale, scores, idx, count, out, ws,
                                           ws_bytes, stream);
  }
  const hipError_t e = launch_score(a, q, G, scores, win.lo, win.hi, hist, stream);
  if (e != hipSuccess) return launched(e);
  if (!one_sweep)
    return long_select_attend(a, q, G, win, k, scale, scores, idx, count, out, ws, th, ws_bytes,
                              stream);
  return launched(launch_select_attend(a, q, G, scores, win.lo, win.hi, k, hist, scale, idx, count,
                                       part, out, stream));
}

skv_status sparsekv_select_attend_resume(const skv_kv* kv, const void* q, int32_t G,
                                         skv_window win, int32_t k, float scale,
                                         const float* scores, int32_t* idx, int32_t* count,
                                         float* out, void* ws, size_t ws_bytes,
                                         hipStream_t stream) {
  if (!kv_ok(kv) || !q || !scores || !idx || !count || !out || G < 1 || k < 1) return SKV_EINVAL;
  if (k > kv->L_max || !win.lo || !win.hi || !isfinite(scale)) return SKV_EINVAL;
  const KvArgs a = to_args(kv);
  const int rows = kv->B * kv->H;
  const size_t th = topk_workspace_bytes(rows, kv->L_max);
  float* part = (float*)((char*)ws + th);
  debug_validate(kv, win, nullptr, 0, stream);
  if (kv->v == nullptr) {
    // latent KV: rows longer than one sweep finish the top-k inside the
    // attention kernel; shorter ones take the one-workgroup top-k first
    if (!mla_supported(a, G) || !topk_supported(kv->L_max)) return SKV_EUNSUPPORTED;
    if (!ws || ws_bytes < th + mla_select_attend_partial_bytes(a, G, k)) return SKV_EWORKSPACE;
    if (mla_list_supported(a, G, k))
      return launched(launch_mla_list_attend(a, q, G, scores, win.lo, win.hi, k, ws, scale, idx,
                                             count, part, out, stream));
    const hipError_t e = launch_topk(scores, rows, kv->H, kv->L_max, win.lo, win.hi, k, idx, count,
                                     ws, true, stream);
    if (e != hipSuccess) return launched(e);
    return launched(launch_mla_attend(a, q, G, idx, k, win.lo, win.hi, scale, out, part,
                                      ws_bytes - th, stream));
  }
  if (select_attend_supported(a, G)) {
    if (!ws || ws_bytes < th + select_attend_partial_bytes(a, G)) return SKV_EWORKSPACE;
    return launched(launch_select_attend(a, q, G, scores, win.lo, win.hi, k, (uint32_t*)ws, scale,
                                         idx, count, part, out, stream));
  }
  if (!long_select_attend_supported(a, G)) return SKV_EUNSUPPORTED;
  if (!ws || ws_bytes < th + attend_workspace_bytes(a, G, k)) return SKV_EWORKSPACE;
  return long_select_attend(a, q, G, win, k, scale, scores, idx, count, out, ws, th, ws_bytes,
                            stream);
}

skv_status sparsekv_indexer_attend(const skv_kv* ikv, const void* iq, int32_t iG,
                                   const skv_kv* kv, const void* q, int32_t G, skv_window win,
                                   int32_t k, float scale, float* scores, int32_t* idx,
                                   int32_t* count, float* out, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
  if (!kv_ok(ikv) || !kv_ok(kv) || !iq || !q || !scores || !idx || !count || !out) return SKV_EINVAL;
  if (iG < 1 || G < 1 || k < 1 || k > kv->L_max || !win.lo || !win.hi || !isfinite(scale))
    return SKV_EINVAL;
  if (kv->v != nullptr || ikv->B != kv->B || ikv->H != kv->H || ikv->L_max != kv->L_max)
    return SKV_EINVAL;
  const KvArgs ia = to_args(ikv), a = to_args(kv);
  if (!score_supported(ikv, iG) || !mla_supported(a, G) || !topk_supported(kv->L_max))
    return SKV_EUNSUPPORTED;
  const int rows = kv->B * kv->H;
  const size_t th = topk_workspace_bytes(rows, kv->L_max);
  if (!ws || ws_bytes < th + mla_select_attend_partial_bytes(a, G, k)) return SKV_EWORKSPACE;
  // long rows: the indexer's scan lists segment candidates and the latent
  // attention kernel selects from them; otherwise the histogram scan and
  // sparsekv_select_attend_resume
  if (sparsekv_segments(kv, G, k) > 0 && score_seg_supported(ia, iG)) {
    const skv_status st =
        sparsekv_score_segments(ikv, iq, iG, win, k, scores, ws, ws_bytes, stream);
    if (st != SKV_OK) return st;
    return sparsekv_select_attend_segments(kv, q, G, win, k, scale, scores, idx, count, out, ws,
                                           ws_bytes, stream);
  }
  const skv_status st = sparsekv_score_hist(ikv, iq, iG, win, scores, ws, ws_bytes, stream);
  if (st != SKV_OK) return st;
  return sparsekv_select_attend_resume(kv, q, G, win, k, scale, scores, idx, count, out, ws,
                                       ws_bytes, stream);
}

int32_t sparsekv_segments(const skv_kv* kv, int32_t G, int32_t k) {
  if (!kv_ok(kv) || G < 1 || k < 1 || k > kv->L_max) return 0;
  const KvArgs a = to_args(kv);
  const int rows = kv->B * kv->H;
  // GQA rows: only when several workgroups share a row (fewer than
  // kFinishAttendMinRows rows).  With one workgroup per row, the row's own
  // listing is cheaper than the segment lists: the token pool's scan took
  // 517 against 488 us with them (4,096 workgroups, each ending with the
  // segment's listing) and the selecting kernel 49.7 against 67.3 us
  const bool consumer = kv->v == nullptr ? mla_list_supported(a, G, k)
                                         : finish_attend_seg_supported(a, G, k) &&
                                               rows < kFinishAttendMinRows;
  return consumer ? topk_seg_count(rows, kv->L_max, k) : 0;
}

skv_status sparsekv_score_segments(const skv_kv* kv, const void* q, int32_t G, skv_window win,
                                   int32_t k, float* scores, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
  if (!kv_ok(kv) || !q || !scores || G < 1 || k < 1 || k > kv->L_max || !win.lo || !win.hi)
    return SKV_EINVAL;
  const KvArgs a = to_args(kv);
  const int rows = kv->B * kv->H;
  const int n_seg = topk_seg_count(rows, kv->L_max, k);
  if (n_seg == 0 || !score_seg_supported(a, G)) return SKV_EUNSUPPORTED;
  if (!ws || ws_bytes < topk_workspace_bytes(rows, kv->L_max)) return SKV_EWORKSPACE;
  debug_validate(kv, win, nullptr, 0, stream);
  return launched(launch_score_seg(a, q, G, scores, win.lo, win.hi, ws, n_seg, stream));
}

skv_status sparsekv_select_attend_segments(const skv_kv* kv, const void* q, int32_t G,
                                           skv_window win, int32_t k, float scale,
                                           const float* scores, int32_t* idx, int32_t* count,
                                           float* out, void* ws, size_t ws_bytes,
                                           hipStream_t stream) {
  if (!kv_ok(kv) || !q || !scores || !idx || !count || !out || G < 1 || k < 1) return SKV_EINVAL;
  if (k > kv->L_max || !win.lo || !win.hi || !isfinite(scale)) return SKV_EINVAL;
  const int n_seg = sparsekv_segments(kv, G, k);
  if (n_seg == 0) return SKV_EUNSUPPORTED;
  const KvArgs a = to_args(kv);
  const int rows = kv->B * kv->H;
  const size_t th = topk_workspace_bytes(rows, kv->L_max);
  const size_t pb = kv->v == nullptr ? mla_select_attend_partial_bytes(a, G, k)
                                     : attend_workspace_bytes(a, G, k);
  if (!ws || ws_bytes < th + pb) return SKV_EWORKSPACE;
  debug_validate(kv, win, nullptr, 0, stream);
  float* part = (float*)((char*)ws + th);
  if (kv->v == nullptr)
    return launched(launch_mla_list_attend(a, q, G, scores, win.lo, win.hi, k, ws, scale, idx,
                                           count, part, out, stream, n_seg));
  return launched(launch_finish_attend(a, q, G, scores, win.lo, win.hi, k, ws, scale, idx, count,
                                       out, part, stream, n_seg));
}

size_t sparsekv_select_attend_noalloc_bytes(const skv_kv* kv, int32_t G) {
  if (!kv || kv->B < 1 || kv->H < 1 || G < 1 || kv->d_k < 1) return 0;
  return noalloc_hist_bytes(kv->B * kv->H) + select_attend_partial_bytes(to_args(kv), G);
}

skv_status sparsekv_select_attend_noalloc(const skv_kv* kv, const void* q, int32_t G,
                                          skv_window win, int32_t k, float scale, float* scores,
                                          int32_t* idx, int32_t* count, float* out,
                                          hipStream_t stream) {
  if (!kv_ok(kv) || !q || !scores || !idx || !count || !out || G < 1 || k < 1) return SKV_EINVAL;
  if (k > kv->L_max || !win.lo || !win.hi || !isfinite(scale)) return SKV_EINVAL;
  const KvArgs a = to_args(kv);
  if (!score_supported(kv, G) || !select_attend_supported(a, G)) return SKV_EUNSUPPORTED;
  const int rows = kv->B * kv->H;
  const size_t hb = noalloc_hist_bytes(rows);
  if (hb + select_attend_partial_bytes(a, G) > kScratchBytes) return SKV_EWORKSPACE;
  debug_validate(kv, win, nullptr, 0, stream);
  void* base = nullptr;
  if (scratch_for_current_device(&base) != hipSuccess) return SKV_ELAUNCH;
  uint32_t* hist = (uint32_t*)base;
  float* part = (float*)((char*)base + hb);
  // the histograms start at zero whatever an earlier call left (a fill
  // kernel, not a memset node, so the call can be captured in a graph)
  const int64_t n16 = (int64_t)hb / 16;
  zero_words_kernel<<<(unsigned)std::min<int64_t>(1024, (n16 + 255) / 256), 256, 0, stream>>>(
      (uint4*)hist, n16);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return launched(e);
  e = launch_score(a, q, G, scores, win.lo, win.hi, hist, stream);
  if (e != hipSuccess) return launched(e);
  return launched(launch_select_attend(a, q, G, scores, win.lo, win.hi, k, hist, scale, idx, count,
                                       part, out, stream));
}

size_t sparsekv_block_summary_bytes(int32_t n_blocks, int32_t H, int32_t d_k) {
  if (n_blocks < 1 || H < 1 || d_k < 1) return 0;
  return (size_t)((n_blocks + 15) / 16) * H * 16 * 2 * d_k * 2;
}

skv_status sparsekv_block_summarize(const skv_kv* kv, int32_t b, int32_t j0, int32_t j1,
                                    void* summ, hipStream_t stream) {
  if (!kv_ok(kv) || !summ || b < 0 || b >= kv->B || j0 < 0 || j1 < j0) return SKV_EINVAL;
  if (j1 > kv->L_max / 16) return SKV_EINVAL;
  if (!block_summary_supported(to_args(kv))) return SKV_EUNSUPPORTED;
  return launched(launch_block_summaries(to_args(kv), b, j0, j1, summ, stream));
}

skv_status sparsekv_block_summarize_last(const skv_kv* kv, void* summ, hipStream_t stream) {
  if (!kv_ok(kv) || !summ) return SKV_EINVAL;
  if (!block_summary_supported(to_args(kv))) return SKV_EUNSUPPORTED;
  return launched(launch_block_summaries_last(to_args(kv), summ, stream));
}

skv_status sparsekv_block_select(const skv_kv* kv, void* summ, const void* q, int32_t G,
                                 skv_window win, int32_t K, float* blk_scores, int32_t* blk_idx,
                                 int32_t* blk_count, int32_t* tok_idx, void* ws, size_t ws_bytes,
                                 hipStream_t stream) {
  if (!kv_ok(kv) || !summ || !q || !blk_scores || !blk_idx || !blk_count || !tok_idx)
    return SKV_EINVAL;
  if (G < 1 || K < 1 || K > kv->L_max / 16 || !win.lo || !win.hi) return SKV_EINVAL;
  const KvArgs a = to_args(kv);
  if (!block_select_supported(a, G)) return SKV_EUNSUPPORTED;
  if (!ws || ws_bytes < block_select_ws_bytes(a, G)) return SKV_EWORKSPACE;
  debug_validate(kv, win, nullptr, 0, stream);
  return launched(launch_block_select(a, summ, q, G, win.lo, win.hi, K, blk_scores, blk_idx,
                                      blk_count, tok_idx, ws, stream));
}

size_t sparsekv_workspace_size(skv_op op, const skv_kv* kv, int32_t G, int32_t k,
                               const skv_index* index) {
  switch (op) {
    case SKV_OP_SCORE:
    case SKV_OP_ENCODE:
      return 0;
    case SKV_OP_TOPK:
    case SKV_OP_SELECT:
      if (!kv || kv->B < 1 || kv->H < 1 || kv->L_max < 1) return 0;
      return topk_workspace_bytes(kv->B * kv->H, kv->L_max);
    case SKV_OP_GATHER_ATTEND:
      if (!kv_ok(kv) || G < 1 || k < 0) return 0;
      if (kv->v == nullptr) return mla_workspace_bytes(to_args(kv), G, k);
      return attend_workspace_bytes(to_args(kv), G, k);
    case SKV_OP_RETRIEVE:
      return sparsekv_retrieve_workspace_size(index, G, 1.0f, k);
    case SKV_OP_SELECT_ATTEND:
      if (!kv_ok(kv) || G < 1 || k < 0) return 0;
      return topk_workspace_bytes(kv->B * kv->H, kv->L_max) +
             (kv->v == nullptr ? mla_select_attend_partial_bytes(to_args(kv), G, k)
                               : std::max(select_attend_partial_bytes(to_args(kv), G),
                                          attend_workspace_bytes(to_args(kv), G, k)));
    case SKV_OP_BLOCK_SELECT:
      if (!kv_ok(kv) || G < 1) return 0;
      return block_select_ws_bytes(to_args(kv), G);
  }
  return 0;
}

const char* sparsekv_status_string(skv_status s) {
  switch (s) {
    case SKV_OK: return "ok";
    case SKV_EINVAL: return "invalid argument";
    case SKV_EUNSUPPORTED: return "unsupported shape or dtype";
    case SKV_EWORKSPACE: return "workspace too small";
    case SKV_ELAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

int32_t sparsekv_version(void) { return 1; }

}  // extern "C"
