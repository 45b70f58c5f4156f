// Validation of the device-resident data the decode step takes on trust:
// sequence lengths, windows, table entries inside the pool, no slot mapped
// twice (vToken reading notes, section 3.5 invariant I2; section 4.6 checks
// the invariants around every migration), selected positions in range and
// distinct.  Reads only seq_len, the tables, lo / hi and idx -- never the K/V
// pools -- so invalid tables never form an address into them.  Flags are
// OR-ed into a device word (SKV_FLAG_* in sparsekv.h).
//
// In builds compiled with SKV_DEBUG every entry point that reads tables,
// windows or selected positions first runs these checks into a flag word the
// library holds per device (sparsekv_debug_status reads and clears it); such
// builds allocate their check workspace with hipMalloc and are not meant for
// graph capture.
#include <algorithm>
#include <mutex>

#include "../../include/sparsekv.h"
#include "skv_internal.h"

namespace skv {

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void zero_u32_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kThreads)
    p[i] = 0u;
}

// One workgroup: seq_len in [0, L_max]; 0 <= lo <= hi <= seq_len.
__global__ __launch_bounds__(kThreads) void check_seq_kernel(const int32_t* seq_len, int B,
                                                             int L_max, const int32_t* lo,
                                                             const int32_t* hi, int32_t* flags) {
  __shared__ int f;
  if (threadIdx.x == 0) f = 0;
  __syncthreads();
  int mine = 0;
  for (int b = threadIdx.x; b < B; b += kThreads) {
    const int s = seq_len[b];
    if (s < 0 || s > L_max) mine |= SKV_FLAG_BAD_SEQ_LEN;
    if (lo && hi) {
      const int sc = min(max(s, 0), L_max);
      const int l = lo[b], h = hi[b];
      if (l < 0 || l > h || h > sc) mine |= SKV_FLAG_BAD_WINDOW;
    }
  }
  if (mine) atomicOr(&f, mine);
  __syncthreads();
  if (threadIdx.x == 0 && f) atomicOr(flags, f);
}

// Grid (ceil(L_max / 256), B): token-table entries of t < seq_len[b]; a
// valid slot is claimed (claims [16 n_blocks], zeroed before) when the pool
// size is known, a second claim is a duplicate.
__global__ __launch_bounds__(kThreads) void check_token_table_kernel(
    const int32_t* tt, const int32_t* seq_len, int L_max, int n_blocks, uint32_t* claims,
    int32_t* flags) {
  __shared__ int f;
  if (threadIdx.x == 0) f = 0;
  __syncthreads();
  const int b = blockIdx.y, t = blockIdx.x * kThreads + threadIdx.x;
  const int n = min(max(seq_len[b], 0), L_max);
  int mine = 0;
  if (t < n) {
    const int e = tt[(int64_t)b * L_max + t];
    if (e < -1 || (n_blocks > 0 && (int64_t)e >= (int64_t)n_blocks * 16)) {
      mine = SKV_FLAG_BAD_SLOT;
    } else if (e >= 0 && n_blocks > 0) {
      if (atomicAdd(&claims[e], 1u) != 0u) mine = SKV_FLAG_DUP_SLOT;
    }
  }
  if (mine) atomicOr(&f, mine);
  __syncthreads();
  if (threadIdx.x == 0 && f) atomicOr(flags, f);
}

// Grid (ceil(L_max / 16 / 256), B): block-table entries of the blocks holding
// t < seq_len[b]; -1 is an unmapped block; claims [n_blocks].
__global__ __launch_bounds__(kThreads) void check_block_table_kernel(
    const int32_t* bt, const int32_t* seq_len, int L_max, int n_blocks, uint32_t* claims,
    int32_t* flags) {
  __shared__ int f;
  if (threadIdx.x == 0) f = 0;
  __syncthreads();
  const int b = blockIdx.y, j = blockIdx.x * kThreads + threadIdx.x;
  const int n = min(max(seq_len[b], 0), L_max);
  int mine = 0;
  if (j < (n + 15) / 16) {
    const int e = bt[(int64_t)b * (L_max / 16) + j];
    if (e < -1 || (n_blocks > 0 && e >= n_blocks)) {
      mine = SKV_FLAG_BAD_SLOT;
    } else if (e >= 0 && n_blocks > 0) {
      if (atomicAdd(&claims[e], 1u) != 0u) mine = SKV_FLAG_DUP_SLOT;
    }
  }
  if (mine) atomicOr(&f, mine);
  __syncthreads();
  if (threadIdx.x == 0 && f) atomicOr(flags, f);
}

// Grid (ceil(k / 256), rows): idx entries in [-1, L_max); a position named
// twice in a row is found through the row's bitmap (bits [rows][L_max],
// zeroed before).
__global__ __launch_bounds__(kThreads) void check_idx_kernel(const int32_t* idx, int k, int L_max,
                                                             uint32_t* bits, int32_t* flags) {
  __shared__ int f;
  if (threadIdx.x == 0) f = 0;
  __syncthreads();
  const int row = blockIdx.y, i = blockIdx.x * kThreads + threadIdx.x;
  int mine = 0;
  if (i < k) {
    const int e = idx[(int64_t)row * k + i];
    if (e < -1 || e >= L_max) {
      mine = SKV_FLAG_BAD_IDX;
    } else if (e >= 0) {
      const uint32_t bit = 1u << (e & 31);
      uint32_t* w = bits + (int64_t)row * ((L_max + 31) / 32) + (e >> 5);
      if (atomicOr(w, bit) & bit) mine = SKV_FLAG_DUP_IDX;
    }
  }
  if (mine) atomicOr(&f, mine);
  __syncthreads();
  if (threadIdx.x == 0 && f) atomicOr(flags, f);
}

bool validate_kv_ok(const skv_kv* kv) {
  return kv && kv->seq_len && kv->B >= 1 && kv->H >= 1 && kv->L_max >= 1 && kv->n_blocks >= 0 &&
         (kv->block == 0 || (kv->block == 16 && kv->L_max % 16 == 0));
}

size_t claims_words(const skv_kv* kv) {
  if (kv->n_blocks <= 0) return 0;
  if (kv->token_table) return (size_t)kv->n_blocks * 16;
  if (kv->block_table) return (size_t)kv->n_blocks;
  return 0;
}

size_t bits_words(const skv_kv* kv, int k) {
  return k > 0 ? (size_t)kv->B * kv->H * ((kv->L_max + 31) / 32) : 0;
}

size_t validate_ws(const skv_kv* kv, int k) {
  return (claims_words(kv) + bits_words(kv, k)) * 4;
}

hipError_t launch_validate(const skv_kv* kv, skv_window win, const int32_t* idx, int k,
                           int32_t* flags, void* ws, hipStream_t st) {
  const size_t nc = claims_words(kv), nb = idx ? bits_words(kv, k) : 0;
  uint32_t* claims = (uint32_t*)ws;
  uint32_t* bits = claims + nc;
  if (nc + nb) {
    const int64_t n = (int64_t)(nc + nb);
    zero_u32_kernel<<<(unsigned)std::min<int64_t>(2048, (n + kThreads - 1) / kThreads), kThreads,
                      0, st>>>(claims, n);
  }
  check_seq_kernel<<<1, kThreads, 0, st>>>(kv->seq_len, kv->B, kv->L_max, win.lo, win.hi, flags);
  if (kv->token_table)
    check_token_table_kernel<<<dim3((kv->L_max + kThreads - 1) / kThreads, kv->B), kThreads, 0,
                               st>>>(kv->token_table, kv->seq_len, kv->L_max, kv->n_blocks, claims,
                                     flags);
  else if (kv->block_table)
    check_block_table_kernel<<<dim3((kv->L_max / 16 + kThreads - 1) / kThreads, kv->B), kThreads,
                               0, st>>>(kv->block_table, kv->seq_len, kv->L_max, kv->n_blocks,
                                        claims, flags);
  if (idx && k > 0)
    check_idx_kernel<<<dim3((k + kThreads - 1) / kThreads, kv->B * kv->H), kThreads, 0, st>>>(
        idx, k, kv->L_max, bits, flags);
  return hipGetLastError();
}

#ifdef SKV_DEBUG
// The debug build's per-device flag word and check workspace.
__device__ int32_t debug_flags;
constexpr int kMaxDevices = 64;
std::mutex g_mu;
int32_t* g_flags[kMaxDevices] = {};
void* g_ws[kMaxDevices] = {};
size_t g_ws_bytes[kMaxDevices] = {};

int32_t* debug_flag_word(int dev) {
  if (!g_flags[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(debug_flags)) != hipSuccess) return nullptr;
    g_flags[dev] = (int32_t*)p;
  }
  return g_flags[dev];
}
#endif

}  // namespace

// Called first by the entry points of a debug build (a no-op otherwise).
void debug_validate(const skv_kv* kv, skv_window win, const int32_t* idx, int k, hipStream_t st) {
#ifdef SKV_DEBUG
  if (!validate_kv_ok(kv)) return;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return;
  std::lock_guard<std::mutex> lock(g_mu);
  int32_t* flags = debug_flag_word(dev);
  if (!flags) return;
  const size_t need = validate_ws(kv, idx ? k : 0);
  if (need > g_ws_bytes[dev]) {
    if (g_ws[dev]) (void)hipFree(g_ws[dev]);   // a failure here only leaks the old buffer
    g_ws[dev] = nullptr;
    g_ws_bytes[dev] = 0;
    if (hipMalloc(&g_ws[dev], need) != hipSuccess) return;
    g_ws_bytes[dev] = need;
  }
  // a failed launch stays the thread's last HIP error, which the calling
  // entry point's own launch check reports
  (void)launch_validate(kv, win, idx, idx ? k : 0, flags, g_ws[dev], st);
#else
  (void)kv; (void)win; (void)idx; (void)k; (void)st;
#endif
}

}  // namespace skv

using namespace skv;

extern "C" {

size_t sparsekv_validate_ws_bytes(const skv_kv* kv, int32_t k) {
  if (!validate_kv_ok(kv) || k < 0) return 0;
  return validate_ws(kv, k);
}

skv_status sparsekv_validate(const skv_kv* kv, skv_window win, const int32_t* idx, int32_t k,
                             int32_t* flags, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!validate_kv_ok(kv) || !flags || k < 0 || (k > 0 && !idx) || (!win.lo != !win.hi))
    return SKV_EINVAL;
  if (kv->block == 16 && !kv->token_table && !kv->block_table) return SKV_EINVAL;
  const size_t need = validate_ws(kv, idx ? k : 0);
  if (need && (!ws || ws_bytes < need)) return SKV_EWORKSPACE;
  return launch_validate(kv, win, idx, idx ? k : 0, flags, ws, stream) == hipSuccess ? SKV_OK
                                                                                    : SKV_ELAUNCH;
}

skv_status sparsekv_debug_status(int32_t* flags) {
  if (!flags) return SKV_EINVAL;
#ifdef SKV_DEBUG
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SKV_ELAUNCH;
  std::lock_guard<std::mutex> lock(g_mu);
  int32_t* word = debug_flag_word(dev);
  if (!word) return SKV_ELAUNCH;
  if (hipDeviceSynchronize() != hipSuccess) return SKV_ELAUNCH;
  if (hipMemcpy(flags, word, sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess)
    return SKV_ELAUNCH;
  const int32_t zero = 0;
  if (hipMemcpy(word, &zero, sizeof(int32_t), hipMemcpyHostToDevice) != hipSuccess)
    return SKV_ELAUNCH;
  return SKV_OK;
#else
  *flags = 0;
  return SKV_EUNSUPPORTED;
#endif
}

int32_t sparsekv_is_debug_build(void) {
#ifdef SKV_DEBUG
  return 1;
#else
  return 0;
#endif
}

}  // extern "C"
