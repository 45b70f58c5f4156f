// Exact top-k per (sequence, KV head) row of fp32 scores.
//
// What is computed: the k largest finite scores among t in [lo[b], hi[b]),
// ties broken toward the lower t, -0.0 equal to +0.0, returned as a set in
// ascending t with -1 padding (ECHO-OSDI26 wiki page, observation 5: the
// final selection is an exact top-k, whatever was prefetched).
//
// gfx950 design: one 1024-thread workgroup per row, radix select on an
// order-preserving 32-bit key (sign-flipped float bits), digits of 12, 12 and
// 8 bits with LDS histograms (4096 / 4096 / 256 bins).  Each pass counts only
// the keys that still match the prefix chosen so far, a block scan over the
// bins finds the bin that holds the k-th largest key, and the pass stops early
// once that bin is taken whole.  Rows of up to 32768 candidates keep their keys
// in LDS (128 KB of the 160 KB) after the first read; longer rows re-read the
// scores (L2-resident).  The final compaction walks the row in index order
// with wave ballots, so the output is sorted and the lowest indices win ties.
// ECHO describes an 8-bit, 256-bin histogram on the top score bits as prior
// art; the wider first digit here splits fp32 exponents by 3 mantissa bits,
// which keeps the threshold bin small for score distributions that span a few
// octaves.
#include "skv_device.h"

namespace skv {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kLdsCap = 32768;   // keys cached in LDS
constexpr int kBins = 4096;

__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u & 0x7f800000u) == 0x7f800000u) return 0u;   // inf / nan: not a candidate
  if (u == 0x80000000u) u = 0u;                        // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);   // finite keys are >= 0x00800000
}

struct Shared {
  uint32_t hist[kBins];
  int wsum[kWaves][2];
  int sel_bin, sel_above;
};

template <bool LDS>
__global__ __launch_bounds__(kThreads) void topk_kernel(const float* scores, int H, int L_max,
                                                        const int32_t* lo_p, const int32_t* hi_p,
                                                        int k, int32_t* idx, int32_t* count) {
  __shared__ Shared sh;
  extern __shared__ uint32_t keys[];   // [kLdsCap] when LDS
  const int row = blockIdx.x;
  const int b = row / H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* srow = scores + (int64_t)row * L_max;
  int32_t* orow = idx + (int64_t)row * k;

  const int lo = max(0, min(lo_p[b], L_max));
  const int hi = max(lo, min(hi_p[b], L_max));
  const int n = hi - lo;

  auto key_at = [&](int i) -> uint32_t {
    if constexpr (LDS) return keys[i];
    else return score_key(srow[lo + i]);
  };

  // ---- radix passes -------------------------------------------------------
  uint32_t prefix = 0, mask = 0;
  int need = 0;
  bool take_all = false;
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 20 : (pass == 1 ? 8 : 0);
    const int nb = pass < 2 ? 4096 : 256;
    for (int i = tid; i < nb; i += kThreads) sh.hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kThreads) {
      uint32_t key;
      if (pass == 0) {
        key = score_key(srow[lo + i]);
        if constexpr (LDS) keys[i] = key;
      } else {
        key = key_at(i);
      }
      if (key != 0u && (key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & (nb - 1)], 1u);
    }
    __syncthreads();
    // bins owned by this thread: [tid*per, tid*per + per), per = nb / kThreads (or 1)
    const int per = nb >= kThreads ? nb / kThreads : 1;
    const int b0 = tid * per;
    int tot = 0;
    if (b0 < nb)
      for (int j = 0; j < per; ++j) tot += (int)sh.hist[b0 + j];
    // inclusive scan of thread totals over the block
    const int wex = wave_excl_scan(tot, lane);
    if (lane == 63) sh.wsum[wave][0] = wex + tot;
    __syncthreads();
    int before = wex, all = 0;
    for (int w = 0; w < kWaves; ++w) {
      const int v = sh.wsum[w][0];
      if (w < wave) before += v;
      all += v;
    }
    if (pass == 0) {
      need = min(k, all);             // all = number of finite candidates
      if (need == all) {              // every candidate selected
        take_all = true;
        __syncthreads();
        break;
      }
    }
    // keys in bins above this thread's bins: all - before - tot
    if (b0 < nb) {
      int above = all - before - tot;
      for (int j = per - 1; j >= 0; --j) {
        const int c = (int)sh.hist[b0 + j];
        if (above < need && need <= above + c) {
          sh.sel_bin = b0 + j;
          sh.sel_above = above;
        }
        above += c;
      }
    }
    __syncthreads();
    const int bin = sh.sel_bin;
    const int above = sh.sel_above;
    const int in_bin = (int)sh.hist[bin];
    need -= above;
    prefix |= (uint32_t)bin << shift;
    mask |= (uint32_t)(nb - 1) << shift;
    __syncthreads();
    if (need == in_bin) {             // the whole bin is taken
      take_all = true;
      break;
    }
  }
  if (take_all) need = 0x7fffffff;
  // Selection rule: (key & mask) > prefix, or (key & mask) == prefix and it is
  // among the first `need` such keys in index order.

  // ---- ordered compaction -------------------------------------------------
  // wave w owns the contiguous segment [w*seg, (w+1)*seg) of the window
  const int seg = (n + kWaves - 1) / kWaves;
  const int s0 = min(n, wave * seg), s1 = min(n, s0 + seg);
  int c_above = 0, c_eq = 0;
  for (int i0 = s0; i0 < s1; i0 += 64) {
    const int i = i0 + lane;
    uint32_t key = 0;
    if (i < s1) key = key_at(i);
    const uint32_t km = key & mask;
    const bool ok = key != 0u;
    const uint64_t ba = __ballot(ok && km > prefix);
    const uint64_t be = __ballot(ok && km == prefix);
    c_above += __popcll(ba);
    c_eq += __popcll(be);
  }
  if (lane == 0) {
    sh.wsum[wave][0] = c_above;
    sh.wsum[wave][1] = c_eq;
  }
  __syncthreads();
  int off_above = 0, off_eq = 0;
  for (int w = 0; w < wave; ++w) {
    off_above += sh.wsum[w][0];
    off_eq += sh.wsum[w][1];
  }
  const uint64_t lt = lanemask_lt(lane);
  for (int i0 = s0; i0 < s1; i0 += 64) {
    const int i = i0 + lane;
    uint32_t key = 0;
    if (i < s1) key = key_at(i);
    const uint32_t km = key & mask;
    const bool ok = key != 0u;
    const bool is_above = ok && km > prefix;
    const bool is_eq = ok && km == prefix;
    const uint64_t ba = __ballot(is_above);
    const uint64_t be = __ballot(is_eq);
    const int a_before = off_above + __popcll(ba & lt);
    const int e_before = off_eq + __popcll(be & lt);
    const bool sel = is_above || (is_eq && e_before < need);
    const int dst = a_before + min(e_before, need);
    if (sel && dst < k) orow[dst] = lo + i;
    off_above += __popcll(ba);
    off_eq += __popcll(be);
  }
  // number selected = min(k, candidates); pad the rest
  int n_sel = 0;
  {
    int tot_above = 0, tot_eq = 0;
    for (int w = 0; w < kWaves; ++w) {
      tot_above += sh.wsum[w][0];
      tot_eq += sh.wsum[w][1];
    }
    n_sel = tot_above + min(tot_eq, need);
  }
  for (int i = n_sel + tid; i < k; i += kThreads) orow[i] = -1;
  if (tid == 0) count[row] = n_sel;
}

}  // namespace

hipError_t launch_topk(const float* scores, int rows, int H, int L_max, const int32_t* lo,
                       const int32_t* hi, int k, int32_t* idx, int32_t* count, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (L_max <= kLdsCap) {
    const size_t dyn = (size_t)L_max * sizeof(uint32_t);
    static bool attr_set = false;
    if (!attr_set) {
      hipError_t e = hipFuncSetAttribute((const void*)topk_kernel<true>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                         (int)(kLdsCap * sizeof(uint32_t)));
      if (e != hipSuccess) return e;
      attr_set = true;
    }
    topk_kernel<true><<<rows, kThreads, dyn, s>>>(scores, H, L_max, lo, hi, k, idx, count);
  } else {
    topk_kernel<false><<<rows, kThreads, 0, s>>>(scores, H, L_max, lo, hi, k, idx, count);
  }
  return hipGetLastError();
}

}  // namespace skv
