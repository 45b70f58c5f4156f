// Exact top-k per (sequence, KV head) row of fp32 scores.
//
// What is computed: the k largest finite scores among t in [lo[b], hi[b]),
// ties broken toward the lower t, -0.0 equal to +0.0, returned as a set in
// ascending t with -1 padding (ECHO-OSDI26 wiki page, observation 5: the
// final selection is an exact top-k, whatever was prefetched).
//
// gfx950 design: a radix select on an order-preserving 32-bit key
// (sign-flipped float bits), one 1024-thread workgroup per row.  The row's
// keys stay in registers (32 per lane for rows of up to 32768 scores; longer
// rows are re-read per pass) while the workgroup
//   1. takes the histogram of the top 12 key bits (built by the score scan
//      when the two are fused, else here with LDS atomics) and finds the bin
//      b0 that holds the k-th largest key while the row's scores arrive;
//   2. resolves the exact 32-bit threshold T and the number of keys equal to
//      T to take (lowest positions first) with two more digits of 12 and 8
//      bits, histogramming only the keys whose prefix still matches;
//   3. writes the selected positions in ascending order: per group of 4
//      consecutive keys per lane, one DPP prefix sum of the packed counts of
//      keys above and equal to T places every lane's keys; one barrier
//      exchanges the waves' totals.
// Everything after the one load of the row happens in registers and LDS with
// DPP scans, so the kernel is a short chain of barriers rather than a chain
// of memory round trips.  ECHO describes an 8-bit, 256-bin histogram of the top score
// bits as prior art; a 12-bit first digit splits each fp32 octave into 8
// bins, which keeps the threshold bin small for score distributions that span
// a few octaves.  The kernel zeroes the row histogram it read, so a
// zero-filled workspace stays valid across calls.
#include "skv_device.h"
#include "skv_topk.h"

namespace skv {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kGroups = 8;                   // groups of 4 consecutive keys per lane per sweep
constexpr int kSeg = 256 * kGroups;          // positions per wave per sweep
constexpr int kSweep = kWaves * kSeg;        // positions per sweep (32768)
constexpr int kBins = 4096;

__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u & 0x7f800000u) == 0x7f800000u) return 0u;   // inf / nan: not a candidate
  if (u == 0x80000000u) u = 0u;                        // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);   // finite keys are >= 0x00800000
}

struct RowWindow {
  int lo, hi, n;
};

__device__ __forceinline__ RowWindow window(const int32_t* lo_p, const int32_t* hi_p, int b,
                                            int L_max) {
  RowWindow w;
  w.lo = max(0, min(lo_p[b], L_max));
  w.hi = max(w.lo, min(hi_p[b], L_max));
  w.n = w.hi - w.lo;
  return w;
}

__device__ __forceinline__ int wave_total(int incl) { return __builtin_amdgcn_readlane(incl, 63); }

// In a wave whose lane l holds the counts of 4 bins b + 4 l .. b + 4 l + 3
// (c[0..3]) and `above` = entries in bins above this lane's: if the
// need-th largest entry lies in one of this lane's bins, write
// {bin, entries above it, entries in it} to trio.
__device__ __forceinline__ void pick_bin(const uint4& c, int first_bin, int above, int need,
                                         int* trio) {
  const int cs[4] = {(int)c.x, (int)c.y, (int)c.z, (int)c.w};
#pragma unroll
  for (int j = 3; j >= 0; --j) {
    if (above < need && need <= above + cs[j]) {
      trio[0] = first_bin + j;
      trio[1] = above;
      trio[2] = cs[j];
    }
    above += cs[j];
  }
}

// Row kernel.  In sweep s, lane l of wave w holds the keys of the positions
// s * kSweep + w * kSeg + 256 g + 4 l + e (g < kGroups, e < 4) relative to
// lo: every load instruction reads 1 KB of consecutive scores.
// RES: the whole window fits one sweep and stays in registers.
template <bool RES>
__global__ __launch_bounds__(kThreads) void topk_row_kernel(const float* scores, int H, int L_max,
                                                            const int32_t* lo_p,
                                                            const int32_t* hi_p, int k,
                                                            uint32_t* ghist, int32_t* idx,
                                                            int32_t* count) {
  __shared__ uint32_t hist[kBins];           // top 12 bits, then bits 19..8 of bin b0's keys
  __shared__ uint32_t dh[256];               // bits 7..0 of the keys matching 24 bits
  __shared__ int wt[kWaves], wa[kWaves], we[kWaves];
  __shared__ int trio[3];
  const int row = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const RowWindow w = window(lo_p, hi_p, row / H, L_max);
  const float* s = scores + (int64_t)row * L_max + w.lo;
  const int n_sweeps = (w.n + kSweep - 1) / kSweep;
  const bool vec = ((uintptr_t)s & 15) == 0;   // 16-byte loads where aligned

  // scores of sweep sw (positions past the window read as -inf)
  auto load_raw = [&](int sw, float (&v)[kGroups][4]) {
    const int p0 = sw * kSweep + wave * kSeg + 4 * lane;
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      const int p = p0 + 256 * g;
      if (vec && p + 4 <= w.n) {
        const float4 f = *(const float4*)(s + p);
        v[g][0] = f.x;
        v[g][1] = f.y;
        v[g][2] = f.z;
        v[g][3] = f.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[g][e] = p + e < w.n ? s[p + e] : -INFINITY;
      }
    }
  };
  auto to_keys = [&](const float (&v)[kGroups][4], uint32_t (&kk)[kGroups][4]) {
#pragma unroll
    for (int g = 0; g < kGroups; ++g)
#pragma unroll
      for (int e = 0; e < 4; ++e) kk[g][e] = score_key(v[g][e]);
  };
  // the row histogram is loaded first and the resident scores next, so the
  // threshold-bin search overlaps the scores' arrival
  uint4* gh4 = ghist ? (uint4*)(ghist + (int64_t)row * kBins) : nullptr;
  uint4 gv = make_uint4(0u, 0u, 0u, 0u);
  if (gh4) gv = gh4[threadIdx.x];
  float fv[RES ? kGroups : 1][4];
  if constexpr (RES) load_raw(0, fv);
  uint32_t kr[RES ? kGroups : 1][4];
  // f(key) over every key of the window (keys outside it are 0)
  auto for_keys = [&](auto&& f) {
    if constexpr (RES) {
#pragma unroll
      for (int g = 0; g < kGroups; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) f(kr[g][e]);
    } else {
      for (int sw = 0; sw < n_sweeps; ++sw) {
        float v[kGroups][4];
        uint32_t kk[kGroups][4];
        load_raw(sw, v);
        to_keys(v, kk);
#pragma unroll
        for (int g = 0; g < kGroups; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e) f(kk[g][e]);
      }
    }
  };
  // The need-th largest entry of a kBins-bin histogram held in hist: wave w
  // covers bins 256 w .. 256 w + 255, lane l four of them.  Two barriers.
  // Also returns the histogram's total in *total.
  auto search4096 = [&](int need, int* total) {
    const uint4 c4 = *(const uint4*)(hist + 4 * threadIdx.x);
    const int cnt = (int)(c4.x + c4.y + c4.z + c4.w);
    const int incl = wave_incl_scan(cnt);
    const int tot_w = wave_total(incl);
    if (lane == 0) wt[wave] = tot_w;
    lds_barrier();
    int all = 0, above_w = 0;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
      all += wt[v];
      if (v > wave) above_w += wt[v];
    }
    *total = all;
    const int nd = need < 0 ? min(-need, all) : need;   // need < 0: min(-need, total)
    if (nd >= 1 && nd < all) pick_bin(c4, 4 * threadIdx.x, above_w + (tot_w - incl), nd, trio);
    lds_barrier();
    return nd;
  };

  // 1. histogram of the top 12 bits
  if (gh4) {
    *(uint4*)(hist + 4 * threadIdx.x) = gv;
  } else {
    if constexpr (RES) to_keys(fv, kr);
    *(uint4*)(hist + 4 * threadIdx.x) = make_uint4(0u, 0u, 0u, 0u);
    lds_barrier();
    for_keys([&](uint32_t key) {
      if (key) atomicAdd(&hist[key >> 20], 1u);
    });
  }
  if (threadIdx.x < 256) dh[threadIdx.x] = 0u;
  lds_barrier();
  int n_cand;
  const int k_sel = search4096(-k, &n_cand);   // k_sel = min(k, n_cand)
  if constexpr (RES) {
    if (gh4) to_keys(fv, kr);
  }

  // 2. threshold: select key > T, plus the first need_eq keys equal to T
  uint32_t T = 0u;   // k_sel == n_cand: every finite key (key > 0)
  int need_eq = 0;
  if (k_sel <= 0) {
    T = 0xffffffffu;   // nothing: finite keys are below 0xff800000
  } else if (k_sel < n_cand) {
    const int b0 = trio[0], above = trio[1], in_bin = trio[2];
    int need = k_sel - above;
    T = ((uint32_t)b0 << 20) - 1u;   // the whole bin b0 is taken
    if (need < in_bin) {
      // bits 19..8 of the keys of bin b0 (finite keys have top bits >= 8,
      // so b0 >= 8 and empty slots never match)
      lds_barrier();   // everyone has read trio and the top-bit counts
      *(uint4*)(hist + 4 * threadIdx.x) = make_uint4(0u, 0u, 0u, 0u);
      lds_barrier();
      for_keys([&](uint32_t key) {
        if ((key >> 20) == (uint32_t)b0) atomicAdd(&hist[(key >> 8) & 0xfffu], 1u);
      });
      lds_barrier();
      int unused;
      search4096(need, &unused);
      const int b1 = trio[0], ab1 = trio[1], ib1 = trio[2];
      need -= ab1;
      const uint32_t pre24 = ((uint32_t)b0 << 12) | (uint32_t)b1;
      if (need == ib1) {
        T = (pre24 << 8) - 1u;
        need = 0;
      } else {
        // bits 7..0 of the keys matching the top 24 bits
        for_keys([&](uint32_t key) {
          if ((key >> 8) == pre24) atomicAdd(&dh[key & 0xffu], 1u);
        });
        lds_barrier();
        if (wave == 0) {
          const uint4 d4 = *(const uint4*)(dh + 4 * lane);
          const int il = wave_incl_scan((int)(d4.x + d4.y + d4.z + d4.w));
          pick_bin(d4, 4 * lane, wave_total(il) - il, need, trio);
        }
        lds_barrier();
        const int b2 = trio[0], ab2 = trio[1], ib2 = trio[2];
        need -= ab2;
        T = (pre24 << 8) | (uint32_t)b2;
        if (need == ib2) {
          T -= 1u;
          need = 0;
        }
      }
      need_eq = need;
    }
  }

  // 3. ordered write.  Per group g the lanes' counts of keys above T and
  //    equal to T are packed into one int and prefix-summed across the wave;
  //    one barrier exchanges the waves' totals.
  int32_t* orow = idx + (int64_t)row * k;
  int a_base = 0, e_base = 0;   // keys above / equal to T in earlier sweeps
  auto emit = [&](const uint32_t (&kk)[kGroups][4], int sw) {
    int cg[kGroups];
    int lane_tot = 0;
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      int c = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) c += (kk[g][e] > T) ? 1 : ((kk[g][e] != 0u && kk[g][e] == T) ? 0x10000 : 0);
      cg[g] = c;
      lane_tot += c;
    }
    const int wt_pk = wave_total(wave_incl_scan(lane_tot));   // packed wave totals
    lds_barrier();   // wa / we of the previous sweep are consumed
    if (lane == 0) {
      wa[wave] = wt_pk & 0xffff;
      we[wave] = wt_pk >> 16;
    }
    lds_barrier();
    int oa = a_base, oe = e_base;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
      if (v < wave) {
        oa += wa[v];
        oe += we[v];
      }
      a_base += wa[v];
      e_base += we[v];
    }
    const int pos0 = w.lo + sw * kSweep + wave * kSeg + 4 * lane;
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      const int ig = wave_incl_scan(cg[g]);
      const int gt = wave_total(ig);
      int ab = oa + ((ig - cg[g]) & 0xffff), eb = oe + ((ig - cg[g]) >> 16);
      if (cg[g] & 0xffff || (cg[g] >> 16 && eb < need_eq)) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t key = kk[g][e];
          if (key > T) {
            const int dst = ab + min(eb, need_eq);
            if (dst < k) orow[dst] = pos0 + 256 * g + e;
            ++ab;
          } else if (key != 0u && key == T) {
            if (eb < need_eq && ab + eb < k) orow[ab + eb] = pos0 + 256 * g + e;
            ++eb;
          }
        }
      }
      oa += gt & 0xffff;
      oe += gt >> 16;
    }
  };
  if constexpr (RES) {
    emit(kr, 0);
  } else {
    for (int sw = 0; sw < n_sweeps; ++sw) {
      float v[kGroups][4];
      uint32_t kk[kGroups][4];
      load_raw(sw, v);
      to_keys(v, kk);
      emit(kk, sw);
    }
  }
  const int n_sel = min(k, a_base + min(e_base, need_eq));
  for (int i = n_sel + threadIdx.x; i < k; i += kThreads) orow[i] = -1;
  if (threadIdx.x == 0) count[row] = n_sel;
  if (gh4) gh4[threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);   // zero for the next call
}

}  // namespace

size_t topk_workspace_bytes(int rows, int L_max) {
  (void)L_max;
  return TopkWs::bytes(rows);
}

bool topk_supported(int L_max) { return L_max >= 1; }

hipError_t launch_topk(const float* scores, int rows, int H, int L_max, const int32_t* lo,
                       const int32_t* hi, int k, int32_t* idx, int32_t* count, void* wsp,
                       bool hist_ready, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  uint32_t* gh = hist_ready ? TopkWs::carve(wsp).hist : nullptr;
  if (L_max <= kSweep)
    topk_row_kernel<true><<<rows, kThreads, 0, s>>>(scores, H, L_max, lo, hi, k, gh, idx, count);
  else
    topk_row_kernel<false><<<rows, kThreads, 0, s>>>(scores, H, L_max, lo, hi, k, gh, idx, count);
  return hipGetLastError();
}

}  // namespace skv
