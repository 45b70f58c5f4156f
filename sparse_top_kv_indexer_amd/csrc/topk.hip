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
#include "skv_rowsel.h"
#include "skv_topk.h"

namespace skv {

namespace {

// RES: the whole window fits one sweep and stays in registers; otherwise the
// scores are re-read from memory for every pass over the keys.
template <bool RES>
__global__ __launch_bounds__(kRowThreads) void topk_row_kernel(const float* scores, int H,
                                                               int L_max, const int32_t* lo_p,
                                                               const int32_t* hi_p, int k,
                                                               uint32_t* ghist, int32_t* idx,
                                                               int32_t* count,
                                                               const int32_t* map_a,
                                                               const int32_t* map_b, int map_ld) {
  __shared__ RowSelLds L;
  const int row = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = row_wave();
  const RowWindow w = row_window(lo_p, hi_p, row / H, L_max);
  const float* s = scores + (int64_t)row * L_max + w.lo;
  const int n_sweeps = (w.n + kSweep - 1) / kSweep;
  const bool vec = ((uintptr_t)s & 15) == 0;   // 16-byte loads where aligned

  // the row histogram is loaded first and the resident scores next, so the
  // threshold-bin search overlaps the scores' arrival
  uint4* gh4 = ghist ? (uint4*)(ghist + (int64_t)row * kBins) : nullptr;
  uint4 gv = make_uint4(0u, 0u, 0u, 0u);
  if (gh4) gv = gh4[threadIdx.x];
  float fv[RES ? kGroups : 1][4];
  if constexpr (RES) row_load(s, w, vec, 0, fv);
  uint32_t kr[RES ? kGroups : 1][4];
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
        row_load(s, w, vec, sw, v);
        row_keys(v, kk);
#pragma unroll
        for (int g = 0; g < kGroups; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e) f(kk[g][e]);
      }
    }
  };

  // 1. histogram of the top 12 bits
  if (gh4) {
    *(uint4*)(L.hist + 4 * threadIdx.x) = gv;
  } else {
    if constexpr (RES) row_keys(fv, kr);
    *(uint4*)(L.hist + 4 * threadIdx.x) = make_uint4(0u, 0u, 0u, 0u);
    lds_barrier();
    for_keys([&](uint32_t key) {
      if (key) atomicAdd(&L.hist[key >> 20], 1u);
    });
  }
  if (threadIdx.x < 256) L.dh[threadIdx.x] = 0u;
  lds_barrier();

  // 2. threshold
  uint32_t T;
  int need_eq, k_sel;
  row_threshold(
      L, k,
      [&]() {
        if constexpr (RES) {
          if (gh4) row_keys(fv, kr);
        }
      },
      for_keys, &T, &need_eq, &k_sel);

  // 3. ordered write
  int32_t* orow = idx + (int64_t)row * k;
  // mapped positions: the selected positions are collected in LDS (the
  // histogram is no longer needed) and mapped in one pass at the end, so the
  // two dependent loads per key are not serialised inside the emit loop
  const bool map_lds = map_a && k <= kBins;
  int a_base = 0, e_base = 0;   // keys above / equal to T in earlier sweeps
  auto emit_sweep = [&](const uint32_t (&kk)[kGroups][4], int sw) {
    int cg[kGroups];
    const int lt = row_counts(kk, T, cg);
    int oa, oe, ta, te;
    row_wave_offsets(L, lt, &oa, &oe, &ta, &te);
    const int pos0 = w.lo + sw * kSweep + wave * kSeg + 4 * lane;
    row_emit(kk, cg, T, need_eq, a_base + oa, e_base + oe, [&](int dst, int g, int e) {
      if (dst < k) {
        const int p = pos0 + 256 * g + e;
        if (!map_a) orow[dst] = p;
        else if (map_lds) L.hist[dst] = (uint32_t)p;
        else orow[dst] = map_b[map_a[(int64_t)row * map_ld + p]];
      }
    });
    a_base += ta;
    e_base += te;
  };
  if constexpr (RES) {
    emit_sweep(kr, 0);
  } else {
    for (int sw = 0; sw < n_sweeps; ++sw) {
      float v[kGroups][4];
      uint32_t kk[kGroups][4];
      row_load(s, w, vec, sw, v);
      row_keys(v, kk);
      emit_sweep(kk, sw);
    }
  }
  const int n_sel = min(k, a_base + min(e_base, need_eq));
  if (map_lds) {
    lds_barrier();
    for (int i = threadIdx.x; i < n_sel; i += kRowThreads)
      orow[i] = map_b[map_a[(int64_t)row * map_ld + (int)L.hist[i]]];
  }
  for (int i = n_sel + threadIdx.x; i < k; i += kRowThreads) orow[i] = -1;
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
                       bool hist_ready, hipStream_t s, const int32_t* map_a,
                       const int32_t* map_b, int map_ld) {
  if (rows <= 0) return hipSuccess;
  uint32_t* gh = hist_ready ? TopkWs::carve(wsp).hist : nullptr;
  if (L_max <= kSweep)
    topk_row_kernel<true><<<rows, kRowThreads, 0, s>>>(scores, H, L_max, lo, hi, k, gh, idx, count,
                                                          map_a, map_b, map_ld);
  else
    topk_row_kernel<false><<<rows, kRowThreads, 0, s>>>(scores, H, L_max, lo, hi, k, gh, idx, count,
                                                          map_a, map_b, map_ld);
  return hipGetLastError();
}

}  // namespace skv
