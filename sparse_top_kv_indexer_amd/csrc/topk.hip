// Exact top-k per (sequence, KV head) row of fp32 scores.
//
// What is computed: the k largest finite scores among t in [lo[b], hi[b]),
// ties broken toward the lower t, -0.0 equal to +0.0, returned as a set in
// ascending t with -1 padding (ECHO-OSDI26 wiki page, observation 5: the
// final selection is an exact top-k, whatever was prefetched).
//
// gfx950 design: a radix select on an order-preserving 32-bit key
// (sign-flipped float bits) whose first digit is the top 12 bits.  ECHO
// describes an 8-bit, 256-bin histogram of the top score bits as prior art; a
// 12-bit first digit splits each fp32 octave into 8 bins, which keeps the
// threshold bin small for score distributions that span a few octaves.
//   0. the row's top-12-bit histogram: built by the score scan when the two
//      are fused, else by topk_hist_kernel (one 256-thread workgroup per
//      8192-slot slice, LDS atomics, non-zero bins added into the row's);
//   1. topk_compact_kernel, one workgroup per slice of 1024, 2048, 4096 or
//      8192 slots (the largest that still gives about 2048 workgroups, so a
//      few long rows spread over every compute unit): every workgroup finds
//      the bin b0 that holds the k-th largest key from the histogram and
//      lists its slice's keys in bins >= b0, with their positions, in
//      position order (a DPP prefix sum per group of 4 slots and one atomic
//      per workgroup on the row's list counter place them; each slice's
//      share is padded to a multiple of 4 entries with key 0); the list
//      holds the keys above b0 plus the bin's, typically k plus a few
//      hundred;
//   2. topk_finish_kernel, one 1024-thread workgroup per row: reads the list
//      slice by slice (16 consecutive ranks per lane, as four 16-byte
//      loads), resolves the exact threshold T and the number of keys equal
//      to T to take (lowest positions first) with two more digits of 12 and
//      8 bits over the listed keys of bin b0, and writes the selected
//      positions in ascending order with one prefix sum over the list,
//      staged in LDS so the stores to the output are consecutive words.
// The per-key work over the whole row is spread over all compute units and
// the row is read once (twice without the fused histogram).  A row whose
// list would exceed kRowList keys (many keys tied around the threshold) is
// selected by the finishing workgroup alone, re-reading the row per digit.
// Rows of at most one 32768-slot sweep are selected by one workgroup each,
// with the keys in registers: one kernel beats two or three there.
// The finishing kernel zeroes the row's histogram and list counter, so a
// zero-filled workspace stays valid across calls.
#include <type_traits>

#include "skv_listsel.h"
#include "skv_rowsel.h"
#include "skv_topk.h"

namespace skv {

namespace {

constexpr int kSliceThreads = 256;           // 4 waves x 256 NG slots = kSliceUnit NG
static_assert(kSliceThreads * 4 == kSliceUnit, "slice layout");

// Window of row `row`, its read base and this lane's first slot in slice sl
// of NG groups per lane (slots sl * kSliceUnit NG + wave * 256 NG + 256 g +
// 4 lane + e, g < NG).
struct SliceView {
  RowWindow w;
  const float* s;
  bool vec;
  int p0;
};

template <int NG>
__device__ __forceinline__ SliceView slice_view(const float* scores, int row, int H, int L_max,
                                                const int32_t* lo_p, const int32_t* hi_p, int sl) {
  SliceView v;
  v.w = row_window(lo_p, hi_p, row / H, L_max);
  v.s = row_base(scores, (int64_t)row * L_max, v.w, &v.vec);
  v.p0 = sl * kSliceUnit * NG + (threadIdx.x >> 6) * 256 * NG + 4 * (threadIdx.x & 63);
  return v;
}

// ------------------------------------------------------------ histogram --
// Grid rows * slices, 256 threads: the slice's top-12-bit key counts.
__global__ __launch_bounds__(kSliceThreads) void topk_hist_kernel(const float* scores, int H,
                                                                  int L_max, const int32_t* lo_p,
                                                                  const int32_t* hi_p,
                                                                  uint32_t* ghist, int n_slices,
                                                                  int copies) {
  __shared__ uint32_t lh[kBins];
  const int row = blockIdx.x / n_slices, sl = blockIdx.x - row * n_slices;
  const SliceView v = slice_view<kGroups>(scores, row, H, L_max, lo_p, hi_p, sl);
  if (sl * kSliceUnit * kGroups >= v.w.ns) return;   // the whole slice lies past the window
  float f[kGroups][4];
  slots_load(v.s, v.w, v.vec, v.p0, f);
#pragma unroll
  for (int u = 0; u < kBins / 4 / kSliceThreads; ++u)
    ((uint4*)lh)[threadIdx.x + u * kSliceThreads] = make_uint4(0u, 0u, 0u, 0u);
  lds_barrier();
#pragma unroll
  for (int g = 0; g < kGroups; ++g)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t key = score_key(f[g][e]);
      if (key) atomicAdd(&lh[key >> 20], 1u);
    }
  lds_barrier();
  uint32_t* gh = ghist + ((int64_t)row * copies + sl % copies) * kBins;
  for (int i = threadIdx.x; i < kBins; i += kSliceThreads) {
    const uint32_t c = lh[i];
    if (c) atomicAdd(&gh[i], c);
  }
}

// -------------------------------------------------------------- listing --
// Workgroups of the listing: rows * slices, or with 8 rows or more
// ceil(rows / 8) * 8 * slices, mapped so that the slices of a row run on one
// XCD (workgroups go to the 8 XCDs round-robin by id): every slice reads its
// row's whole histogram, and each XCD's L2 then fetches the histograms of its
// own rows only, not of every row.  Fewer rows spread their slices over all
// XCDs.
inline int64_t listing_wgs(int rows, int n_slices) {
  return rows >= 8 ? (int64_t)((rows + 7) / 8) * 8 * n_slices : (int64_t)rows * n_slices;
}
__device__ __forceinline__ void listing_slot(int rows, int n_slices, int& row, int& sl) {
  const int x = blockIdx.x;
  if (rows >= 8) {
    const int per = 8 * n_slices, grp = x / per, rem = x - grp * per;
    row = grp * 8 + (rem & 7);
    sl = rem >> 3;
  } else {
    row = x / n_slices;
    sl = x - row * n_slices;
  }
}

// Grid listing_wgs(rows, slices of NG groups per lane), 256 threads; COPIES:
// the rows' histogram copies (ws.copies), a compile-time constant so that one
// copy costs no registers for the others.
template <int NG, int COPIES>
__global__ __launch_bounds__(kSliceThreads) void topk_compact_kernel(
    const float* scores, int rows, int H, int L_max, const int32_t* lo_p, const int32_t* hi_p,
    int k, TopkWs ws, int n_slices) {
  __shared__ int wsum[4], wlist[4];
  __shared__ int sh[3];   // smallest listed key, listed count, this slice's list offset
  int row, sl;
  listing_slot(rows, n_slices, row, sl);
  if (row >= rows) return;   // the padding workgroups of the last group of 8 rows
  const int lane = threadIdx.x & 63, wave = row_wave();
  const SliceView v = slice_view<NG>(scores, row, H, L_max, lo_p, hi_p, sl);
  const bool any = sl * kSliceUnit * NG < v.w.ns;
  float f[NG][4];
  if (any) slots_load(v.s, v.w, v.vec, v.p0, f);

  // the bin of the k-th largest key: thread t holds bins 16 t .. 16 t + 15
  // (summed over the row's histogram copies)
  int c[16];
  {
    const uint4* gh = (const uint4*)(ws.hist + (int64_t)row * COPIES * kBins) + 4 * threadIdx.x;
    uint4 x[COPIES][4];
#pragma unroll
    for (int cp = 0; cp < COPIES; ++cp)
#pragma unroll
      for (int u = 0; u < 4; ++u) x[cp][u] = gh[cp * (kBins / 4) + u];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      c[4 * u] = c[4 * u + 1] = c[4 * u + 2] = c[4 * u + 3] = 0;
#pragma unroll
      for (int cp = 0; cp < COPIES; ++cp) {
        c[4 * u] += (int)x[cp][u].x;
        c[4 * u + 1] += (int)x[cp][u].y;
        c[4 * u + 2] += (int)x[cp][u].z;
        c[4 * u + 3] += (int)x[cp][u].w;
      }
    }
  }
  int tsum = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) tsum += c[j];
  const int incl = wave_incl_scan(tsum);
  if (lane == 63) wsum[wave] = incl;
  lds_barrier();
  int total = 0, upto = incl;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    total += wsum[u];
    if (u < wave) upto += wsum[u];
  }
  const int k_sel = min(k, total);
  if (threadIdx.x == 0 && (k_sel <= 0 || k_sel == total)) {
    sh[0] = k_sel <= 0 ? -1 : 1;   // nothing, or every finite key (key >= 1)
    sh[1] = k_sel <= 0 ? 0 : total;
  }
  // only the thread whose 16 bins hold the k-th key walks them
  if (k_sel > 0 && k_sel < total && total - upto < k_sel && k_sel <= total - upto + tsum) {
    int above = total - upto;   // keys in the bins above this thread's
#pragma unroll
    for (int j = 15; j >= 0; --j) {
      if (above < k_sel && k_sel <= above + c[j]) {
        sh[0] = (int)((uint32_t)(16 * threadIdx.x + j) << 20);
        sh[1] = above + c[j];
      }
      above += c[j];
    }
  }
  lds_barrier();
  const uint32_t lower = (uint32_t)sh[0];
  const int listed = sh[1];
  // every slice's share of the list is padded to a multiple of 4 entries
  if (listed + 3 * n_slices > kRowList) {   // the finishing workgroup selects this row alone
    if (sl == 0 && threadIdx.x == 0) {
      ws.meta[2 * row] = (int)lower;
      ws.meta[2 * row + 1] = -1;
    }
    return;
  }
  if (sl == 0 && threadIdx.x == 0) {
    ws.meta[2 * row] = (int)lower;
    ws.meta[2 * row + 1] = listed;
  }

  // this slice's keys >= lower, in position order (lower >= 1, so an empty
  // slot's key 0 is never listed)
  uint32_t kk[NG][4];
  int cg[NG], ig[NG], wt = 0;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    int n = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kk[g][e] = any ? score_key(f[g][e]) : 0u;
      n += kk[g][e] >= lower;
    }
    cg[g] = n;
    ig[g] = wave_incl_scan(n);
    wt += wave_total(ig[g]);
  }
  if (lane == 0) wlist[wave] = wt;
  lds_barrier();
  int o = 0, t_wg = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if (u < wave) o += wlist[u];
    t_wg += wlist[u];
  }
  if (threadIdx.x == 0) {
    // the share is padded to a multiple of 4 entries with key 0 (never
    // selected), so the finishing workgroup reads it 16 bytes at a time
    const int t_pad = (t_wg + 3) & ~3;
    const int base = t_pad ? atomicAdd(&ws.ctr[(int64_t)row * kCtrStride], t_pad) : 0;
    sh[2] = base;
    ws.slc[((int64_t)row * n_slices + sl) * 2] = base;
    ws.slc[((int64_t)row * n_slices + sl) * 2 + 1] = t_wg;
  }
  lds_barrier();
  o += sh[2];
  uint32_t* lk = ws.lkey + (int64_t)row * kRowList;
  int32_t* lp = ws.lpos + (int64_t)row * kRowList;
  if (threadIdx.x < ((t_wg + 3) & ~3) - t_wg) lk[sh[2] + t_wg + threadIdx.x] = 0u;   // padding
  const int pos0 = v.w.lo - v.w.o + v.p0;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    int d = o + ig[g] - cg[g];
    if (cg[g]) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (kk[g][e] >= lower) {
          if (d < kRowList) {
            lk[d] = kk[g][e];
            lp[d] = pos0 + 256 * g + e;
          }
          ++d;
        }
    }
    o += wave_total(ig[g]);
  }
}

// ------------------------------------------------------------ finishing --
// pre[w] = set bits of map[0 .. w) for the W <= 4096 words of a position
// bitmap, 4 words per thread (two barriers).
__device__ __forceinline__ void bitmap_prefix(const uint32_t* map, int* pre, int W, RowSelLds& L) {
  const int lane = threadIdx.x & 63, wave = row_wave();
  const int w0 = 4 * threadIdx.x;
  int c[4], tot = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    c[u] = w0 + u < W ? __popc(map[w0 + u]) : 0;
    tot += c[u];
  }
  const int inc = wave_incl_scan(tot);
  lds_barrier();   // earlier readers of L.wt are done
  if (lane == 63) L.wt[wave] = inc;
  lds_barrier();
  int before = inc - tot;
#pragma unroll
  for (int v = 0; v < kRowWaves; ++v)
    if (v < wave) before += L.wt[v];
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (w0 + u < W) {
      pre[w0 + u] = before;
      before += c[u];
    }
  lds_barrier();
}

// Grid rows, 1024 threads: rows of one sweep, each selected by its workgroup
// alone with the keys in registers (one kernel instead of two or three);
// ghist: the rows' histograms from the scan, or null.  NG groups of 4 keys
// per lane: rows of up to 4096 NG slots.
template <int MAP, int NG>
__global__ __launch_bounds__(kRowThreads) void topk_alone_kernel(
    const float* scores, int H, int L_max, const int32_t* lo_p, const int32_t* hi_p, int k,
    uint32_t* ghist, int32_t* idx, int32_t* count, const int32_t* map_a, const int32_t* map_b,
    int map_ld) {
  __shared__ RowSelLds L;
  __shared__ int klist_n;
  const int row = blockIdx.x;
  row_select_alone<true, MAP, NG>(scores, row, H, L_max, lo_p, hi_p, k,
                         ghist ? ghist + (int64_t)row * kBins : nullptr, ghist != nullptr,
                         idx + (int64_t)row * k, count, map_a, map_b, map_ld, L, nullptr, klist_n);
}

// Grid rows, 1024 threads.
template <int MAP>
__global__ __launch_bounds__(kRowThreads) void topk_finish_kernel(
    const float* scores, int H, int L_max, const int32_t* lo_p, const int32_t* hi_p, int k,
    TopkWs ws, int n_slices, int32_t* idx, int32_t* count, const int32_t* map_a,
    const int32_t* map_b, int map_ld) {
  __shared__ RowSelLds L;
  __shared__ uint32_t klist[kListCap];
  __shared__ int klist_n;
  __shared__ int s_off[kMaxSlices + 1], s_at[kMaxSlices];
  const int row = blockIdx.x;
  int32_t* orow = idx + (int64_t)row * k;
  uint4* gh4 = (uint4*)(ws.hist + (int64_t)row * ws.copies * kBins);
  const uint4 gv = hist_bins_summed(ws, row);
  if (ws.meta[2 * row + 1] < 0) {
    row_select_alone<false, MAP>(scores, row, H, L_max, lo_p, hi_p, k, (uint32_t*)gh4, true, orow,
                                 count, map_a, map_b, map_ld, L, klist, klist_n, nullptr, true, gv);
  } else {
    // the selection is staged in LDS (the list buffer of the fallback) when
    // it fits, then written in one coalesced pass
    const bool stage = k <= kListCap;
    const int n_sel = list_select(ws, row, k, n_slices, gv, L, s_off, s_at, [&](int dst, int p,
                                                                               uint32_t) {
      if (stage) klist[dst] = (uint32_t)p;
      else if constexpr (MAP == 0) orow[dst] = p;
      else orow[dst] = map_b[map_a[(int64_t)row * map_ld + p]];
    });
    if (stage) {
      lds_barrier();
      for (int i = threadIdx.x; i < n_sel; i += kRowThreads) {
        const int p = (int)klist[i];
        orow[i] = MAP == 0 ? p : map_b[map_a[(int64_t)row * map_ld + p]];
      }
    }
    for (int i = n_sel + threadIdx.x; i < k; i += kRowThreads) orow[i] = -1;
    if (threadIdx.x == 0) count[row] = n_sel;
  }
  // zero for the next call: every copy of the row's histogram, its list counter
  for (int cp = 0; cp < ws.copies; ++cp) gh4[cp * (kBins / 4) + threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
  if (threadIdx.x == 0) ws.ctr[(int64_t)row * kCtrStride] = 0;
}

// --------------------------------------------------- prefiltered top-k --
// Threshold-prefiltered exact top-k (ECHO-OSDI26 wiki page, observation 3 and
// core method 3: the k-th largest index score of a step moves smoothly, so an
// EMA with alpha = 0.5 of the past steps' k-th scores predicts the next
// step's).  The scan listed the window's keys whose score reaches the row's
// prediction thr[row] (ws.lkey / ws.lpos, count ws.ctr).  If at least k keys
// survived, the k-th largest key of the row is among them together with every
// key at or above it, so the exact selection is resolved over the survivors
// alone: threshold digits over their histogram, equal keys ranked by position
// through a bitmap of the window, and the output placed in ascending order
// by prefix popcounts of a second bitmap.  Fewer than k survivors, a list
// overflow or a window over 131072 slots: the full row is selected by this
// workgroup, re-reading it per pass.  Either way thr[row] becomes
// alpha kth + (1 - alpha) thr[row] (kth when thr[row] is -inf; -inf when the
// window has fewer than k candidates), and the list counter is zeroed.
constexpr int kMapWords = 4096;   // position bitmaps: windows of up to 131072 slots

template <int MAP>
__global__ __launch_bounds__(kRowThreads) void topk_survivor_kernel(
    const float* scores, int H, int L_max, const int32_t* lo_p, const int32_t* hi_p, int k,
    TopkWs ws, float* thr, float alpha, int32_t* used, int32_t* idx, int32_t* count,
    const int32_t* map_a, const int32_t* map_b, int map_ld) {
  __shared__ RowSelLds L;
  __shared__ uint32_t klist[kListCap];
  __shared__ int klist_n;
  __shared__ uint32_t selmap[kMapWords], eqmap[kMapWords];
  __shared__ int wpre[kMapWords];
  __shared__ uint32_t s_min;
  constexpr int kPer = kRowList / kRowThreads;   // survivors per lane
  const int row = blockIdx.x;
  int32_t* orow = idx + (int64_t)row * k;
  const int m = ws.ctr[(int64_t)row * kCtrStride];
  const float thr_old = thr[row];
  const RowWindow w = row_window(lo_p, hi_p, row / H, L_max);
  const bool listed = m >= k && m <= kRowList && w.n <= kMapWords * 32;
  int k_sel;
  uint32_t mink;
  if (!listed) {
    row_select_alone<false, MAP>(scores, row, H, L_max, lo_p, hi_p, k, nullptr, false, orow,
                                 count, map_a, map_b, map_ld, L, klist, klist_n, &s_min);
    lds_barrier();
    mink = s_min;
    k_sel = count[row];   // written by thread 0, which alone reads it below
  } else {
    uint32_t key[kPer];
    int pos[kPer];
    const uint32_t* lk = ws.lkey + (int64_t)row * kRowList;
    const int32_t* lp = ws.lpos + (int64_t)row * kRowList;
    // survivors in any order (bitmaps place them): lane-interleaved, so every
    // load instruction reads consecutive words
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int r = u * kRowThreads + threadIdx.x;
      key[u] = r < m ? lk[r] : 0u;
      pos[u] = r < m ? lp[r] : 0;
      if (pos[u] < w.lo || pos[u] >= w.hi) key[u] = 0u;   // only window positions were listed
    }
    *(uint4*)(L.hist + 4 * threadIdx.x) = make_uint4(0u, 0u, 0u, 0u);
    if (threadIdx.x < 256) L.dh[threadIdx.x] = 0u;
    *(uint4*)(selmap + 4 * threadIdx.x) = make_uint4(0u, 0u, 0u, 0u);
    *(uint4*)(eqmap + 4 * threadIdx.x) = make_uint4(0u, 0u, 0u, 0u);
    lds_barrier();
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      if (key[u]) atomicAdd(&L.hist[key[u] >> 20], 1u);
    lds_barrier();
    uint32_t T;
    int need_eq;
    row_threshold(
        L, k, []() {},
        [&](auto&& f) {
#pragma unroll
          for (int u = 0; u < kPer; ++u) f(key[u]);
        },
        &T, &need_eq, &k_sel);
    const int W = (w.n + 31) >> 5;
    // keys equal to T: the first need_eq by position are taken
    if (need_eq > 0) {
#pragma unroll
      for (int u = 0; u < kPer; ++u)
        if (key[u] != 0u && key[u] == T) {
          const int b = pos[u] - w.lo;
          atomicOr(&eqmap[b >> 5], 1u << (b & 31));
        }
      lds_barrier();
      bitmap_prefix(eqmap, wpre, W, L);
    }
    bool sel[kPer];
    uint32_t mk = 0xffffffffu;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int b = pos[u] - w.lo;
      bool t = key[u] > T;
      if (!t && need_eq > 0 && key[u] != 0u && key[u] == T)
        t = wpre[b >> 5] + __popc(eqmap[b >> 5] & ((1u << (b & 31)) - 1u)) < need_eq;
      sel[u] = t;
      if (t) {
        atomicOr(&selmap[b >> 5], 1u << (b & 31));
        mk = min(mk, key[u]);
      }
    }
    lds_barrier();
    bitmap_prefix(selmap, wpre, W, L);
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      if (sel[u]) {
        const int b = pos[u] - w.lo;
        const int dst = wpre[b >> 5] + __popc(selmap[b >> 5] & ((1u << (b & 31)) - 1u));
        if (dst < k) {
          if constexpr (MAP == 0) orow[dst] = pos[u];
          else if constexpr (MAP == 1) L.hist[dst] = (uint32_t)pos[u];
          else orow[dst] = map_b[map_a[(int64_t)row * map_ld + pos[u]]];
        }
      }
    if constexpr (MAP == 1) {
      lds_barrier();
      for (int i = threadIdx.x; i < k_sel; i += kRowThreads)
        orow[i] = map_b[map_a[(int64_t)row * map_ld + (int)L.hist[i]]];
    }
    for (int i = k_sel + threadIdx.x; i < k; i += kRowThreads) orow[i] = -1;
    if (threadIdx.x == 0) count[row] = k_sel;
    mink = block_min_u32(mk, (uint32_t*)L.wt);
  }
  if (threadIdx.x == 0) {
    const float kth = (k_sel >= k && mink != 0xffffffffu) ? key_score(mink) : -INFINITY;
    thr[row] = (thr_old == -INFINITY || kth == -INFINITY) ? kth
                                                          : alpha * kth + (1.f - alpha) * thr_old;
    if (used) used[row] = listed ? 1 : 0;
    ws.ctr[(int64_t)row * kCtrStride] = 0;
  }
}

}  // namespace

size_t topk_workspace_bytes(int rows, int L_max) { return TopkWs::bytes(rows, L_max); }

bool topk_supported(int L_max) { return L_max >= 1 && topk_slices(L_max) <= kMaxSlices; }

int topk_listing_slices(int rows, int L_max) {
  return topk_slices_ng(L_max, topk_slice_groups(rows, L_max));
}

hipError_t launch_topk_listing(const float* scores, int rows, int H, int L_max, const int32_t* lo,
                               const int32_t* hi, int k, void* wsp, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const TopkWs ws = TopkWs::carve(wsp, rows, L_max);
  const int ng_l = topk_slice_groups(rows, L_max);
  const int ns = topk_slices_ng(L_max, ng_l);
  if (ns > kMaxSlices || ns > topk_slices(L_max) || listing_wgs(rows, ns) > 0x7fffffff)
    return hipErrorInvalidValue;
  if (ws.copies != 1 && ws.copies != kHistCopiesMax) return hipErrorInvalidValue;
  auto list = [&](auto kern) {
    kern<<<(unsigned)listing_wgs(rows, ns), kSliceThreads, 0, s>>>(scores, rows, H, L_max, lo, hi,
                                                                  k, ws, ns);
  };
  auto by_ng = [&](auto copies_c) {
    constexpr int CP = decltype(copies_c)::value;
    if (ng_l == 1) list(topk_compact_kernel<1, CP>);
    else if (ng_l == 2) list(topk_compact_kernel<2, CP>);
    else if (ng_l == 4) list(topk_compact_kernel<4, CP>);
    else list(topk_compact_kernel<kGroups, CP>);
  };
  if (ws.copies == 1) by_ng(std::integral_constant<int, 1>{});
  else by_ng(std::integral_constant<int, kHistCopiesMax>{});
  return hipGetLastError();
}

hipError_t launch_topk(const float* scores, int rows, int H, int L_max, const int32_t* lo,
                       const int32_t* hi, int k, int32_t* idx, int32_t* count, void* wsp,
                       bool hist_ready, hipStream_t s, const int32_t* map_a,
                       const int32_t* map_b, int map_ld) {
  if (rows <= 0) return hipSuccess;
  const TopkWs ws = TopkWs::carve(wsp, rows, L_max);
  const int ng_l = topk_slice_groups(rows, L_max);
  const int ns = topk_slices_ng(L_max, ng_l);           // listing slices per row
  const int ns_h = topk_slices_ng(L_max, kGroups);      // histogram slices per row
  if (ns > kMaxSlices || ns > topk_slices(L_max) || (int64_t)rows * ns > 0x7fffffff)
    return hipErrorInvalidValue;
  const int map = map_a ? (k <= kBins ? 1 : 2) : 0;
  if (row_slots_max(L_max) <= kSweep) {
    // rows of one sweep: one workgroup per row
    uint32_t* gh = hist_ready ? ws.hist : nullptr;
    // the fewest groups per lane that hold the row: every pass over the
    // keys is that much shorter
    const int slots = row_slots_max(L_max);
    const int ng = slots <= 4096 ? 1 : slots <= 8192 ? 2 : slots <= 16384 ? 4
                 : slots <= 24576 ? 6 : kGroups;
    auto go = [&](auto kern) {
      kern<<<rows, kRowThreads, 0, s>>>(scores, H, L_max, lo, hi, k, gh, idx, count, map_a, map_b,
                                        map_ld);
    };
    auto by_ng = [&](auto map_c) {
      constexpr int M = decltype(map_c)::value;
      if (ng == 1) go(topk_alone_kernel<M, 1>);
      else if (ng == 2) go(topk_alone_kernel<M, 2>);
      else if (ng == 4) go(topk_alone_kernel<M, 4>);
      else if (ng == 6) go(topk_alone_kernel<M, 6>);
      else go(topk_alone_kernel<M, kGroups>);
    };
    if (map == 0) by_ng(std::integral_constant<int, 0>{});
    else if (map == 1) by_ng(std::integral_constant<int, 1>{});
    else by_ng(std::integral_constant<int, 2>{});
    return hipGetLastError();
  }
  if (!hist_ready)
    topk_hist_kernel<<<(unsigned)(rows * ns_h), kSliceThreads, 0, s>>>(scores, H, L_max, lo, hi,
                                                                         ws.hist, ns_h, ws.copies);
  const hipError_t e = launch_topk_listing(scores, rows, H, L_max, lo, hi, k, wsp, s);
  if (e != hipSuccess) return e;
  if (map == 0)
    topk_finish_kernel<0><<<rows, kRowThreads, 0, s>>>(scores, H, L_max, lo, hi, k, ws, ns, idx,
                                                       count, map_a, map_b, map_ld);
  else if (map == 1)
    topk_finish_kernel<1><<<rows, kRowThreads, 0, s>>>(scores, H, L_max, lo, hi, k, ws, ns, idx,
                                                       count, map_a, map_b, map_ld);
  else
    topk_finish_kernel<2><<<rows, kRowThreads, 0, s>>>(scores, H, L_max, lo, hi, k, ws, ns, idx,
                                                       count, map_a, map_b, map_ld);
  return hipGetLastError();
}

bool topk_survivors_supported(int L_max) { return topk_supported(L_max); }

hipError_t launch_topk_survivors(const float* scores, int rows, int H, int L_max,
                                 const int32_t* lo, const int32_t* hi, int k, int32_t* idx,
                                 int32_t* count, void* wsp, float* thr, float alpha,
                                 int32_t* used, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const TopkWs ws = TopkWs::carve(wsp, rows, L_max);
  topk_survivor_kernel<0><<<rows, kRowThreads, 0, s>>>(scores, H, L_max, lo, hi, k, ws, thr, alpha,
                                                       used, idx, count, nullptr, nullptr, 0);
  return hipGetLastError();
}

}  // namespace skv
