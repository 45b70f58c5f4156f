// Row selection routines shared by the top-k kernels and the kernels that
// fuse the end of the top-k with the attention: the whole selection of one
// row by one workgroup (row_select_alone) and the exact selection of a row
// from the list the slice-listing kernel left in the top-k workspace
// (list_select).  Both take the exact top-k of the row's window (ties to the
// lower position, -0 = +0; ECHO-OSDI26 wiki page, observation 5).
#pragma once

#include "skv_rowsel.h"
#include "skv_topk.h"

namespace skv {

namespace {

constexpr int kListCap = 16384;              // fallback: LDS list of the threshold bin's keys

// The score whose order-preserving key is `key`.
__device__ __forceinline__ float key_score(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// Minimum of v over the 1024-thread workgroup (two barriers; red: 16 words).
__device__ __forceinline__ uint32_t block_min_u32(uint32_t v, uint32_t* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o, 64));
  lds_barrier();   // earlier readers of red are done
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  lds_barrier();
  uint32_t m = 0xffffffffu;
#pragma unroll
  for (int i = 0; i < kRowWaves; ++i) m = min(m, red[i]);
  return m;
}

// The whole selection of one row by one workgroup, re-reading the row from
// memory for every pass (rows whose list would overflow).  The threshold
// bin's keys are compacted into an LDS list when they fit, so the lower
// digits need no further pass over the row.
// RES: the row is one sweep, whose keys stay in registers across the passes.
// MAP: how a selected position p is written: 0 as p; 1 (k <= 4096) as
// map_b[map_a[row][p]], the positions gathered in LDS first and mapped in one
// pass; 2 mapped as each key is emitted; 3 (k <= 4096) not at all: the
// positions stay in L.hist[0 .. n_sel) in ascending order, and nothing is
// written to memory (orow, count and the histogram are left as they are).  A
// compile-time choice, so every instantiation has one kind of store in its
// emission loop.  klist may be null: the threshold bin's keys are then
// re-read from the row for every digit.  With use_pre, gv_pre is this
// thread's 4 bins of the row's histogram (bins 4 t .. 4 t + 3), already
// summed, and ghist_row is not read.  Returns the number selected.
template <bool RES, int MAP, int NG = kGroups>
__device__ __forceinline__ int row_select_alone(const float* scores, int row, int H, int L_max,
                                 const int32_t* lo_p, const int32_t* hi_p, int k,
                                 uint32_t* ghist_row, bool hist_ready, int32_t* orow,
                                 int32_t* count, const int32_t* map_a, const int32_t* map_b,
                                 int map_ld, RowSelLds& L, uint32_t* klist, int& klist_n,
                                 uint32_t* min_key = nullptr, bool use_pre = false,
                                 uint4 gv_pre = make_uint4(0u, 0u, 0u, 0u)) {
  const int lane = threadIdx.x & 63;
  RowWindow w = row_window(lo_p, hi_p, row / H, L_max);
  bool vec;
  const float* s = row_base(scores, (int64_t)row * L_max, w, &vec);
  const int n_sweeps = RES ? 1 : (w.ns + kSweep - 1) / kSweep;
  uint4* gh4 = (uint4*)ghist_row;
  const uint4 gv = use_pre ? gv_pre : hist_ready ? gh4[threadIdx.x] : make_uint4(0u, 0u, 0u, 0u);
  // RES: the row's scores are loaded now and turned into keys once the
  // first digit's search (from the scan's histogram) has overlapped their
  // arrival
  static_assert(RES || NG == kGroups, "short rows keep their keys in registers");
  uint32_t kr[RES ? NG : 1][4];
  float fr[RES ? NG : 1][4];
  if constexpr (RES) row_load(s, w, vec, 0, fr);

  // F(keys, sweep) for every sweep, the next sweep's loads in flight while
  // one is processed
  auto for_sweeps = [&](auto&& F) {
    if constexpr (RES) {
      F(kr, 0);
      return;
    }
    float va[kGroups][4], vb[kGroups][4];
    row_load(s, w, vec, 0, va);
    for (int sw = 0; sw < n_sweeps; sw += 2) {
      if (sw + 1 < n_sweeps) row_load(s, w, vec, sw + 1, vb);
      {
        uint32_t kk[kGroups][4];
        row_keys(va, kk);
        F(kk, sw);
      }
      if (sw + 1 < n_sweeps) {
        if (sw + 2 < n_sweeps) row_load(s, w, vec, sw + 2, va);
        uint32_t kk[kGroups][4];
        row_keys(vb, kk);
        F(kk, sw + 1);
      }
    }
  };
  bool use_list = false;
  auto for_keys = [&](auto&& f) {
    if (use_list) {
      const int nl = min(klist_n, kListCap);
      for (int i = threadIdx.x; i < nl; i += kRowThreads) f(klist[i]);
    } else {
      for_sweeps([&](const auto& kk, int) {
        constexpr int ng = sizeof(kk) / sizeof(kk[0]);
#pragma unroll
        for (int g = 0; g < ng; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e) f(kk[g][e]);
      });
    }
  };
  // one pass compacts the keys of bin b0 into klist (a wave prefix sum of
  // the lanes' match counts places them; one LDS atomic per wave and sweep)
  auto prepare = [&](int b0, int in_bin) {
    if (RES || !klist || in_bin > kListCap) return;
    if (threadIdx.x == 0) klist_n = 0;
    lds_barrier();
    for_sweeps([&](const auto& kk, int) {
      constexpr int ng = sizeof(kk) / sizeof(kk[0]);
      int c = 0;
#pragma unroll
      for (int g = 0; g < ng; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) c += (kk[g][e] >> 20) == (uint32_t)b0;
      const int incl = wave_incl_scan(c);
      int base = 0;
      if (lane == 63) base = atomicAdd(&klist_n, incl);
      int o = __builtin_amdgcn_readlane(base, 63) + incl - c;
      if (c) {
#pragma unroll
        for (int g = 0; g < ng; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if ((kk[g][e] >> 20) == (uint32_t)b0) {
              if (o < kListCap) klist[o] = kk[g][e];
              ++o;
            }
      }
    });
    lds_barrier();
    use_list = true;
  };

  *(uint4*)(L.hist + 4 * threadIdx.x) = gv;
  if (threadIdx.x < 256) L.dh[threadIdx.x] = 0u;
  lds_barrier();
  if (!hist_ready) {   // the top-12-bit histogram, with LDS atomics
    if constexpr (RES) row_keys(fr, kr);
    for_keys([&](uint32_t key) {
      if (key) atomicAdd(&L.hist[key >> 20], 1u);
    });
    lds_barrier();
  }
  uint32_t T;
  int need_eq, k_sel;
  row_threshold_p(
      L, k,
      [&]() {
        if constexpr (RES) {
          if (hist_ready) row_keys(fr, kr);
        }
      },
      prepare, for_keys, &T, &need_eq, &k_sel);

  int a_base = 0, e_base = 0;   // keys above / equal to T in earlier sweeps
  uint32_t mk = 0xffffffffu;    // smallest selected key of this lane
  for (int sw = 0; sw < n_sweeps; ++sw) {
    uint32_t kk[NG][4];
    if constexpr (RES) {
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) kk[g][e] = kr[g][e];
    } else {
      float f[NG][4];
      row_load(s, w, vec, sw, f);
      row_keys(f, kk);
    }
    int cg[NG];
    const int lt = row_counts(kk, T, cg);
    int oa, oe, ta, te;
    row_wave_offsets(L, lt, &oa, &oe, &ta, &te);
    const int pos0 = w.lo - w.o + row_slot0<NG>(sw);
    row_emit(kk, cg, T, need_eq, a_base + oa, e_base + oe, [&](int dst, int g, int e) {
      if (dst < k) {
        const int p = pos0 + 256 * g + e;
        if constexpr (MAP == 0) orow[dst] = p;
        else if constexpr (MAP == 1 || MAP == 3) L.hist[dst] = (uint32_t)p;
        else orow[dst] = map_b[map_a[(int64_t)row * map_ld + p]];
        mk = min(mk, kk[g][e]);
      }
    });
    a_base += ta;
    e_base += te;
  }
  const int n_sel = min(k, a_base + min(e_base, need_eq));
  if constexpr (MAP == 3) {
    lds_barrier();   // the emitted positions are in L.hist
    return n_sel;
  }
  if constexpr (MAP == 1) {
    lds_barrier();
    for (int i = threadIdx.x; i < n_sel; i += kRowThreads)
      orow[i] = map_b[map_a[(int64_t)row * map_ld + (int)L.hist[i]]];
  }
  for (int i = n_sel + threadIdx.x; i < k; i += kRowThreads) orow[i] = -1;
  if (threadIdx.x == 0) count[row] = n_sel;
  if (hist_ready) gh4[threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
  if (min_key) {
    const uint32_t m = block_min_u32(mk, (uint32_t*)L.wt);
    if (threadIdx.x == 0) *min_key = m;
  }
  return n_sel;
}


// Steps 2 and 3 of a list selection: the listed keys (every key of the bins
// at or above the k-th key's bin, in position order) are held KPER
// consecutive list ranks per lane (lane t: ranks KPER t .. KPER t + KPER - 1,
// key 0 past the list's end, which is never selected), pos their positions.
// Resolves the exact threshold T and the number of keys equal to T to take
// (lowest positions first) with two more digits over the listed keys, then
// calls emit(dst, pos, key) for every selected key with dst < k, dst being
// its rank in ascending position order.  gv: this thread's 4 bins of the
// row's first-digit histogram.  Returns min(k, finite candidates).
template <int KPER, typename Emit>
__device__ __forceinline__ int select_listed(int k, uint4 gv, RowSelLds& L,
                                             const uint32_t (&key)[KPER], const int (&pos)[KPER],
                                             Emit&& emit, int* first_bin = nullptr) {
  // threshold over the listed keys
  *(uint4*)(L.hist + 4 * threadIdx.x) = gv;
  if (threadIdx.x < 256) L.dh[threadIdx.x] = 0u;
  lds_barrier();
  uint32_t T;
  int need_eq, k_sel;
  row_threshold(
      L, k, []() {},
      [&](auto&& f) {
#pragma unroll
        for (int u = 0; u < KPER; ++u) f(key[u]);
      },
      &T, &need_eq, &k_sel, first_bin);

  // ranks: the lane's entries are consecutive list ranks
  int c = 0;
#pragma unroll
  for (int u = 0; u < KPER; ++u)
    c += key[u] > T ? 1 : ((key[u] != 0u && key[u] == T) ? 0x10000 : 0);
  const int inc = wave_incl_scan(c);
  int oa, oe, ta, te;
  row_wave_offsets(L, c, &oa, &oe, &ta, &te);
  int ab = oa + ((inc - c) & 0xffff), eb = oe + ((inc - c) >> 16);
  if (c) {
#pragma unroll
    for (int u = 0; u < KPER; ++u) {
      int dst = -1;
      if (key[u] > T) {
        dst = ab + min(eb, need_eq);
        ++ab;
      } else if (key[u] != 0u && key[u] == T) {
        if (eb < need_eq) dst = ab + eb;
        ++eb;
      }
      if (dst >= 0 && dst < k) emit(dst, pos[u], key[u]);
    }
  }
  return min(k, ta + min(te, need_eq));
}

// Exact selection of row `row` from the list the slice-listing kernel left in
// ws (every key of the bins at or above the k-th key's bin, slice by slice in
// position order; ws.meta[2 row + 1] >= 0): reads the slices' list offsets
// into s_off / s_at (n_slices <= the arrays' room), the list (kPer
// consecutive ranks per lane, as 16-byte loads), resolves the exact threshold
// T and the number of keys equal to T to take (lowest positions first) with
// two more digits over the listed keys, then calls emit(dst, pos, key) for
// every selected key with dst < k, dst being its rank in ascending position
// order (key: its order-preserving score key, key_score(key) the score).
// gv: this thread's 4 bins (4 t .. 4 t + 3) of the row's histogram, summed
// over its copies.  Only reads memory; every workgroup of a row may run it.
// Returns the number selected, min(k, finite candidates).
template <typename Emit>
__device__ __forceinline__ int list_select(const TopkWs& ws, int row, int k, int n_slices, uint4 gv,
                                           RowSelLds& L, int* s_off, int* s_at, Emit&& emit) {
  constexpr int kPer = kRowList / kRowThreads;   // list entries per lane
  const int lane = threadIdx.x & 63, wave = row_wave();
  const int32_t* slc = ws.slc + (int64_t)row * n_slices * 2;
  // 1. the list, slice by slice: s_off = first list rank of each slice (ranks
  // count every slice's share padded to a multiple of 4, as stored)
  int run = 0;
  for (int b0 = 0; b0 < n_slices; b0 += kRowThreads) {
    const int sl = b0 + threadIdx.x;
    const int n = ((sl < n_slices ? slc[2 * sl + 1] : 0) + 3) & ~3;
    if (sl < n_slices) s_at[sl] = slc[2 * sl];
    const int inc = wave_incl_scan(n);
    if (lane == 63) L.wt[wave] = inc;
    lds_barrier();
    int before = run + inc - n, all = 0;
#pragma unroll
    for (int u = 0; u < kRowWaves; ++u) {
      if (u < wave) before += L.wt[u];
      all += L.wt[u];
    }
    if (sl < n_slices) s_off[sl] = before;
    run += all;
    lds_barrier();
  }
  const int m = min(run, kRowList);
  if (threadIdx.x == 0) s_off[n_slices] = run;
  lds_barrier();
  // list ranks kPer * tid .. kPer * tid + kPer - 1: the slice holding a rank
  // is the last one whose first rank is not above it
  uint32_t key[kPer];
  int pos[kPer];
  const uint32_t* lk = ws.lkey + (int64_t)row * kRowList;
  const int32_t* lp = ws.lpos + (int64_t)row * kRowList;
  {
    const int r0 = kPer * threadIdx.x;
    int sl = 0;
    if (r0 < m) {
      int a = 0, b = n_slices - 1;
      while (a < b) {
        const int mid = (a + b + 1) >> 1;
        if (s_off[mid] <= r0) a = mid;
        else b = mid - 1;
      }
      sl = a;
    }
    // four ranks at a time: a slice's share starts on a multiple of 4 and
    // holds a multiple of 4 entries, so they are 16 consecutive bytes
#pragma unroll
    for (int u = 0; u < kPer; u += 4) {
      const int r = r0 + u;
      uint4 kq = make_uint4(0u, 0u, 0u, 0u);
      int4 pq = make_int4(0, 0, 0, 0);
      if (r < m) {
        while (s_off[sl + 1] <= r) ++sl;
        const int at = s_at[sl] + (r - s_off[sl]);
        if (at + 4 <= kRowList) {
          kq = *(const uint4*)(lk + at);
          pq = *(const int4*)(lp + at);
        }
      }
      key[u] = kq.x;
      key[u + 1] = kq.y;
      key[u + 2] = kq.z;
      key[u + 3] = kq.w;
      pos[u] = pq.x;
      pos[u + 1] = pq.y;
      pos[u + 2] = pq.z;
      pos[u + 3] = pq.w;
    }
  }

  return select_listed<kPer>(k, gv, L, key, pos, emit);
}

// Exact selection of row `row` by a workgroup that lists the row itself, for
// kernels that own a whole row (no slice-listing kernel before them): the bin
// b0 of the k-th largest key from the row's histogram (gv: this thread's 4
// bins, summed over the copies), then one pass over the window's scores (the
// next sweep's loads in flight while one is listed) keeps every key of the
// bins >= b0 with its position in LDS (lk, lp: KPER * kRowThreads entries), in
// position order, and select_listed finishes over them: emit(dst, pos, key)
// for every selected key, dst its rank in ascending position order.  Returns
// the number selected, or -1 when the listed keys would not fit (the caller
// then selects the row alone).
template <int KPER, typename Emit>
__device__ __forceinline__ int local_list_select(const float* scores, int row, int H, int L_max,
                                                 const int32_t* lo_p, const int32_t* hi_p, int k,
                                                 uint4 gv, RowSelLds& L, uint32_t* lk, int32_t* lp,
                                                 Emit&& emit) {
  constexpr int kCap = KPER * kRowThreads;
  constexpr int NG = 4;                                // groups of 4 slots per lane per sweep
  constexpr int kSw = kRowWaves * 256 * NG;            // slots per sweep
  static_assert(KPER % 4 == 0, "16-byte list reads");
  const int lane = threadIdx.x & 63, wave = row_wave();
  RowWindow w = row_window(lo_p, hi_p, row / H, L_max);
  bool vec;
  const float* s = row_base(scores, (int64_t)row * L_max, w, &vec);
  const int n_sweeps = (w.ns + kSw - 1) / kSw;
  float va[NG][4], vb[NG][4];
  if (n_sweeps > 0) row_load<NG, true>(s, w, vec, 0, va);

  // 1. the bin of the k-th largest key; every key of the bins above it and of
  //    the bin itself is listed (lower = its first key)
  *(uint4*)(L.hist + 4 * threadIdx.x) = gv;
  lds_barrier();
  int total;
  const int k_sel = row_search4096(L, -k, &total);   // min(k, total)
  if (k_sel <= 0) return 0;
  uint32_t lower = 1u;   // k_sel == total: every finite key (finite keys are >= 1)
  int listed = total;
  if (k_sel < total) {
    lower = (uint32_t)L.trio[0] << 20;
    listed = L.trio[1] + L.trio[2];
  }
  if (listed > kCap) return -1;

  // 2. the listing, sweep by sweep; in a sweep wave w holds slots
  //    w 256 NG + 256 g + 4 lane + e, so ranks go wave, group, lane, element
  //    (the keys are formed twice, for the counts and for the stores, rather
  //    than held)
  int base = 0;
  auto list_sweep = [&](const float (&f)[NG][4], int sw) {
    int cg[NG], ig[NG], wt = 0;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      int c = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) c += score_key(f[g][e]) >= lower;
      cg[g] = c;
      ig[g] = wave_incl_scan(c);
      wt += wave_total(ig[g]);
    }
    lds_barrier();   // earlier readers of L.wt are done
    if (lane == 0) L.wt[wave] = wt;
    lds_barrier();
    int o = base, all = 0;
#pragma unroll
    for (int u = 0; u < kRowWaves; ++u) {
      if (u < wave) o += L.wt[u];
      all += L.wt[u];
    }
    const int pos0 = w.lo - w.o + row_slot0<NG>(sw);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      int d = o + ig[g] - cg[g];
      if (cg[g]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t key = score_key(f[g][e]);
          if (key >= lower) {
            if (d < kCap) {
              lk[d] = key;
              lp[d] = pos0 + 256 * g + e;
            }
            ++d;
          }
        }
      }
      o += wave_total(ig[g]);
    }
    base += all;
  };
  for (int sw = 0; sw < n_sweeps; sw += 2) {
    if (sw + 1 < n_sweeps) row_load<NG, true>(s, w, vec, sw + 1, vb);
    list_sweep(va, sw);
    if (sw + 1 < n_sweeps) {
      if (sw + 2 < n_sweeps) row_load<NG, true>(s, w, vec, sw + 2, va);
      list_sweep(vb, sw + 1);
    }
  }
  if (base > kCap) return -1;   // (the histogram promised fewer)
  lds_barrier();                // the list is complete

  // 3. ranks KPER t .. KPER t + KPER - 1 per lane, then the exact threshold
  uint32_t key[KPER];
  int pos[KPER];
#pragma unroll
  for (int u = 0; u < KPER; u += 4) {
    const int r = KPER * threadIdx.x + u;
    const uint4 kq = r < base ? *(const uint4*)(lk + r) : make_uint4(0u, 0u, 0u, 0u);
    const int4 pq = r < base ? *(const int4*)(lp + r) : make_int4(0, 0, 0, 0);
    key[u] = r < base ? kq.x : 0u;
    key[u + 1] = r + 1 < base ? kq.y : 0u;
    key[u + 2] = r + 2 < base ? kq.z : 0u;
    key[u + 3] = r + 3 < base ? kq.w : 0u;
    pos[u] = pq.x;
    pos[u + 1] = pq.y;
    pos[u + 2] = pq.z;
    pos[u + 3] = pq.w;
  }
  return select_listed<KPER>(k, gv, L, key, pos, emit);
}

// Exact selection of row `row` from the segment candidates the score scan
// listed in ws (topk_seg_count: S segments of m = kSegSlots / S slots, keys
// in position order): lane t takes slots KPER t .. KPER t + KPER - 1, all in
// one segment (keys past the segment's count read as 0, never selected), and
// select_listed finishes over them: emit(dst, pos, key) for every selected
// key, dst its rank in ascending position order.  The candidates are the top
// of every segment, so their keys share their leading bits and would crowd
// into a few bins of the first 12-bit digit (same-address LDS atomics: 2.6 us
// for 7,000 candidates in about 4 bins); the keys are shifted left past the
// bits all candidates share but one, whose place takes a set top bit (order
// and distinctness kept, no key 0 or in a low bin), which spreads them over
// the digit's bins.  The result
// is the row's exact top-k when no key left out can rank among it: every
// segment's cut (all its unlisted keys are below it, a multiple of 2^20) is
// at most the smallest key of the k-th candidate's first-digit bin, and no
// segment left keys out if fewer than k were listed.  Returns the number
// selected, or -1 when that does not hold (the caller then selects the row
// alone).
template <typename Emit>
__device__ __forceinline__ int seg_select(const TopkWs& ws, int row, int S, int k, RowSelLds& L,
                                          Emit&& emit) {
  constexpr int KPER = kSegSlots / kRowThreads;
  static_assert(KPER == 8, "two 16-byte loads of keys and of positions per lane");
  const int lane = threadIdx.x & 63, wave = row_wave();
  const int m = kSegSlots / S;   // a power of two >= 16
  const int64_t rb = (int64_t)row * kRowList;
  const int slot0 = KPER * threadIdx.x;
  const int seg = slot0 / m, o = slot0 - seg * m;
  const int n_in = ws.seg_n()[rb + seg];
  const uint4 ka = *(const uint4*)(ws.seg_key() + rb + slot0);
  const uint4 kb = *(const uint4*)(ws.seg_key() + rb + slot0 + 4);
  const int4 pa = *(const int4*)(ws.seg_pos() + rb + slot0);
  const int4 pb = *(const int4*)(ws.seg_pos() + rb + slot0 + 4);
  uint32_t cut = (int)threadIdx.x < S ? ws.seg_cut()[rb + threadIdx.x] : 0u;
  *(uint4*)(L.hist + 4 * threadIdx.x) = make_uint4(0u, 0u, 0u, 0u);
  const uint32_t kv8[8] = {ka.x, ka.y, ka.z, ka.w, kb.x, kb.y, kb.z, kb.w};
  const int pv8[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
  uint32_t key[KPER];
  int pos[KPER];
  uint32_t kand = 0xffffffffu, kor = 0u;   // over the candidates
#pragma unroll
  for (int u = 0; u < KPER; ++u) {
    key[u] = o + u < n_in ? kv8[u] : 0u;
    pos[u] = pv8[u];
    if (key[u]) {
      kand &= key[u];
      kor |= key[u];
    }
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    cut = max(cut, (uint32_t)__shfl_xor((int)cut, d, 64));
    kand &= (uint32_t)__shfl_xor((int)kand, d, 64);
    kor |= (uint32_t)__shfl_xor((int)kor, d, 64);
  }
  if (lane == 0) {
    L.wa[wave] = (int)cut;
    L.we[wave] = (int)kand;
    L.wt[wave] = (int)kor;
  }
  lds_barrier();   // L.hist is zero, the waves' reductions are in
  uint32_t max_cut = 0u;
  kand = 0xffffffffu;
  kor = 0u;
#pragma unroll
  for (int v = 0; v < kRowWaves; ++v) {
    max_cut = max(max_cut, (uint32_t)L.wa[v]);
    kand &= (uint32_t)L.we[v];
    kor |= (uint32_t)L.wt[v];
  }
  const uint32_t diff = kand ^ kor;                  // bits where some candidates differ
  const int sh = kor == 0u ? 0 : min(diff ? __clz(diff) : 32, 24);
  const uint32_t prefix = sh ? (kand & ~(0xffffffffu >> sh)) : 0u;
  // shifted keys keep the top bit set: never 0 and never in a low bin,
  // which the later digits take as empty slots
#pragma unroll
  for (int u = 0; u < KPER; ++u) {
    if (sh && key[u]) key[u] = 0x80000000u | (key[u] << (sh - 1));
    if (key[u]) atomicAdd(&L.hist[key[u] >> 20], 1u);
  }
  lds_barrier();
  const uint4 gv = *(const uint4*)(L.hist + 4 * threadIdx.x);
  auto orig = [&](uint32_t kk) { return sh ? (prefix | ((kk & 0x7fffffffu) >> (sh - 1))) : kk; };
  int b0;   // the first-digit bin of the k-th candidate (-1: not below every candidate)
  const int n_sel = select_listed<KPER>(
      k, gv, L, key, pos, [&](int dst, int p, uint32_t kk) { emit(dst, p, orig(kk)); }, &b0);
  if (max_cut == 0u) return n_sel;   // every window key was listed
  return (n_sel == k && b0 >= 0 && max_cut <= orig((uint32_t)b0 << 20)) ? n_sel : -1;
}

// The selection of a row whose list overflowed, for kernels that finish the
// selection themselves: the row alone, re-read per digit, the positions left
// in L.hist[0 .. n) ascending (k <= 4096).  Rare; kept out of line so its
// registers do not weigh on the attention that follows.
__device__ __noinline__ int fallback_select(const float* scores, int row, int H, int L_max,
                                           const int32_t* lo_p, const int32_t* hi_p, int k,
                                           uint32_t* ghist_row, RowSelLds& L, int& klist_n,
                                           uint4 gv) {
  return row_select_alone<false, 3>(scores, row, H, L_max, lo_p, hi_p, k, ghist_row, true, nullptr,
                                    nullptr, nullptr, nullptr, 0, L, nullptr, klist_n, nullptr,
                                    true, gv);
}

// The same without a first-digit histogram in memory (the segment
// candidates' scan leaves none): the histogram is counted from the row.
__device__ __noinline__ int fallback_select_nohist(const float* scores, int row, int H, int L_max,
                                                  const int32_t* lo_p, const int32_t* hi_p, int k,
                                                  RowSelLds& L, int& klist_n) {
  return row_select_alone<false, 3>(scores, row, H, L_max, lo_p, hi_p, k, nullptr, false, nullptr,
                                    nullptr, nullptr, nullptr, 0, L, nullptr, klist_n);
}

// This thread's 4 bins (4 t .. 4 t + 3) of row `row`'s first-digit
// histogram, summed over its copies (1 or kHistCopiesMax).  The copies' loads
// are all issued before the first is used: as a loop over a run-time count
// they went one round trip at a time.
__device__ __forceinline__ uint4 hist_bins_summed(const TopkWs& ws, int row) {
  const uint4* g = (const uint4*)(ws.hist + (int64_t)row * ws.copies * kBins) + threadIdx.x;
  if (ws.copies != kHistCopiesMax) return g[0];
  uint4 x[kHistCopiesMax];
#pragma unroll
  for (int cp = 0; cp < kHistCopiesMax; ++cp) x[cp] = g[cp * (kBins / 4)];
  uint4 v = x[0];
#pragma unroll
  for (int cp = 1; cp < kHistCopiesMax; ++cp) {
    v.x += x[cp].x;
    v.y += x[cp].y;
    v.z += x[cp].z;
    v.w += x[cp].w;
  }
  return v;
}

}  // namespace

}  // namespace skv
