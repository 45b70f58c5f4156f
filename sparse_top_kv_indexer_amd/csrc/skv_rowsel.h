// Exact top-k selection of one row of fp32 scores by one 1024-thread
// workgroup: the building blocks shared by the standalone top-k kernel and the
// fused select + attend kernel.
//
// Keys: an order-preserving 32-bit image of the score (sign-flipped float
// bits; -0.0 maps to +0.0; inf and nan map to 0, which is never selected).
// Selected: every key > T plus the first need_eq keys equal to T, in
// position order (ties go to the lower position).
//
// Layout: the row is read from the 16-byte boundary at or below the window
// start, w.o slots before it; in sweep s, lane l of wave w holds the slots
// j = s * kSweep + w * kSeg + 256 g + 4 l + e (g < kGroups, e < 4), slot j
// being position lo - o + j, so every load instruction reads 1 KB of
// consecutive scores with 16-byte loads whatever the window's alignment.
// Slots outside [o, o + n) read as -inf.  Short rows use NG < kGroups groups
// per lane (a wave then holds 256 NG slots of a 4096 NG-slot sweep), so every
// wave still holds a share of the row and each pass runs over NG groups.
#pragma once

#include "skv_device.h"

namespace skv {

constexpr int kRowThreads = 1024;
constexpr int kRowWaves = kRowThreads / 64;
constexpr int kGroups = 8;                    // groups of 4 consecutive keys per lane per sweep
constexpr int kSeg = 256 * kGroups;           // positions per wave per sweep
constexpr int kSweep = kRowWaves * kSeg;      // positions per sweep (32768)
constexpr int kBins = 4096;

__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u & 0x7f800000u) == 0x7f800000u) return 0u;   // inf / nan: not a candidate
  if (u == 0x80000000u) u = 0u;                        // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);   // finite keys are >= 0x00800000
}

struct RowWindow {
  int lo, hi, n;
  int o;        // slots between the 16-byte boundary and the window start
  int ns;       // slots to read: o + n
  bool whole;   // L_max % 4 == 0: a 16-byte piece holding a window slot lies
                // inside the scores array (rows start on 4-slot steps)
};

__device__ __forceinline__ RowWindow row_window(const int32_t* lo_p, const int32_t* hi_p, int b,
                                                int L_max) {
  RowWindow w;
  w.lo = max(0, min(lo_p[b], L_max));
  w.hi = max(w.lo, min(hi_p[b], L_max));
  w.n = w.hi - w.lo;
  w.o = 0;
  w.ns = w.n;
  w.whole = (L_max & 3) == 0;
  return w;
}

// The pointer rows are read from: the window start itself, or, when the
// scores array starts on a 16-byte boundary (*vec = true), the boundary at
// or below it (never before the array), with w.o / w.ns set accordingly.
__device__ __forceinline__ const float* row_base(const float* scores, int64_t row_off,
                                                 RowWindow& w, bool* vec) {
  const float* start = scores + row_off + w.lo;
  *vec = ((uintptr_t)scores & 15) == 0;
  if (!*vec) return start;
  w.o = (int)(((uintptr_t)start & 15) >> 2);
  w.ns = w.o + w.n;
  return start - w.o;
}

// Sweeps needed for rows of at most L_max slots whose window start may sit up
// to 3 slots past a 16-byte boundary that lies before the row start.
__host__ __device__ __forceinline__ int row_slots_max(int L_max) {
  return L_max % 4 == 0 ? L_max : L_max + 3;
}

__device__ __forceinline__ int wave_total(int incl) { return __builtin_amdgcn_readlane(incl, 63); }

// This thread's wave index, known to the compiler to be uniform.
__device__ __forceinline__ int row_wave() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// In a wave whose lane holds the counts c of 4 bins first_bin .. first_bin + 3
// and `above` = entries in bins above them: if the need-th largest entry lies
// in one of these bins, write {bin, entries above it, entries in it} to trio.
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

struct RowSelLds {
  uint32_t hist[kBins];   // top 12 key bits, then bits 19..8 of bin b0's keys
  uint32_t dh[256];       // bits 7..0 of the keys matching the top 24 bits
  int wt[kRowWaves], wa[kRowWaves], we[kRowWaves];
  int trio[3];
};

// Scores of the slots p0 + 256 g + e (s from row_base); slots outside the
// window read as -inf.  With 16-byte-aligned rows of a multiple of 4 slots
// (vec and w.whole), every group is one 16-byte load, all of them issued
// before any is used, and the slots outside the window are masked by
// position (a piece that holds a window slot lies inside the array).
// Otherwise a 16-byte load covers slots j .. j + 3 only when all of them lie
// before the window end, so nothing past the row is read; that form compiles
// to branches that wait for each group's load before issuing the next
// (the token pool's listing: 26.0 us that way, 24.9 us with the first form).
// NT: non-temporal loads, for a row this workgroup alone reads, once.
template <bool NT>
__device__ __forceinline__ float4 load_f4(const float* p) {
  if constexpr (NT) {
    typedef float f32x4n_t __attribute__((ext_vector_type(4)));
    const f32x4n_t v = __builtin_nontemporal_load((const f32x4n_t*)p);
    return make_float4(v.x, v.y, v.z, v.w);
  } else {
    return *(const float4*)p;
  }
}

template <int NG, bool NT = false>
__device__ __forceinline__ void slots_load(const float* s, const RowWindow& w, bool vec, int p0,
                                           float (&v)[NG][4]) {
  if (vec && w.whole) {
    float4 f[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int p = p0 + 256 * g;
      f[g] = p < w.ns ? load_f4<NT>(s + p)
                      : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int p = p0 + 256 * g;
      const float fe[4] = {f[g].x, f[g].y, f[g].z, f[g].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) v[g][e] = (p + e >= w.o && p + e < w.ns) ? fe[e] : -INFINITY;
    }
    return;
  }
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int p = p0 + 256 * g;
    if (vec && p + 4 <= w.ns) {
      const float4 f = load_f4<NT>(s + p);
      v[g][0] = f.x;
      v[g][1] = f.y;
      v[g][2] = f.z;
      v[g][3] = f.w;
      if (p < w.o) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (p + e < w.o) v[g][e] = -INFINITY;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        v[g][e] = (p + e >= w.o && p + e < w.ns) ? s[p + e] : -INFINITY;
    }
  }
}

// This lane's first slot of sweep sw with NG groups per lane.
template <int NG>
__device__ __forceinline__ int row_slot0(int sw) {
  const int lane = threadIdx.x & 63, wave = row_wave();
  return sw * (kRowWaves * 256 * NG) + wave * (256 * NG) + 4 * lane;
}

// The slots p0 + 256 g + e of sweep sw for this lane (see the layout above).
template <int NG, bool NT = false>
__device__ __forceinline__ void row_load(const float* s, const RowWindow& w, bool vec, int sw,
                                         float (&v)[NG][4]) {
  slots_load<NG, NT>(s, w, vec, row_slot0<NG>(sw), v);
}

template <int NG>
__device__ __forceinline__ void row_keys(const float (&v)[NG][4], uint32_t (&kk)[NG][4]) {
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int e = 0; e < 4; ++e) kk[g][e] = score_key(v[g][e]);
}

// The need-th largest entry of the kBins-bin histogram in L.hist (wave w
// covers bins 256 w .. 256 w + 255): two barriers; *total receives the
// histogram's total.  need < 0 asks for the min(-need, total)-th; the
// effective rank is returned and, when 1 <= rank < total, L.trio holds
// {bin, entries above it, entries in it} afterwards.
__device__ __forceinline__ int row_search4096(RowSelLds& L, int need, int* total) {
  const int lane = threadIdx.x & 63, wave = row_wave();
  const uint4 c4 = *(const uint4*)(L.hist + 4 * threadIdx.x);
  const int incl = wave_incl_scan((int)(c4.x + c4.y + c4.z + c4.w));
  const int tot_w = wave_total(incl);
  if (lane == 0) L.wt[wave] = tot_w;
  lds_barrier();
  int all = 0, above_w = 0;
#pragma unroll
  for (int v = 0; v < kRowWaves; ++v) {
    all += L.wt[v];
    if (v > wave) above_w += L.wt[v];
  }
  *total = all;
  const int nd = need < 0 ? min(-need, all) : need;
  if (nd >= 1 && nd < all) pick_bin(c4, 4 * threadIdx.x, above_w + (tot_w - incl), nd, L.trio);
  lds_barrier();
  return nd;
}

// Threshold of the row once L.hist holds its top-12-bit histogram (and a
// barrier has passed).  keys_ready() runs after the first search (callers
// convert resident scores to keys there, overlapping their arrival);
// prepare(b0, in_bin) runs (by the whole workgroup) before the lower digits
// are resolved within bin b0 of in_bin keys; for_keys(f) then calls f(key)
// for every key of the window, or at least for every key of bin b0.
template <class KeysReady, class Prepare, class ForKeys>
__device__ __forceinline__ void row_threshold_p(RowSelLds& L, int k, KeysReady&& keys_ready,
                                                Prepare&& prepare, ForKeys&& for_keys,
                                                uint32_t* T_out, int* need_eq_out,
                                                int* k_sel_out, int* first_bin = nullptr) {
  const int lane = threadIdx.x & 63, wave = row_wave();
  int n_cand;
  const int k_sel = row_search4096(L, -k, &n_cand);   // min(k, n_cand)
  keys_ready();
  uint32_t T = 0u;   // k_sel == n_cand: every finite key (key > 0)
  int need_eq = 0;
  if (first_bin) *first_bin = -1;
  if (k_sel <= 0) {
    T = 0xffffffffu;   // nothing: finite keys are below 0xff800000
  } else if (k_sel < n_cand) {
    const int b0 = L.trio[0], above = L.trio[1], in_bin = L.trio[2];
    if (first_bin) *first_bin = b0;
    int need = k_sel - above;
    T = ((uint32_t)b0 << 20) - 1u;   // the whole bin b0 is taken
    if (need < in_bin && in_bin <= 64) {
      // few keys in bin b0: one wave sorts them (bitonic, one key per lane)
      // and reads the need-th largest, instead of two more digit passes
      lds_barrier();   // everyone has read trio
      if (threadIdx.x == 0) L.wa[0] = 0;
      lds_barrier();
      for_keys([&](uint32_t key) {
        if ((key >> 20) == (uint32_t)b0) {
          const int i = atomicAdd(&L.wa[0], 1);
          if (i < 64) L.dh[i] = key;
        }
      });
      lds_barrier();
      if (wave == 0) {
        uint32_t v = lane < in_bin ? L.dh[lane] : 0u;
#pragma unroll
        for (int sz = 2; sz <= 64; sz <<= 1)
#pragma unroll
          for (int j = sz >> 1; j >= 1; j >>= 1) {
            const uint32_t o = (uint32_t)__shfl_xor((int)v, j, 64);
            // descending runs where (lane & sz) == 0; the lower lane keeps the larger
            const bool lower = (lane & j) == 0;
            const bool desc = (lane & sz) == 0;
            v = (lower == desc) ? max(v, o) : min(v, o);
          }
        const uint32_t t_key = (uint32_t)__shfl((int)v, need - 1, 64);
        const int gt = __popcll(__ballot(v > t_key));
        if (lane == 0) {
          L.trio[0] = (int)t_key;
          L.trio[1] = need - gt;
        }
      }
      lds_barrier();
      T = (uint32_t)L.trio[0];
      need_eq = L.trio[1];
    } else if (need < in_bin) {
      prepare(b0, in_bin);
      // bits 19..8 of the keys of bin b0 (finite keys have top bits >= 8, so
      // b0 >= 8 and empty slots never match)
      lds_barrier();   // everyone has read trio and the top-bit counts
      *(uint4*)(L.hist + 4 * threadIdx.x) = make_uint4(0u, 0u, 0u, 0u);
      lds_barrier();
      for_keys([&](uint32_t key) {
        if ((key >> 20) == (uint32_t)b0) atomicAdd(&L.hist[(key >> 8) & 0xfffu], 1u);
      });
      lds_barrier();
      int unused;
      row_search4096(L, need, &unused);
      const int b1 = L.trio[0], ab1 = L.trio[1], ib1 = L.trio[2];
      need -= ab1;
      const uint32_t pre24 = ((uint32_t)b0 << 12) | (uint32_t)b1;
      if (need == ib1) {
        T = (pre24 << 8) - 1u;
        need = 0;
      } else {
        // bits 7..0 of the keys matching the top 24 bits
        for_keys([&](uint32_t key) {
          if ((key >> 8) == pre24) atomicAdd(&L.dh[key & 0xffu], 1u);
        });
        lds_barrier();
        if (wave == 0) {
          const uint4 d4 = *(const uint4*)(L.dh + 4 * lane);
          const int il = wave_incl_scan((int)(d4.x + d4.y + d4.z + d4.w));
          pick_bin(d4, 4 * lane, wave_total(il) - il, need, L.trio);
        }
        lds_barrier();
        const int b2 = L.trio[0], ab2 = L.trio[1], ib2 = L.trio[2];
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
  *T_out = T;
  *need_eq_out = need_eq;
  *k_sel_out = k_sel;
}

template <class KeysReady, class ForKeys>
__device__ __forceinline__ void row_threshold(RowSelLds& L, int k, KeysReady&& keys_ready,
                                              ForKeys&& for_keys, uint32_t* T_out,
                                              int* need_eq_out, int* k_sel_out,
                                              int* first_bin = nullptr) {
  row_threshold_p(L, k, keys_ready, [](int, int) {}, for_keys, T_out, need_eq_out, k_sel_out,
                  first_bin);
}

// Per group g, the lane's counts of keys above T (low 16 bits) and equal to T
// (high 16 bits); returns the lane's total, packed the same way.
template <int NG>
__device__ __forceinline__ int row_counts(const uint32_t (&kk)[NG][4], uint32_t T,
                                          int (&cg)[NG]) {
  int tot = 0;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    int c = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      c += (kk[g][e] > T) ? 1 : ((kk[g][e] != 0u && kk[g][e] == T) ? 0x10000 : 0);
    cg[g] = c;
    tot += c;
  }
  return tot;
}

// Exchange the waves' packed totals (two barriers): *oa / *oe receive the keys
// above / equal to T in the waves before this one, *ta / *te the workgroup's.
__device__ __forceinline__ void row_wave_offsets(RowSelLds& L, int lane_tot, int* oa, int* oe,
                                                 int* ta, int* te) {
  const int lane = threadIdx.x & 63, wave = row_wave();
  const int wt_pk = wave_total(wave_incl_scan(lane_tot));
  lds_barrier();   // earlier readers of wa / we are done
  if (lane == 0) {
    L.wa[wave] = wt_pk & 0xffff;
    L.we[wave] = wt_pk >> 16;
  }
  lds_barrier();
  int a = 0, e = 0, sa = 0, se = 0;
#pragma unroll
  for (int v = 0; v < kRowWaves; ++v) {
    if (v < wave) {
      a += L.wa[v];
      e += L.we[v];
    }
    sa += L.wa[v];
    se += L.we[v];
  }
  *oa = a;
  *oe = e;
  *ta = sa;
  *te = se;
}

// The wave's selected keys in position order: emit(dst, g, e) for every key
// taken, dst = its rank among the selected keys of the row.  oa / oe: keys
// above / equal to T before this wave's positions.
template <int NG, class Emit>
__device__ __forceinline__ void row_emit(const uint32_t (&kk)[NG][4], const int (&cg)[NG],
                                         uint32_t T, int need_eq, int oa, int oe, Emit&& emit) {
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int ig = wave_incl_scan(cg[g]);
    const int gt = wave_total(ig);
    int ab = oa + ((ig - cg[g]) & 0xffff), eb = oe + ((ig - cg[g]) >> 16);
    if ((cg[g] & 0xffff) || ((cg[g] >> 16) && eb < need_eq)) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t key = kk[g][e];
        if (key > T) {
          emit(ab + min(eb, need_eq), g, e);
          ++ab;
        } else if (key != 0u && key == T) {
          if (eb < need_eq) emit(ab + eb, g, e);
          ++eb;
        }
      }
    }
    oa += gt & 0xffff;
    oe += gt >> 16;
  }
}

}  // namespace skv
