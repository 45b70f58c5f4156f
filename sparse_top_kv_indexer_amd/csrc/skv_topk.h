// Workspace layout of the exact top-k (topk.hip).  Per row: the 4096-bin
// histogram of the top 12 key bits (filled by the score scan when the two
// are fused) and the fill counter of the row's key list; both must be zero
// when a call starts and every call leaves them zero again.  Then the row's
// list bounds, the per-slice list placement and the list itself.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace skv {

// A listing workgroup covers 1024 ng row slots (256 threads, ng groups of 4
// slots per lane, ng in 1, 2, 4, 8): few long rows get small slices so the
// listing still spreads over the whole chip, many rows get large ones so the
// per-workgroup work (reading the row's histogram) stays small.
constexpr int kSliceUnit = 1024;    // row slots per listing workgroup and group per lane
constexpr int kRowList = 16384;     // keys a row's list holds
constexpr int kMaxSlices = 4096;    // rows of up to 8 * kSliceUnit * kMaxSlices slots
constexpr int kListWgs = 2048;      // listing workgroups a call aims for
// A row's list counter sits alone in a 256-byte line: the listing workgroups
// of every row add to their row's counter, and counters sharing a line would
// queue behind each other at the one place device atomics are resolved.
constexpr int kCtrStride = 64;

__host__ __device__ inline int topk_slices_ng(int L_max, int ng) {
  const int64_t slots = L_max % 4 == 0 ? (int64_t)L_max : (int64_t)L_max + 3;
  const int64_t per = (int64_t)kSliceUnit * ng;
  return (int)((slots + per - 1) / per);
}

// Groups per lane of the listing workgroups of `rows` rows: the largest of
// 8, 4, 2, 1 that still gives kListWgs workgroups, or the smallest that
// keeps a row within kMaxSlices slices.
inline int topk_slice_groups(int rows, int L_max) {
  int ng = 8;
  while (ng > 1 && (int64_t)rows * topk_slices_ng(L_max, ng) < kListWgs &&
         topk_slices_ng(L_max, ng / 2) <= kMaxSlices)
    ng /= 2;
  return ng;
}

// Copies of a row's first-digit histogram.  A few long rows are scanned by
// hundreds of workgroups each, and their once-per-workgroup flushes of the
// histogram queue behind each other on the row's bins (device atomics on few
// addresses are slow); with several copies, workgroup w adds into copy
// w % copies and every reader sums the copies.  Two copies: for one row of
// 131,072 keys the scan took 14.4 us with one copy and 12.0-12.6 us with
// 2, 4 or 8, while every listing workgroup, which reads all copies, took 5.7,
// 6.4 and 7.8 us.  Producer and consumers derive the count from (rows, L_max)
// alone.
constexpr int kHistCopiesMax = 2;
__host__ __device__ inline int topk_hist_copies(int rows, int L_max) {
  const int64_t slots = L_max % 4 == 0 ? (int64_t)L_max : (int64_t)L_max + 3;
  return (rows <= 4 && slots > 32768) ? kHistCopiesMax : 1;
}

// Slice entries a row's workspace holds: the most any call may use.
__host__ __device__ inline int topk_slices(int L_max) {
  int ng = 1;
  while (ng < 8 && topk_slices_ng(L_max, ng) > kMaxSlices) ng *= 2;
  return topk_slices_ng(L_max, ng);
}

// Segment candidates of few long rows (k <= kSegMaxK): the score scan gives
// each of a row's S workgroups one segment of at most kSegMaxKeys keys, and
// each lists the segment's keys of its highest histogram bins that fit in
// m = kSegSlots / S slots, in position order, with the count listed and a cut
// (0: the segment listed every key of the window; else every key it left
// out is below the cut).  A row's exact top-k is the top-k of its listed keys
// whenever no cut lies above the k-th of them.  The lists live in the row's
// key-list region of the workspace: keys and positions in slots
// [0, kSegSlots) of lkey / lpos, counts and cuts after the keys.
constexpr int kSegSlots = 8192;     // listed slots per row
constexpr int kSegMaxKeys = 4096;   // keys per segment
constexpr int kSegMax = 512;        // segments per row
constexpr int kSegMaxK = 2048;      // k served (a quarter of the slots)

// Segments per row for `rows` rows of L_max slots and k, or 0 when the
// segment candidates do not serve the call (rows of at most 16,384 slots):
// a power of two giving about 512 workgroups in all (one per resident slot
// of the scan), at most 256 unless a segment would exceed kSegMaxKeys keys
// (one row of 131,072: 256 segments scanned in 12.0 us, 512 in 12.6; 32
// rows of 32,768: 16 segments 54.8 us, 32 segments 56.4 us).
inline int topk_seg_count(int rows, int L_max, int k) {
  const int64_t slots = L_max % 4 == 0 ? (int64_t)L_max : (int64_t)L_max + 3;
  if (rows < 1 || k < 1 || k > kSegMaxK || slots <= 16384) return 0;
  int S = 256;
  while (S > 1 && (int64_t)rows * S > 512) S >>= 1;
  const int64_t cpr = ((int64_t)L_max + 15) / 16;
  while (S < kSegMax && cpr > (int64_t)S * (kSegMaxKeys / 16)) S <<= 1;
  return cpr <= (int64_t)S * (kSegMaxKeys / 16) ? S : 0;
}

struct TopkWs {
  uint32_t* hist;   // [rows][copies][4096]
  int32_t* ctr;     // [rows][kCtrStride] keys listed so far (element 0 of each line)
  int32_t* meta;    // [rows][2]: smallest listed key, listed count (-1: too many)
  int32_t* slc;     // [rows][slices][2]: list offset and count of each slice
  uint32_t* lkey;   // [rows][kRowList] listed keys, slice by slice in position order
  int32_t* lpos;    // [rows][kRowList] their positions
  int copies;       // histogram copies per row (topk_hist_copies)

  static size_t align(size_t x) { return (x + 255) & ~(size_t)255; }
  static size_t zero_bytes(int rows, int L_max) {
    return align((size_t)rows * topk_hist_copies(rows, L_max) * 4096 * 4) +
           align((size_t)rows * kCtrStride * 4);
  }
  static size_t bytes(int rows, int L_max) {
    return zero_bytes(rows, L_max) + align((size_t)rows * 8) +
           align((size_t)rows * topk_slices(L_max) * 8) + 2 * align((size_t)rows * kRowList * 4);
  }
  // segment candidates of row r: key / pos slot i at r * kRowList + i,
  // count and cut of segment j at r * kRowList + j
  __host__ __device__ uint32_t* seg_key() const { return lkey; }
  __host__ __device__ int32_t* seg_pos() const { return lpos; }
  __host__ __device__ int32_t* seg_n() const { return (int32_t*)(lkey + kSegSlots); }
  __host__ __device__ uint32_t* seg_cut() const { return lkey + kSegSlots + kSegMax; }
  static TopkWs carve(void* p, int rows, int L_max) {
    TopkWs w;
    char* c = (char*)p;
    w.copies = topk_hist_copies(rows, L_max);
    w.hist = (uint32_t*)c;
    c += align((size_t)rows * w.copies * 4096 * 4);
    w.ctr = (int32_t*)c;
    c += align((size_t)rows * kCtrStride * 4);
    w.meta = (int32_t*)c;
    c += align((size_t)rows * 8);
    w.slc = (int32_t*)c;
    c += align((size_t)rows * topk_slices(L_max) * 8);
    w.lkey = (uint32_t*)c;
    c += align((size_t)rows * kRowList * 4);
    w.lpos = (int32_t*)c;
    return w;
  }
};

}  // namespace skv
