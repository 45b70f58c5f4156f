// Workspace layout of the exact top-k (topk.hip).  Per row: the 4096-bin
// histogram of the top 12 key bits (filled by the score scan when the two
// are fused) and the fill counter of the row's key list; both must be zero
// when a call starts and every call leaves them zero again.  Then the row's
// list bounds, the per-slice list placement and the list itself.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace skv {

constexpr int kSlice = 8192;        // row slots per listing workgroup
constexpr int kRowList = 16384;     // keys a row's list holds
constexpr int kMaxSlices = 4096;    // rows of up to kSlice * kMaxSlices slots

__host__ __device__ inline int topk_slices(int L_max) {
  const int64_t slots = L_max % 4 == 0 ? (int64_t)L_max : (int64_t)L_max + 3;
  return (int)((slots + kSlice - 1) / kSlice);
}

struct TopkWs {
  uint32_t* hist;   // [rows][4096]
  int32_t* ctr;     // [rows] keys listed so far
  int32_t* meta;    // [rows][2]: smallest listed key, listed count (-1: too many)
  int32_t* slc;     // [rows][slices][2]: list offset and count of each slice
  uint32_t* lkey;   // [rows][kRowList] listed keys, slice by slice in position order
  int32_t* lpos;    // [rows][kRowList] their positions

  static size_t align(size_t x) { return (x + 255) & ~(size_t)255; }
  static size_t zero_bytes(int rows) {
    return align((size_t)rows * 4096 * 4) + align((size_t)rows * 4);
  }
  static size_t bytes(int rows, int L_max) {
    return zero_bytes(rows) + align((size_t)rows * 8) +
           align((size_t)rows * topk_slices(L_max) * 8) + 2 * align((size_t)rows * kRowList * 4);
  }
  static TopkWs carve(void* p, int rows, int L_max) {
    TopkWs w;
    char* c = (char*)p;
    w.hist = (uint32_t*)c;
    c += align((size_t)rows * 4096 * 4);
    w.ctr = (int32_t*)c;
    c += align((size_t)rows * 4);
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
