// Workspace layout of the exact top-k: one 4096-bin histogram of the top 12
// key bits per row, filled by the score scan when the two are fused.  The
// region must be zero when a call starts; every call leaves it zero again.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace skv {

struct TopkWs {
  uint32_t* hist;   // [rows][4096]

  static size_t align(size_t x) { return (x + 255) & ~(size_t)255; }
  static size_t zero_bytes(int rows) { return align((size_t)rows * 4096 * 4); }
  static size_t bytes(int rows) { return zero_bytes(rows); }
  static TopkWs carve(void* p) {
    TopkWs w;
    w.hist = (uint32_t*)p;
    return w;
  }
};

}  // namespace skv
