// Workspace layout of the multi-workgroup exact top-k.  The first region
// (the row histograms) must be zero when a call starts; every call leaves it
// zero again.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace skv {

constexpr int kTopkTile = 4096;   // scores per workgroup tile

struct TopkWs {
  uint32_t* hist;       // [rows][4096] row histogram of the key's top 12 bits
  int32_t* row_info;    // [rows][4] mode, threshold bin, keys above it, k selected
  int32_t* tile_in;     // [rows][n_tiles] keys of the tile inside the threshold bin
  int32_t* tile_above;  // [rows][n_tiles] keys of the tile above the threshold bin
  uint32_t* cand_key;   // [rows][n_tiles][4096] each tile's keys inside the threshold bin

  static size_t align(size_t x) { return (x + 255) & ~(size_t)255; }
  static size_t zero_bytes(int rows) { return align((size_t)rows * 4096 * 4); }
  static size_t bytes(int rows, int L_max, int n_tiles) {
    (void)L_max;
    return zero_bytes(rows) + align((size_t)rows * 16) + 2 * align((size_t)rows * n_tiles * 4) +
           align((size_t)rows * n_tiles * 4096 * 4);
  }
  static TopkWs carve(void* p, int rows, int L_max, int n_tiles) {
    char* c = (char*)p;
    TopkWs w;
    w.hist = (uint32_t*)c;       c += align((size_t)rows * 4096 * 4);
    w.row_info = (int32_t*)c;    c += align((size_t)rows * 16);
    w.tile_in = (int32_t*)c;     c += align((size_t)rows * n_tiles * 4);
    w.tile_above = (int32_t*)c;  c += align((size_t)rows * n_tiles * 4);
    w.cand_key = (uint32_t*)c;
    return w;
  }
};

}  // namespace skv
