// Token-table compaction (vToken reading notes, sections 3.2-3.5 and 4.6):
// the relocation plan on the host (stage 1 eligibility by the waste ratio of
// Eq. (1), stage 2 headroom, stage 3 order-preserving packing that must free
// strictly more blocks than it consumes), the copy + apply_moves on the GPU,
// and the two invariant checks as GPU reductions: I1, a hash of every live
// token's id and K/V words that does not depend on where the token is
// stored, and I2, the number of live tokens that share a slot or point
// outside the pool.
//
// The copy runs one workgroup per 16 consecutive moves and head: a plan fills
// one target block per 16 moves, and a block's 16 rows of one head are one
// contiguous run in the pool, so the writes are whole 4 KB runs (d = 128,
// bf16) while the reads gather the scattered source rows.
#include <math.h>

#include <algorithm>
#include <numeric>
#include <vector>

#include "../../include/sparsekv.h"
#include "skv_device.h"
#include "skv_internal.h"

namespace skv {

namespace {

constexpr int kS = 16;   // tokens per block

// Grid (ceil(n_moves / 16), H): one workgroup per 16 moves and head; thread
// work item (r, m, c): row r (0 = K, 1 = V), move m of the group, 16-byte
// chunk c of the row.  Four items' loads are issued before their stores.
// The workgroups of head 0 then point the token table at the targets.
// A move whose sequence, token or either slot lies outside the table or the
// pool of n_slots slots is skipped (no row is read or written for it) and,
// once per move, counted into *err when err is given.
__device__ __forceinline__ bool move_ok(const skv_move& mv, int B, int L_max, int64_t n_slots) {
  return mv.b >= 0 && mv.b < B && mv.t >= 0 && mv.t < L_max && mv.src >= 0 && mv.src < n_slots &&
         mv.dst >= 0 && mv.dst < n_slots;
}

__global__ __launch_bounds__(256) void compact_copy_kernel(char* k, char* v, int H, int row_k,
                                                           int row_v, const skv_move* moves,
                                                           int n_moves, int32_t* token_table,
                                                           int B, int L_max, int64_t n_slots,
                                                           int32_t* err) {
  const int m0 = blockIdx.x * 16, h = blockIdx.y;
  const int nm = min(16, n_moves - m0);
  const int ck = row_k / 16, cv = row_v / 16;
  const int n_items = nm * (ck + cv);
  for (int i0 = threadIdx.x; i0 < n_items; i0 += 4 * 256) {
    u32x4_t w[4];
    int64_t dst[4];
    char* base[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int it = i0 + u * 256;
      dst[u] = -1;
      if (it >= n_items) continue;
      int rem = it;
      const bool is_v = rem >= nm * ck;
      if (is_v) rem -= nm * ck;
      const int cpr = is_v ? cv : ck;
      const int m = rem / cpr, c = rem - m * cpr;
      const skv_move mv = moves[m0 + m];
      if (!move_ok(mv, B, L_max, n_slots)) continue;
      const int row = is_v ? row_v : row_k;
      base[u] = is_v ? v : k;
      const int64_t so = (((int64_t)(mv.src / kS) * H + h) * kS + mv.src % kS) * row + 16 * c;
      dst[u] = (((int64_t)(mv.dst / kS) * H + h) * kS + mv.dst % kS) * row + 16 * c;
      w[u] = *(const u32x4_t*)(base[u] + so);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (dst[u] >= 0) *(u32x4_t*)(base[u] + dst[u]) = w[u];
  }
  if (h == 0 && threadIdx.x < nm) {
    const skv_move mv = moves[m0 + threadIdx.x];
    if (move_ok(mv, B, L_max, n_slots))
      token_table[(int64_t)mv.b * L_max + mv.t] = mv.dst;
    else if (err)
      atomicAdd(err, 1);
  }
}

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t x, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)x, m, 64), hi = __shfl_xor((uint32_t)(x >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}

__global__ __launch_bounds__(256) void zero_hash_kernel(uint64_t* hash, int32_t* count, int B) {
  for (int i = threadIdx.x; i < B; i += blockDim.x) {
    hash[i] = 0ull;
    count[i] = 0;
  }
}

constexpr int kHashTok = 512;   // tokens per hashing workgroup

// Grid (ceil(L_max / kHashTok), B): tokens kHashTok x .. of sequence b.  The
// chunk's live tokens are gathered first (any order: the hash is a sum), so
// dead tokens cost nothing after that.  A row (token, head h, K or V) is cut
// into P <= 256 16-byte pieces; thread i < (256 / P) P takes piece i % P of
// the rows hr = i / P, i / P + 256 / P, ... (hr = h R + r) of every live
// token, eight tokens' loads in flight at a time.  Per 64-bit word j of a
// row: mix64((s + (j + 1) gamma) ^ w_j) with s = mix64((t H + h) R + r);
// per-thread sums, one workgroup sum, one 64-bit atomic per workgroup (the
// sequence's sum is where every workgroup of the sequence meets, so the
// atomics are kept few).
__global__ __launch_bounds__(256) void live_hash_kernel(KvArgs kv, int P, uint64_t* hash,
                                                        int32_t* count) {
  __shared__ int64_t ls[kHashTok];   // live slots of the chunk
  __shared__ int lt[kHashTok];       // their tokens
  __shared__ uint64_t wsum[4];
  __shared__ int n_live;
  const int b = blockIdx.y, t0 = blockIdx.x * kHashTok;
  if (threadIdx.x == 0) n_live = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < kHashTok; i += 256) {
    const int64_t slot = slot_of(kv, b, t0 + i);
    if (slot >= 0) {
      const int j = atomicAdd(&n_live, 1);
      ls[j] = slot;
      lt[j] = t0 + i;
    }
  }
  __syncthreads();
  const int n = n_live;
  const int R = kv.v ? 2 : 1, HR = kv.H * R;
  const int es = kv.bf16 ? 2 : 4;
  const int p = threadIdx.x % P, rows_par = 256 / P;
  const int q0 = threadIdx.x < rows_par * P ? threadIdx.x / P : HR;   // the rest sit out
  const uint64_t gamma = 0x9e3779b97f4a7c15ull;
  uint64_t acc = 0;
  for (int tb = 0; tb < n; tb += 8) {
    for (int hr = q0; hr < HR; hr += rows_par) {
      const int h = hr / R, r = hr - h * R;
      const int d = r ? kv.d_v : kv.d_k;
      const char* base = (const char*)(r ? kv.v : kv.k);
      u32x4_t w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (tb + u < n)
          w[u] = *(const u32x4_t*)(base + row_elem(kv, b, h, ls[tb + u], d) * es + 16 * p);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (tb + u >= n) continue;
        const uint64_t s = mix64(((uint64_t)lt[tb + u] * kv.H + h) * R + r);
        const uint64_t w0 = (uint64_t)w[u][0] | ((uint64_t)w[u][1] << 32);
        const uint64_t w1 = (uint64_t)w[u][2] | ((uint64_t)w[u][3] << 32);
        acc += mix64((s + (uint64_t)(2 * p + 1) * gamma) ^ w0);
        acc += mix64((s + (uint64_t)(2 * p + 2) * gamma) ^ w1);
      }
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc += shfl_xor64(acc, m);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint64_t tot = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    if (tot) atomicAdd((unsigned long long*)&hash[b], (unsigned long long)tot);
    if (n) atomicAdd(&count[b], n);
  }
}

__global__ __launch_bounds__(256) void unique_init_kernel(int32_t* owner, int64_t n_slots,
                                                          int32_t* result) {
  const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (int64_t i = i0; i < n_slots; i += (int64_t)gridDim.x * blockDim.x) owner[i] = 0;
  if (i0 < 2) result[i0] = 0;
}

// Grid (ceil(L_max / 256), B): a live token claims its slot; a claim that
// finds the slot taken counts a duplicate, a slot outside the pool counts as
// out of range.
__global__ __launch_bounds__(256) void unique_claim_kernel(KvArgs kv, int64_t n_slots,
                                                           int32_t* owner, int32_t* result) {
  const int b = blockIdx.y, t = blockIdx.x * 256 + threadIdx.x;
  const int64_t slot = slot_of(kv, b, t);
  if (slot < 0) return;
  if (slot >= n_slots) {
    atomicAdd(&result[1], 1);
    return;
  }
  if (atomicAdd(&owner[slot], 1) != 0) atomicAdd(&result[0], 1);
}

KvArgs kv_args(const skv_kv* kv) {
  KvArgs a;
  a.k = kv->k;
  a.v = kv->v;
  a.bf16 = kv->dtype == SKV_BF16;
  a.B = kv->B;
  a.H = kv->H;
  a.d_k = kv->d_k;
  a.d_v = kv->d_v;
  a.block = kv->block;
  a.L_max = kv->L_max;
  a.block_table = kv->block_table;
  a.token_table = kv->token_table;
  a.seq_len = kv->seq_len;
  return a;
}

bool pool_ok(const skv_kv* kv) {
  return kv && kv->k && kv->seq_len && kv->B >= 1 && kv->H >= 1 && kv->L_max >= 1 &&
         kv->L_max % kS == 0 && kv->block == kS && kv->d_k >= 1 && kv->d_v >= 1 &&
         (kv->dtype == SKV_BF16 || kv->dtype == SKV_F32) && (kv->v == nullptr || kv->d_v == kv->d_k);
}

}  // namespace

}  // namespace skv

using namespace skv;

extern "C" {

double sparsekv_waste_ratio(const int32_t* n_live, int32_t n) {
  if (!n_live || n < 1) return 0.0;
  double s = 0.0;
  for (int i = 0; i < n; ++i) s += n_live[i];
  return 1.0 - s / ((double)n * kS);
}

skv_status sparsekv_compact_plan(const int32_t* token_table, const int32_t* seq_len, int32_t B,
                                 int32_t L_max, int32_t n_blocks, const int32_t* counts, int32_t b,
                                 const int32_t* free_blocks, int32_t n_free, double theta_F,
                                 int32_t max_src, skv_move* moves, int32_t* n_moves,
                                 int32_t* src_blocks, int32_t* n_src, int32_t* n_dst) {
  if (!token_table || !seq_len || !moves || !n_moves || !src_blocks || !n_src || !n_dst)
    return SKV_EINVAL;
  if (B < 1 || L_max < 1 || n_blocks < 1 || b < 0 || b >= B || max_src < 1 || n_free < 0 ||
      (n_free > 0 && !free_blocks))
    return SKV_EINVAL;
  *n_moves = *n_src = *n_dst = 0;
  const int64_t n_slots = (int64_t)n_blocks * kS;
  for (int i = 0; i < n_free; ++i)
    if (free_blocks[i] < 0 || free_blocks[i] >= n_blocks) return SKV_EINVAL;
  // live tokens per block over every sequence (the caller's running counts
  // when given), and this sequence's own
  std::vector<int32_t> all;
  if (!counts) {
    all.assign(n_blocks, 0);
    for (int s = 0; s < B; ++s) {
      const int len = std::min(seq_len[s], L_max);
      const int32_t* row = token_table + (int64_t)s * L_max;
      for (int t = 0; t < len; ++t)
        if (row[t] >= 0) {
          if (row[t] >= n_slots) return SKV_EINVAL;
          ++all[row[t] / kS];
        }
    }
    counts = all.data();
  }
  {
    std::vector<char> seen(n_blocks, 0);
    for (int i = 0; i < n_free; ++i) {
      const int32_t p = free_blocks[i];
      if (counts[p] != 0 || seen[p]) return SKV_EINVAL;
      seen[p] = 1;
    }
  }
  std::vector<int32_t> own(n_blocks, 0);
  const int len = std::min(seq_len[b], L_max);
  const int32_t* row = token_table + (int64_t)b * L_max;
  for (int t = 0; t < len; ++t)
    if (row[t] >= 0) {
      if (row[t] >= n_slots) return SKV_EINVAL;
      ++own[row[t] / kS];
    }
  // stage 1: the waste ratio over the blocks holding this sequence's tokens
  int64_t live = 0, n_mine = 0;
  for (int p = 0; p < n_blocks; ++p)
    if (own[p]) {
      live += counts[p];
      ++n_mine;
    }
  if (n_mine == 0) return SKV_OK;
  const double F = 1.0 - (double)live / ((double)n_mine * kS);
  if (!(F > theta_F)) return SKV_OK;
  // candidates: private blocks that are not full, emptiest first
  std::vector<int32_t> cand;
  for (int p = 0; p < n_blocks; ++p)
    if (own[p] && own[p] == counts[p] && counts[p] < kS) cand.push_back(p);
  std::stable_sort(cand.begin(), cand.end(),
                   [&](int32_t x, int32_t y) { return counts[x] < counts[y]; });
  if ((int)cand.size() > max_src) cand.resize(max_src);
  // stages 2 and 3: shrink until it frees more than it takes and fits the headroom
  int64_t T = 0;
  for (int32_t p : cand) T += counts[p];
  while (!cand.empty()) {
    const int64_t tgt = (T + kS - 1) / kS;
    if ((int64_t)cand.size() > tgt && tgt <= n_free) break;
    T -= counts[cand.back()];
    cand.pop_back();
  }
  if (cand.empty()) return SKV_OK;
  std::vector<char> is_src(n_blocks, 0);
  for (int32_t p : cand) is_src[p] = 1;
  int i = 0;
  for (int t = 0; t < len; ++t)
    if (row[t] >= 0 && is_src[row[t] / kS]) {
      skv_move& mv = moves[i];
      mv.b = b;
      mv.t = t;
      mv.src = row[t];
      mv.dst = free_blocks[i / kS] * kS + i % kS;
      ++i;
    }
  *n_moves = i;
  std::sort(cand.begin(), cand.end());
  for (size_t j = 0; j < cand.size(); ++j) src_blocks[j] = cand[j];
  *n_src = (int32_t)cand.size();
  *n_dst = (i + kS - 1) / kS;
  return SKV_OK;
}

skv_status sparsekv_compact_apply(const skv_kv* kv, int32_t n_blocks, const skv_move* moves,
                                  int32_t n_moves, int32_t* err, hipStream_t stream) {
  if (!pool_ok(kv) || !kv->token_table || n_blocks < 1 || n_moves < 0 || (n_moves > 0 && !moves))
    return SKV_EINVAL;
  const int es = kv->dtype == SKV_BF16 ? 2 : 4;
  const int row_k = kv->d_k * es, row_v = kv->v ? kv->d_v * es : 0;
  if (row_k % 16 || row_v % 16) return SKV_EUNSUPPORTED;
  if (n_moves == 0) return SKV_OK;
  compact_copy_kernel<<<dim3((n_moves + 15) / 16, kv->H), 256, 0, stream>>>(
      (char*)kv->k, (char*)kv->v, kv->H, row_k, row_v, moves, n_moves,
      (int32_t*)kv->token_table, kv->B, kv->L_max, (int64_t)n_blocks * kS, err);
  return hipGetLastError() == hipSuccess ? SKV_OK : SKV_ELAUNCH;
}

skv_status sparsekv_live_hash(const skv_kv* kv, uint64_t* hash, int32_t* count,
                              hipStream_t stream) {
  if (!kv || !kv->k || !kv->seq_len || !hash || !count || kv->B < 1 || kv->H < 1 ||
      kv->L_max < 1 || kv->d_k < 1)
    return SKV_EINVAL;
  if (kv->dtype != SKV_BF16 && kv->dtype != SKV_F32) return SKV_EINVAL;
  if (kv->block != 0 && kv->block != kS) return SKV_EINVAL;
  if (kv->v && kv->d_v != kv->d_k) return SKV_EINVAL;
  // rows of at most 256 16-byte pieces
  const int es = kv->dtype == SKV_BF16 ? 2 : 4;
  const int row = kv->d_k * es;
  if (row % 16 || row / 16 > 256) return SKV_EUNSUPPORTED;
  KvArgs a = kv_args(kv);
  if (!kv->v) a.d_v = kv->d_k;
  zero_hash_kernel<<<1, 256, 0, stream>>>(hash, count, kv->B);
  live_hash_kernel<<<dim3((kv->L_max + kHashTok - 1) / kHashTok, kv->B), 256, 0, stream>>>(
      a, row / 16, hash, count);
  return hipGetLastError() == hipSuccess ? SKV_OK : SKV_ELAUNCH;
}

size_t sparsekv_check_unique_ws_bytes(int32_t n_blocks) {
  return n_blocks < 1 ? 0 : (size_t)n_blocks * kS * 4;
}

skv_status sparsekv_check_unique(const skv_kv* kv, int32_t n_blocks, int32_t* result, void* ws,
                                 size_t ws_bytes, hipStream_t stream) {
  if (!kv || !kv->seq_len || !result || n_blocks < 1 || kv->B < 1 || kv->L_max < 1) return SKV_EINVAL;
  if (kv->block != kS || (kv->block_table == nullptr) == (kv->token_table == nullptr))
    return SKV_EINVAL;
  if (!ws || ws_bytes < sparsekv_check_unique_ws_bytes(n_blocks)) return SKV_EWORKSPACE;
  const int64_t n_slots = (int64_t)n_blocks * kS;
  const KvArgs a = kv_args(kv);
  const int grid0 = (int)std::min<int64_t>(4096, (n_slots + 255) / 256);
  unique_init_kernel<<<grid0, 256, 0, stream>>>((int32_t*)ws, n_slots, result);
  unique_claim_kernel<<<dim3((kv->L_max + 255) / 256, kv->B), 256, 0, stream>>>(
      a, n_slots, (int32_t*)ws, result);
  return hipGetLastError() == hipSuccess ? SKV_OK : SKV_ELAUNCH;
}

}  // extern "C"
