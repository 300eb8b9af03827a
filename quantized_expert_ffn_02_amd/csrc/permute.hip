// Token permutation by expert: a stable counting sort of the routed entries
// r = t*k + i (and the shared-expert entries r = T*k + t as group E), done as
// histogram -> prefix sum -> stable scatter, all on the device with integer
// arithmetic only (so the result is the same on every run).
//
// The pages motivate it: per token only 10 of a layer's 512 experts run (page
// "Strata Runs 125B Qwen3.8-Flash-Next on a 12GB Gaming GPU", section "How a
// 125B model fits in 12 GB"), and a prompt chunk of up to 8,192 tokens (page
// "Strata Runs a 125-Billion-Parameter Qwen Model on a 12 GB Gaming GPU ...")
// has to be grouped by expert before each expert's weights are read once.
#include "device.h"
#include "internal.h"

namespace moe {

static constexpr int kChunk = 1024;   // entries per histogram / scatter chunk

int permute_chunks(int n_entries) { return (n_entries + kChunk - 1) / kChunk; }

__device__ __forceinline__ int group_of(const int32_t* __restrict__ ids, int r, int Tk, int E) {
  return r < Tk ? ids[r] : E;
}

// Per-chunk histogram over G = E + 1 groups: counts[chunk][g].
__global__ __launch_bounds__(256) void k_perm_hist(const int32_t* __restrict__ ids, int Tk, int n, int E,
                                                   int32_t* __restrict__ counts) {
  __shared__ int h[1024];
  const int G = E + 1;
  for (int g = threadIdx.x; g < G; g += blockDim.x) h[g] = 0;
  __syncthreads();
  const int r0 = blockIdx.x * kChunk;
  const int r1 = min(n, r0 + kChunk);
  for (int r = r0 + threadIdx.x; r < r1; r += blockDim.x) {
    const int g = group_of(ids, r, Tk, E);
    if ((unsigned)g <= (unsigned)E) atomicAdd(&h[g], 1);   // out-of-range ids are dropped
  }
  __syncthreads();
  for (int g = threadIdx.x; g < G; g += blockDim.x) counts[(size_t)blockIdx.x * G + g] = h[g];
}

// Exclusive scan of v over the 1024 threads of a block (v = 0 past the end).
__device__ int block_exclusive_scan_1024(int v, int* total) {
  __shared__ int wsum[16];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int base = 0, all = 0;
  for (int i = 0; i < 16; ++i) {
    const int s = wsum[i];
    if (i < w) base += s;
    all += s;
  }
  __syncthreads();
  *total = all;
  return base + incl - v;
}

// One block of 1024 threads, thread g = group: totals, offsets and per-chunk
// bases.  A group's per-chunk counts are read kScanBatch at a time (indices
// clamped, extra values dropped), so a thread waits for one memory round trip
// per batch rather than per chunk.
static constexpr int kScanBatch = 16;

struct PlanOut {
  int min_rows = 0, items_per = 1, tile_rows = 1;
  int mx_rows = 0;   // groups of 1 .. mx_rows entries: fp8 x fp4 tiles of at most kMxTileRows rows
  int32_t *tiles = nullptr, *n_tiles = nullptr, *items = nullptr, *n_items = nullptr;
};

// Plan of the groups (as k_plan computes it) from thread g's group start and
// count; every thread of the block calls it.  A small group is cut into
// ceil(cnt / kMxTileRows) fp8 x fp4 tiles of (nearly) equal rows (rows |
// kTileMx), which follow all the fp16 tiles, so the longer fp16 tiles are
// dispatched first; n_tiles[1] counts the fp16 tiles.
__device__ void plan_groups(const PlanOut& P, int g, int start, int cnt) {
  const bool big = cnt >= P.min_rows;
  const bool mx = big && cnt > 0 && cnt <= P.mx_rows;
  const int nmx = mx ? (cnt + kMxTileRows - 1) / kMxTileRows : 0;
  const int nt = big && !mx ? (cnt + P.tile_rows - 1) / P.tile_rows : 0;
  const int ni = big ? 0 : (cnt + P.items_per - 1) / P.items_per;
  // with fp8 x fp4 tiles (batches below a prompt chunk: fewer than 2^20 fp16 tiles,
  // fewer than 2^11 fp8 x fp4 tiles) one scan counts both kinds: fp16 tiles in the
  // low 20 bits, fp8 x fp4 tiles above them
  int tot_tm = 0, tot_i = 0;
  const int ptm = P.mx_rows > 0 ? block_exclusive_scan_1024(nt | (nmx << 20), &tot_tm)
                                : block_exclusive_scan_1024(nt, &tot_tm);
  // with min_rows <= 1 every non-empty group takes tiles: no work items, no scan for them
  const int pi = P.min_rows > 1 ? block_exclusive_scan_1024(ni, &tot_i) : 0;
  const int low = P.mx_rows > 0 ? (1 << 20) - 1 : -1;
  const int pt = ptm & low, pm = P.mx_rows > 0 ? ptm >> 20 : 0;
  const int tot_t = tot_tm & low, tot_m = P.mx_rows > 0 ? tot_tm >> 20 : 0;
  for (int i = 0; i < nt; ++i) {
    P.tiles[3 * (pt + i)] = g;
    P.tiles[3 * (pt + i) + 1] = start + i * P.tile_rows;
    P.tiles[3 * (pt + i) + 2] = min(P.tile_rows, cnt - i * P.tile_rows);
  }
  for (int i = 0; i < nmx; ++i) {
    const int r0 = i * cnt / nmx, r1 = (i + 1) * cnt / nmx;
    P.tiles[3 * (tot_t + pm + i)] = g;
    P.tiles[3 * (tot_t + pm + i) + 1] = start + r0;
    P.tiles[3 * (tot_t + pm + i) + 2] = (r1 - r0) | kTileMx;
  }
  for (int i = 0; i < ni; ++i) {
    P.items[3 * (pi + i)] = g;
    P.items[3 * (pi + i) + 1] = start + i * P.items_per;
    P.items[3 * (pi + i) + 2] = min(P.items_per, cnt - i * P.items_per);
  }
  if (g == 0) {
    P.n_tiles[0] = tot_t + tot_m;
    P.n_tiles[1] = tot_t;
    *P.n_items = tot_i;
  }
}

// P.tiles != NULL: the plan is made here too (the offsets are this block's).
__global__ __launch_bounds__(1024) void k_perm_scan(const int32_t* __restrict__ counts, int n_chunks, int E,
                                                    int32_t* __restrict__ base, int32_t* __restrict__ offsets,
                                                    PlanOut P) {
  const int G = E + 1;
  const int g = threadIdx.x;
  const int gg = g < G ? g : 0;
  int tot = 0;
  for (int c0 = 0; c0 < n_chunks; c0 += kScanBatch) {
    int v[kScanBatch];
#pragma unroll
    for (int j = 0; j < kScanBatch; ++j) v[j] = counts[(size_t)min(c0 + j, n_chunks - 1) * G + gg];
#pragma unroll
    for (int j = 0; j < kScanBatch; ++j) tot += c0 + j < n_chunks ? v[j] : 0;
  }
  int n_all = 0;
  const int off = block_exclusive_scan_1024(g < G ? tot : 0, &n_all);
  if (g < G) {
    offsets[g] = off;
    int run = off;
    for (int c0 = 0; c0 < n_chunks; c0 += kScanBatch) {
      int v[kScanBatch];
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) v[j] = counts[(size_t)min(c0 + j, n_chunks - 1) * G + g];
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) {
        if (c0 + j < n_chunks) {
          base[(size_t)(c0 + j) * G + g] = run;
          run += v[j];
        }
      }
    }
  }
  if (g == 0) offsets[G] = n_all;
  if (P.tiles) plan_groups(P, g, g < G ? off : 0, g < G ? tot : 0);
}

// The same scan with the whole count matrix staged in LDS as 16-bit values (a
// chunk counts at most kChunk = 1,024 entries of a group): the block loads it
// in one cooperative pass, every load of a thread in flight at once, so it
// waits for memory about once instead of once per batch of chunks and pass.  For count
// matrices of up to kScanLdsCounts values (88 chunks x 513 groups at 8,192
// tokens is 45,144).
static constexpr int kScanLdsCounts = 49152;   // 96 KB of LDS

__global__ __launch_bounds__(1024) void k_perm_scan_lds(const int32_t* __restrict__ counts, int n_chunks, int E,
                                                        int32_t* __restrict__ base, int32_t* __restrict__ offsets,
                                                        PlanOut P) {
  __shared__ uint16_t cs[kScanLdsCounts];
  const int G = E + 1, N = n_chunks * G;
  constexpr int PER = kScanLdsCounts / 1024;   // values per thread, all loads issued before the first store
  int v[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = threadIdx.x + j * 1024;
    v[j] = i < N ? counts[i] : 0;
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = threadIdx.x + j * 1024;
    if (i < N) cs[i] = (uint16_t)v[j];
  }
  __syncthreads();
  const int g = threadIdx.x;
  int tot = 0;
  if (g < G)
    for (int c = 0; c < n_chunks; ++c) tot += cs[c * G + g];
  int n_all = 0;
  const int off = block_exclusive_scan_1024(g < G ? tot : 0, &n_all);
  if (g < G) {
    offsets[g] = off;
    int run = off;
    for (int c = 0; c < n_chunks; ++c) {
      base[(size_t)c * G + g] = run;
      run += cs[c * G + g];
    }
  }
  if (g == 0) offsets[G] = n_all;
  if (P.tiles) plan_groups(P, g, g < G ? off : 0, g < G ? tot : 0);
}

// One wave per chunk: entries in ascending r, 64 at a time; the rank of an
// entry among equal-group entries of its batch comes from ballots over the
// group's bits, and a per-group running count in LDS carries across batches.
__global__ __launch_bounds__(64) void k_perm_scatter(const int32_t* __restrict__ ids, int Tk, int n, int E,
                                                     const int32_t* __restrict__ base,
                                                     int32_t* __restrict__ sorted_rows,
                                                     int32_t* __restrict__ row_to_sorted) {
  __shared__ int run[1024];
  const int G = E + 1;
  const int lane = threadIdx.x;
  for (int g = lane; g < G; g += 64) run[g] = 0;
  __syncthreads();
  const int r0 = blockIdx.x * kChunk;
  const int r1 = min(n, r0 + kChunk);
  const int32_t* __restrict__ cbase = base + (size_t)blockIdx.x * G;
  for (int b = r0; b < r1; b += 64) {
    const int r = b + lane;
    int g = r < r1 ? group_of(ids, r, Tk, E) : 0;
    const bool valid = r < r1 && (unsigned)g <= (unsigned)E;
    if (!valid) g = 0;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 10; ++bit) {
      const bool on = (g >> bit) & 1;
      const uint64_t m = __ballot(on);
      peers &= on ? m : ~m;
    }
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int rank = __popcll(peers & below);
    int prior = 0;
    if (valid) prior = run[g];
    __syncthreads();
    if (valid) {
      const int pos = cbase[g] + prior + rank;
      sorted_rows[pos] = r;
      row_to_sorted[r] = pos;
      const bool last = (peers >> lane) == 1ull;   // highest lane of this group in the batch
      if (last) run[g] = prior + __popcll(peers);
    }
    __syncthreads();
  }
}

static hipError_t permute_multi(const int32_t* ids, int T, int k, int E, int with_shared, int32_t* offsets,
                                int32_t* sorted_rows, int32_t* row_to_sorted, int32_t* counts, int32_t* base,
                                const PlanOut& plan, hipStream_t s) {
  const int Tk = T * k;
  const int n = Tk + (with_shared ? T : 0);
  const int nc = permute_chunks(n);
  MOE_LAUNCH(k_perm_hist, dim3(nc), dim3(256), 0, s, ids, Tk, n, E, counts);
  if ((size_t)nc * (E + 1) <= (size_t)kScanLdsCounts)
    MOE_LAUNCH(k_perm_scan_lds, dim3(1), dim3(1024), 0, s, counts, nc, E, base, offsets, plan);
  else
    MOE_LAUNCH(k_perm_scan, dim3(1), dim3(1024), 0, s, counts, nc, E, base, offsets, plan);
  MOE_LAUNCH(k_perm_scatter, dim3(nc), dim3(64), 0, s, ids, Tk, n, E, base, sorted_rows, row_to_sorted);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* ids, int T, int k, int E, int with_shared, int32_t* offsets,
                          int32_t* sorted_rows, int32_t* row_to_sorted, int32_t* counts, int32_t* base,
                          hipStream_t s) {
  return permute_multi(ids, T, k, E, with_shared, offsets, sorted_rows, row_to_sorted, counts, base, PlanOut(), s);
}

// ---------------------------------------------------------------------------
// Permutation and plan of a batch of up to kPermSmallMax entries in ONE block
// of 16 waves (the four launches above cost more than the work at these
// sizes).  Wave w owns the contiguous entries [w P, (w + 1) P): per-wave
// group counts in LDS, a block scan gives the offsets and then each wave's
// base per group (waves in order), and every wave scatters its own entries in
// ascending r, 64 at a time, ranking equal groups inside a batch with ballots
// over the group bits -- the same stable order as the multi-block path.  The
// plan (tiles of groups with at least min_rows entries, work items of the
// rest) follows from the offsets, as k_plan computes it.
// ---------------------------------------------------------------------------
static constexpr int kPermSmallMax = 16384;

__global__ __launch_bounds__(1024) void k_perm_plan_small(const int32_t* __restrict__ ids, int Tk, int n, int E,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ sorted_rows,
                                                          int32_t* __restrict__ row_to_sorted, int min_rows,
                                                          int items_per, int tile_rows, int32_t* __restrict__ tiles,
                                                          int32_t* __restrict__ n_tiles, int32_t* __restrict__ items,
                                                          int32_t* __restrict__ n_items, int mx_rows) {
  __shared__ int hw[16][1024];
  __shared__ int s_off[1025];
  const int G = E + 1;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < 16 * 1024; i += 1024) (&hw[0][0])[i] = 0;
  __syncthreads();
  const int per = (n + 15) / 16;
  const int r0 = min(n, w * per), r1 = min(n, r0 + per);
  for (int r = r0 + lane; r < r1; r += 64) {
    const int g = group_of(ids, r, Tk, E);
    if ((unsigned)g <= (unsigned)E) atomicAdd(&hw[w][g], 1);   // out-of-range ids are dropped
  }
  __syncthreads();
  int tot = 0;
  if (tid < G)
    for (int i = 0; i < 16; ++i) tot += hw[i][tid];
  int n_all = 0;
  const int off = block_exclusive_scan_1024(tid < G ? tot : 0, &n_all);
  if (tid < G) {
    offsets[tid] = off;
    s_off[tid] = off;
    int run = off;
    for (int i = 0; i < 16; ++i) {
      const int c = hw[i][tid];
      hw[i][tid] = run;
      run += c;
    }
  }
  if (tid == 0) {
    offsets[G] = n_all;
    s_off[G] = n_all;
  }
  __syncthreads();
  // per-wave scatter (no block barrier inside: the waves' ranges differ in
  // length; a wave's LDS reads of hw[w][g] precede its own update in order)
  for (int b = r0; b < r1; b += 64) {
    const int r = b + lane;
    int g = r < r1 ? group_of(ids, r, Tk, E) : 0;
    const bool valid = r < r1 && (unsigned)g <= (unsigned)E;
    if (!valid) g = 0;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 10; ++bit) {
      const bool on = (g >> bit) & 1;
      const uint64_t m = __ballot(on);
      peers &= on ? m : ~m;
    }
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int rank = __popcll(peers & below);
    const int prior = valid ? hw[w][g] : 0;
    if (valid) {
      const int pos = prior + rank;
      sorted_rows[pos] = r;
      row_to_sorted[r] = pos;
      if ((peers >> lane) == 1ull) hw[w][g] = prior + __popcll(peers);   // the group's highest lane
    }
  }
  __syncthreads();
  PlanOut P;
  P.min_rows = min_rows;
  P.items_per = items_per;
  P.tile_rows = tile_rows;
  P.mx_rows = mx_rows;
  P.tiles = tiles;
  P.n_tiles = n_tiles;
  P.items = items;
  P.n_items = n_items;
  const int start = tid < G ? s_off[tid] : 0;
  plan_groups(P, tid, start, tid < G ? s_off[tid + 1] - start : 0);
}

hipError_t launch_permute_plan(const int32_t* ids, int T, int k, int E, int with_shared, int32_t* offsets,
                               int32_t* sorted_rows, int32_t* row_to_sorted, int32_t* counts, int32_t* base,
                               int min_rows, int items_per, int tile_rows, int32_t* tiles, int32_t* n_tiles,
                               int32_t* items, int32_t* n_items, hipStream_t s, int mx_rows) {
  const int Tk = T * k;
  const int n = Tk + (with_shared ? T : 0);
  if (n <= kPermSmallMax && E + 1 <= 1024) {
    MOE_LAUNCH(k_perm_plan_small, dim3(1), dim3(1024), 0, s, ids, Tk, n, E, offsets, sorted_rows, row_to_sorted,
               min_rows, items_per, tile_rows, tiles, n_tiles, items, n_items, mx_rows);
    return hipGetLastError();
  }
  PlanOut P;
  P.min_rows = min_rows;
  P.items_per = items_per;
  P.tile_rows = tile_rows;
  P.mx_rows = mx_rows;
  P.tiles = tiles;
  P.n_tiles = n_tiles;
  P.items = items;
  P.n_items = n_items;
  return permute_multi(ids, T, k, E, with_shared, offsets, sorted_rows, row_to_sorted, counts, base, P, s);
}

// Work items from offsets: group g yields ceil(count / items_per) items, placed
// after the items of every lower group.
__global__ __launch_bounds__(1024) void k_items_from_offsets(const int32_t* __restrict__ offsets, int E,
                                                             int items_per, int32_t* __restrict__ items,
                                                             int32_t* __restrict__ n_items) {
  const int G = E + 1;
  const int g = threadIdx.x;
  const int start = g < G ? offsets[g] : 0;
  const int cnt = g < G ? offsets[g + 1] - start : 0;
  const int ni = (cnt + items_per - 1) / items_per;
  int total = 0;
  const int pos = block_exclusive_scan_1024(ni, &total);
  for (int i = 0; i < ni; ++i) {
    items[(size_t)(pos + i) * 3 + 0] = g;
    items[(size_t)(pos + i) * 3 + 1] = start + i * items_per;
    items[(size_t)(pos + i) * 3 + 2] = min(items_per, cnt - i * items_per);
  }
  if (g == 0) *n_items = total;
}

hipError_t launch_items_from_offsets(const int32_t* offsets, int E, int items_per, int32_t* items,
                                     int32_t* n_items, hipStream_t s) {
  MOE_LAUNCH(k_items_from_offsets, dim3(1), dim3(1024), 0, s, offsets, E, items_per, items, n_items);
  return hipGetLastError();
}

// Expert-cache miss list: one block walks the entries in chunks of 1024 in
// ascending r; a block scan of the miss flags gives each miss its position.
__global__ __launch_bounds__(1024) void k_miss_list(const int32_t* __restrict__ ids, int Tk,
                                                    const int32_t* __restrict__ slot_map,
                                                    int32_t* __restrict__ miss_rows, int32_t* __restrict__ n_miss) {
  int base = 0;
  for (int r0 = 0; r0 < Tk; r0 += 1024) {
    const int r = r0 + threadIdx.x;
    const bool miss = r < Tk && slot_map[ids[r]] < 0;
    int total = 0;
    const int pos = block_exclusive_scan_1024(miss ? 1 : 0, &total);
    if (miss) miss_rows[base + pos] = r;
    base += total;
  }
  if (threadIdx.x == 0) *n_miss = base;
}

hipError_t launch_miss_list(const int32_t* ids, int Tk, const int32_t* slot_map, int32_t* miss_rows, int32_t* n_miss,
                            hipStream_t s) {
  MOE_LAUNCH(k_miss_list, dim3(1), dim3(1024), 0, s, ids, Tk, slot_map, miss_rows, n_miss);
  return hipGetLastError();
}

}  // namespace moe
