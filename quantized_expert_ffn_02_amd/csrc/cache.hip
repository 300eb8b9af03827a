// Adaptive expert cache: usage counters, and slot refills from host memory.
//
// The GPU keeps a cache of the most used experts, which adapts as the conversation
// goes on, while every expert stays in pinned system memory ("Strata Runs 125B
// Qwen3.8-Flash-Next on a 12GB Gaming GPU at Up to 94 Tokens/s", section "How a 125B
// model fits in 12 GB"; the aireport.net page: a learned cache of the few thousand
// most used experts).  Here:
//   - moe_expert_usage adds each expert's number of selections to a counter, after
//     halving the old counts decay_shift times (integer, so exact);
//   - moe_cache_plan (cache_plan.cpp, host) picks the moves;
//   - moe_cache_refill unmaps the slots a move overwrites (and the incoming experts)
//     on the compute stream, then copies the incoming experts' weights from host
//     memory into their slots on a copy stream, so the copies overlap later compute;
//   - moe_cache_commit maps the incoming experts on the compute stream once the
//     copies are done.
// Every call on the compute stream sees one slot table: an expert is either mapped
// to a slot whose weights are complete, or unmapped (a miss).
#include <hip/hip_runtime.h>

#include "internal.h"

namespace moe {

struct MoveList {
  static constexpr int kMax = 64;
  int32_t expert[kMax];
  int32_t slot[kMax];
  int32_t n;
};

// counts[e] = (counts[e] >> shift) + #{i : ids[i] == e}, one block, E <= 1024.
__global__ __launch_bounds__(1024) void k_expert_usage(const int32_t* __restrict__ ids, int n, int E,
                                                       uint32_t* __restrict__ counts, int shift) {
  __shared__ uint32_t hist[1024];
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int e = ids[i];
    if ((unsigned)e < (unsigned)E) atomicAdd(&hist[e], 1u);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) counts[e] = (counts[e] >> shift) + hist[e];
}

// row[e] = -1 where row[e] is one of the moves' slots or e is one of the moves' experts.
__global__ __launch_bounds__(256) void k_cache_unmap(int32_t* __restrict__ row, int E, MoveList m) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  const int32_t v = row[e];
  bool hit = false;
  for (int i = 0; i < m.n; ++i) hit |= (v >= 0 && v == m.slot[i]) || e == m.expert[i];
  if (hit) row[e] = -1;
}

__global__ __launch_bounds__(64) void k_cache_map(int32_t* __restrict__ row, MoveList m) {
  const int i = threadIdx.x;
  if (i < m.n) row[m.expert[i]] = m.slot[i];
}

}  // namespace moe

using namespace moe;

namespace {

int check_moves(const int32_t* experts, const int32_t* slots, int32_t n, int32_t E, int32_t n_slots, MoveList* m) {
  if (n < 0 || n > MoveList::kMax) return MOE_EINVAL;
  if (n > 0 && (!experts || !slots)) return MOE_EINVAL;
  for (int i = 0; i < n; ++i) {
    if (experts[i] < 0 || experts[i] >= E || slots[i] < 0 || slots[i] >= n_slots) return MOE_EINVAL;
    for (int j = 0; j < i; ++j)
      if (experts[j] == experts[i] || slots[j] == slots[i]) return MOE_EINVAL;
    m->expert[i] = experts[i];
    m->slot[i] = slots[i];
  }
  m->n = n;
  return MOE_OK;
}

// Bytes per expert of each tensor of a quantized bank (lo/codes, hi, scales; w13 then w2).
void tensor_bytes(const moe_bank_t& b, size_t out[6]) {
  const size_t n13 = (size_t)2 * b.inter * b.hidden, n2 = (size_t)b.hidden * b.inter;
  const bool q3 = b.fmt == MOE_FMT_Q3;
  out[0] = n13 / 4;
  out[1] = q3 ? n13 / 8 : 0;
  out[2] = n13 / 32 * 2;
  out[3] = n2 / 4;
  out[4] = q3 ? n2 / 8 : 0;
  out[5] = n2 / 32 * 2;
}

}  // namespace

extern "C" {

int moe_expert_usage(const int32_t* topk_ids, int32_t n_ids, int32_t E, uint32_t* counts, int32_t decay_shift,
                     void* stream) {
  if (!counts || E < 1 || E > 1024 || n_ids < 0 || decay_shift < 0 || decay_shift > 31) return MOE_EINVAL;
  if (n_ids > 0 && !topk_ids) return MOE_EINVAL;
  hipLaunchKernelGGL(k_expert_usage, dim3(1), dim3(1024), 0, (hipStream_t)stream, topk_ids, (int)n_ids, (int)E,
                     counts, (int)decay_shift);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

int moe_cache_refill(const moe_bank_t* host_bank, const moe_bank_t* slot_pool, int32_t* slot_of, int32_t layer_idx,
                     int32_t n_layers, int32_t E, const int32_t* move_experts, const int32_t* move_slots,
                     int32_t n_moves, void* done_event, void* stream, void* copy_stream) {
  if (!host_bank || !slot_pool || !slot_of || !done_event || E < 1) return MOE_EINVAL;
  if (n_layers < 1 || layer_idx < 0 || layer_idx >= n_layers) return MOE_EINVAL;
  const moe_bank_t& hb = *host_bank;
  const moe_bank_t& pb = *slot_pool;
  if ((hb.fmt != MOE_FMT_Q2 && hb.fmt != MOE_FMT_Q3) || hb.fmt != pb.fmt) return MOE_EUNSUPPORTED;
  if (hb.hidden != pb.hidden || hb.inter != pb.inter || hb.n_experts != E || pb.n_experts < 1) return MOE_EINVAL;
  if (!hb.w13 || !hb.w13_scale || !hb.w2 || !hb.w2_scale || !pb.w13 || !pb.w13_scale || !pb.w2 || !pb.w2_scale)
    return MOE_EINVAL;
  if (hb.fmt == MOE_FMT_Q3 && (!hb.w13_hi || !hb.w2_hi || !pb.w13_hi || !pb.w2_hi)) return MOE_EINVAL;
  MoveList m;
  int rc = check_moves(move_experts, move_slots, n_moves, E, pb.n_experts, &m);
  if (rc) return rc;
  hipStream_t s = (hipStream_t)stream;
  hipStream_t c = copy_stream ? (hipStream_t)copy_stream : s;
  int32_t* row = slot_of + (size_t)layer_idx * E;
  if (m.n > 0) {
    hipLaunchKernelGGL(k_cache_unmap, dim3((E + 255) / 256), dim3(256), 0, s, row, (int)E, m);
    if (hipGetLastError() != hipSuccess) return MOE_EHIP;
    if (c != s) {
      // the copies start once every kernel enqueued before the unmap has finished
      hipEvent_t ev;
      if (hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess) return MOE_EHIP;
      hipError_t e1 = hipEventRecord(ev, s);
      hipError_t e2 = e1 == hipSuccess ? hipStreamWaitEvent(c, ev, 0) : e1;
      (void)hipEventDestroy(ev);
      if (e2 != hipSuccess) return MOE_EHIP;
    }
    size_t bytes[6];
    tensor_bytes(hb, bytes);
    const char* src[6] = {(const char*)hb.w13, (const char*)hb.w13_hi, (const char*)hb.w13_scale,
                          (const char*)hb.w2, (const char*)hb.w2_hi, (const char*)hb.w2_scale};
    char* dst[6] = {(char*)pb.w13, (char*)pb.w13_hi, (char*)pb.w13_scale,
                    (char*)pb.w2, (char*)pb.w2_hi, (char*)pb.w2_scale};
    for (int i = 0; i < m.n; ++i)
      for (int t = 0; t < 6; ++t) {
        if (!bytes[t]) continue;
        if (hipMemcpyAsync(dst[t] + (size_t)m.slot[i] * bytes[t], src[t] + (size_t)m.expert[i] * bytes[t], bytes[t],
                           hipMemcpyHostToDevice, c) != hipSuccess)
          return MOE_EHIP;
      }
  }
  return hipEventRecord((hipEvent_t)done_event, c) == hipSuccess ? MOE_OK : MOE_EHIP;
}

int moe_cache_commit(int32_t* slot_of, int32_t layer_idx, int32_t n_layers, int32_t E, int32_t n_slots,
                     const int32_t* move_experts, const int32_t* move_slots, int32_t n_moves, void* done_event,
                     void* stream) {
  if (!slot_of || E < 1 || n_slots < 1) return MOE_EINVAL;
  if (n_layers < 1 || layer_idx < 0 || layer_idx >= n_layers) return MOE_EINVAL;
  MoveList m;
  int rc = check_moves(move_experts, move_slots, n_moves, E, n_slots, &m);
  if (rc) return rc;
  hipStream_t s = (hipStream_t)stream;
  if (done_event && hipStreamWaitEvent(s, (hipEvent_t)done_event, 0) != hipSuccess) return MOE_EHIP;
  if (m.n == 0) return MOE_OK;
  hipLaunchKernelGGL(k_cache_map, dim3(1), dim3(64), 0, s, slot_of + (size_t)layer_idx * E, m);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

}  // extern "C"
