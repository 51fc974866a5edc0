// Allocation-free varlen attention: the same kernels as the cached-plan entry
// point, with the tile plan (the attention's work queue) in a file-scope
// device array instead of a hipMalloc'd buffer, for callers that cannot
// allocate device memory (graph-captured code, tight serving loops, harnesses
// that forbid it).
//
// The plan is not uploaded: a small kernel on the caller's stream expands a
// per-segment table passed by value into the array.  Work items are the same
// (segment, head, query tile) items as the cached plan's, segments longest
// first, consecutive items dealt in chunks of 16 to the XCDs round-robin
// (workgroup b runs on XCD b % n_xcd); there is no per-XCD load balancing.
// Each output row depends only on its own item, so the output is bitwise the
// cached-plan entry point's.
//
// Every call on one device shares that device's array.  A per-device event,
// recorded after each attention launch that read the array and waited on by
// the next call's plan kernel, orders the calls on the GPU even when they come
// on different streams, so a later call never rewrites a plan an earlier
// kernel is still reading; host threads take a per-device lock around the
// wait, the two launches and the record.
#include <mutex>
#include <unordered_map>

#include "common.h"

namespace h3a {

// The plan storage: kNoAllocMaxItems work items (2 MiB) per GPU, held until
// the process ends.  In host code `scratch` is only a symbol; its device
// address comes from hipGetSymbolAddress.
static __device__ __align__(256) WorkItem scratch[kNoAllocMaxItems];

namespace {

constexpr int kPlanThreads = 256;
constexpr int kChunk = 16;  // consecutive items of one XCD

// Entry b of the padded plan: position p = b / n_xcd in XCD b % n_xcd's queue,
// which holds chunks xcd, xcd + n_xcd, ... of the natural item order
// (segment-major, then head, then query tile).
__global__ void __launch_bounds__(kPlanThreads) noalloc_plan_kernel(NoAllocPlanArgs a, WorkItem* __restrict__ out) {
  const int32_t b = int32_t(blockIdx.x) * kPlanThreads + int32_t(threadIdx.x);
  if (b >= a.n_blocks) return;
  const int32_t xcd = b % a.n_xcd, pos = b / a.n_xcd;
  const int64_t i = (int64_t(pos / kChunk) * a.n_xcd + xcd) * kChunk + pos % kChunk;
  WorkItem w{0, 0, 0, 0, 0, 0, 0, 0};
  if (i < a.n_items) {
    int32_t lo = 0, hi = a.nseg - 1;  // last segment whose first item is <= i
    while (lo < hi) {
      const int32_t mid = (lo + hi + 1) / 2;
      if (a.first[mid] <= i) lo = mid;
      else hi = mid - 1;
    }
    const int32_t local = int32_t(i - a.first[lo]);
    const int32_t tiles = (a.len[lo] + a.block_m - 1) / a.block_m;
    w.seg_start = a.start[lo];
    w.seg_len = a.len[lo];
    w.q_start = (local % tiles) * a.block_m;
    w.head = local / tiles;
  }
  out[b] = w;
}

struct DeviceState {
  WorkItem* items = nullptr;  // this device's copy of `scratch`
  hipEvent_t released = nullptr;  // after the last attention launch that read it
  bool used = false;
  std::mutex mu;
};

std::mutex g_states_mu;

DeviceState& state_of(int device) {
  static auto* states = new std::unordered_map<int, DeviceState>();  // intentionally leaked
  std::lock_guard<std::mutex> lock(g_states_mu);
  return (*states)[device];
}

}  // namespace

hipError_t launch_attn_noalloc(const NoAllocPlanArgs& plan, bool bf16, const void* q, const void* k, const void* v,
                               void* o, int32_t D, int64_t sq, int64_t sk, int64_t sv, int64_t so, float scale,
                               int32_t kv_group, bool causal, hipStream_t stream) {
  if (plan.n_blocks <= 0) return hipSuccess;
  if (plan.n_blocks > kNoAllocMaxItems || plan.nseg < 1 || plan.nseg > kNoAllocMaxSegs || plan.n_xcd < 1)
    return hipErrorInvalidValue;
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return e;
  DeviceState& st = state_of(device);
  std::lock_guard<std::mutex> lock(st.mu);
  if (st.items == nullptr) {
    // Set-up, once per device, with that device current: the array's address
    // on this device and the event that orders calls through it.
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&st.released, hipEventDisableTiming)) != hipSuccess) return e;
    st.items = static_cast<WorkItem*>(p);
  }
  if (st.used && (e = hipStreamWaitEvent(stream, st.released, 0)) != hipSuccess) return e;
  const unsigned grid = unsigned((plan.n_blocks + kPlanThreads - 1) / kPlanThreads);
  hipLaunchKernelGGL(noalloc_plan_kernel, dim3(grid), dim3(kPlanThreads), 0, stream, plan, st.items);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  e = bf16 ? launch_attn_fwd_bf16(q, k, v, o, D, sq, sk, sv, so, st.items, plan.n_blocks, scale, kv_group, causal,
                                  stream)
           : launch_attn_fwd_f32(q, k, v, o, D, sq, sk, sv, so, st.items, plan.n_blocks, scale, kv_group, causal,
                                 stream);
  if (e != hipSuccess) return e;
  if ((e = hipEventRecord(st.released, stream)) != hipSuccess) return e;
  st.used = true;
  return hipSuccess;
}

}  // namespace h3a
