// The h3a C ABI: argument validation, error reporting, the attention plan
// cache, and dispatch to the kernel launchers.  Every check runs before any
// HIP call, so invalid requests fail without touching the device.
//
// Error style follows the pages' fail-loudly-by-name rule: a missing tensor
// throws by name rather than reading as zeros and shape disagreements throw
// rather than mis-slice (vllm.cpp PR #26, commits on the streamed bf16 stager
// and the condition-noise row accounting); here that becomes a status code
// plus a message naming the argument.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <list>
#include <mutex>
#include <new>
#include <stdexcept>
#include <string>
#include <unordered_map>
#include <vector>

#include "h3a.h"
#include "common.h"

namespace {

thread_local std::string g_last_error;

h3a_status fail(h3a_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  try {
    g_last_error = buf;
  } catch (...) {  // keep the status even if the message cannot be stored
  }
  return st;
}

// Turns the exception being handled into a status: nothing thrown inside the
// library (host allocations of plans, keys and tables) crosses the C ABI.
h3a_status fail_exception(const char* fn) noexcept {
  try {
    throw;
  } catch (const std::bad_alloc&) {
    return fail(H3A_EUNSUPPORTED, "%s: host memory allocation failed", fn);
  } catch (const std::exception& e) {
    return fail(H3A_EUNSUPPORTED, "%s: %s", fn, e.what());
  } catch (...) {
    return fail(H3A_EUNSUPPORTED, "%s: unexpected C++ exception", fn);
  }
}

h3a_status fail_hip(const char* what, hipError_t e) {
  return fail(H3A_EHIP, "%s: HIP error %d (%s)", what, int(e), hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t elem_size(h3a_dtype dt) { return dt == H3A_BF16 ? 2 : 4; }

// Byte range [lo, hi) touched by a [S, H, D] tensor with token stride `stride`.
struct Range {
  uintptr_t lo, hi;
};
Range tensor_range(const void* p, int64_t S, int64_t H, int64_t D, int64_t stride, size_t esz) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  if (S <= 0) return {lo, lo};
  return {lo, lo + uintptr_t(((S - 1) * stride + H * D) * int64_t(esz))};
}

// Whether two token-major tensors, [S, Ha, D] at a and [S, Hb, D] at b, can
// share an element.  Disjoint byte ranges never do.  With equal token
// strides the rows of one tensor sit at a fixed offset from the other's (e.g.
// the q, k, v slices of one fused [S, Hq + 2 Hkv, D] buffer); they are
// disjoint when that offset, taken modulo the stride, puts b's row after a's
// and before a's next one.  Anything else is treated as overlapping.
bool may_overlap(const void* a, int64_t sa, int64_t Ha, const void* b, int64_t sb, int64_t Hb, int64_t S,
                 int64_t D, size_t esz) {
  const Range ra = tensor_range(a, S, Ha, D, sa, esz), rb = tensor_range(b, S, Hb, D, sb, esz);
  if (!(ra.lo < rb.hi && rb.lo < ra.hi)) return false;
  if (sa != sb) return true;
  const int64_t stride_b = sa * int64_t(esz);
  const int64_t row_a = Ha * D * int64_t(esz), row_b = Hb * D * int64_t(esz);
  const int64_t diff = int64_t(reinterpret_cast<uintptr_t>(b) - reinterpret_cast<uintptr_t>(a));
  const int64_t phase = ((diff % stride_b) + stride_b) % stride_b;
  return !(phase >= row_a && phase + row_b <= stride_b);
}

// Validates a token-major [S, H, D] operand.
h3a_status check_operand(const char* name, const void* p, int64_t S, int32_t H, int32_t D,
                         int64_t stride, size_t esz) {
  if (S > 0 && p == nullptr) return fail(H3A_EINVAL, "%s is NULL", name);
  if (stride < int64_t(H) * D)
    return fail(H3A_ESHAPE, "%s: token stride %lld is smaller than H*D = %lld", name,
                (long long)stride, (long long)(int64_t(H) * D));
  if (!aligned(p, 16)) return fail(H3A_EUNSUPPORTED, "%s is not 16-byte aligned", name);
  if ((stride * int64_t(esz)) % 16 != 0)
    return fail(H3A_EUNSUPPORTED, "%s: token stride %lld elements is not a multiple of 16 bytes", name,
                (long long)stride);
  // The attention kernels address up to 64 rows of a tensor with 32-bit
  // buffer offsets.
  if (stride * int64_t(esz) * 64 > int64_t(INT32_MAX))
    return fail(H3A_EUNSUPPORTED, "%s: token stride %lld elements is too large (64 rows must fit in 2 GiB)", name,
                (long long)stride);
  return H3A_OK;
}

// ---------------------------------------------------------------------------
// Attention plan cache: device copies of the tile plan keyed by the
// cu_seqlens content, heads, block size and device.
// ---------------------------------------------------------------------------
struct Plan {
  h3a::WorkItem* dev = nullptr;  // one allocation: the items, then the split variant below
  int64_t n = 0;
  // Split variant (bidirectional plans whose longest items would set the
  // time): items cutting some keys into ranges, the merge list, and the
  // partial-row workspace they share.  Only calls outside stream capture use
  // it; its workspace is reused by every such call, so each call waits for
  // the previous one's merge (event `released`) before writing it.
  h3a::WorkItem* sdev = nullptr;
  int64_t sn = 0;
  h3a::MergeItem* merges = nullptr;
  int64_t n_merges = 0;
  h3a::SplitArgs sp{};
  hipEvent_t released = nullptr;
  bool used = false;
  int device = 0;       // where dev lives
  bool pinned = false;  // used under stream capture: a graph may hold dev, never evict it
};

// What one call uses: the cached plan (valid while the cache lock is held)
// and whether the call's stream is capturing.
struct PlanUse {
  Plan* plan = nullptr;
  bool capturing = false;
};

constexpr size_t kMaxPlans = 256;

// Largest plan built: 2^26 items (2 GiB of host vector).  Any packing whose
// q, k, v fit in one GPU's memory needs far fewer (S * H / 128 items; under
// 2^23 for 288 GB), so larger requests are malformed and are rejected before
// anything is allocated.
constexpr int64_t kMaxPlanItems = int64_t(1) << 26;

// Whether the plan for cu_seqlens fits kMaxPlanItems (counted without building it).
bool plan_fits(const int32_t* cu, int32_t nseg, int32_t H, int32_t block_m) {
  int64_t tiles = 0;  // at most S + nseg < 2^33
  for (int32_t s = 0; s < nseg; ++s) tiles += (int64_t(cu[s + 1]) - cu[s] + block_m - 1) / block_m;
  return tiles <= kMaxPlanItems / H;
}

struct PlanCache {
  std::mutex mu;
  std::unordered_map<std::string, Plan> map;
  std::list<std::string> order;  // insertion order, oldest first
};

PlanCache& plan_cache() {
  static PlanCache* c = new PlanCache();  // intentionally leaked: usable during exit
  return *c;
}

// Split policy for plans built from now on (h3a_set_split_policy).
std::atomic<int32_t> g_split_policy{h3a::kSplitAuto};

struct DeviceShape {
  int cus = 0;
  int n_xcd = 1;
};

DeviceShape shape_of(int device) {
  static std::mutex mu;
  static std::unordered_map<int, DeviceShape> known;
  std::lock_guard<std::mutex> lock(mu);
  auto it = known.find(device);
  if (it != known.end()) return it->second;
  DeviceShape d;
  // MI355X: 8 XCDs of 32 CUs; the dispatcher deals workgroups round-robin.
  if (hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) d.cus = 0;
  if (d.cus >= 64 && d.cus % 32 == 0) d.n_xcd = d.cus / 32;
  known[device] = d;
  return d;
}

void free_plan(Plan& p) {
  if (p.dev != nullptr) (void)hipFree(p.dev);
  if (p.released != nullptr) (void)hipEventDestroy(p.released);
  p.dev = nullptr;
  p.released = nullptr;
}

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// On success `*hold` owns the cache lock: the caller launches the kernels that
// read the plan before releasing it, so no other thread can evict (free) the
// plan between this lookup and that launch.  An eviction synchronises the
// device first, so launches already made have finished with the plan.
// A call on a capturing stream only looks the plan up: building one allocates,
// copies synchronously and may synchronise the device for an eviction, none of
// which a capture allows.  The plan it uses is pinned, since the captured
// graph keeps its device pointer for every later replay: pinned plans are
// never evicted, only h3a_release_caches frees them.  split_ok: the caller's
// kernels handle split items (the bf16-tile kernels; not the fp32 one).
h3a_status get_plan(const int32_t* cu, int32_t nseg, int32_t H, int32_t block_m, bool causal, bool split_ok,
                    hipStream_t stream, PlanUse* out, std::unique_lock<std::mutex>* hold) {
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return fail_hip("hipGetDevice", e);
  hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
  if ((e = hipStreamIsCapturing(stream, &capture)) != hipSuccess) return fail_hip("hipStreamIsCapturing", e);
  const bool capturing = capture != hipStreamCaptureStatusNone;
  const DeviceShape shape = shape_of(device);
  const int32_t policy = split_ok && !causal ? g_split_policy.load() : h3a::kSplitNever;
  std::string key;
  key.reserve(24 + size_t(nseg + 1) * 4);
  const int32_t hdr[6] = {device, H, block_m, shape.n_xcd, causal ? 1 : 0, policy};
  key.append(reinterpret_cast<const char*>(hdr), sizeof(hdr));
  key.append(reinterpret_cast<const char*>(cu), size_t(nseg + 1) * sizeof(int32_t));

  PlanCache& pc = plan_cache();
  std::unique_lock<std::mutex> lock(pc.mu);
  auto it = pc.map.find(key);
  if (it != pc.map.end()) {
    if (capturing) it->second.pinned = true;
    out->plan = &it->second;
    out->capturing = capturing;
    *hold = std::move(lock);
    return H3A_OK;
  }
  if (capturing)
    return fail(H3A_EUNSUPPORTED,
                "stream is capturing and the tile plan for this cu_seqlens / head count / device is not cached: "
                "make one attention call with it outside capture first");
  if (!plan_fits(cu, nseg, H, block_m))
    return fail(H3A_EUNSUPPORTED, "attention plan would exceed %lld work items", (long long)kMaxPlanItems);
  std::vector<h3a::WorkItem> items = h3a::plan_tiles(cu, nseg, H, block_m, shape.n_xcd, causal);
  std::vector<h3a::WorkItem> sitems;
  std::vector<h3a::MergeItem> merges;
  int64_t n_parts = 0;
  if (policy != h3a::kSplitNever && shape.cus > 0) {
    sitems = h3a::plan_tiles_split(cu, nseg, H, block_m, shape.n_xcd, 2 * shape.cus, causal, policy, &merges,
                                   &n_parts);
    if (merges.empty()) sitems.clear();
  }
  Plan p;
  p.n = int64_t(items.size());
  p.device = device;
  if (p.n > 0) {
    if (p.n > int64_t(INT32_MAX) || int64_t(sitems.size()) > int64_t(INT32_MAX))
      return fail(H3A_EUNSUPPORTED, "attention plan has %lld items", (long long)p.n);
    // Evict the oldest plan no captured graph uses (if every cached plan is
    // pinned, the cache grows instead).
    auto old = pc.order.begin();
    while (old != pc.order.end() && pc.map.at(*old).pinned) ++old;
    if (pc.map.size() >= kMaxPlans && old != pc.order.end()) {
      // Evicting frees device memory an earlier launch may still read: wait
      // for the device the victim lives on (not necessarily the current one).
      auto victim = pc.map.find(*old);
      if (victim != pc.map.end()) {
        if (victim->second.dev != nullptr) {
          const int vdev = victim->second.device;
          if (vdev != device && (e = hipSetDevice(vdev)) != hipSuccess)
            return fail_hip("hipSetDevice (plan eviction)", e);
          e = hipDeviceSynchronize();
          if (e == hipSuccess) free_plan(victim->second);
          const hipError_t back = vdev != device ? hipSetDevice(device) : hipSuccess;
          if (e != hipSuccess) return fail_hip("hipDeviceSynchronize (plan eviction)", e);
          if (back != hipSuccess) return fail_hip("hipSetDevice (plan eviction)", back);
        }
        pc.map.erase(victim);
      }
      pc.order.erase(old);
    }
    // [items | split items | merges | per-row (max, sum) | partial rows (D <= 128)]
    const size_t o_items = 0, b_items = round256(items.size() * sizeof(h3a::WorkItem));
    const size_t o_sitems = o_items + b_items, b_sitems = round256(sitems.size() * sizeof(h3a::WorkItem));
    const size_t o_merges = o_sitems + b_sitems, b_merges = round256(merges.size() * sizeof(h3a::MergeItem));
    const size_t rows = size_t(n_parts) * size_t(block_m);
    const size_t o_ml = o_merges + b_merges, b_ml = round256(rows * 2 * sizeof(float));
    const size_t o_po = o_ml + b_ml, b_po = round256(rows * 128 * sizeof(float));
    char* base = nullptr;
    e = hipMalloc(reinterpret_cast<void**>(&base), o_po + b_po);
    if (e != hipSuccess) return fail_hip("hipMalloc (attention plan)", e);
    p.dev = reinterpret_cast<h3a::WorkItem*>(base + o_items);
    // Synchronous uploads: the plan is complete before any stream can use it.
    e = hipMemcpy(p.dev, items.data(), items.size() * sizeof(h3a::WorkItem), hipMemcpyHostToDevice);
    if (e == hipSuccess && !sitems.empty()) {
      p.sdev = reinterpret_cast<h3a::WorkItem*>(base + o_sitems);
      p.sn = int64_t(sitems.size());
      p.merges = reinterpret_cast<h3a::MergeItem*>(base + o_merges);
      p.n_merges = int64_t(merges.size());
      p.sp = h3a::SplitArgs{reinterpret_cast<float*>(base + o_po), reinterpret_cast<float*>(base + o_ml)};
      e = hipMemcpy(p.sdev, sitems.data(), sitems.size() * sizeof(h3a::WorkItem), hipMemcpyHostToDevice);
      if (e == hipSuccess)
        e = hipMemcpy(p.merges, merges.data(), merges.size() * sizeof(h3a::MergeItem), hipMemcpyHostToDevice);
      if (e == hipSuccess) e = hipEventCreateWithFlags(&p.released, hipEventDisableTiming);
    }
    if (e != hipSuccess) {
      free_plan(p);
      return fail_hip("hipMemcpy / hipEventCreate (attention plan)", e);
    }
  }
  auto ins = pc.map.emplace(key, p);
  pc.order.push_back(key);
  out->plan = &ins.first->second;
  out->capturing = false;
  *hold = std::move(lock);
  return H3A_OK;
}

// Launches the attention over a plan: the split variant (then the merge pass)
// outside capture when the plan has one, else the plain items.  launch(items,
// n, sp) enqueues the attention kernel.  Called with the cache lock held.
template <typename F>
h3a_status run_plan(const PlanUse& u, hipStream_t stream, void* o, int32_t D, int64_t stride_o, const char* what,
                    F&& launch) {
  Plan& p = *u.plan;
  hipError_t e;
  if (p.n_merges == 0 || u.capturing) {
    if ((e = launch(p.dev, p.n, h3a::SplitArgs{})) != hipSuccess) return fail_hip(what, e);
    return H3A_OK;
  }
  // the previous split call's merge must have read the workspace
  if (p.used && (e = hipStreamWaitEvent(stream, p.released, 0)) != hipSuccess)
    return fail_hip("hipStreamWaitEvent (split workspace)", e);
  if ((e = launch(p.sdev, p.sn, p.sp)) != hipSuccess) return fail_hip(what, e);
  if ((e = h3a::launch_attn_merge(p.merges, p.n_merges, p.sp, o, D, stride_o, stream)) != hipSuccess)
    return fail_hip("split merge launch", e);
  if ((e = hipEventRecord(p.released, stream)) != hipSuccess) return fail_hip("hipEventRecord (split workspace)", e);
  p.used = true;
  return H3A_OK;
}

h3a_status check_cu_seqlens(const int32_t* cu, int32_t nseg, int64_t S) {
  if (cu == nullptr) return fail(H3A_EINVAL, "cu_seqlens is NULL");
  if (nseg < 1) return fail(H3A_EINVAL, "nseg = %d must be >= 1", nseg);
  if (cu[0] != 0) return fail(H3A_EINVAL, "cu_seqlens[0] = %d must be 0", cu[0]);
  for (int32_t s = 0; s < nseg; ++s)
    if (cu[s + 1] < cu[s])
      return fail(H3A_EINVAL, "cu_seqlens decreases at index %d (%d -> %d)", s + 1, cu[s], cu[s + 1]);
  if (int64_t(cu[nseg]) != S)
    return fail(H3A_ESHAPE, "cu_seqlens[nseg] = %d but S = %lld", cu[nseg], (long long)S);
  return H3A_OK;
}

// A packed array of E8M0 block scales: `bytes` long, aligned to `align`
// (the kernels read D / 32 scales of a row as one word).
h3a_status check_scales(const char* name, const void* p, int64_t bytes, int64_t align) {
  if (bytes == 0) return H3A_OK;
  if (p == nullptr) return fail(H3A_EINVAL, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(p) % uintptr_t(align) != 0)
    return fail(H3A_EUNSUPPORTED, "%s is not %lld-byte aligned", name, (long long)align);
  return H3A_OK;
}

Range byte_range(const void* p, int64_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + uintptr_t(bytes)};
}

bool ranges_hit(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi; }

// Argument checks shared by h3a_varlen_attn_fwd_ex and its allocation-free
// variant: every error they report, before anything is launched.
h3a_status check_attn_ex(const void* q, const void* k, const void* v, const void* o, h3a_dtype dtype, int64_t S,
                         int32_t Hq, int32_t Hkv, int32_t D, int64_t stride_q, int64_t stride_k, int64_t stride_v,
                         int64_t stride_o, const int32_t* cu_seqlens, int32_t nseg, float scale, int32_t causal) {
  if (dtype != H3A_F32 && dtype != H3A_BF16) return fail(H3A_EDTYPE, "unknown dtype %d", int(dtype));
  if (S < 0) return fail(H3A_EINVAL, "S = %lld must be >= 0", (long long)S);
  if (S > int64_t(INT32_MAX)) return fail(H3A_EUNSUPPORTED, "S = %lld exceeds INT32_MAX", (long long)S);
  if (Hq < 1) return fail(H3A_EINVAL, "H = %d must be >= 1", Hq);
  if (Hkv < 1) return fail(H3A_EINVAL, "Hkv = %d must be >= 1", Hkv);
  if (Hq % Hkv != 0) return fail(H3A_ESHAPE, "Hkv = %d does not divide H = %d", Hkv, Hq);
  if (causal != 0 && causal != 1) return fail(H3A_EINVAL, "causal = %d must be 0 or 1", causal);
  if (D != 64 && D != 128) return fail(H3A_EUNSUPPORTED, "head_dim %d (supported: 64, 128)", D);
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(H3A_EINVAL, "scale = %g must be finite and > 0", double(scale));
  h3a_status st;
  if ((st = check_cu_seqlens(cu_seqlens, nseg, S)) != H3A_OK) return st;
  const size_t esz = elem_size(dtype);
  if ((st = check_operand("q", q, S, Hq, D, stride_q, esz)) != H3A_OK) return st;
  if ((st = check_operand("k", k, S, Hkv, D, stride_k, esz)) != H3A_OK) return st;
  if ((st = check_operand("v", v, S, Hkv, D, stride_v, esz)) != H3A_OK) return st;
  if ((st = check_operand("o", o, S, Hq, D, stride_o, esz)) != H3A_OK) return st;
  if (S == 0) return H3A_OK;
  auto overlaps = [&](const void* x, int64_t sx, int32_t h) {
    return may_overlap(o, stride_o, Hq, x, sx, h, S, D, esz);
  };
  if (overlaps(q, stride_q, Hq)) return fail(H3A_EINVAL, "o overlaps q");
  if (overlaps(k, stride_k, Hkv)) return fail(H3A_EINVAL, "o overlaps k");
  if (overlaps(v, stride_v, Hkv)) return fail(H3A_EINVAL, "o overlaps v");
  return H3A_OK;
}

}  // namespace

extern "C" {

const char* h3a_last_error(void) { return g_last_error.c_str(); }

int32_t h3a_version(void) { return 200; }

h3a_status h3a_set_split_policy(int32_t policy) {
  try {
    if (policy != H3A_SPLIT_AUTO && policy != H3A_SPLIT_NEVER && policy != H3A_SPLIT_ALWAYS)
      return fail(H3A_EINVAL, "unknown split policy %d", policy);
    static_assert(int(H3A_SPLIT_AUTO) == h3a::kSplitAuto && int(H3A_SPLIT_NEVER) == h3a::kSplitNever &&
                      int(H3A_SPLIT_ALWAYS) == h3a::kSplitAlways,
                  "split policy values");
    g_split_policy.store(policy);
    return H3A_OK;
  } catch (...) {
    return fail_exception("h3a_set_split_policy");
  }
}

void h3a_release_caches(void) {
  try {
    PlanCache& pc = plan_cache();
    std::lock_guard<std::mutex> lock(pc.mu);
    // Wait for every device that holds a plan (kernels enqueued earlier may
    // still read it), then free them all.
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return;
    std::vector<int> devices;
    for (auto& kv : pc.map)
      if (kv.second.dev && std::find(devices.begin(), devices.end(), kv.second.device) == devices.end())
        devices.push_back(kv.second.device);
    for (int d : devices) {
      // a device that cannot be reached or is in error: keep the plans rather
      // than free memory a kernel may still use
      if ((d != cur && hipSetDevice(d) != hipSuccess) || hipDeviceSynchronize() != hipSuccess) {
        (void)hipSetDevice(cur);
        return;
      }
    }
    (void)hipSetDevice(cur);
    for (auto& kv : pc.map) free_plan(kv.second);
    pc.map.clear();
    pc.order.clear();
  } catch (...) {  // nothing may cross the C ABI; the cache is left as it was
  }
}

h3a_status h3a_build_rope_table_ex(const int32_t* segments, int32_t nseg, const h3a_rope_spec* spec,
                                   float* cos_sin, int64_t S, int32_t* cu_seqlens_out,
                                   hipStream_t stream) {
  try {
    if (segments == nullptr) return fail(H3A_EINVAL, "segments is NULL");
    if (nseg < 1) return fail(H3A_EINVAL, "nseg = %d must be >= 1", nseg);
    if (spec == nullptr) return fail(H3A_EINVAL, "spec is NULL");
    const int32_t mode = spec->mode;
    if (mode < H3A_ROPE_GRID || mode > H3A_ROPE_INTERLEAVED) return fail(H3A_EINVAL, "unknown rotary table mode %d", mode);
    const int32_t* axis_dims = spec->axis_dims;
    int64_t R = 0;
    for (int a = 0; a < 3; ++a) {
      if (axis_dims[a] < 0 || axis_dims[a] % 2 != 0)
        return fail(H3A_EINVAL, "axis_dims[%d] = %d must be even and >= 0", a, axis_dims[a]);
      R += axis_dims[a];
    }
    if (R > 128) return fail(H3A_EUNSUPPORTED, "rotated dims %lld > 128", (long long)R);
    const double base = spec->base;
    if (!(base > 0.0) || !std::isfinite(base)) return fail(H3A_EINVAL, "base = %g must be finite and > 0", base);
    if (mode == H3A_ROPE_LINSPACE)
      for (int a = 0; a < 3; ++a)
        if (!std::isfinite(spec->start[a]) || !std::isfinite(spec->stop[a]))
          return fail(H3A_EINVAL, "linspace start/stop of axis %d must be finite", a);
    int64_t total = 0;
    for (int32_t s = 0; s < nseg; ++s) {
      const int32_t* g = segments + 4 * int64_t(s);
      if (g[0] < 1 || g[1] < 1 || g[2] < 1)
        return fail(H3A_EINVAL, "segment %d grid (%d, %d, %d) must be >= 1 on every axis", s, g[0], g[1], g[2]);
      const int64_t cap = int64_t(g[0]) * g[1] * g[2];
      if (cap > int64_t(INT32_MAX))
        return fail(H3A_EINVAL, "segment %d grid %d x %d x %d exceeds INT32_MAX tokens", s, g[0], g[1], g[2]);
      if (g[3] < 0) return fail(H3A_EINVAL, "segment %d length %d is negative", s, g[3]);
      if (mode != H3A_ROPE_NORMALIZED && int64_t(g[3]) > cap)
        return fail(H3A_EINVAL, "segment %d length %d outside [0, T*H*W = %lld]", s, g[3], (long long)cap);
      total += g[3];
    }
    if (total != S) return fail(H3A_ESHAPE, "S = %lld but the segment lengths sum to %lld", (long long)S, (long long)total);
    if (S > int64_t(INT32_MAX)) return fail(H3A_EUNSUPPORTED, "S = %lld exceeds INT32_MAX", (long long)S);
    if (R > 0 && S > 0) {
      if (cos_sin == nullptr) return fail(H3A_EINVAL, "cos_sin is NULL");
      if (!aligned(cos_sin, 16)) return fail(H3A_EUNSUPPORTED, "cos_sin is not 16-byte aligned");
    }

    std::vector<int32_t> starts(size_t(nseg) + 1, 0);
    for (int32_t s = 0; s < nseg; ++s) starts[s + 1] = starts[s] + segments[4 * int64_t(s) + 3];
    const int32_t half = int32_t(R / 2);
    std::vector<double> inv_freq;
    std::vector<int32_t> axis_of;
    if (mode == H3A_ROPE_INTERLEAVED) {
      // One ladder base^(-2j/R); angle j takes h while j % 3 == 1 and the h
      // share lasts, w likewise for j % 3 == 2, t otherwise.
      const int32_t n_h = axis_dims[1] / 2, n_w = axis_dims[2] / 2;
      int32_t count[3] = {0, 0, 0};
      for (int32_t j = 0; j < half; ++j) {
        const int32_t a = (j % 3 == 1 && j < 3 * n_h) ? 1 : ((j % 3 == 2 && j < 3 * n_w) ? 2 : 0);
        axis_of.push_back(a);
        ++count[a];
        inv_freq.push_back(std::pow(base, -2.0 * double(j) / double(R)));
      }
      for (int a = 0; a < 3; ++a)
        if (count[a] != axis_dims[a] / 2)
          return fail(H3A_EINVAL, "axis_dims (%d, %d, %d) cannot be interleaved t, h, w", axis_dims[0],
                      axis_dims[1], axis_dims[2]);
    } else {
      for (int a = 0; a < 3; ++a)
        for (int32_t j = 0; j < axis_dims[a] / 2; ++j) {
          inv_freq.push_back(std::pow(base, -2.0 * double(j) / double(axis_dims[a])));
          axis_of.push_back(a);
        }
    }
    if (half > 0 && S > 0) {
      h3a::RopeTableSpec ts{};
      ts.mode = mode;
      ts.half = half;
      ts.inv_freq = inv_freq.data();
      ts.axis_of = axis_of.data();
      for (int a = 0; a < 3; ++a) {
        ts.lin_start[a] = mode == H3A_ROPE_LINSPACE ? spec->start[a] : 0.0;
        ts.lin_stop[a] = mode == H3A_ROPE_LINSPACE ? spec->stop[a] : 0.0;
      }
      hipError_t e = h3a::launch_rope_table(ts, segments, starts.data(), nseg, cos_sin, S, stream);
      if (e != hipSuccess) return fail_hip("rope table launch", e);
    }
    if (cu_seqlens_out != nullptr) std::memcpy(cu_seqlens_out, starts.data(), starts.size() * sizeof(int32_t));
    return H3A_OK;
  } catch (...) {
    return fail_exception("h3a_build_rope_table_ex");
  }
}

h3a_status h3a_build_rope_table(const int32_t* segments, int32_t nseg, const int32_t* axis_dims,
                                double base, float* cos_sin, int64_t S, int32_t* cu_seqlens_out,
                                hipStream_t stream) {
  try {
    if (axis_dims == nullptr) return fail(H3A_EINVAL, "axis_dims is NULL");
    h3a_rope_spec spec{};
    spec.mode = H3A_ROPE_GRID;
    for (int a = 0; a < 3; ++a) spec.axis_dims[a] = axis_dims[a];
    spec.base = base;
    return h3a_build_rope_table_ex(segments, nseg, &spec, cos_sin, S, cu_seqlens_out, stream);
  } catch (...) {
    return fail_exception("h3a_build_rope_table");
  }
}

h3a_status h3a_qk_rmsnorm_rope_ex(const void* q, const void* k, void* q_out, void* k_out,
                                  h3a_dtype dtype, int64_t S, int32_t Hq, int32_t Hk, int32_t D,
                                  int64_t stride_q, int64_t stride_k, int64_t stride_qo,
                                  int64_t stride_ko, const float* gamma_q, const float* gamma_k,
                                  float eps, const float* cos_sin, int32_t rot_dim,
                                  hipStream_t stream) {
  try {
    if (dtype != H3A_F32 && dtype != H3A_BF16) return fail(H3A_EDTYPE, "unknown dtype %d", int(dtype));
    if (S < 0) return fail(H3A_EINVAL, "S = %lld must be >= 0", (long long)S);
    if (S > int64_t(INT32_MAX)) return fail(H3A_EUNSUPPORTED, "S = %lld exceeds INT32_MAX", (long long)S);
    if (Hq < 1) return fail(H3A_EINVAL, "H = %d must be >= 1", Hq);
    if (Hk < 1) return fail(H3A_EINVAL, "Hk = %d must be >= 1", Hk);
    if (D != 64 && D != 128) return fail(H3A_EUNSUPPORTED, "head_dim %d (supported: 64, 128)", D);
    const int V = dtype == H3A_BF16 ? 8 : 4;
    if (rot_dim < 0 || rot_dim > D || rot_dim % 2 != 0)
      return fail(H3A_EINVAL, "rot_dim = %d must be even and in [0, D = %d]", rot_dim, D);
    if ((rot_dim / 2) % V != 0)
      return fail(H3A_EUNSUPPORTED, "rot_dim / 2 = %d must be a multiple of %d for this dtype", rot_dim / 2, V);
    if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(H3A_EINVAL, "eps = %g must be finite and >= 0", double(eps));
    const size_t esz = elem_size(dtype);
    h3a_status st;
    if ((st = check_operand("q", q, S, Hq, D, stride_q, esz)) != H3A_OK) return st;
    if ((st = check_operand("k", k, S, Hk, D, stride_k, esz)) != H3A_OK) return st;
    if ((st = check_operand("q_out", q_out, S, Hq, D, stride_qo, esz)) != H3A_OK) return st;
    if ((st = check_operand("k_out", k_out, S, Hk, D, stride_ko, esz)) != H3A_OK) return st;
    if (gamma_q == nullptr) return fail(H3A_EINVAL, "gamma_q is NULL");
    if (gamma_k == nullptr) return fail(H3A_EINVAL, "gamma_k is NULL");
    if (!aligned(gamma_q, 4) || !aligned(gamma_k, 4)) return fail(H3A_EUNSUPPORTED, "gamma is not 4-byte aligned");
    if (rot_dim > 0 && S > 0) {
      if (cos_sin == nullptr) return fail(H3A_EINVAL, "cos_sin is NULL with rot_dim = %d", rot_dim);
      if (!aligned(cos_sin, 16)) return fail(H3A_EUNSUPPORTED, "cos_sin is not 16-byte aligned");
    }
    if (S == 0) return H3A_OK;
    const bool q_inplace = q_out == q && stride_qo == stride_q;
    const bool k_inplace = k_out == k && stride_ko == stride_k;
    if (!q_inplace && may_overlap(q_out, stride_qo, Hq, q, stride_q, Hq, S, D, esz))
      return fail(H3A_EINVAL, "q_out overlaps q without being q itself");
    if (!k_inplace && may_overlap(k_out, stride_ko, Hk, k, stride_k, Hk, S, D, esz))
      return fail(H3A_EINVAL, "k_out overlaps k without being k itself");
    if (may_overlap(q_out, stride_qo, Hq, k, stride_k, Hk, S, D, esz)) return fail(H3A_EINVAL, "q_out overlaps k");
    if (may_overlap(k_out, stride_ko, Hk, q, stride_q, Hq, S, D, esz)) return fail(H3A_EINVAL, "k_out overlaps q");
    if (may_overlap(q_out, stride_qo, Hq, k_out, stride_ko, Hk, S, D, esz)) return fail(H3A_EINVAL, "q_out overlaps k_out");

    hipError_t e = h3a::launch_qk_rmsnorm_rope(dtype == H3A_BF16, q, k, q_out, k_out, S, Hq, Hk, D, stride_q,
                                               stride_k, stride_qo, stride_ko, gamma_q, gamma_k, eps, cos_sin,
                                               rot_dim, stream);
    if (e != hipSuccess) return fail_hip("qk_rmsnorm_rope launch", e);
    return H3A_OK;
  } catch (...) {
    return fail_exception("h3a_qk_rmsnorm_rope_ex");
  }
}

h3a_status h3a_rmsnorm_rope(const void* x, void* x_out, h3a_dtype dtype, int64_t S, int32_t H, int32_t D,
                            int64_t stride_x, int64_t stride_xo, const float* gamma, float eps,
                            const float* cos_sin, int32_t rot_dim, hipStream_t stream) {
  try {
    if (dtype != H3A_F32 && dtype != H3A_BF16) return fail(H3A_EDTYPE, "unknown dtype %d", int(dtype));
    if (S < 0) return fail(H3A_EINVAL, "S = %lld must be >= 0", (long long)S);
    if (S > int64_t(INT32_MAX)) return fail(H3A_EUNSUPPORTED, "S = %lld exceeds INT32_MAX", (long long)S);
    if (H < 1) return fail(H3A_EINVAL, "H = %d must be >= 1", H);
    if (D != 64 && D != 128) return fail(H3A_EUNSUPPORTED, "head_dim %d (supported: 64, 128)", D);
    const int V = dtype == H3A_BF16 ? 8 : 4;
    if (rot_dim < 0 || rot_dim > D || rot_dim % 2 != 0)
      return fail(H3A_EINVAL, "rot_dim = %d must be even and in [0, D = %d]", rot_dim, D);
    if ((rot_dim / 2) % V != 0)
      return fail(H3A_EUNSUPPORTED, "rot_dim / 2 = %d must be a multiple of %d for this dtype", rot_dim / 2, V);
    if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(H3A_EINVAL, "eps = %g must be finite and >= 0", double(eps));
    const size_t esz = elem_size(dtype);
    h3a_status st;
    if ((st = check_operand("x", x, S, H, D, stride_x, esz)) != H3A_OK) return st;
    if ((st = check_operand("x_out", x_out, S, H, D, stride_xo, esz)) != H3A_OK) return st;
    if (gamma == nullptr) return fail(H3A_EINVAL, "gamma is NULL");
    if (!aligned(gamma, 4)) return fail(H3A_EUNSUPPORTED, "gamma is not 4-byte aligned");
    if (rot_dim > 0 && S > 0) {
      if (cos_sin == nullptr) return fail(H3A_EINVAL, "cos_sin is NULL with rot_dim = %d", rot_dim);
      if (!aligned(cos_sin, 16)) return fail(H3A_EUNSUPPORTED, "cos_sin is not 16-byte aligned");
    }
    if (S == 0) return H3A_OK;
    const bool inplace = x_out == x && stride_xo == stride_x;
    if (!inplace && may_overlap(x_out, stride_xo, H, x, stride_x, H, S, D, esz))
      return fail(H3A_EINVAL, "x_out overlaps x without being x itself");
    // The fused kernel with no q heads: only its k pass runs.
    hipError_t e = h3a::launch_qk_rmsnorm_rope(dtype == H3A_BF16, x, x, x_out, x_out, S, 0, H, D, stride_x,
                                               stride_x, stride_xo, stride_xo, gamma, gamma, eps, cos_sin, rot_dim,
                                               stream);
    if (e != hipSuccess) return fail_hip("rmsnorm_rope launch", e);
    return H3A_OK;
  } catch (...) {
    return fail_exception("h3a_rmsnorm_rope");
  }
}

h3a_status h3a_qk_rmsnorm_rope(const void* q, const void* k, void* q_out, void* k_out,
                               h3a_dtype dtype, int64_t S, int32_t H, int32_t D,
                               int64_t stride_q, int64_t stride_k, int64_t stride_qo,
                               int64_t stride_ko, const float* gamma_q, const float* gamma_k,
                               float eps, const float* cos_sin, int32_t rot_dim,
                               hipStream_t stream) {
  try {
    return h3a_qk_rmsnorm_rope_ex(q, k, q_out, k_out, dtype, S, H, H, D, stride_q, stride_k, stride_qo, stride_ko,
                                  gamma_q, gamma_k, eps, cos_sin, rot_dim, stream);
  } catch (...) {
    return fail_exception("h3a_qk_rmsnorm_rope");
  }
}

h3a_status h3a_varlen_attn_fwd_ex(const void* q, const void* k, const void* v, void* o,
                                  h3a_dtype dtype, int64_t S, int32_t Hq, int32_t Hkv, int32_t D,
                                  int64_t stride_q, int64_t stride_k, int64_t stride_v,
                                  int64_t stride_o, const int32_t* cu_seqlens, int32_t nseg,
                                  float scale, int32_t causal, hipStream_t stream) {
  try {
    h3a_status st = check_attn_ex(q, k, v, o, dtype, S, Hq, Hkv, D, stride_q, stride_k, stride_v, stride_o,
                                  cu_seqlens, nseg, scale, causal);
    if (st != H3A_OK || S == 0) return st;
    const bool bf16 = dtype == H3A_BF16;
    PlanUse plan;
    std::unique_lock<std::mutex> plan_lock;  // held until the launches below are enqueued
    if ((st = get_plan(cu_seqlens, nseg, Hq, bf16 ? h3a::kAttnBlockM_BF16 : h3a::kAttnBlockM_F32, causal != 0, bf16,
                       stream, &plan, &plan_lock)) != H3A_OK)
      return st;
    const int32_t group = Hq / Hkv;
    return run_plan(plan, stream, o, D, stride_o, "varlen attention launch",
                    [&](const h3a::WorkItem* items, int64_t n, const h3a::SplitArgs& sp) {
                      return bf16 ? h3a::launch_attn_fwd_bf16(q, k, v, o, D, stride_q, stride_k, stride_v, stride_o,
                                                              items, n, scale, group, causal != 0, stream, sp)
                                  : h3a::launch_attn_fwd_f32(q, k, v, o, D, stride_q, stride_k, stride_v, stride_o,
                                                             items, n, scale, group, causal != 0, stream);
                    });
  } catch (...) {
    return fail_exception("h3a_varlen_attn_fwd_ex");
  }
}

h3a_status h3a_varlen_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o,
                                       h3a_dtype dtype, int64_t S, int32_t Hq, int32_t Hkv, int32_t D,
                                       int64_t stride_q, int64_t stride_k, int64_t stride_v,
                                       int64_t stride_o, const int32_t* cu_seqlens, int32_t nseg,
                                       float scale, int32_t causal, hipStream_t stream) {
  try {
    h3a_status st = check_attn_ex(q, k, v, o, dtype, S, Hq, Hkv, D, stride_q, stride_k, stride_v, stride_o,
                                  cu_seqlens, nseg, scale, causal);
    if (st != H3A_OK || S == 0) return st;
    const bool bf16 = dtype == H3A_BF16;
    // The segment table, in fixed storage: the non-empty segments, longest
    // first (a stable insertion sort over at most kNoAllocMaxSegs entries).
    h3a::NoAllocPlanArgs a{};
    a.block_m = bf16 ? h3a::kAttnBlockM_BF16 : h3a::kAttnBlockM_F32;
    int32_t n = 0;
    for (int32_t s = 0; s < nseg; ++s) {
      const int32_t len = cu_seqlens[s + 1] - cu_seqlens[s];
      if (len == 0) continue;
      if (n == h3a::kNoAllocMaxSegs)
        return fail(H3A_EUNSUPPORTED, "cu_seqlens has more than %d non-empty segments (the allocation-free "
                    "entry point's limit)", h3a::kNoAllocMaxSegs);
      int32_t j = n++;
      for (; j > 0 && a.len[j - 1] < len; --j) {
        a.len[j] = a.len[j - 1];
        a.start[j] = a.start[j - 1];
      }
      a.len[j] = len;
      a.start[j] = cu_seqlens[s];
    }
    a.nseg = n;
    int64_t items = 0;
    for (int32_t i = 0; i < n; ++i) {
      a.first[i] = int32_t(std::min<int64_t>(items, INT32_MAX));
      items += int64_t((a.len[i] + a.block_m - 1) / a.block_m) * Hq;
    }
    if (items > h3a::kNoAllocMaxItems)
      return fail(H3A_EUNSUPPORTED, "the attention needs %lld work items; the allocation-free entry point holds at "
                  "most %d (use h3a_varlen_attn_fwd_ex)", (long long)items, h3a::kNoAllocMaxItems);
    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess) return fail_hip("hipGetDevice", e);
    a.n_xcd = shape_of(device).n_xcd;
    a.n_items = int32_t(items);
    const int64_t chunks = (items + 15) / 16;
    const int64_t blocks = int64_t(a.n_xcd) * 16 * ((chunks + a.n_xcd - 1) / a.n_xcd);
    if (blocks > h3a::kNoAllocMaxItems)
      return fail(H3A_EUNSUPPORTED, "the attention needs %lld work items once padded over %d XCDs; the "
                  "allocation-free entry point holds at most %d (use h3a_varlen_attn_fwd_ex)", (long long)blocks,
                  a.n_xcd, h3a::kNoAllocMaxItems);
    a.n_blocks = int32_t(blocks);
    e = h3a::launch_attn_noalloc(a, bf16, q, k, v, o, D, stride_q, stride_k, stride_v, stride_o, scale, Hq / Hkv,
                                 causal != 0, stream);
    if (e != hipSuccess) return fail_hip("allocation-free varlen attention launch", e);
    return H3A_OK;
  } catch (...) {
    return fail_exception("h3a_varlen_attn_fwd_noalloc");
  }
}

h3a_status h3a_varlen_attn_fwd_qnorm(const void* q, const void* k, const void* v, void* o, h3a_dtype dtype,
                                     int64_t S, int32_t Hq, int32_t Hkv, int32_t D, int64_t stride_q,
                                     int64_t stride_k, int64_t stride_v, int64_t stride_o,
                                     const int32_t* cu_seqlens, int32_t nseg, float scale, const float* gamma_q,
                                     float eps, const float* cos_sin, int32_t rot_dim, hipStream_t stream) {
  try {
    if (dtype != H3A_BF16)
      return dtype == H3A_F32 ? fail(H3A_EUNSUPPORTED, "dtype: the fused Q norm path is bf16 only")
                              : fail(H3A_EDTYPE, "unknown dtype %d", int(dtype));
    if (S < 0) return fail(H3A_EINVAL, "S = %lld must be >= 0", (long long)S);
    if (S > int64_t(INT32_MAX)) return fail(H3A_EUNSUPPORTED, "S = %lld exceeds INT32_MAX", (long long)S);
    if (Hq < 1) return fail(H3A_EINVAL, "H = %d must be >= 1", Hq);
    if (Hkv < 1) return fail(H3A_EINVAL, "Hkv = %d must be >= 1", Hkv);
    if (Hq % Hkv != 0) return fail(H3A_ESHAPE, "Hkv = %d does not divide H = %d", Hkv, Hq);
    if (D != 64 && D != 128) return fail(H3A_EUNSUPPORTED, "head_dim %d (supported: 64, 128)", D);
    if (!(scale > 0.f) || !std::isfinite(scale)) return fail(H3A_EINVAL, "scale = %g must be finite and > 0", double(scale));
    if (rot_dim < 0 || rot_dim > D || rot_dim % 2 != 0)
      return fail(H3A_EINVAL, "rot_dim = %d must be even and in [0, D = %d]", rot_dim, D);
    if (rot_dim % 32 != 0) return fail(H3A_EUNSUPPORTED, "rot_dim = %d must be a multiple of 32 on the fused path", rot_dim);
    if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(H3A_EINVAL, "eps = %g must be finite and >= 0", double(eps));
    if (gamma_q == nullptr) return fail(H3A_EINVAL, "gamma_q is NULL");
    if (!aligned(gamma_q, 16)) return fail(H3A_EUNSUPPORTED, "gamma_q is not 16-byte aligned");
    h3a_status st;
    if ((st = check_cu_seqlens(cu_seqlens, nseg, S)) != H3A_OK) return st;
    const size_t esz = elem_size(dtype);
    if ((st = check_operand("q", q, S, Hq, D, stride_q, esz)) != H3A_OK) return st;
    if ((st = check_operand("k", k, S, Hkv, D, stride_k, esz)) != H3A_OK) return st;
    if ((st = check_operand("v", v, S, Hkv, D, stride_v, esz)) != H3A_OK) return st;
    if ((st = check_operand("o", o, S, Hq, D, stride_o, esz)) != H3A_OK) return st;
    if (rot_dim > 0 && S > 0) {
      if (cos_sin == nullptr) return fail(H3A_EINVAL, "cos_sin is NULL with rot_dim = %d", rot_dim);
      if (!aligned(cos_sin, 16)) return fail(H3A_EUNSUPPORTED, "cos_sin is not 16-byte aligned");
    }
    if (S == 0) return H3A_OK;
    if (may_overlap(o, stride_o, Hq, q, stride_q, Hq, S, D, esz)) return fail(H3A_EINVAL, "o overlaps q");
    if (may_overlap(o, stride_o, Hq, k, stride_k, Hkv, S, D, esz)) return fail(H3A_EINVAL, "o overlaps k");
    if (may_overlap(o, stride_o, Hq, v, stride_v, Hkv, S, D, esz)) return fail(H3A_EINVAL, "o overlaps v");
    PlanUse plan;
    std::unique_lock<std::mutex> plan_lock;  // held until the launches below are enqueued
    if ((st = get_plan(cu_seqlens, nseg, Hq, h3a::kAttnBlockM_BF16, false, true, stream, &plan, &plan_lock)) != H3A_OK)
      return st;
    return run_plan(plan, stream, o, D, stride_o, "varlen attention (fused q norm) launch",
                    [&](const h3a::WorkItem* items, int64_t n, const h3a::SplitArgs& sp) {
                      return h3a::launch_attn_fwd_bf16_qnorm(q, k, v, o, D, stride_q, stride_k, stride_v, stride_o,
                                                             items, n, scale, Hq / Hkv, gamma_q, eps, cos_sin, S,
                                                             rot_dim, stream, sp);
                    });
  } catch (...) {
    return fail_exception("h3a_varlen_attn_fwd_qnorm");
  }
}

h3a_status h3a_quantize_e4m3(const void* x, void* y, void* y_scale, int64_t S, int32_t H, int32_t D,
                             int64_t stride_x, int64_t stride_y, hipStream_t stream) {
  try {
    if (S < 0) return fail(H3A_EINVAL, "S = %lld must be >= 0", (long long)S);
    if (S > int64_t(INT32_MAX)) return fail(H3A_EUNSUPPORTED, "S = %lld exceeds INT32_MAX", (long long)S);
    if (H < 1) return fail(H3A_EINVAL, "H = %d must be >= 1", H);
    if (D != 64 && D != 128) return fail(H3A_EUNSUPPORTED, "head_dim %d (supported: 64, 128)", D);
    h3a_status st;
    if ((st = check_operand("x", x, S, H, D, stride_x, 2)) != H3A_OK) return st;
    if ((st = check_operand("y", y, S, H, D, stride_y, 1)) != H3A_OK) return st;
    const int64_t sbytes = S * H * (D / 32);
    if ((st = check_scales("y_scale", y_scale, sbytes, 1)) != H3A_OK) return st;
    if (S == 0) return H3A_OK;
    // y (bytes) against x (bf16): plain byte ranges.
    const uintptr_t x0 = reinterpret_cast<uintptr_t>(x), y0 = reinterpret_cast<uintptr_t>(y);
    const uintptr_t x1 = x0 + uintptr_t(((S - 1) * stride_x + int64_t(H) * D) * 2);
    const uintptr_t y1 = y0 + uintptr_t((S - 1) * stride_y + int64_t(H) * D);
    if (x0 < y1 && y0 < x1) return fail(H3A_EINVAL, "y overlaps x");
    const Range rs = byte_range(y_scale, sbytes);
    if (ranges_hit(rs, Range{x0, x1}) || ranges_hit(rs, Range{y0, y1}))
      return fail(H3A_EINVAL, "y_scale overlaps x or y");
    hipError_t e = h3a::launch_quantize_e4m3(x, y, y_scale, S, H, D, stride_x, stride_y, stream);
    if (e != hipSuccess) return fail_hip("quantize_e4m3 launch", e);
    return H3A_OK;
  } catch (...) {
    return fail_exception("h3a_quantize_e4m3");
  }
}

h3a_status h3a_qk_rmsnorm_rope_e4m3(const void* q, const void* k, void* q8, void* k8, void* q_scale, void* k_scale,
                                    int64_t S, int32_t Hq, int32_t Hk, int32_t D, int64_t stride_q, int64_t stride_k,
                                    int64_t stride_q8, int64_t stride_k8, const float* gamma_q, const float* gamma_k,
                                    float eps, const float* cos_sin, int32_t rot_dim, hipStream_t stream) {
  try {
    if (S < 0) return fail(H3A_EINVAL, "S = %lld must be >= 0", (long long)S);
    if (S > int64_t(INT32_MAX)) return fail(H3A_EUNSUPPORTED, "S = %lld exceeds INT32_MAX", (long long)S);
    if (Hq < 1) return fail(H3A_EINVAL, "H = %d must be >= 1", Hq);
    if (Hk < 1) return fail(H3A_EINVAL, "Hk = %d must be >= 1", Hk);
    if (D != 64 && D != 128) return fail(H3A_EUNSUPPORTED, "head_dim %d (supported: 64, 128)", D);
    if (rot_dim < 0 || rot_dim > D || rot_dim % 2 != 0)
      return fail(H3A_EINVAL, "rot_dim = %d must be even and in [0, D = %d]", rot_dim, D);
    if ((rot_dim / 2) % 8 != 0)
      return fail(H3A_EUNSUPPORTED, "rot_dim / 2 = %d must be a multiple of 8 for this dtype", rot_dim / 2);
    if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(H3A_EINVAL, "eps = %g must be finite and >= 0", double(eps));
    h3a_status st;
    if ((st = check_operand("q", q, S, Hq, D, stride_q, 2)) != H3A_OK) return st;
    if ((st = check_operand("k", k, S, Hk, D, stride_k, 2)) != H3A_OK) return st;
    if ((st = check_operand("q8", q8, S, Hq, D, stride_q8, 1)) != H3A_OK) return st;
    if ((st = check_operand("k8", k8, S, Hk, D, stride_k8, 1)) != H3A_OK) return st;
    const int64_t qsb = S * Hq * (D / 32), ksb = S * Hk * (D / 32);
    if ((st = check_scales("q_scale", q_scale, qsb, 1)) != H3A_OK) return st;
    if ((st = check_scales("k_scale", k_scale, ksb, 1)) != H3A_OK) return st;
    if (gamma_q == nullptr) return fail(H3A_EINVAL, "gamma_q is NULL");
    if (gamma_k == nullptr) return fail(H3A_EINVAL, "gamma_k is NULL");
    if (!aligned(gamma_q, 4) || !aligned(gamma_k, 4)) return fail(H3A_EUNSUPPORTED, "gamma is not 4-byte aligned");
    if (rot_dim > 0 && S > 0) {
      if (cos_sin == nullptr) return fail(H3A_EINVAL, "cos_sin is NULL with rot_dim = %d", rot_dim);
      if (!aligned(cos_sin, 16)) return fail(H3A_EUNSUPPORTED, "cos_sin is not 16-byte aligned");
    }
    if (S == 0) return H3A_OK;
    // the byte outputs against every other tensor: plain byte ranges
    const Range rq = tensor_range(q, S, Hq, D, stride_q, 2), rk = tensor_range(k, S, Hk, D, stride_k, 2);
    const Range rq8 = tensor_range(q8, S, Hq, D, stride_q8, 1), rk8 = tensor_range(k8, S, Hk, D, stride_k8, 1);
    auto hit = [](const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi; };
    if (hit(rq8, rq) || hit(rq8, rk)) return fail(H3A_EINVAL, "q8 overlaps q or k");
    if (hit(rk8, rq) || hit(rk8, rk)) return fail(H3A_EINVAL, "k8 overlaps q or k");
    if (may_overlap(q8, stride_q8, Hq, k8, stride_k8, Hk, S, D, 1)) return fail(H3A_EINVAL, "q8 overlaps k8");
    const Range rqs = byte_range(q_scale, qsb), rks = byte_range(k_scale, ksb);
    for (const Range& r : {rq, rk, rq8, rk8})
      if (ranges_hit(rqs, r) || ranges_hit(rks, r)) return fail(H3A_EINVAL, "q_scale or k_scale overlaps a tensor");
    if (ranges_hit(rqs, rks)) return fail(H3A_EINVAL, "q_scale overlaps k_scale");
    hipError_t e = h3a::launch_qk_rmsnorm_rope_e4m3(q, k, q8, k8, q_scale, k_scale, S, Hq, Hk, D, stride_q, stride_k,
                                                    stride_q8, stride_k8, gamma_q, gamma_k, eps, cos_sin, rot_dim,
                                                    stream);
    if (e != hipSuccess) return fail_hip("qk_rmsnorm_rope_e4m3 launch", e);
    return H3A_OK;
  } catch (...) {
    return fail_exception("h3a_qk_rmsnorm_rope_e4m3");
  }
}

h3a_status h3a_varlen_attn_fwd_fp8qk(const void* q8, const void* k8, const void* q_scale, const void* k_scale,
                                     const void* v, void* o, int64_t S, int32_t Hq, int32_t Hkv, int32_t D,
                                     int64_t stride_q, int64_t stride_k, int64_t stride_v, int64_t stride_o,
                                     const int32_t* cu_seqlens, int32_t nseg, float scale, int32_t causal,
                                     hipStream_t stream) {
  try {
    if (S < 0) return fail(H3A_EINVAL, "S = %lld must be >= 0", (long long)S);
    if (S > int64_t(INT32_MAX)) return fail(H3A_EUNSUPPORTED, "S = %lld exceeds INT32_MAX", (long long)S);
    if (Hq < 1) return fail(H3A_EINVAL, "H = %d must be >= 1", Hq);
    if (Hkv < 1) return fail(H3A_EINVAL, "Hkv = %d must be >= 1", Hkv);
    if (Hq % Hkv != 0) return fail(H3A_ESHAPE, "Hkv = %d does not divide H = %d", Hkv, Hq);
    if (causal != 0 && causal != 1) return fail(H3A_EINVAL, "causal = %d must be 0 or 1", causal);
    if (D != 64 && D != 128) return fail(H3A_EUNSUPPORTED, "head_dim %d (supported: 64, 128)", D);
    if (!(scale > 0.f) || !std::isfinite(scale)) return fail(H3A_EINVAL, "scale = %g must be finite and > 0", double(scale));
    h3a_status st;
    if ((st = check_cu_seqlens(cu_seqlens, nseg, S)) != H3A_OK) return st;
    if ((st = check_operand("q", q8, S, Hq, D, stride_q, 1)) != H3A_OK) return st;
    if ((st = check_operand("k", k8, S, Hkv, D, stride_k, 1)) != H3A_OK) return st;
    if ((st = check_operand("v", v, S, Hkv, D, stride_v, 2)) != H3A_OK) return st;
    if ((st = check_operand("o", o, S, Hq, D, stride_o, 2)) != H3A_OK) return st;
    const int64_t qsb = S * Hq * (D / 32), ksb = S * Hkv * (D / 32);
    if ((st = check_scales("q_scale", q_scale, qsb, D / 32)) != H3A_OK) return st;
    if ((st = check_scales("k_scale", k_scale, ksb, D / 32)) != H3A_OK) return st;
    if (S == 0) return H3A_OK;
    // o (bf16) against the byte-coded q and k, their scales, and v (bf16)
    const Range ro = tensor_range(o, S, Hq, D, stride_o, 2);
    const Range rq = tensor_range(q8, S, Hq, D, stride_q, 1), rk = tensor_range(k8, S, Hkv, D, stride_k, 1);
    if (ro.lo < rq.hi && rq.lo < ro.hi) return fail(H3A_EINVAL, "o overlaps q");
    if (ro.lo < rk.hi && rk.lo < ro.hi) return fail(H3A_EINVAL, "o overlaps k");
    if (ranges_hit(ro, byte_range(q_scale, qsb)) || ranges_hit(ro, byte_range(k_scale, ksb)))
      return fail(H3A_EINVAL, "o overlaps q_scale or k_scale");
    if (may_overlap(o, stride_o, Hq, v, stride_v, Hkv, S, D, 2)) return fail(H3A_EINVAL, "o overlaps v");
    PlanUse plan;
    std::unique_lock<std::mutex> plan_lock;  // held until the launches below are enqueued
    if ((st = get_plan(cu_seqlens, nseg, Hq, h3a::kAttnBlockM_BF16, causal != 0, true, stream, &plan, &plan_lock)) !=
        H3A_OK)
      return st;
    return run_plan(plan, stream, o, D, stride_o, "varlen attention (fp8 qk) launch",
                    [&](const h3a::WorkItem* items, int64_t n, const h3a::SplitArgs& sp) {
                      return h3a::launch_attn_fwd_fp8qk(q8, k8, q_scale, k_scale, v, o, D, stride_q, stride_k,
                                                        S * (D / 32), S * (D / 32), stride_v, stride_o, items, n,
                                                        scale, Hq / Hkv, causal != 0, stream, sp);
                    });
  } catch (...) {
    return fail_exception("h3a_varlen_attn_fwd_fp8qk");
  }
}

h3a_status h3a_quantize_i8_rows(const void* x, void* y, void* y_scale, int64_t S, int32_t H, int32_t D,
                                int64_t stride_x, int64_t stride_y, hipStream_t stream) {
  try {
    if (S < 0) return fail(H3A_EINVAL, "S = %lld must be >= 0", (long long)S);
    if (S > int64_t(INT32_MAX)) return fail(H3A_EUNSUPPORTED, "S = %lld exceeds INT32_MAX", (long long)S);
    if (H < 1) return fail(H3A_EINVAL, "H = %d must be >= 1", H);
    if (D != 64 && D != 128) return fail(H3A_EUNSUPPORTED, "head_dim %d (supported: 64, 128)", D);
    h3a_status st;
    if ((st = check_operand("x", x, S, H, D, stride_x, 2)) != H3A_OK) return st;
    if ((st = check_operand("y", y, S, H, D, stride_y, 1)) != H3A_OK) return st;
    const int64_t sbytes = S * H * 4;
    if ((st = check_scales("y_scale", y_scale, sbytes, 4)) != H3A_OK) return st;
    if (S == 0) return H3A_OK;
    const Range rx = tensor_range(x, S, H, D, stride_x, 2), ry = tensor_range(y, S, H, D, stride_y, 1);
    if (ranges_hit(rx, ry)) return fail(H3A_EINVAL, "y overlaps x");
    const Range rs = byte_range(y_scale, sbytes);
    if (ranges_hit(rs, rx) || ranges_hit(rs, ry)) return fail(H3A_EINVAL, "y_scale overlaps x or y");
    hipError_t e = h3a::launch_quantize_i8_rows(x, y, y_scale, S, H, D, stride_x, stride_y, stream);
    if (e != hipSuccess) return fail_hip("quantize_i8_rows launch", e);
    return H3A_OK;
  } catch (...) {
    return fail_exception("h3a_quantize_i8_rows");
  }
}

h3a_status h3a_qk_rmsnorm_rope_i8q(const void* q, const void* k, void* q8, void* k_out, void* q_scale,
                                   int64_t S, int32_t Hq, int32_t Hk, int32_t D, int64_t stride_q, int64_t stride_k,
                                   int64_t stride_q8, int64_t stride_ko, const float* gamma_q, const float* gamma_k,
                                   float eps, const float* cos_sin, int32_t rot_dim, hipStream_t stream) {
  try {
    if (S < 0) return fail(H3A_EINVAL, "S = %lld must be >= 0", (long long)S);
    if (S > int64_t(INT32_MAX)) return fail(H3A_EUNSUPPORTED, "S = %lld exceeds INT32_MAX", (long long)S);
    if (Hq < 1) return fail(H3A_EINVAL, "H = %d must be >= 1", Hq);
    if (Hk < 1) return fail(H3A_EINVAL, "Hk = %d must be >= 1", Hk);
    if (D != 64 && D != 128) return fail(H3A_EUNSUPPORTED, "head_dim %d (supported: 64, 128)", D);
    if (rot_dim < 0 || rot_dim > D || rot_dim % 2 != 0)
      return fail(H3A_EINVAL, "rot_dim = %d must be even and in [0, D = %d]", rot_dim, D);
    if ((rot_dim / 2) % 8 != 0)
      return fail(H3A_EUNSUPPORTED, "rot_dim / 2 = %d must be a multiple of 8 for this dtype", rot_dim / 2);
    if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(H3A_EINVAL, "eps = %g must be finite and >= 0", double(eps));
    h3a_status st;
    if ((st = check_operand("q", q, S, Hq, D, stride_q, 2)) != H3A_OK) return st;
    if ((st = check_operand("k", k, S, Hk, D, stride_k, 2)) != H3A_OK) return st;
    if ((st = check_operand("q8", q8, S, Hq, D, stride_q8, 1)) != H3A_OK) return st;
    if ((st = check_operand("k_out", k_out, S, Hk, D, stride_ko, 2)) != H3A_OK) return st;
    const int64_t qsb = S * Hq * 4;
    if ((st = check_scales("q_scale", q_scale, qsb, 4)) != H3A_OK) return st;
    if (gamma_q == nullptr) return fail(H3A_EINVAL, "gamma_q is NULL");
    if (gamma_k == nullptr) return fail(H3A_EINVAL, "gamma_k is NULL");
    if (!aligned(gamma_q, 4) || !aligned(gamma_k, 4)) return fail(H3A_EUNSUPPORTED, "gamma is not 4-byte aligned");
    if (rot_dim > 0 && S > 0) {
      if (cos_sin == nullptr) return fail(H3A_EINVAL, "cos_sin is NULL with rot_dim = %d", rot_dim);
      if (!aligned(cos_sin, 16)) return fail(H3A_EUNSUPPORTED, "cos_sin is not 16-byte aligned");
    }
    if (S == 0) return H3A_OK;
    // k_out may be k itself (each token is read before it is written); q8 and
    // q_scale are byte ranges that may touch nothing else
    const bool k_inplace = k_out == k && stride_ko == stride_k;
    if (!k_inplace && may_overlap(k_out, stride_ko, Hk, k, stride_k, Hk, S, D, 2))
      return fail(H3A_EINVAL, "k_out overlaps k without being k itself");
    if (may_overlap(k_out, stride_ko, Hk, q, stride_q, Hq, S, D, 2)) return fail(H3A_EINVAL, "k_out overlaps q");
    const Range rq = tensor_range(q, S, Hq, D, stride_q, 2), rk = tensor_range(k, S, Hk, D, stride_k, 2);
    const Range rko = tensor_range(k_out, S, Hk, D, stride_ko, 2);
    const Range rq8 = tensor_range(q8, S, Hq, D, stride_q8, 1), rqs = byte_range(q_scale, qsb);
    for (const Range& r : {rq, rk, rko}) {
      if (ranges_hit(rq8, r)) return fail(H3A_EINVAL, "q8 overlaps q, k or k_out");
      if (ranges_hit(rqs, r)) return fail(H3A_EINVAL, "q_scale overlaps q, k or k_out");
    }
    if (ranges_hit(rqs, rq8)) return fail(H3A_EINVAL, "q_scale overlaps q8");
    hipError_t e = h3a::launch_qk_rmsnorm_rope_i8q(q, k, q8, k_out, q_scale, S, Hq, Hk, D, stride_q, stride_k,
                                                   stride_q8, stride_ko, gamma_q, gamma_k, eps, cos_sin, rot_dim,
                                                   stream);
    if (e != hipSuccess) return fail_hip("qk_rmsnorm_rope_i8q launch", e);
    return H3A_OK;
  } catch (...) {
    return fail_exception("h3a_qk_rmsnorm_rope_i8q");
  }
}

h3a_status h3a_i8_key_blocks(const int32_t* cu_seqlens, int32_t nseg, int64_t* n_blocks) {
  try {
    if (n_blocks == nullptr) return fail(H3A_EINVAL, "n_blocks is NULL");
    if (cu_seqlens == nullptr) return fail(H3A_EINVAL, "cu_seqlens is NULL");
    if (nseg < 1) return fail(H3A_EINVAL, "nseg = %d must be >= 1", nseg);
    h3a_status st;
    if ((st = check_cu_seqlens(cu_seqlens, nseg, cu_seqlens[nseg])) != H3A_OK) return st;
    *n_blocks = h3a::vt_e4m3_columns(cu_seqlens, nseg) / h3a::kVtTile;
    return H3A_OK;
  } catch (...) {
    return fail_exception("h3a_i8_key_blocks");
  }
}

namespace {

// The key quantiser, plain or on centred keys (mu: fp32 [nseg][H][D]).
h3a_status quantize_i8_keys_impl(bool centered, const void* x, const float* mu, void* y, void* y_scale, int64_t S,
                                 int32_t H, int32_t D, int64_t stride_x, int64_t stride_y, int64_t n_blocks,
                                 const int32_t* cu_seqlens, int32_t nseg, hipStream_t stream) {
  if (S < 0) return fail(H3A_EINVAL, "S = %lld must be >= 0", (long long)S);
  if (S > int64_t(INT32_MAX)) return fail(H3A_EUNSUPPORTED, "S = %lld exceeds INT32_MAX", (long long)S);
  if (H < 1) return fail(H3A_EINVAL, "H = %d must be >= 1", H);
  if (D != 64 && D != 128) return fail(H3A_EUNSUPPORTED, "head_dim %d (supported: 64, 128)", D);
  h3a_status st;
  if ((st = check_cu_seqlens(cu_seqlens, nseg, S)) != H3A_OK) return st;
  const int64_t need = h3a::vt_e4m3_columns(cu_seqlens, nseg) / h3a::kVtTile;
  if (n_blocks != need)
    return fail(H3A_ESHAPE, "n_blocks = %lld but cu_seqlens has %lld blocks of 64 keys", (long long)n_blocks,
                (long long)need);
  if ((st = check_operand("x", x, S, H, D, stride_x, 2)) != H3A_OK) return st;
  if ((st = check_operand("y", y, S, H, D, stride_y, 1)) != H3A_OK) return st;
  const int64_t sbytes = int64_t(H) * n_blocks * 4;
  if ((st = check_scales("y_scale", y_scale, sbytes, 4)) != H3A_OK) return st;
  const int64_t mbytes = int64_t(nseg) * H * D * 4;
  if (centered && (st = check_scales("mu", mu, mbytes, 16)) != H3A_OK) return st;
  if (S == 0) return H3A_OK;
  const Range rx = tensor_range(x, S, H, D, stride_x, 2), ry = tensor_range(y, S, H, D, stride_y, 1);
  if (ranges_hit(rx, ry)) return fail(H3A_EINVAL, "y overlaps x");
  const Range rs = byte_range(y_scale, sbytes);
  if (ranges_hit(rs, rx) || ranges_hit(rs, ry)) return fail(H3A_EINVAL, "y_scale overlaps x or y");
  if (centered) {
    const Range rm = byte_range(mu, mbytes);
    if (ranges_hit(rm, ry) || ranges_hit(rm, rs)) return fail(H3A_EINVAL, "mu overlaps y or y_scale");
  }
  hipError_t e = h3a::launch_quantize_i8_keys(x, y, y_scale, cu_seqlens, nseg, H, D, stride_x, stride_y, n_blocks,
                                              stream, mu);
  if (e != hipSuccess) return fail_hip("quantize_i8_keys launch", e);
  return H3A_OK;
}

}  // namespace

h3a_status h3a_quantize_i8_keys(const void* x, void* y, void* y_scale, int64_t S, int32_t H, int32_t D,
                                int64_t stride_x, int64_t stride_y, int64_t n_blocks, const int32_t* cu_seqlens,
                                int32_t nseg, hipStream_t stream) {
  try {
    return quantize_i8_keys_impl(false, x, nullptr, y, y_scale, S, H, D, stride_x, stride_y, n_blocks,
                                 cu_seqlens, nseg, stream);
  } catch (...) {
    return fail_exception("h3a_quantize_i8_keys");
  }
}

h3a_status h3a_quantize_i8_keys_centered(const void* x, const void* mu, void* y, void* y_scale, int64_t S, int32_t H,
                                         int32_t D, int64_t stride_x, int64_t stride_y, int64_t n_blocks,
                                         const int32_t* cu_seqlens, int32_t nseg, hipStream_t stream) {
  try {
    return quantize_i8_keys_impl(true, x, static_cast<const float*>(mu), y, y_scale, S, H,
                                 D, stride_x, stride_y, n_blocks, cu_seqlens, nseg, stream);
  } catch (...) {
    return fail_exception("h3a_quantize_i8_keys_centered");
  }
}

h3a_status h3a_i8_key_mean_chunks(const int32_t* cu_seqlens, int32_t nseg, int64_t* n_chunks) {
  try {
    if (n_chunks == nullptr) return fail(H3A_EINVAL, "n_chunks is NULL");
    if (cu_seqlens == nullptr) return fail(H3A_EINVAL, "cu_seqlens is NULL");
    if (nseg < 1) return fail(H3A_EINVAL, "nseg = %d must be >= 1", nseg);
    h3a_status st;
    if ((st = check_cu_seqlens(cu_seqlens, nseg, cu_seqlens[nseg])) != H3A_OK) return st;
    *n_chunks = h3a::key_mean_chunks(cu_seqlens, nseg);
    return H3A_OK;
  } catch (...) {
    return fail_exception("h3a_i8_key_mean_chunks");
  }
}

h3a_status h3a_segment_key_means(const void* k, void* partial, void* mu, int64_t S, int32_t H, int32_t D,
                                 int64_t stride_k, int64_t n_chunks, const int32_t* cu_seqlens, int32_t nseg,
                                 hipStream_t stream) {
  try {
    if (S < 0) return fail(H3A_EINVAL, "S = %lld must be >= 0", (long long)S);
    if (S > int64_t(INT32_MAX)) return fail(H3A_EUNSUPPORTED, "S = %lld exceeds INT32_MAX", (long long)S);
    if (H < 1) return fail(H3A_EINVAL, "H = %d must be >= 1", H);
    if (D != 64 && D != 128) return fail(H3A_EUNSUPPORTED, "head_dim %d (supported: 64, 128)", D);
    h3a_status st;
    if ((st = check_cu_seqlens(cu_seqlens, nseg, S)) != H3A_OK) return st;
    const int64_t need = h3a::key_mean_chunks(cu_seqlens, nseg);
    if (n_chunks != need)
      return fail(H3A_ESHAPE, "n_chunks = %lld but cu_seqlens has %lld chunks of 256 keys", (long long)n_chunks,
                  (long long)need);
    if ((st = check_operand("k", k, S, H, D, stride_k, 2)) != H3A_OK) return st;
    const int64_t pbytes = n_chunks * H * D * 4, mbytes = int64_t(nseg) * H * D * 4;
    if ((st = check_scales("partial", partial, pbytes, 4)) != H3A_OK) return st;
    if ((st = check_scales("mu", mu, mbytes, 4)) != H3A_OK) return st;
    const Range rp = byte_range(partial, pbytes), rm = byte_range(mu, mbytes);
    if (ranges_hit(rp, rm)) return fail(H3A_EINVAL, "partial overlaps mu");
    if (S > 0) {
      const Range rk = tensor_range(k, S, H, D, stride_k, 2);
      if (ranges_hit(rp, rk) || ranges_hit(rm, rk)) return fail(H3A_EINVAL, "partial or mu overlaps k");
    }
    hipError_t e = h3a::launch_segment_key_means(k, partial, mu, cu_seqlens, nseg, H, D, stride_k, n_chunks, stream);
    if (e != hipSuccess) return fail_hip("segment_key_means launch", e);
    return H3A_OK;
  } catch (...) {
    return fail_exception("h3a_segment_key_means");
  }
}

h3a_status h3a_varlen_attn_fwd_i8qk(const void* q8, const void* k8, const void* q_scale, const void* k_scale,
                                    const void* v, void* o, int64_t S, int32_t Hq, int32_t Hkv, int32_t D,
                                    int64_t stride_q, int64_t stride_k, int64_t stride_v, int64_t stride_o,
                                    const int32_t* cu_seqlens, int32_t nseg, float scale, int32_t causal,
                                    hipStream_t stream) {
  try {
    if (S < 0) return fail(H3A_EINVAL, "S = %lld must be >= 0", (long long)S);
    if (S > int64_t(INT32_MAX)) return fail(H3A_EUNSUPPORTED, "S = %lld exceeds INT32_MAX", (long long)S);
    if (Hq < 1) return fail(H3A_EINVAL, "H = %d must be >= 1", Hq);
    if (Hkv < 1) return fail(H3A_EINVAL, "Hkv = %d must be >= 1", Hkv);
    if (Hq % Hkv != 0) return fail(H3A_ESHAPE, "Hkv = %d does not divide H = %d", Hkv, Hq);
    if (causal != 0 && causal != 1) return fail(H3A_EINVAL, "causal = %d must be 0 or 1", causal);
    if (D != 64 && D != 128) return fail(H3A_EUNSUPPORTED, "head_dim %d (supported: 64, 128)", D);
    if (!(scale > 0.f) || !std::isfinite(scale)) return fail(H3A_EINVAL, "scale = %g must be finite and > 0", double(scale));
    h3a_status st;
    if ((st = check_cu_seqlens(cu_seqlens, nseg, S)) != H3A_OK) return st;
    // the kernel finds a segment's key blocks from its padded column (an int32)
    const int64_t cols = h3a::vt_e4m3_columns(cu_seqlens, nseg);
    if (cols > int64_t(INT32_MAX))
      return fail(H3A_EUNSUPPORTED, "the segments' 64-key blocks cover %lld keys, more than INT32_MAX", (long long)cols);
    const int64_t n_blocks = cols / h3a::kVtTile;
    if ((st = check_operand("q", q8, S, Hq, D, stride_q, 1)) != H3A_OK) return st;
    if ((st = check_operand("k", k8, S, Hkv, D, stride_k, 1)) != H3A_OK) return st;
    if ((st = check_operand("v", v, S, Hkv, D, stride_v, 2)) != H3A_OK) return st;
    if ((st = check_operand("o", o, S, Hq, D, stride_o, 2)) != H3A_OK) return st;
    const int64_t qsb = S * Hq * 4, ksb = int64_t(Hkv) * n_blocks * 4;
    if ((st = check_scales("q_scale", q_scale, qsb, 4)) != H3A_OK) return st;
    if ((st = check_scales("k_scale", k_scale, ksb, 4)) != H3A_OK) return st;
    if (S == 0) return H3A_OK;
    // o (bf16) against the byte-coded q and k, their scales, and v (bf16)
    const Range ro = tensor_range(o, S, Hq, D, stride_o, 2);
    const Range rq = tensor_range(q8, S, Hq, D, stride_q, 1), rk = tensor_range(k8, S, Hkv, D, stride_k, 1);
    if (ranges_hit(ro, rq)) return fail(H3A_EINVAL, "o overlaps q");
    if (ranges_hit(ro, rk)) return fail(H3A_EINVAL, "o overlaps k");
    if (ranges_hit(ro, byte_range(q_scale, qsb)) || ranges_hit(ro, byte_range(k_scale, ksb)))
      return fail(H3A_EINVAL, "o overlaps q_scale or k_scale");
    if (may_overlap(o, stride_o, Hq, v, stride_v, Hkv, S, D, 2)) return fail(H3A_EINVAL, "o overlaps v");
    PlanUse plan;
    std::unique_lock<std::mutex> plan_lock;  // held until the launches below are enqueued
    if ((st = get_plan(cu_seqlens, nseg, Hq, h3a::kAttnBlockM_BF16, causal != 0, true, stream, &plan, &plan_lock)) !=
        H3A_OK)
      return st;
    return run_plan(plan, stream, o, D, stride_o, "varlen attention (int8 qk) launch",
                    [&](const h3a::WorkItem* items, int64_t n, const h3a::SplitArgs& sp) {
                      return h3a::launch_attn_fwd_i8qk(q8, k8, q_scale, k_scale, v, o, D, stride_q, stride_k, S * 4,
                                                       n_blocks * 4, stride_v, stride_o, items, n, scale, Hq / Hkv,
                                                       causal != 0, stream, sp);
                    });
  } catch (...) {
    return fail_exception("h3a_varlen_attn_fwd_i8qk");
  }
}

h3a_status h3a_varlen_attn_fwd_i8qk_fp8pv(const void* q8, const void* k8, const void* vt8, const void* q_scale,
                                          const void* k_scale, const void* vt_scale, void* o, int64_t S, int32_t Hq,
                                          int32_t Hkv, int32_t D, int64_t stride_q, int64_t stride_k, int64_t vt_cols,
                                          int64_t stride_o, const int32_t* cu_seqlens, int32_t nseg, float scale,
                                          int32_t causal, hipStream_t stream) {
  try {
    if (S < 0) return fail(H3A_EINVAL, "S = %lld must be >= 0", (long long)S);
    if (S > int64_t(INT32_MAX)) return fail(H3A_EUNSUPPORTED, "S = %lld exceeds INT32_MAX", (long long)S);
    if (Hq < 1) return fail(H3A_EINVAL, "H = %d must be >= 1", Hq);
    if (Hkv < 1) return fail(H3A_EINVAL, "Hkv = %d must be >= 1", Hkv);
    if (Hq % Hkv != 0) return fail(H3A_ESHAPE, "Hkv = %d does not divide H = %d", Hkv, Hq);
    if (causal != 0 && causal != 1) return fail(H3A_EINVAL, "causal = %d must be 0 or 1", causal);
    if (D != 64 && D != 128) return fail(H3A_EUNSUPPORTED, "head_dim %d (supported: 64, 128)", D);
    if (!(scale > 0.f) || !std::isfinite(scale)) return fail(H3A_EINVAL, "scale = %g must be finite and > 0", double(scale));
    h3a_status st;
    if ((st = check_cu_seqlens(cu_seqlens, nseg, S)) != H3A_OK) return st;
    if ((st = check_operand("q", q8, S, Hq, D, stride_q, 1)) != H3A_OK) return st;
    if ((st = check_operand("k", k8, S, Hkv, D, stride_k, 1)) != H3A_OK) return st;
    if ((st = check_operand("o", o, S, Hq, D, stride_o, 2)) != H3A_OK) return st;
    // the padded columns of the V^T layout are also the k scales' key blocks
    const int64_t need = h3a::vt_e4m3_columns(cu_seqlens, nseg);
    if (vt_cols != need)
      return fail(H3A_ESHAPE, "vt_cols = %lld but the padded layout of cu_seqlens has %lld columns", (long long)vt_cols,
                  (long long)need);
    if (int64_t(D) * vt_cols > int64_t(INT32_MAX))
      return fail(H3A_EUNSUPPORTED, "D * vt_cols = %lld exceeds INT32_MAX", (long long)(int64_t(D) * vt_cols));
    const int64_t n_blocks = vt_cols / h3a::kVtTile;
    const int64_t qsb = S * Hq * 4, ksb = int64_t(Hkv) * n_blocks * 4, vsb = int64_t(Hkv) * vt_cols * (D / 32);
    if ((st = check_scales("q_scale", q_scale, qsb, 4)) != H3A_OK) return st;
    if ((st = check_scales("k_scale", k_scale, ksb, 4)) != H3A_OK) return st;
    if ((st = check_scales("vt_scale", vt_scale, vsb, D / 32)) != H3A_OK) return st;
    if (S == 0) return H3A_OK;
    if (vt8 == nullptr) return fail(H3A_EINVAL, "vt8 is NULL");
    if (!aligned(vt8, 16)) return fail(H3A_EUNSUPPORTED, "vt8 is not 16-byte aligned");
    const Range ro = tensor_range(o, S, Hq, D, stride_o, 2);
    const Range rq = tensor_range(q8, S, Hq, D, stride_q, 1), rk = tensor_range(k8, S, Hkv, D, stride_k, 1);
    const uintptr_t t0 = reinterpret_cast<uintptr_t>(vt8), t1 = t0 + uintptr_t(int64_t(Hkv) * D * vt_cols);
    if (ranges_hit(ro, rq)) return fail(H3A_EINVAL, "o overlaps q");
    if (ranges_hit(ro, rk)) return fail(H3A_EINVAL, "o overlaps k");
    if (ro.lo < t1 && t0 < ro.hi) return fail(H3A_EINVAL, "o overlaps vt8");
    for (const Range& r : {byte_range(q_scale, qsb), byte_range(k_scale, ksb), byte_range(vt_scale, vsb)})
      if (ranges_hit(ro, r)) return fail(H3A_EINVAL, "o overlaps a scale array");
    PlanUse plan;
    std::unique_lock<std::mutex> plan_lock;  // held until the launches below are enqueued
    if ((st = get_plan(cu_seqlens, nseg, Hq, h3a::kAttnBlockM_BF16, causal != 0, true, stream, &plan, &plan_lock)) !=
        H3A_OK)
      return st;
    return run_plan(plan, stream, o, D, stride_o, "varlen attention (int8 qk, fp8 pv) launch",
                    [&](const h3a::WorkItem* items, int64_t n, const h3a::SplitArgs& sp) {
                      return h3a::launch_attn_fwd_i8qk_fp8pv(q8, k8, vt8, q_scale, k_scale, vt_scale, o, D, stride_q,
                                                             stride_k, S * 4, n_blocks * 4, vt_cols, stride_o, items,
                                                             n, scale, Hq / Hkv, causal != 0, stream, sp);
                    });
  } catch (...) {
    return fail_exception("h3a_varlen_attn_fwd_i8qk_fp8pv");
  }
}

h3a_status h3a_vt_e4m3_columns(const int32_t* cu_seqlens, int32_t nseg, int64_t* columns) {
  try {
    if (columns == nullptr) return fail(H3A_EINVAL, "columns is NULL");
    if (cu_seqlens == nullptr) return fail(H3A_EINVAL, "cu_seqlens is NULL");
    if (nseg < 1) return fail(H3A_EINVAL, "nseg = %d must be >= 1", nseg);
    h3a_status st;
    if ((st = check_cu_seqlens(cu_seqlens, nseg, cu_seqlens[nseg])) != H3A_OK) return st;
    *columns = h3a::vt_e4m3_columns(cu_seqlens, nseg);
    return H3A_OK;
  } catch (...) {
    return fail_exception("h3a_vt_e4m3_columns");
  }
}

h3a_status h3a_prepare_vt_e4m3(const void* v, void* vt8, void* vt_scale, int64_t S, int32_t Hkv, int32_t D,
                               int64_t stride_v, int64_t vt_cols, const int32_t* cu_seqlens, int32_t nseg,
                               hipStream_t stream) {
  try {
    if (S < 0) return fail(H3A_EINVAL, "S = %lld must be >= 0", (long long)S);
    if (S > int64_t(INT32_MAX)) return fail(H3A_EUNSUPPORTED, "S = %lld exceeds INT32_MAX", (long long)S);
    if (Hkv < 1) return fail(H3A_EINVAL, "Hkv = %d must be >= 1", Hkv);
    if (D != 64 && D != 128) return fail(H3A_EUNSUPPORTED, "head_dim %d (supported: 64, 128)", D);
    h3a_status st;
    if ((st = check_cu_seqlens(cu_seqlens, nseg, S)) != H3A_OK) return st;
    if ((st = check_operand("v", v, S, Hkv, D, stride_v, 2)) != H3A_OK) return st;
    const int64_t need = h3a::vt_e4m3_columns(cu_seqlens, nseg);
    if (vt_cols != need)
      return fail(H3A_ESHAPE, "vt_cols = %lld but the padded layout of cu_seqlens has %lld columns", (long long)vt_cols,
                  (long long)need);
    if (int64_t(D) * vt_cols > int64_t(INT32_MAX))
      return fail(H3A_EUNSUPPORTED, "D * vt_cols = %lld exceeds INT32_MAX", (long long)(int64_t(D) * vt_cols));
    if (need == 0) return H3A_OK;
    if (vt8 == nullptr) return fail(H3A_EINVAL, "vt8 is NULL");
    if (!aligned(vt8, 16)) return fail(H3A_EUNSUPPORTED, "vt8 is not 16-byte aligned");
    const int64_t vsb = int64_t(Hkv) * vt_cols * (D / 32);
    if ((st = check_scales("vt_scale", vt_scale, vsb, D / 32)) != H3A_OK) return st;
    const Range rv = tensor_range(v, S, Hkv, D, stride_v, 2);
    const uintptr_t t0 = reinterpret_cast<uintptr_t>(vt8), t1 = t0 + uintptr_t(int64_t(Hkv) * D * vt_cols);
    if (rv.lo < t1 && t0 < rv.hi) return fail(H3A_EINVAL, "vt8 overlaps v");
    const Range rs = byte_range(vt_scale, vsb);
    if (ranges_hit(rs, rv) || ranges_hit(rs, Range{t0, t1})) return fail(H3A_EINVAL, "vt_scale overlaps v or vt8");
    hipError_t e = h3a::launch_prepare_vt_e4m3(v, stride_v, cu_seqlens, nseg, Hkv, D, vt8, vt_scale, vt_cols, stream);
    if (e != hipSuccess) return fail_hip("prepare_vt_e4m3 launch", e);
    return H3A_OK;
  } catch (...) {
    return fail_exception("h3a_prepare_vt_e4m3");
  }
}

h3a_status h3a_varlen_attn_fwd_fp8(const void* q8, const void* k8, const void* vt8, const void* q_scale,
                                   const void* k_scale, const void* vt_scale, void* o, int64_t S, int32_t Hq,
                                   int32_t Hkv, int32_t D, int64_t stride_q, int64_t stride_k, int64_t vt_cols,
                                   int64_t stride_o, const int32_t* cu_seqlens, int32_t nseg, float scale,
                                   int32_t causal, hipStream_t stream) {
  try {
    if (S < 0) return fail(H3A_EINVAL, "S = %lld must be >= 0", (long long)S);
    if (S > int64_t(INT32_MAX)) return fail(H3A_EUNSUPPORTED, "S = %lld exceeds INT32_MAX", (long long)S);
    if (Hq < 1) return fail(H3A_EINVAL, "H = %d must be >= 1", Hq);
    if (Hkv < 1) return fail(H3A_EINVAL, "Hkv = %d must be >= 1", Hkv);
    if (Hq % Hkv != 0) return fail(H3A_ESHAPE, "Hkv = %d does not divide H = %d", Hkv, Hq);
    if (causal != 0 && causal != 1) return fail(H3A_EINVAL, "causal = %d must be 0 or 1", causal);
    if (D != 64 && D != 128) return fail(H3A_EUNSUPPORTED, "head_dim %d (supported: 64, 128)", D);
    if (!(scale > 0.f) || !std::isfinite(scale)) return fail(H3A_EINVAL, "scale = %g must be finite and > 0", double(scale));
    h3a_status st;
    if ((st = check_cu_seqlens(cu_seqlens, nseg, S)) != H3A_OK) return st;
    if ((st = check_operand("q", q8, S, Hq, D, stride_q, 1)) != H3A_OK) return st;
    if ((st = check_operand("k", k8, S, Hkv, D, stride_k, 1)) != H3A_OK) return st;
    if ((st = check_operand("o", o, S, Hq, D, stride_o, 2)) != H3A_OK) return st;
    const int64_t need = h3a::vt_e4m3_columns(cu_seqlens, nseg);
    if (vt_cols != need)
      return fail(H3A_ESHAPE, "vt_cols = %lld but the padded layout of cu_seqlens has %lld columns", (long long)vt_cols,
                  (long long)need);
    if (int64_t(D) * vt_cols > int64_t(INT32_MAX))
      return fail(H3A_EUNSUPPORTED, "D * vt_cols = %lld exceeds INT32_MAX", (long long)(int64_t(D) * vt_cols));
    const int64_t qsb = S * Hq * (D / 32), ksb = S * Hkv * (D / 32), vsb = int64_t(Hkv) * vt_cols * (D / 32);
    if ((st = check_scales("q_scale", q_scale, qsb, D / 32)) != H3A_OK) return st;
    if ((st = check_scales("k_scale", k_scale, ksb, D / 32)) != H3A_OK) return st;
    if ((st = check_scales("vt_scale", vt_scale, vsb, D / 32)) != H3A_OK) return st;
    if (S == 0) return H3A_OK;
    if (vt8 == nullptr) return fail(H3A_EINVAL, "vt8 is NULL");
    if (!aligned(vt8, 16)) return fail(H3A_EUNSUPPORTED, "vt8 is not 16-byte aligned");
    const Range ro = tensor_range(o, S, Hq, D, stride_o, 2);
    const Range rq = tensor_range(q8, S, Hq, D, stride_q, 1), rk = tensor_range(k8, S, Hkv, D, stride_k, 1);
    const uintptr_t t0 = reinterpret_cast<uintptr_t>(vt8), t1 = t0 + uintptr_t(int64_t(Hkv) * D * vt_cols);
    if (ro.lo < rq.hi && rq.lo < ro.hi) return fail(H3A_EINVAL, "o overlaps q");
    if (ro.lo < rk.hi && rk.lo < ro.hi) return fail(H3A_EINVAL, "o overlaps k");
    if (ro.lo < t1 && t0 < ro.hi) return fail(H3A_EINVAL, "o overlaps vt8");
    for (const Range& r : {byte_range(q_scale, qsb), byte_range(k_scale, ksb), byte_range(vt_scale, vsb)})
      if (ranges_hit(ro, r)) return fail(H3A_EINVAL, "o overlaps a scale array");
    PlanUse plan;
    std::unique_lock<std::mutex> plan_lock;  // held until the launches below are enqueued
    if ((st = get_plan(cu_seqlens, nseg, Hq, h3a::kAttnBlockM_BF16, causal != 0, true, stream, &plan, &plan_lock)) !=
        H3A_OK)
      return st;
    return run_plan(plan, stream, o, D, stride_o, "varlen attention (fp8) launch",
                    [&](const h3a::WorkItem* items, int64_t n, const h3a::SplitArgs& sp) {
                      return h3a::launch_attn_fwd_fp8(q8, k8, vt8, q_scale, k_scale, vt_scale, o, D, stride_q,
                                                      stride_k, S * (D / 32), S * (D / 32), vt_cols, stride_o, items,
                                                      n, scale, Hq / Hkv, causal != 0, stream, sp);
                    });
  } catch (...) {
    return fail_exception("h3a_varlen_attn_fwd_fp8");
  }
}

h3a_status h3a_varlen_attn_fwd(const void* q, const void* k, const void* v, void* o,
                               h3a_dtype dtype, int64_t S, int32_t H, int32_t D,
                               int64_t stride_q, int64_t stride_k, int64_t stride_v,
                               int64_t stride_o, const int32_t* cu_seqlens, int32_t nseg,
                               float scale, hipStream_t stream) {
  try {
    return h3a_varlen_attn_fwd_ex(q, k, v, o, dtype, S, H, H, D, stride_q, stride_k, stride_v, stride_o,
                                  cu_seqlens, nseg, scale, 0, stream);
  } catch (...) {
    return fail_exception("h3a_varlen_attn_fwd");
  }
}

h3a_status h3a_plan_tiles_ex(const int32_t* cu_seqlens, int32_t nseg, int32_t H, int32_t block_m,
                             int32_t n_xcd, int32_t causal, int32_t* items, int64_t cap, int64_t* n_items) {
  try {
    if (n_items == nullptr) return fail(H3A_EINVAL, "n_items is NULL");
    if (H < 1) return fail(H3A_EINVAL, "H = %d must be >= 1", H);
    if (block_m < 1) return fail(H3A_EINVAL, "block_m = %d must be >= 1", block_m);
    if (n_xcd < 1) return fail(H3A_EINVAL, "n_xcd = %d must be >= 1", n_xcd);
    if (causal != 0 && causal != 1) return fail(H3A_EINVAL, "causal = %d must be 0 or 1", causal);
    h3a_status st;
    if (cu_seqlens == nullptr) return fail(H3A_EINVAL, "cu_seqlens is NULL");
    if (nseg < 1) return fail(H3A_EINVAL, "nseg = %d must be >= 1", nseg);
    if ((st = check_cu_seqlens(cu_seqlens, nseg, cu_seqlens[nseg])) != H3A_OK) return st;
    if (!plan_fits(cu_seqlens, nseg, H, block_m))
      return fail(H3A_EUNSUPPORTED, "plan would exceed %lld work items", (long long)kMaxPlanItems);
    std::vector<h3a::WorkItem> plan = h3a::plan_tiles(cu_seqlens, nseg, H, block_m, n_xcd, causal != 0);
    *n_items = int64_t(plan.size());
    if (int64_t(plan.size()) > cap) return fail(H3A_ESHAPE, "cap %lld < plan length %lld", (long long)cap, (long long)plan.size());
    if (!plan.empty() && items == nullptr) return fail(H3A_EINVAL, "items is NULL");
    for (size_t i = 0; i < plan.size(); ++i) {
      items[4 * i + 0] = plan[i].seg_start;
      items[4 * i + 1] = plan[i].seg_len;
      items[4 * i + 2] = plan[i].q_start;
      items[4 * i + 3] = plan[i].head;
    }
    return H3A_OK;
  } catch (...) {
    return fail_exception("h3a_plan_tiles_ex");
  }
}

h3a_status h3a_plan_tiles(const int32_t* cu_seqlens, int32_t nseg, int32_t H, int32_t block_m,
                          int32_t n_xcd, int32_t* items, int64_t cap, int64_t* n_items) {
  try {
    return h3a_plan_tiles_ex(cu_seqlens, nseg, H, block_m, n_xcd, 0, items, cap, n_items);
  } catch (...) {
    return fail_exception("h3a_plan_tiles");
  }
}

}  // extern "C"
