// Expert cache: a global LRU over (layer, expert) keys backed by a device
// slot pool, with the full expert pool in pinned host memory.
//
// FreeToken treats VRAM as a cache over the host-resident pool and streams
// only missing experts over PCIe ("FreeToken Inference Engine: 3x Speed
// Boost for MoE Models", sections "From Static Allocation to Dynamic
// Scheduling" and "RTX 5090 Benchmark"); the cache is one global LRU
// (FreeToken fork README, "About"; setup guide: a shared LRU follows
// token-level routing locality).
//
// Slots.  The device pool has n_slots + 2 slots.  At most n_slots keys are
// resident; free slots wait in a FIFO, so the slot a miss is copied into was
// released at least two evictions earlier (ping-pong staging): its last
// reader has normally long finished, and the copy still waits on that
// reader's event before overwriting it.
//
// Order of LRU updates.  cache_slot_table_lookup applies the layer's ids in
// order: a hit refreshes the key; a miss evicts the least recently used key
// not looked up earlier in this (step, layer) and inserts the new key at
// once, with its destination slot.  prefetch_expert then moves the bytes
// and installs the slot in the device table in stream order.
#include <algorithm>
#include <chrono>
#include <deque>
#include <cmath>
#include <set>
#include <unordered_map>
#include <vector>

#include <hsa/hsa.h>
#include <hsa/hsa_ext_amd.h>

#include "device_common.h"
#include "hsa_copy.h"
#include "ffn.h"

namespace moe {

constexpr int kTableUpdates = 16;
struct TableUpdate {
  int n;
  int idx[kTableUpdates];
  int val[kTableUpdates];
};

__global__ void table_update_kernel(int32_t* table, TableUpdate u) {
  const int i = threadIdx.x;
  if (i < u.n) table[u.idx[i]] = u.val[i];
}

// Moves whole slots of the device pool: moves[m] = (from, to), slot indices
// into src and dst.  blockIdx.y strides over the moves, blockIdx.x and the
// threads over the 16-byte words of a slot.  No slot is both a source and a
// destination, so src and dst may be one pool.
__global__ void slot_move_kernel(const uint4* src, uint4* dst, const int2* moves, int n_moves,
                                 long long words_per_slot) {
  for (int m = blockIdx.y; m < n_moves; m += gridDim.y) {
    const int2 mv = moves[m];
    const uint4* from = src + (long long)mv.x * words_per_slot;
    uint4* to = dst + (long long)mv.y * words_per_slot;
    for (long long w = (long long)blockIdx.x * blockDim.x + threadIdx.x; w < words_per_slot;
         w += (long long)gridDim.x * blockDim.x)
      to[w] = from[w];
  }
}

// Rows of y_pairs computed on the host: pair p's row is read from src
// (coherent pinned host memory, [P][H]) when its expert is a host miss.
__global__ void host_rows_kernel(const float4* __restrict__ src, const int32_t* __restrict__ host_mask,
                                 const int32_t* __restrict__ ids, float4* __restrict__ y, int H4) {
  const int p = blockIdx.y;
  if (!host_mask[ids[p]]) return;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < H4; i += gridDim.x * blockDim.x)
    y[(size_t)p * H4 + i] = src[(size_t)p * H4 + i];
}

// The layer's expert masks (resident, copied misses, host misses) travel
// as bits in the kernel arguments and are expanded on the device, so no
// copy-engine transfer, which could queue behind expert copies still in
// flight on another stream, stands between the lookup and the FFN.
struct MaskBits {
  int E;
  uint32_t bits[3][kMaxE / 32];
};

__global__ void mask_write_kernel(int32_t* __restrict__ mask, MaskBits m) {
  for (int i = threadIdx.x; i < 3 * m.E; i += blockDim.x) {
    const int j = i / m.E, e = i - j * m.E;
    mask[i] = (m.bits[j][e >> 5] >> (e & 31)) & 1u;
  }
}

// The layer's tokens into coherent pinned host memory for the host
// executor, written by the GPU itself (no copy-engine transfer).
__global__ void rows_to_host_kernel(const float4* __restrict__ src, float4* __restrict__ dst, int n4) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += gridDim.x * blockDim.x) dst[i] = src[i];
}

constexpr int kEventRing = 256;
constexpr int kCtlStagePairs = 1024;  // T*k of one cache_decode_layer call
constexpr int kFlagPad = 64;          // the ids-ready flag sits on a line of its own after the ids

}  // namespace moe

using namespace moe;

struct moe_cache {
  int device = 0;
  int L = 0, E = 0, n_slots = 0, qtype = 0, H = 0, I = 0;
  size_t slot_bytes = 0;
  uint8_t* d_pool = nullptr;
  const uint8_t* h_pool = nullptr;
  int32_t* d_table = nullptr;            // [L][E]
  std::vector<int32_t> table;            // host shadow: key -> slot or -1
  std::vector<int> slot_key;             // slot -> key or -1
  std::vector<uint64_t> stamp;           // key -> recency stamp
  std::vector<uint64_t> protect;         // key -> lookup epoch
  std::set<std::pair<uint64_t, int>> lru;  // (stamp, key) of resident keys
  std::vector<int> free_fifo;            // free slots, oldest release first
  size_t free_head = 0;
  struct Pending { int slot; int victim_key; };
  std::unordered_map<int, Pending> pending;  // key -> destination (copy not issued)
  std::vector<int> slot_event;           // slot -> index into events or -1
  std::vector<int> slot_ready;           // slot -> index into copy_events of its last copy, or -1
  std::vector<int> layer_slots;          // slots touched by the current lookup
  hipEvent_t events[kEventRing] = {};       // layer-done events (compute stream)
  hipEvent_t copy_events[kEventRing] = {};  // copy-done events (copy streams)
  int next_event = 0, next_copy_event = 0;
  uint64_t clock = 0, epoch = 0;
  int64_t hits = 0, misses = 0;
  // staging of cache_decode_layer, allocated with the cache: the routed ids
  // (pinned host), the hit / miss expert masks (pinned host and device)
  int32_t* h_ids = nullptr;   // coherent [kCtlStagePairs + kFlagPad]: ids, then the ids-ready flag
  int32_t ids_seq = 0;        // the last value the routing kernel was told to raise the flag to
  int32_t* h_mask = nullptr;  // [3][E]: hits, copied misses, host misses
  int32_t* d_mask = nullptr;  // [3][E]
  hipEvent_t ids_ready = nullptr;
  // misses computed on the host (cache_set_miss_policy), staging made when
  // such a policy is first set
  int policy = MOE_MISS_COPY;
  int host_threads = 1;
  float* h_x = nullptr;   // pinned [kCtlStagePairs][H]: the layer's tokens
  float* h_y = nullptr;   // pinned [kCtlStagePairs][H]: host-computed pair rows
  float* d_yh = nullptr;  // device [kCtlStagePairs][H]: destination of the copy-rate calibration
  std::vector<float> h_scratch;  // [kCtlStagePairs][I]
  hipEvent_t copy_t0 = nullptr, copy_t1 = nullptr;  // around one layer's copies
  int timed_copies = 0;                             // copies between them, not yet read
  double rate_pcie = 0.0, rate_host = 0.0;          // bytes per second
  int64_t n_copied = 0, n_host = 0;
  std::vector<int32_t> last_copy, last_host;
  int last_host_only = 0;  // the first of last_host that were not inserted
  std::deque<int> inflight;  // copy_events of background copies, oldest first
  // MOE_MISS_HOST_COPY's background copies go through the HSA runtime's
  // asynchronous copy with a completion signal the host polls, not through a
  // HIP stream: an event recorded on a copy stream becomes a barrier packet
  // on that stream's hardware queue, and when the caller's compute stream
  // shares the queue (HIP shares a few queues among all streams) its
  // kernels would wait for the copy.  Set up with the policy; if it cannot
  // be, those copies take the copy stream.
  bool hsa_ok = false;
  hsa_agent_t hsa_gpu{}, hsa_cpu{};
  hsa_signal_t hsa_sig[kEventRing] = {};
  int next_sig = 0;
  std::vector<int> slot_sig;  // slot -> hsa_sig of its last background copy, or -1
  std::deque<int> inflight_sig;
};

// Background copies allowed in flight under MOE_MISS_HOST_COPY; a miss
// beyond them is computed on the host and not inserted.
constexpr int kCopyBacklog = 8;

static bool sig_done(const moe_cache* c, int si) { return hsa_signal_load_scacquire(c->hsa_sig[si]) == 0; }
static void sig_wait(const moe_cache* c, int si) {
  while (hsa_signal_wait_scacquire(c->hsa_sig[si], HSA_SIGNAL_CONDITION_EQ, 0, UINT64_MAX, HSA_WAIT_STATE_BLOCKED) != 0) {
  }
}
// Every background copy has landed (before the pool is moved or freed).
static void wait_all_sigs(moe_cache* c) {
  if (!c->hsa_ok) return;
  for (int i = 0; i < kEventRing; ++i) sig_wait(c, i);
  c->inflight_sig.clear();
  std::fill(c->slot_sig.begin(), c->slot_sig.end(), -1);
}

struct AgentSearch {
  int domain, bus, device;
  hsa_agent_t gpu{}, cpu{};
  bool have_gpu = false, have_cpu = false;
};
static hsa_status_t find_agents(hsa_agent_t a, void* data) {
  auto* q = static_cast<AgentSearch*>(data);
  hsa_device_type_t type;
  if (hsa_agent_get_info(a, HSA_AGENT_INFO_DEVICE, &type) != HSA_STATUS_SUCCESS) return HSA_STATUS_SUCCESS;
  if (type == HSA_DEVICE_TYPE_CPU && !q->have_cpu) {
    q->cpu = a;
    q->have_cpu = true;
  } else if (type == HSA_DEVICE_TYPE_GPU && !q->have_gpu) {
    uint32_t bdf = 0, domain = 0;
    if (hsa_agent_get_info(a, (hsa_agent_info_t)HSA_AMD_AGENT_INFO_BDFID, &bdf) == HSA_STATUS_SUCCESS &&
        hsa_agent_get_info(a, (hsa_agent_info_t)HSA_AMD_AGENT_INFO_DOMAIN, &domain) == HSA_STATUS_SUCCESS &&
        (int)domain == q->domain && (int)(bdf >> 8) == q->bus && (int)((bdf >> 3) & 31) == q->device) {
      q->gpu = a;
      q->have_gpu = true;
    }
  }
  return HSA_STATUS_SUCCESS;
}

namespace moe {
bool hsa_agents_of(int device, hsa_agent_t* gpu, hsa_agent_t* cpu) {
  AgentSearch q{};
  if (hipDeviceGetAttribute(&q.domain, hipDeviceAttributePciDomainID, device) != hipSuccess ||
      hipDeviceGetAttribute(&q.bus, hipDeviceAttributePciBusId, device) != hipSuccess ||
      hipDeviceGetAttribute(&q.device, hipDeviceAttributePciDeviceId, device) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  if (hsa_iterate_agents(find_agents, &q) != HSA_STATUS_SUCCESS || !q.have_gpu || !q.have_cpu) return false;
  *gpu = q.gpu;
  *cpu = q.cpu;
  return true;
}
}  // namespace moe

// The HSA agents of the cache's device and of the host, and the signals.
static void hsa_setup(moe_cache* c) {
  if (c->hsa_ok) return;
  if (hsa_init() != HSA_STATUS_SUCCESS) return;
  hsa_agent_t gpu{}, cpu{};
  if (!hsa_agents_of(c->device, &gpu, &cpu)) {
    hsa_shut_down();
    return;
  }
  int made = 0;
  for (; made < kEventRing; ++made)
    if (hsa_signal_create(0, 0, nullptr, &c->hsa_sig[made]) != HSA_STATUS_SUCCESS) break;
  if (made < kEventRing) {
    for (int i = 0; i < made; ++i) hsa_signal_destroy(c->hsa_sig[i]);
    hsa_shut_down();
    return;
  }
  c->hsa_gpu = gpu;
  c->hsa_cpu = cpu;
  c->slot_sig.assign(c->slot_key.size(), -1);
  c->hsa_ok = true;
}

static int pop_free(moe_cache* c) {
  if (c->free_head >= c->free_fifo.size()) return -1;
  const int s = c->free_fifo[c->free_head++];
  if (c->free_head > 4096 && c->free_head * 2 > c->free_fifo.size()) {
    c->free_fifo.erase(c->free_fifo.begin(), c->free_fifo.begin() + (long)c->free_head);
    c->free_head = 0;
  }
  return s;
}

extern "C" {

int cache_slot_table_destroy(moe_cache* c);

int cache_slot_table_create(int L, int E, int n_slots, int qtype, int H, int I, void* d_pool,
                            const void* h_pool, moe_cache** out) {
  clear_error();
  if (!out) return set_error(MOE_ERR_INVALID_ARG, "cache_slot_table_create: out is NULL");
  if (!qtype_supported(qtype))
    return set_error(MOE_ERR_UNSUPPORTED_QTYPE, "cache_slot_table_create: block type %d is not supported", qtype);
  if (L < 1 || E < 1 || E > kMaxE || n_slots < 1)
    return set_error(MOE_ERR_INVALID_ARG, "cache_slot_table_create: L=%d E=%d n_slots=%d", L, E, n_slots);
  if (H <= 0 || I <= 0 || H % kGroupWeights || I % kGroupWeights)
    return set_error(MOE_ERR_INVALID_ARG, "cache_slot_table_create: H=%d I=%d must be multiples of %d", H, I,
                     kGroupWeights);
  if (!d_pool || !h_pool) return set_error(MOE_ERR_INVALID_ARG, "cache_slot_table_create: NULL pool");
  if (!aligned(d_pool, 16)) return set_error(MOE_ERR_ALIGNMENT, "cache_slot_table_create: d_pool not 16-byte aligned");
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, h_pool);
  if (e != hipSuccess || attr.type != hipMemoryTypeHost) {
    (void)hipGetLastError();
    return set_error(MOE_ERR_NOT_PINNED,
                     "cache_slot_table_create: the host expert pool is not pinned (allocate it with hipHostMalloc)");
  }
  int dev = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return hip_error(e, "hipGetDevice");
  moe_cache* c = new moe_cache;
  c->device = dev;
  c->L = L; c->E = E; c->n_slots = n_slots; c->qtype = qtype; c->H = H; c->I = I;
  c->slot_bytes = slot_bytes_of(qtype, H, I);
  c->d_pool = (uint8_t*)d_pool;
  c->h_pool = (const uint8_t*)h_pool;
  const int keys = L * E;
  c->table.assign(keys, -1);
  c->stamp.assign(keys, 0);
  c->protect.assign(keys, 0);
  c->slot_key.assign(n_slots + 2, -1);
  c->slot_event.assign(n_slots + 2, -1);
  c->slot_ready.assign(n_slots + 2, -1);
  for (int s = 0; s < n_slots + 2; ++s) c->free_fifo.push_back(s);
  if ((e = hipMalloc(&c->d_table, sizeof(int32_t) * keys)) != hipSuccess) {
    delete c;
    return hip_error(e, "hipMalloc(slot table)");
  }
  if ((e = hipMemcpy(c->d_table, c->table.data(), sizeof(int32_t) * keys, hipMemcpyHostToDevice)) != hipSuccess) {
    (void)hipFree(c->d_table);
    delete c;
    return hip_error(e, "hipMemcpy(slot table)");
  }
  for (int i = 0; i < 2 * kEventRing; ++i) {
    hipEvent_t* ev = i < kEventRing ? &c->events[i] : &c->copy_events[i - kEventRing];
    if ((e = hipEventCreateWithFlags(ev, hipEventDisableTiming)) != hipSuccess) {
      cache_slot_table_destroy(c);
      return hip_error(e, "hipEventCreate");
    }
  }
  if ((e = hipHostMalloc((void**)&c->h_ids, sizeof(int32_t) * (kCtlStagePairs + kFlagPad), hipHostMallocCoherent)) !=
          hipSuccess ||
      (e = hipHostMalloc((void**)&c->h_mask, sizeof(int32_t) * 3 * E, hipHostMallocDefault)) != hipSuccess ||
      (e = hipMalloc(&c->d_mask, sizeof(int32_t) * 3 * E)) != hipSuccess ||
      (e = hipEventCreateWithFlags(&c->ids_ready, hipEventDisableTiming)) != hipSuccess) {
    cache_slot_table_destroy(c);
    return hip_error(e, "cache staging allocation");
  }
  std::fill(c->h_mask, c->h_mask + 3 * E, 0);
  std::fill(c->h_ids, c->h_ids + kCtlStagePairs + kFlagPad, 0);
  *out = c;
  return MOE_OK;
}

int cache_slot_table_destroy(moe_cache* c) {
  clear_error();
  if (!c) return MOE_OK;
  (void)hipDeviceSynchronize();
  if (c->hsa_ok) {
    wait_all_sigs(c);
    for (int i = 0; i < kEventRing; ++i) hsa_signal_destroy(c->hsa_sig[i]);
    hsa_shut_down();
  }
  for (int i = 0; i < kEventRing; ++i) {
    if (c->events[i]) (void)hipEventDestroy(c->events[i]);
    if (c->copy_events[i]) (void)hipEventDestroy(c->copy_events[i]);
  }
  if (c->d_table) (void)hipFree(c->d_table);
  if (c->h_ids) (void)hipHostFree(c->h_ids);
  if (c->h_mask) (void)hipHostFree(c->h_mask);
  if (c->d_mask) (void)hipFree(c->d_mask);
  if (c->ids_ready) (void)hipEventDestroy(c->ids_ready);
  if (c->h_x) (void)hipHostFree(c->h_x);
  if (c->h_y) (void)hipHostFree(c->h_y);
  if (c->d_yh) (void)hipFree(c->d_yh);
  if (c->copy_t0) (void)hipEventDestroy(c->copy_t0);
  if (c->copy_t1) (void)hipEventDestroy(c->copy_t1);
  delete c;
  return MOE_OK;
}

const int32_t* cache_slot_table_device(moe_cache* c) { return c ? c->d_table : nullptr; }

int cache_slot_table_stats(moe_cache* c, int64_t* hits, int64_t* misses) {
  clear_error();
  if (!c) return set_error(MOE_ERR_INVALID_ARG, "cache_slot_table_stats: cache is NULL");
  if (hits) *hits = c->hits;
  if (misses) *misses = c->misses;
  return MOE_OK;
}

// The LRU lookup of cache_slot_table_lookup.  Ids marked in `host` (or all
// none when it is NULL) are misses computed on the host: counted as misses
// and otherwise left out (no refresh, no insertion), slot -1.
static int lookup_impl(moe_cache* c, int layer, const int32_t* ids, int n, const int32_t* host, int32_t* slots_out,
                       int32_t* miss_ids, int* n_miss) {
  if (!c) return set_error(MOE_ERR_INVALID_ARG, "cache_slot_table_lookup: cache is NULL");
  if (layer < 0 || layer >= c->L || n < 0 || (n > 0 && (!ids || !slots_out)) || !n_miss)
    return set_error(MOE_ERR_INVALID_ARG, "cache_slot_table_lookup: layer=%d n=%d", layer, n);
  for (int i = 0; i < n; ++i)
    if (ids[i] < 0 || ids[i] >= c->E)
      return set_error(MOE_ERR_INVALID_ARG, "cache_slot_table_lookup: expert id %d of layer %d not in [0, %d)",
                       ids[i], layer, c->E);
  {
    std::vector<int32_t> distinct;
    for (int i = 0; i < n; ++i)
      if (!host || !host[ids[i]]) distinct.push_back(ids[i]);
    std::sort(distinct.begin(), distinct.end());
    const long nd = std::unique(distinct.begin(), distinct.end()) - distinct.begin();
    if (nd > c->n_slots)
      return set_error(MOE_ERR_CAPACITY, "cache_slot_table_lookup: layer %d needs %ld distinct experts, cache holds %d",
                       layer, nd, c->n_slots);
  }
  if (!c->layer_slots.empty())
    return set_error(MOE_ERR_INVALID_ARG,
                     "cache_slot_table_lookup: the previous lookup's layer was not marked done "
                     "(cache_mark_layer_done) so its slots could be overwritten while in use");
  ++c->epoch;
  int nm = 0;
  for (int i = 0; i < n; ++i) {
    const int key = layer * c->E + ids[i];
    if (host && host[ids[i]]) {
      ++c->misses;
      slots_out[i] = -1;
      continue;
    }
    ++c->clock;
    if (c->table[key] >= 0) {
      ++c->hits;
      c->lru.erase({c->stamp[key], key});
    } else {
      ++c->misses;
      int victim = -1;
      if ((int)c->lru.size() >= c->n_slots) {
        for (auto it = c->lru.begin(); it != c->lru.end(); ++it) {
          if (c->protect[it->second] != c->epoch) {
            victim = it->second;
            break;
          }
        }
        if (victim < 0)
          return set_error(MOE_ERR_CAPACITY,
                           "cache_slot_table_lookup: all %d slots hold experts of layer %d's current lookup",
                           c->n_slots, layer);
        const int vs = c->table[victim];
        c->lru.erase({c->stamp[victim], victim});
        c->table[victim] = -1;
        c->slot_key[vs] = -1;
        c->free_fifo.push_back(vs);
        auto pv = c->pending.find(victim);
        if (pv != c->pending.end()) c->pending.erase(pv);  // evicted before its copy was issued
      }
      const int s = pop_free(c);
      c->table[key] = s;
      c->slot_key[s] = key;
      c->pending[key] = moe_cache::Pending{s, victim};
      if (miss_ids) {
        bool seen = false;
        for (int m = 0; m < nm; ++m) seen |= miss_ids[m] == ids[i];
        if (!seen) miss_ids[nm++] = ids[i];
      } else {
        ++nm;
      }
    }
    c->stamp[key] = c->clock;
    c->protect[key] = c->epoch;
    c->lru.insert({c->clock, key});
    slots_out[i] = c->table[key];
    c->layer_slots.push_back(c->table[key]);
  }
  *n_miss = nm;
  return MOE_OK;
}

int cache_slot_table_lookup(moe_cache* c, int layer, const int32_t* ids, int n, int32_t* slots_out,
                            int32_t* miss_ids, int* n_miss) {
  clear_error();
  return lookup_impl(c, layer, ids, n, nullptr, slots_out, miss_ids, n_miss);
}

static int issue_copy(moe_cache* c, int key, moe_cache::Pending pd, hipStream_t cs, hipStream_t ks,
                      bool compute_waits);

int prefetch_expert(moe_cache* c, int layer, int expert, void* copy_stream, void* compute_stream,
                    int32_t* slot_out) {
  clear_error();
  if (!c) return set_error(MOE_ERR_INVALID_ARG, "prefetch_expert: cache is NULL");
  if (layer < 0 || layer >= c->L || expert < 0 || expert >= c->E)
    return set_error(MOE_ERR_INVALID_ARG, "prefetch_expert: layer=%d expert=%d", layer, expert);
  const int key = layer * c->E + expert;
  auto it = c->pending.find(key);
  if (it == c->pending.end()) {
    if (c->table[key] < 0)
      return set_error(MOE_ERR_NOT_RESIDENT,
                       "prefetch_expert: layer %d expert %d was not looked up (no destination slot)", layer, expert);
    if (slot_out) *slot_out = c->table[key];
    return MOE_OK;  // resident already
  }
  const moe_cache::Pending pd = it->second;
  c->pending.erase(it);
  int rc = issue_copy(c, key, pd, (hipStream_t)copy_stream, (hipStream_t)compute_stream, true);
  if (rc) return rc;
  if (slot_out) *slot_out = pd.slot;
  return MOE_OK;
}

// The copy of key into its destination slot on copy stream cs, after the
// slot's previous reader; the slot table update on compute stream ks.  With
// compute_waits, ks waits for the copy (the expert is used in stream order);
// without, the caller must not let a kernel read the slot before the copy's
// event (slot_ready) has completed.
static int issue_copy(moe_cache* c, int key, moe_cache::Pending pd, hipStream_t cs, hipStream_t ks,
                      bool compute_waits) {
  hipError_t e = hipSetDevice(c->device);
  if (e != hipSuccess) return hip_error(e, "hipSetDevice");
  // a background copy into the slot (HSA, no stream to wait on) comes first
  if (c->hsa_ok && c->slot_sig[pd.slot] >= 0) {
    sig_wait(c, c->slot_sig[pd.slot]);
    c->slot_sig[pd.slot] = -1;
  }
  // an earlier copy into the slot (possibly on another stream) comes first
  if (c->slot_ready[pd.slot] >= 0 &&
      (e = hipStreamWaitEvent(cs, c->copy_events[c->slot_ready[pd.slot]], 0)) != hipSuccess)
    return hip_error(e, "hipStreamWaitEvent(earlier copy)");
  // the slot's previous reader must be done before the copy overwrites it
  if (c->slot_event[pd.slot] >= 0) {
    if ((e = hipStreamWaitEvent(cs, c->events[c->slot_event[pd.slot]], 0)) != hipSuccess)
      return hip_error(e, "hipStreamWaitEvent(copy)");
  }
  if ((e = hipMemcpyAsync(c->d_pool + (size_t)pd.slot * c->slot_bytes, c->h_pool + (size_t)key * c->slot_bytes,
                          c->slot_bytes, hipMemcpyHostToDevice, cs)) != hipSuccess)
    return hip_error(e, "hipMemcpyAsync(expert)");
  const int ce = c->next_copy_event;
  hipEvent_t done = c->copy_events[ce];
  c->next_copy_event = (c->next_copy_event + 1) % kEventRing;
  if ((e = hipEventRecord(done, cs)) != hipSuccess) return hip_error(e, "hipEventRecord(copy)");
  c->slot_ready[pd.slot] = ce;
  if (compute_waits && (e = hipStreamWaitEvent(ks, done, 0)) != hipSuccess)
    return hip_error(e, "hipStreamWaitEvent(compute)");
  TableUpdate u{};
  u.idx[u.n] = key; u.val[u.n] = pd.slot; ++u.n;
  if (pd.victim_key >= 0 && c->table[pd.victim_key] < 0) {
    u.idx[u.n] = pd.victim_key; u.val[u.n] = -1; ++u.n;
  }
  launch(table_update_kernel, 1, 64, 0, ks, c->d_table, u);
  return check_launch("table_update_kernel");
}

// A background copy of key into its destination slot through the HSA
// runtime (completion signal polled by the host), then the slot table
// update on compute stream ks.  The slot's earlier copy is a dependency of
// the copy itself; its earlier readers have finished, which the host
// checks (the LRU evicts only keys of earlier layers, whose kernels precede
// this layer's routing, already complete).  No kernel may read the slot
// before the signal reads zero.
static int issue_copy_hsa(moe_cache* c, int key, moe_cache::Pending pd, hipStream_t ks) {
  hipError_t e = hipSetDevice(c->device);
  if (e != hipSuccess) return hip_error(e, "hipSetDevice");
  if (c->slot_ready[pd.slot] >= 0) {  // an earlier copy on a stream
    if ((e = hipEventSynchronize(c->copy_events[c->slot_ready[pd.slot]])) != hipSuccess)
      return hip_error(e, "hipEventSynchronize(earlier copy)");
    c->slot_ready[pd.slot] = -1;
  }
  if (c->slot_event[pd.slot] >= 0 && (e = hipEventSynchronize(c->events[c->slot_event[pd.slot]])) != hipSuccess)
    return hip_error(e, "hipEventSynchronize(reader)");
  const int si = c->next_sig;
  c->next_sig = (c->next_sig + 1) % kEventRing;
  sig_wait(c, si);  // the ring is far longer than the backlog: normally done
  hsa_signal_t dep[1];
  uint32_t n_dep = 0;
  if (c->slot_sig[pd.slot] >= 0 && !sig_done(c, c->slot_sig[pd.slot])) dep[n_dep++] = c->hsa_sig[c->slot_sig[pd.slot]];
  hsa_signal_store_screlease(c->hsa_sig[si], 1);
  const hsa_status_t st = hsa_amd_memory_async_copy(c->d_pool + (size_t)pd.slot * c->slot_bytes, c->hsa_gpu,
                                                    c->h_pool + (size_t)key * c->slot_bytes, c->hsa_cpu,
                                                    c->slot_bytes, n_dep, n_dep ? dep : nullptr, c->hsa_sig[si]);
  if (st != HSA_STATUS_SUCCESS) {
    hsa_signal_store_screlease(c->hsa_sig[si], 0);
    return set_error(MOE_ERR_HIP, "hsa_amd_memory_async_copy(expert) failed (status %d)", (int)st);
  }
  c->slot_sig[pd.slot] = si;
  c->inflight_sig.push_back(si);
  TableUpdate u{};
  u.idx[u.n] = key; u.val[u.n] = pd.slot; ++u.n;
  if (pd.victim_key >= 0 && c->table[pd.victim_key] < 0) {
    u.idx[u.n] = pd.victim_key; u.val[u.n] = -1; ++u.n;
  }
  launch(table_update_kernel, 1, 64, 0, ks, c->d_table, u);
  return check_launch("table_update_kernel");
}

int cache_mark_layer_done(moe_cache* c, int layer, void* compute_stream) {
  clear_error();
  if (!c) return set_error(MOE_ERR_INVALID_ARG, "cache_mark_layer_done: cache is NULL");
  if (layer < 0 || layer >= c->L) return set_error(MOE_ERR_INVALID_ARG, "cache_mark_layer_done: layer=%d", layer);
  hipError_t e = hipSetDevice(c->device);
  if (e != hipSuccess) return hip_error(e, "hipSetDevice");
  const int ev = c->next_event;
  c->next_event = (c->next_event + 1) % kEventRing;
  if ((e = hipEventRecord(c->events[ev], (hipStream_t)compute_stream)) != hipSuccess)
    return hip_error(e, "hipEventRecord(layer done)");
  for (int s : c->layer_slots) c->slot_event[s] = ev;
  c->layer_slots.clear();
  ++c->epoch;  // the layer's keys are no longer protected
  return MOE_OK;
}

int cache_slot_table_resize(moe_cache* c, int n_slots, void* d_pool, void* stream) {
  clear_error();
  if (!c) return set_error(MOE_ERR_INVALID_ARG, "cache_slot_table_resize: cache is NULL");
  if (n_slots < 1) return set_error(MOE_ERR_INVALID_ARG, "cache_slot_table_resize: n_slots=%d", n_slots);
  if (!c->layer_slots.empty() || !c->pending.empty())
    return set_error(MOE_ERR_INVALID_ARG,
                     "cache_slot_table_resize: a lookup is in progress (copies not issued or layer not marked done)");
  uint8_t* pool = d_pool ? (uint8_t*)d_pool : c->d_pool;
  if (!aligned(pool, 16)) return set_error(MOE_ERR_ALIGNMENT, "cache_slot_table_resize: d_pool not 16-byte aligned");
  const bool same = pool == c->d_pool;
  const int count = n_slots + 2;
  // the n_slots most recently used keys stay; the rest are evicted
  std::vector<int> mru;
  for (auto it = c->lru.rbegin(); it != c->lru.rend(); ++it) mru.push_back(it->second);
  const int kept = std::min((int)mru.size(), n_slots);
  std::vector<int32_t> table = c->table;
  for (int i = kept; i < (int)mru.size(); ++i) table[mru[i]] = -1;
  std::vector<int> slot_key(count, -1);
  std::vector<int2> moves;
  std::vector<int> order(mru.begin(), mru.begin() + kept);
  std::sort(order.begin(), order.end(), [&](int a, int b) { return table[a] < table[b]; });
  if (same) {  // keys already below the new slot count stay where they are
    std::vector<int> movers;
    for (int key : order) {
      if (table[key] < count) slot_key[table[key]] = key;
      else movers.push_back(key);
    }
    int next = 0;
    for (int key : movers) {
      while (slot_key[next] >= 0) ++next;
      moves.push_back(make_int2(table[key], next));
      table[key] = next;
      slot_key[next] = key;
    }
  } else {  // every kept key is copied, packed from slot 0 in its old slot order
    for (int i = 0; i < kept; ++i) {
      moves.push_back(make_int2(table[order[i]], i));
      table[order[i]] = i;
      slot_key[i] = order[i];
    }
  }
  hipError_t e = hipSetDevice(c->device);
  if (e != hipSuccess) return hip_error(e, "hipSetDevice");
  // every earlier reader of the pool and every expert copy, on any stream
  // or through the HSA runtime
  if ((e = hipDeviceSynchronize()) != hipSuccess) return hip_error(e, "hipDeviceSynchronize");
  wait_all_sigs(c);
  hipStream_t st = (hipStream_t)stream;
  int2* d_moves = nullptr;
  if (!moves.empty()) {
    if ((e = hipMalloc(&d_moves, sizeof(int2) * moves.size())) != hipSuccess) return hip_error(e, "hipMalloc(moves)");
    e = hipMemcpyAsync(d_moves, moves.data(), sizeof(int2) * moves.size(), hipMemcpyHostToDevice, st);
    if (e != hipSuccess) {
      (void)hipFree(d_moves);
      return hip_error(e, "hipMemcpyAsync(moves)");
    }
    const long long words = (long long)(c->slot_bytes / 16);
    const int bx = (int)std::min<long long>((words + 1023) / 1024, 1024);
    const int by = (int)std::min<size_t>(moves.size(), 4096);
    launch(slot_move_kernel, dim3(bx, by), 256, 0, st, (const uint4*)c->d_pool, (uint4*)pool,
           (const int2*)d_moves, (int)moves.size(), words);
    int rc = check_launch("slot_move_kernel");
    if (rc) {
      (void)hipStreamSynchronize(st);
      (void)hipFree(d_moves);
      return rc;
    }
  }
  e = hipMemcpyAsync(c->d_table, table.data(), sizeof(int32_t) * table.size(), hipMemcpyHostToDevice, st);
  const hipError_t es = hipStreamSynchronize(st);
  if (d_moves) (void)hipFree(d_moves);
  if (e != hipSuccess) return hip_error(e, "hipMemcpyAsync(slot table)");
  if (es != hipSuccess) return hip_error(es, "hipStreamSynchronize");
  for (int i = kept; i < (int)mru.size(); ++i) c->lru.erase({c->stamp[mru[i]], mru[i]});
  c->table.swap(table);
  c->slot_key.swap(slot_key);
  c->slot_event.assign(count, -1);
  c->slot_ready.assign(count, -1);
  if (c->hsa_ok) c->slot_sig.assign(count, -1);
  c->free_fifo.clear();
  c->free_head = 0;
  for (int s = 0; s < count; ++s)
    if (c->slot_key[s] < 0) c->free_fifo.push_back(s);
  c->n_slots = n_slots;
  c->d_pool = pool;
  return MOE_OK;
}

static double now_s() {
  return std::chrono::duration<double>(std::chrono::steady_clock::now().time_since_epoch()).count();
}

static void update_rate(double& rate, double sample) {
  if (!(sample > 0.0) || !std::isfinite(sample)) return;
  rate = rate > 0.0 ? 0.75 * rate + 0.25 * sample : sample;
}

// Bytes per second of expert copies and of the host executor, measured
// once when a policy that needs them is set (the running estimates then
// follow every layer).
static int calibrate_rates(moe_cache* c) {
  hipError_t e = hipSetDevice(c->device);
  if (e != hipSuccess) return hip_error(e, "hipSetDevice");
  const size_t stage = sizeof(float) * (size_t)kCtlStagePairs * c->H;
  const size_t chunk = std::min(c->slot_bytes, stage);
  double best = 1e30;
  for (int r = 0; r < 3; ++r) {
    const double t0 = now_s();
    const uint8_t* src = c->h_pool + (size_t)(r % (c->L * c->E)) * c->slot_bytes;  // chunk <= slot_bytes
    if ((e = hipMemcpy(c->d_yh, src, chunk, hipMemcpyHostToDevice)) != hipSuccess)
      return hip_error(e, "hipMemcpy(calibration)");
    best = std::min(best, now_s() - t0);
  }
  c->rate_pcie = (double)chunk / best;
  std::fill(c->h_x, c->h_x + c->H, 0.0f);
  best = 1e30;
  for (int r = 0; r < 3; ++r) {
    const uint8_t* slot = c->h_pool + (size_t)(r % (c->L * c->E)) * c->slot_bytes;
    const int one = 1, tok0 = 0;
    const int* tp = &tok0;
    const double t0 = now_s();
    int rc = host_experts_ffn(c->qtype, c->H, c->I, 1, &slot, &one, &tp, &tp, c->h_x, c->h_y, c->h_scratch.data(),
                              c->host_threads, true);
    if (rc) return rc;
    best = std::min(best, now_s() - t0);
  }
  c->rate_host = (double)c->slot_bytes / best;
  return MOE_OK;
}

int cache_set_miss_policy(moe_cache* c, int policy, int host_threads) {
  clear_error();
  if (!c) return set_error(MOE_ERR_INVALID_ARG, "cache_set_miss_policy: cache is NULL");
  if (policy != MOE_MISS_COPY && policy != MOE_MISS_HOST && policy != MOE_MISS_QSTAR && policy != MOE_MISS_HOST_COPY)
    return set_error(MOE_ERR_INVALID_ARG, "cache_set_miss_policy: policy %d unknown", policy);
  if (host_threads < 0) return set_error(MOE_ERR_INVALID_ARG, "cache_set_miss_policy: host_threads=%d", host_threads);
  c->host_threads = host_threads == 0 ? default_host_threads() : host_threads;
  if (c->policy == MOE_MISS_HOST_COPY && policy != MOE_MISS_HOST_COPY) {
    // the other policies read a resident slot without checking that its
    // copy has landed: let every background copy land first
    hipError_t e = hipSetDevice(c->device);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_error(e, "cache_set_miss_policy: background copies");
    wait_all_sigs(c);
    c->inflight.clear();
    std::fill(c->slot_ready.begin(), c->slot_ready.end(), -1);
  }
  if (policy != MOE_MISS_COPY && !c->h_x) {
    hipError_t e = hipSetDevice(c->device);
    if (e != hipSuccess) return hip_error(e, "hipSetDevice");
    const size_t rows = (size_t)kCtlStagePairs * c->H;
    // coherent: the GPU writes h_x and reads h_y in place
    if ((e = hipHostMalloc((void**)&c->h_x, sizeof(float) * rows, hipHostMallocCoherent)) != hipSuccess ||
        (e = hipHostMalloc((void**)&c->h_y, sizeof(float) * rows, hipHostMallocCoherent)) != hipSuccess ||
        (e = hipMalloc(&c->d_yh, sizeof(float) * rows)) != hipSuccess ||
        (e = hipEventCreate(&c->copy_t0)) != hipSuccess || (e = hipEventCreate(&c->copy_t1)) != hipSuccess) {
      if (c->h_x) (void)hipHostFree(c->h_x);
      if (c->h_y) (void)hipHostFree(c->h_y);
      if (c->d_yh) (void)hipFree(c->d_yh);
      if (c->copy_t0) (void)hipEventDestroy(c->copy_t0);
      if (c->copy_t1) (void)hipEventDestroy(c->copy_t1);
      c->h_x = c->h_y = c->d_yh = nullptr;
      c->copy_t0 = c->copy_t1 = nullptr;
      return hip_error(e, "cache_set_miss_policy: staging");
    }
    c->h_scratch.assign((size_t)kCtlStagePairs * c->I, 0.0f);
  }
  if (policy == MOE_MISS_HOST_COPY) hsa_setup(c);
  if (policy == MOE_MISS_QSTAR && (c->rate_pcie <= 0.0 || c->rate_host <= 0.0)) {
    int rc = calibrate_rates(c);
    if (rc) return rc;
  }
  c->policy = policy;
  return MOE_OK;
}

int cache_miss_stats(moe_cache* c, int64_t* copied, int64_t* host, double* pcie_gbs, double* host_gbs) {
  clear_error();
  if (!c) return set_error(MOE_ERR_INVALID_ARG, "cache_miss_stats: cache is NULL");
  if (copied) *copied = c->n_copied;
  if (host) *host = c->n_host;
  if (pcie_gbs) *pcie_gbs = c->rate_pcie / 1e9;
  if (host_gbs) *host_gbs = c->rate_host / 1e9;
  return MOE_OK;
}

int cache_last_misses(moe_cache* c, int32_t* copy_ids, int* n_copy, int32_t* host_ids, int* n_host,
                      int* n_host_only) {
  clear_error();
  if (!c || !n_copy || !n_host) return set_error(MOE_ERR_INVALID_ARG, "cache_last_misses: NULL argument");
  *n_copy = (int)c->last_copy.size();
  *n_host = (int)c->last_host.size();
  if (n_host_only) *n_host_only = c->last_host_only;
  if (copy_ids) std::copy(c->last_copy.begin(), c->last_copy.end(), copy_ids);
  if (host_ids) std::copy(c->last_host.begin(), c->last_host.end(), host_ids);
  return MOE_OK;
}

// How many of n missing experts go to the host: the split that finishes
// both sides soonest at the measured rates (copies and host work run at the
// same time), the fewest host experts on a tie.
static int qstar_split(const moe_cache* c, int n) {
  const double B = (double)c->slot_bytes;
  const double kHostFixed = 20e-6;  // waking the workers, moving the rows back
  int best = 0;
  double best_t = n * B / c->rate_pcie;
  for (int m = 1; m <= n; ++m) {
    const double t = std::max((n - m) * B / c->rate_pcie, m * B / c->rate_host + kHostFixed);
    if (t < best_t) {
      best_t = t;
      best = m;
    }
  }
  return best;
}

int cache_decode_layer(moe_cache* c, moe_ctx* ctx, int layer, const float* x, const float* router_w,
                       const float* bias, const float* logits_in, int T, int k, float* logits_out,
                       int32_t* topk_ids, float* topk_w, int32_t* expert_offsets, int32_t* sorted_pairs,
                       int32_t* pair_pos, int32_t* active, float* y_pairs, void* ws, size_t ws_bytes, float* out,
                       void* copy_stream, void* compute_stream) {
  clear_error();
  if (!c || !ctx) return set_error(MOE_ERR_INVALID_ARG, "cache_decode_layer: cache or ctx is NULL");
  if (layer < 0 || layer >= c->L) return set_error(MOE_ERR_INVALID_ARG, "cache_decode_layer: layer=%d", layer);
  if (T < 0 || k < 1 || (long long)T * k > kCtlStagePairs)
    return set_error(MOE_ERR_INVALID_ARG, "cache_decode_layer: T*k must be in [0, %d] (T=%d k=%d)", kCtlStagePairs,
                     T, k);
  if (T == 0) return MOE_OK;
  if (!out) return set_error(MOE_ERR_INVALID_ARG, "cache_decode_layer: out is NULL");
  const int E = c->E, P = T * k;
  const bool host_ok = c->policy != MOE_MISS_COPY;
  // the routing kernel writes the ids into the coherent staging and then
  // raises the flag to a value no earlier call used
  int32_t* flag = c->h_ids + kCtlStagePairs;
  const int32_t seq = c->ids_seq = c->ids_seq == INT32_MAX ? 1 : c->ids_seq + 1;
  int rc = route_permute_impl(ctx, x, MOE_DTYPE_F32, router_w, bias, logits_in, T, c->H, E, k, logits_out, topk_ids,
                              topk_w, expert_offsets, sorted_pairs, pair_pos, active, nullptr, 0, c->h_ids, flag, seq,
                              compute_stream);
  if (rc) return rc;
  hipStream_t cs = (hipStream_t)compute_stream, ps = (hipStream_t)copy_stream;
  hipError_t e;
  if (host_ok) {
    const int n4 = T * c->H / 4;
    launch(rows_to_host_kernel, std::min(64, (n4 + 255) / 256), 256, 0, cs, (const float4*)x, (float4*)c->h_x, n4);
    if ((rc = check_launch("rows_to_host_kernel"))) return rc;
  }
  if ((e = hipEventRecord(c->ids_ready, cs)) != hipSuccess) return hip_error(e, "hipEventRecord(ids)");
  // wait for the flag, not for the kernel's end; the event bounds the wait:
  // once it has completed the flag must be up
  for (unsigned it = 1;; ++it) {
    if (__atomic_load_n(flag, __ATOMIC_ACQUIRE) == seq) break;
    if (it % 64 == 0) {
      e = hipEventQuery(c->ids_ready);
      if (e == hipSuccess) {
        if (__atomic_load_n(flag, __ATOMIC_ACQUIRE) == seq) break;
        return set_error(MOE_ERR_HIP, "cache_decode_layer: the routing kernel ended without publishing the ids");
      }
      if (e != hipErrorNotReady) return hip_error(e, "hipEventQuery(ids)");
    }
  }
  // the previous layer's copies have long finished: fold their rate in
  if (c->timed_copies > 0 && hipEventQuery(c->copy_t1) == hipSuccess) {
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, c->copy_t0, c->copy_t1) == hipSuccess && ms > 0.0f)
      update_rate(c->rate_pcie, c->timed_copies * (double)c->slot_bytes / (ms * 1e-3));
    c->timed_copies = 0;
  }
  // which experts are missing, in the order the router named them
  std::vector<int32_t> host_flag(E, 0), missing;
  for (int i = 0; i < P; ++i) {
    const int id = c->h_ids[i];
    if (id < 0 || id >= E) return set_error(MOE_ERR_INVALID_ARG, "cache_decode_layer: routed id %d", id);
    if (c->table[layer * E + id] < 0 && std::find(missing.begin(), missing.end(), id) == missing.end())
      missing.push_back(id);
  }
  int n_host = 0;
  if (c->policy == MOE_MISS_HOST) {
    n_host = (int)missing.size();
  } else if (c->policy == MOE_MISS_QSTAR) {
    n_host = qstar_split(c, (int)missing.size());
  } else if (c->policy == MOE_MISS_HOST_COPY) {
    while (!c->inflight.empty() && hipEventQuery(c->copy_events[c->inflight.front()]) == hipSuccess)
      c->inflight.pop_front();
    while (!c->inflight_sig.empty() && sig_done(c, c->inflight_sig.front())) c->inflight_sig.pop_front();
    const int room = std::max(0, kCopyBacklog - (int)c->inflight.size() - (int)c->inflight_sig.size());
    n_host = std::max(0, (int)missing.size() - room);  // host only: not inserted
  }
  c->last_host.assign(missing.end() - n_host, missing.end());
  c->last_host_only = n_host;
  for (int id : c->last_host) host_flag[id] = 1;
  std::vector<int32_t> slots(P), miss(P);
  int n_miss = 0;
  if ((rc = lookup_impl(c, layer, c->h_ids, P, host_ok ? host_flag.data() : nullptr, slots.data(), miss.data(),
                        &n_miss)))
    return rc;
  c->last_copy.assign(miss.begin(), miss.begin() + n_miss);
  const bool both = c->policy == MOE_MISS_HOST_COPY;
  if (both) {
    // the misses are computed here (those past the backlog only here, the
    // others also copied for later); so is a hit whose copy has not landed
    // yet (its slot may not be read before that)
    c->last_host.insert(c->last_host.end(), c->last_copy.begin(), c->last_copy.end());
    for (int i = 0; i < P; ++i) {
      const int id = c->h_ids[i];
      if (std::find(c->last_host.begin(), c->last_host.end(), id) != c->last_host.end()) continue;
      const int slot = c->table[layer * E + id];
      if (slot < 0) continue;
      bool landed = true;
      if (c->hsa_ok && c->slot_sig[slot] >= 0) {
        if (sig_done(c, c->slot_sig[slot])) c->slot_sig[slot] = -1;
        else landed = false;
      }
      const int r = c->slot_ready[slot];
      if (r >= 0) {
        if (hipEventQuery(c->copy_events[r]) == hipSuccess) c->slot_ready[slot] = -1;
        else landed = false;
      }
      if (!landed) c->last_host.push_back(id);
    }
    n_host = (int)c->last_host.size();
  }
  c->n_copied += n_miss;
  c->n_host += n_host;
  // masks: resident experts, copied misses, host misses
  int32_t* hm = c->h_mask;
  std::fill(hm, hm + 3 * E, 0);
  for (int i = 0; i < P; ++i) hm[c->h_ids[i]] = 1;
  for (int i = 0; i < n_miss; ++i) {
    hm[miss[i]] = 0;
    hm[E + miss[i]] = both ? 0 : 1;
  }
  for (int id : c->last_host) {
    hm[id] = 0;
    hm[2 * E + id] = 1;
  }
  bool any_hit = false;
  for (int i = 0; i < P; ++i) any_hit |= hm[c->h_ids[i]] != 0;
  moe_ffn_args a{};
  a.pool_base = c->d_pool;
  a.slot_bytes = c->slot_bytes;
  a.n_slots = c->n_slots + 2;
  a.qtype = c->qtype;
  a.H = c->H;
  a.I = c->I;
  a.T = T;
  a.k = k;
  a.E = E;
  a.slot_table = c->d_table + (size_t)layer * E;
  a.x = x;
  a.x_dtype = MOE_DTYPE_F32;
  a.expert_offsets = expert_offsets;
  a.sorted_pairs = sorted_pairs;
  a.active = active;
  a.y_pairs = y_pairs;
  a.mode = MOE_MODE_DECODE;
  a.ws = ws;
  a.ws_bytes = ws_bytes;
  a.topk_w = topk_w;
  if (n_miss == 0 && n_host == 0) {  // every expert resident: one call with the combine folded in
    a.out = out;
    if ((rc = moe_expert_ffn(ctx, &a, compute_stream))) return rc;
    return cache_mark_layer_done(c, layer, compute_stream);
  }
  {
    MaskBits mb{};
    mb.E = E;
    for (int j = 0; j < 3; ++j)
      for (int id = 0; id < E; ++id)
        if (hm[j * E + id]) mb.bits[j][id >> 5] |= 1u << (id & 31);
    launch(mask_write_kernel, 1, 256, 0, cs, c->d_mask, mb);
    if ((rc = check_launch("mask_write_kernel"))) return rc;
  }
  if (any_hit) {  // the resident experts run while the misses are copied
    a.expert_mask = c->d_mask;
    if ((rc = moe_expert_ffn(ctx, &a, compute_stream))) return rc;
  }
  if (n_miss > 0 && both) {  // in the background: nothing on the compute stream waits for these
    for (int i = 0; i < n_miss; ++i) {
      const int key = layer * E + miss[i];
      auto it = c->pending.find(key);
      if (it == c->pending.end()) continue;
      const moe_cache::Pending pd = it->second;
      c->pending.erase(it);
      if (c->hsa_ok) {
        if ((rc = issue_copy_hsa(c, key, pd, cs))) return rc;
        continue;
      }
      if ((rc = issue_copy(c, key, pd, ps, cs, false))) return rc;
      c->inflight.push_back(c->slot_ready[pd.slot]);
    }
  } else if (n_miss > 0) {
    const bool timed = host_ok && c->timed_copies == 0;
    if (timed) {  // the copies' own time: wait for the slots' readers first
      for (int i = 0; i < n_miss; ++i) {
        const auto it = c->pending.find(layer * E + miss[i]);
        if (it == c->pending.end()) continue;
        const int slot = it->second.slot;
        if (c->slot_event[slot] >= 0 && (e = hipStreamWaitEvent(ps, c->events[c->slot_event[slot]], 0)) != hipSuccess)
          return hip_error(e, "hipStreamWaitEvent(copy)");
      }
      if ((e = hipEventRecord(c->copy_t0, ps)) != hipSuccess) return hip_error(e, "hipEventRecord(copy start)");
    }
    for (int i = 0; i < n_miss; ++i)
      if ((rc = prefetch_expert(c, layer, miss[i], copy_stream, compute_stream, nullptr))) return rc;
    if (timed) {
      if ((e = hipEventRecord(c->copy_t1, ps)) != hipSuccess) return hip_error(e, "hipEventRecord(copy end)");
      c->timed_copies = n_miss;
    }
    a.expert_mask = c->d_mask + E;
    if ((rc = moe_expert_ffn(ctx, &a, compute_stream))) return rc;
  }
  if (n_host > 0) {  // on the host cores while the GPU works through the above
    std::vector<const uint8_t*> hs(n_host);
    std::vector<std::vector<int>> tok(n_host), yrow(n_host);
    for (int j = 0; j < n_host; ++j) hs[j] = c->h_pool + (size_t)(layer * E + c->last_host[j]) * c->slot_bytes;
    for (int p = 0; p < P; ++p)
      for (int j = 0; j < n_host; ++j)
        if (c->h_ids[p] == c->last_host[j]) {
          tok[j].push_back(p / k);
          yrow[j].push_back(p);
        }
    std::vector<int> cnt(n_host);
    std::vector<const int*> tp(n_host), yp(n_host);
    for (int j = 0; j < n_host; ++j) {
      cnt[j] = (int)tok[j].size();
      tp[j] = tok[j].data();
      yp[j] = yrow[j].data();
    }
    // the tokens were staged behind the routing kernel
    if ((e = hipEventSynchronize(c->ids_ready)) != hipSuccess) return hip_error(e, "hipEventSynchronize(x)");
    const double t0 = now_s();
    if ((rc = host_experts_ffn(c->qtype, c->H, c->I, n_host, hs.data(), cnt.data(), tp.data(), yp.data(), c->h_x,
                               c->h_y, c->h_scratch.data(), c->host_threads, true)))
      return rc;
    update_rate(c->rate_host, n_host * (double)c->slot_bytes / (now_s() - t0));
    const int H4 = c->H / 4;
    launch(host_rows_kernel, dim3((H4 + 255) / 256, P), 256, 0, cs, (const float4*)c->h_y,
           (const int32_t*)(c->d_mask + 2 * E), (const int32_t*)topk_ids, (float4*)y_pairs, H4);
    if ((rc = check_launch("host_rows_kernel"))) return rc;
  }
  if ((rc = moe_combine(ctx, y_pairs, topk_w, T, k, c->H, out, compute_stream))) return rc;
  return cache_mark_layer_done(c, layer, compute_stream);
}

}  // extern "C"
