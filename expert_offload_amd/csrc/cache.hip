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
#include <set>
#include <unordered_map>
#include <vector>

#include "device_common.h"

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

constexpr int kEventRing = 256;
constexpr int kCtlStagePairs = 1024;  // T*k of one cache_decode_layer call

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
  std::vector<int> layer_slots;          // slots touched by the current lookup
  hipEvent_t events[kEventRing] = {};       // layer-done events (compute stream)
  hipEvent_t copy_events[kEventRing] = {};  // copy-done events (copy streams)
  int next_event = 0, next_copy_event = 0;
  uint64_t clock = 0, epoch = 0;
  int64_t hits = 0, misses = 0;
  // staging of cache_decode_layer, allocated with the cache: the routed ids
  // (pinned host), the hit / miss expert masks (pinned host and device)
  int32_t* h_ids = nullptr;   // [kCtlStagePairs]
  int32_t* h_mask = nullptr;  // [2][E]
  int32_t* d_mask = nullptr;  // [2][E]
  hipEvent_t ids_ready = nullptr;
};

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
  if ((e = hipHostMalloc((void**)&c->h_ids, sizeof(int32_t) * kCtlStagePairs, hipHostMallocDefault)) != hipSuccess ||
      (e = hipHostMalloc((void**)&c->h_mask, sizeof(int32_t) * 2 * E, hipHostMallocDefault)) != hipSuccess ||
      (e = hipMalloc(&c->d_mask, sizeof(int32_t) * 2 * E)) != hipSuccess ||
      (e = hipEventCreateWithFlags(&c->ids_ready, hipEventDisableTiming)) != hipSuccess) {
    cache_slot_table_destroy(c);
    return hip_error(e, "cache staging allocation");
  }
  std::fill(c->h_mask, c->h_mask + 2 * E, 0);
  *out = c;
  return MOE_OK;
}

int cache_slot_table_destroy(moe_cache* c) {
  clear_error();
  if (!c) return MOE_OK;
  (void)hipDeviceSynchronize();
  for (int i = 0; i < kEventRing; ++i) {
    if (c->events[i]) (void)hipEventDestroy(c->events[i]);
    if (c->copy_events[i]) (void)hipEventDestroy(c->copy_events[i]);
  }
  if (c->d_table) (void)hipFree(c->d_table);
  if (c->h_ids) (void)hipHostFree(c->h_ids);
  if (c->h_mask) (void)hipHostFree(c->h_mask);
  if (c->d_mask) (void)hipFree(c->d_mask);
  if (c->ids_ready) (void)hipEventDestroy(c->ids_ready);
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

int cache_slot_table_lookup(moe_cache* c, int layer, const int32_t* ids, int n, int32_t* slots_out,
                            int32_t* miss_ids, int* n_miss) {
  clear_error();
  if (!c) return set_error(MOE_ERR_INVALID_ARG, "cache_slot_table_lookup: cache is NULL");
  if (layer < 0 || layer >= c->L || n < 0 || (n > 0 && (!ids || !slots_out)) || !n_miss)
    return set_error(MOE_ERR_INVALID_ARG, "cache_slot_table_lookup: layer=%d n=%d", layer, n);
  for (int i = 0; i < n; ++i)
    if (ids[i] < 0 || ids[i] >= c->E)
      return set_error(MOE_ERR_INVALID_ARG, "cache_slot_table_lookup: expert id %d of layer %d not in [0, %d)",
                       ids[i], layer, c->E);
  {
    std::vector<int32_t> distinct(ids, ids + n);
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
  hipError_t e = hipSetDevice(c->device);
  if (e != hipSuccess) return hip_error(e, "hipSetDevice");
  hipStream_t cs = (hipStream_t)copy_stream, ks = (hipStream_t)compute_stream;
  // the slot's previous reader must be done before the copy overwrites it
  if (c->slot_event[pd.slot] >= 0) {
    if ((e = hipStreamWaitEvent(cs, c->events[c->slot_event[pd.slot]], 0)) != hipSuccess)
      return hip_error(e, "hipStreamWaitEvent(copy)");
  }
  if ((e = hipMemcpyAsync(c->d_pool + (size_t)pd.slot * c->slot_bytes, c->h_pool + (size_t)key * c->slot_bytes,
                          c->slot_bytes, hipMemcpyHostToDevice, cs)) != hipSuccess)
    return hip_error(e, "hipMemcpyAsync(expert)");
  hipEvent_t done = c->copy_events[c->next_copy_event];
  c->next_copy_event = (c->next_copy_event + 1) % kEventRing;
  if ((e = hipEventRecord(done, cs)) != hipSuccess) return hip_error(e, "hipEventRecord(copy)");
  if ((e = hipStreamWaitEvent(ks, done, 0)) != hipSuccess) return hip_error(e, "hipStreamWaitEvent(compute)");
  TableUpdate u{};
  u.idx[u.n] = key; u.val[u.n] = pd.slot; ++u.n;
  if (pd.victim_key >= 0 && c->table[pd.victim_key] < 0) {
    u.idx[u.n] = pd.victim_key; u.val[u.n] = -1; ++u.n;
  }
  launch(table_update_kernel, 1, 64, 0, ks, c->d_table, u);
  int rc = check_launch("table_update_kernel");
  if (rc) return rc;
  if (slot_out) *slot_out = pd.slot;
  return MOE_OK;
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
  if ((e = hipDeviceSynchronize()) != hipSuccess) return hip_error(e, "hipDeviceSynchronize");
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
  c->free_fifo.clear();
  c->free_head = 0;
  for (int s = 0; s < count; ++s)
    if (c->slot_key[s] < 0) c->free_fifo.push_back(s);
  c->n_slots = n_slots;
  c->d_pool = pool;
  return MOE_OK;
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
  int rc = moe_route_permute(ctx, x, MOE_DTYPE_F32, router_w, bias, logits_in, T, c->H, E, k, logits_out, topk_ids,
                             topk_w, expert_offsets, sorted_pairs, pair_pos, active, nullptr, 0, compute_stream);
  if (rc) return rc;
  hipStream_t cs = (hipStream_t)compute_stream;
  hipError_t e = hipMemcpyAsync(c->h_ids, topk_ids, sizeof(int32_t) * P, hipMemcpyDeviceToHost, cs);
  if (e != hipSuccess) return hip_error(e, "hipMemcpyAsync(ids)");
  if ((e = hipEventRecord(c->ids_ready, cs)) != hipSuccess) return hip_error(e, "hipEventRecord(ids)");
  if ((e = hipEventSynchronize(c->ids_ready)) != hipSuccess) return hip_error(e, "hipEventSynchronize(ids)");
  std::vector<int32_t> slots(P), miss(P);
  int n_miss = 0;
  if ((rc = cache_slot_table_lookup(c, layer, c->h_ids, P, slots.data(), miss.data(), &n_miss))) return rc;
  // hit / miss masks; the previous call's upload has run (it precedes this
  // call's routing on the same stream, which the host waited for)
  std::fill(c->h_mask, c->h_mask + 2 * E, 0);
  for (int i = 0; i < P; ++i) c->h_mask[c->h_ids[i]] = 1;
  for (int i = 0; i < n_miss; ++i) {
    c->h_mask[miss[i]] = 0;
    c->h_mask[E + miss[i]] = 1;
  }
  bool any_hit = false;
  for (int i = 0; i < P; ++i) any_hit |= c->h_mask[c->h_ids[i]] != 0;
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
  if (n_miss == 0) {  // every expert resident: one call with the combine folded in
    a.out = out;
    if ((rc = moe_expert_ffn(ctx, &a, compute_stream))) return rc;
    return cache_mark_layer_done(c, layer, compute_stream);
  }
  if ((e = hipMemcpyAsync(c->d_mask, c->h_mask, sizeof(int32_t) * 2 * E, hipMemcpyHostToDevice, cs)) != hipSuccess)
    return hip_error(e, "hipMemcpyAsync(masks)");
  if (any_hit) {  // the resident experts run while the misses are copied
    a.expert_mask = c->d_mask;
    if ((rc = moe_expert_ffn(ctx, &a, compute_stream))) return rc;
  }
  for (int i = 0; i < n_miss; ++i)
    if ((rc = prefetch_expert(c, layer, miss[i], copy_stream, compute_stream, nullptr))) return rc;
  a.expert_mask = c->d_mask + E;
  if ((rc = moe_expert_ffn(ctx, &a, compute_stream))) return rc;
  if ((rc = moe_combine(ctx, y_pairs, topk_w, T, k, c->H, out, compute_stream))) return rc;
  return cache_mark_layer_done(c, layer, compute_stream);
}

}  // extern "C"
