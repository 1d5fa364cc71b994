// KV-cache manager: the per-layer K/V storage around the hot path (append each chunk's rows, drop the
// history of converted layers).  The operations, layouts and error behaviour are documented in
// include/ispa.h.
//
// The pages' inference stage keeps full attention (the whole growing cache) in the F-layers and only
// sink + current chunk in the converted L-layers (technical summary, section 2, stage 3
// "Memory-Efficient Inference"); the memory saving it reports is exactly the history rows those
// layers no longer hold.  Layout: per layer, K rows and V rows each live in a virtual address range
// reserved for the layer's largest size (HIP virtual memory management); physical memory is mapped
// behind a range only as rows arrive, in pieces of whole allocation granules, and the pieces past the
// sink and current chunk are unmapped and released when a layer is converted.  Rows keep their
// addresses while a layer grows (appends never move data), nothing is committed up front, and the
// device memory in use follows the rows held, so the peak of a rollout is the peak of what it holds.
#include "../../include/ispa.h"

#include <hip/hip_runtime.h>

#include <new>
#include <vector>

namespace {

// One virtual range (K or V rows of a layer) with physical pieces mapped from its start.
struct Region {
  char* base = nullptr;   // reserved virtual range [base, base + va)
  size_t va = 0;
  size_t mapped = 0;      // [base, base + mapped) is backed by the pieces, in address order
  std::vector<std::pair<size_t, hipMemGenericAllocationHandle_t>> pieces;
};

size_t round_up(size_t x, size_t g) { return (x + g - 1) / g * g; }

}  // namespace

struct ispa_kv_cache {
  struct Layer {
    Region k, v;
    int32_t n_chunks = 0;    // chunks appended so far (a converted layer holds at most one)
    bool local = false;      // history released: rows are sink + current chunk only
  };
  int device = 0, d = 0, dtype = 0;
  int32_t sink = 0, chunk = 0, max_chunks = 0;
  size_t row_bytes = 0;      // bytes of one row of K (or V)
  size_t gran = 0;           // physical allocation granule
  std::vector<Layer> layers;

  int64_t held_rows(const Layer& L) const {
    return L.local ? (int64_t)sink + (L.n_chunks > 0 ? chunk : 0) : (int64_t)sink + (int64_t)L.n_chunks * chunk;
  }
  hipMemAllocationProp prop() const {
    hipMemAllocationProp p = {};
    p.type = hipMemAllocationTypePinned;
    p.location.type = hipMemLocationTypeDevice;
    p.location.id = device;
    return p;
  }
  // back [base, base + bytes) with physical memory (one new piece for what is missing)
  int ensure(Region& r, size_t bytes) const {
    if (bytes <= r.mapped) return ISPA_OK;
    const size_t add = round_up(bytes - r.mapped, gran);
    if (r.mapped + add > r.va) return ISPA_EINVAL;
    hipMemAllocationProp p = prop();
    hipMemGenericAllocationHandle_t h;
    if (hipMemCreate(&h, add, &p, 0) != hipSuccess) return ISPA_EHIP;
    if (hipMemMap(r.base + r.mapped, add, 0, h, 0) != hipSuccess) {
      (void)hipMemRelease(h);
      return ISPA_EHIP;
    }
    // access is granted over the whole mapped prefix from the start of the reservation (the runtime
    // here rejects a range that starts inside a reservation)
    hipMemAccessDesc acc = {};
    acc.location = p.location;
    acc.flags = hipMemAccessFlagsProtReadWrite;
    if (hipMemSetAccess(r.base, r.mapped + add, &acc, 1) != hipSuccess) {
      (void)hipMemUnmap(r.base + r.mapped, add);
      (void)hipMemRelease(h);
      return ISPA_EHIP;
    }
    r.pieces.emplace_back(add, h);
    r.mapped += add;
    return ISPA_OK;
  }
  // unmap and release the pieces that lie entirely past `bytes`
  int trim(Region& r, size_t bytes) const {
    int st = ISPA_OK;
    while (!r.pieces.empty() && r.mapped - r.pieces.back().first >= bytes) {
      const size_t sz = r.pieces.back().first;
      if (hipMemUnmap(r.base + r.mapped - sz, sz) != hipSuccess) st = ISPA_EHIP;
      if (hipMemRelease(r.pieces.back().second) != hipSuccess) st = ISPA_EHIP;
      r.pieces.pop_back();
      r.mapped -= sz;
    }
    return st;
  }
  int free_region(Region& r) const {
    int st = trim(r, 0);
    if (r.base && hipMemAddressFree(r.base, r.va) != hipSuccess) st = ISPA_EHIP;
    r.base = nullptr;
    r.va = 0;
    return st;
  }
};

namespace {

size_t elem_bytes(int dtype) { return dtype == ISPA_F32 ? 4 : 2; }
bool valid_layer(const ispa_kv_cache* kv, int layer) { return kv && layer >= 0 && layer < (int)kv->layers.size(); }

}  // namespace

extern "C" {

int ispa_kv_create(int n_layers, int d, int dtype, int32_t sink_rows, int32_t chunk_rows, int32_t max_chunks,
                   ispa_kv_cache** out) {
  if (!out) return ISPA_EINVAL;
  *out = nullptr;
  if (n_layers < 1 || d < 1 || d % 8 != 0 || sink_rows < 0 || chunk_rows < 1 || max_chunks < 1) return ISPA_EINVAL;
  if (dtype != ISPA_F32 && dtype != ISPA_BF16 && dtype != ISPA_F16) return ISPA_EINVAL;
  const int64_t cap = (int64_t)sink_rows + (int64_t)max_chunks * chunk_rows;
  if (cap > INT32_MAX) return ISPA_EINVAL;
  ispa_kv_cache* kv = new (std::nothrow) ispa_kv_cache;
  if (!kv) return ISPA_EHIP;
  if (hipGetDevice(&kv->device) != hipSuccess) {
    delete kv;
    return ISPA_EHIP;
  }
  kv->d = d;
  kv->dtype = dtype;
  kv->sink = sink_rows;
  kv->chunk = chunk_rows;
  kv->max_chunks = max_chunks;
  kv->row_bytes = (size_t)d * elem_bytes(dtype);
  hipMemAllocationProp p = kv->prop();
  if (hipMemGetAllocationGranularity(&kv->gran, &p, hipMemAllocationGranularityRecommended) != hipSuccess ||
      kv->gran == 0) {
    delete kv;
    return ISPA_EHIP;
  }
  // physical memory is handed out in 2 MiB pages whatever smaller granule is reported: map whole pages
  // so the mapped bytes are the bytes in use
  kv->gran = round_up(kv->gran > ((size_t)2 << 20) ? kv->gran : ((size_t)2 << 20), kv->gran);
  kv->layers.resize(n_layers);
  const size_t va = round_up((size_t)cap * kv->row_bytes, kv->gran);
  for (auto& L : kv->layers) {
    for (Region* r : {&L.k, &L.v}) {
      void* base = nullptr;
      if (hipMemAddressReserve(&base, va, kv->gran, nullptr, 0) != hipSuccess) {
        ispa_kv_destroy(kv);
        return ISPA_EHIP;
      }
      r->base = (char*)base;
      r->va = va;
      // the sink rows are held from the start (every layer keeps them), so they are mapped now
      if (kv->ensure(*r, (size_t)sink_rows * kv->row_bytes) != ISPA_OK) {
        ispa_kv_destroy(kv);
        return ISPA_EHIP;
      }
    }
  }
  *out = kv;
  return ISPA_OK;
}

int ispa_kv_destroy(ispa_kv_cache* kv) {
  if (!kv) return ISPA_OK;
  int st = ISPA_OK;
  // pending copies into the cache must finish before its memory goes
  if (hipDeviceSynchronize() != hipSuccess) st = ISPA_EHIP;
  for (auto& L : kv->layers)
    for (Region* r : {&L.k, &L.v})
      if (kv->free_region(*r) != ISPA_OK) st = ISPA_EHIP;
  delete kv;
  return st;
}

int ispa_kv_write_sink(ispa_kv_cache* kv, int layer, const void* k, const void* v, void* stream) {
  if (!valid_layer(kv, layer) || !k || !v) return ISPA_EINVAL;
  if (kv->sink == 0) return ISPA_OK;
  auto& L = kv->layers[layer];
  const size_t bytes = (size_t)kv->sink * kv->row_bytes;   // mapped since ispa_kv_create
  const hipStream_t s = (hipStream_t)stream;
  if (hipMemcpyAsync(L.k.base, k, bytes, hipMemcpyDeviceToDevice, s) != hipSuccess) return ISPA_EHIP;
  if (hipMemcpyAsync(L.v.base, v, bytes, hipMemcpyDeviceToDevice, s) != hipSuccess) return ISPA_EHIP;
  return ISPA_OK;
}

int ispa_kv_append_chunk(ispa_kv_cache* kv, int layer, const void* k, const void* v, void* stream) {
  if (!valid_layer(kv, layer) || !k || !v) return ISPA_EINVAL;
  auto& L = kv->layers[layer];
  int64_t row;
  if (L.local) {
    row = kv->sink;   // a converted layer keeps one chunk: the new one replaces it
  } else {
    if (L.n_chunks >= kv->max_chunks) return ISPA_EINVAL;
    row = (int64_t)kv->sink + (int64_t)L.n_chunks * kv->chunk;
  }
  const size_t end = (size_t)(row + kv->chunk) * kv->row_bytes;
  int st = kv->ensure(L.k, end);
  if (st == ISPA_OK) st = kv->ensure(L.v, end);
  if (st != ISPA_OK) return st;
  const size_t bytes = (size_t)kv->chunk * kv->row_bytes;
  const hipStream_t s = (hipStream_t)stream;
  if (hipMemcpyAsync(L.k.base + row * kv->row_bytes, k, bytes, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return ISPA_EHIP;
  if (hipMemcpyAsync(L.v.base + row * kv->row_bytes, v, bytes, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return ISPA_EHIP;
  if (L.local) {
    L.n_chunks = 1;
  } else {
    ++L.n_chunks;
  }
  return ISPA_OK;
}

int ispa_kv_release_history(ispa_kv_cache* kv, int layer, void* stream) {
  if (!valid_layer(kv, layer)) return ISPA_EINVAL;
  auto& L = kv->layers[layer];
  if (L.local) return ISPA_EINVAL;
  const hipStream_t s = (hipStream_t)stream;
  const size_t keep = (size_t)((int64_t)kv->sink + (L.n_chunks > 0 ? kv->chunk : 0)) * kv->row_bytes;
  if (L.n_chunks >= 2) {
    // the current chunk moves next to the sink; with at least one chunk of history between them
    // the two row ranges do not overlap
    const int64_t cur = (int64_t)kv->sink + (int64_t)(L.n_chunks - 1) * kv->chunk;
    const size_t bytes = (size_t)kv->chunk * kv->row_bytes;
    for (Region* r : {&L.k, &L.v})
      if (hipMemcpyAsync(r->base + (size_t)kv->sink * kv->row_bytes, r->base + cur * kv->row_bytes, bytes,
                         hipMemcpyDeviceToDevice, s) != hipSuccess)
        return ISPA_EHIP;
  }
  // earlier work on the stream may still read the history rows, and the copy must land before the
  // memory behind them goes
  if (hipStreamSynchronize(s) != hipSuccess) return ISPA_EHIP;
  int st = kv->trim(L.k, keep);
  if (kv->trim(L.v, keep) != ISPA_OK) st = ISPA_EHIP;
  L.local = true;
  L.n_chunks = L.n_chunks > 0 ? 1 : 0;
  return st;
}

int ispa_kv_layer(const ispa_kv_cache* kv, int layer, void** k, void** v, int32_t* rows) {
  if (!valid_layer(kv, layer) || !k || !v || !rows) return ISPA_EINVAL;
  const auto& L = kv->layers[layer];
  *k = L.k.base;
  *v = L.v.base;
  rows[0] = kv->sink;
  if (L.local) {
    rows[1] = 0;
    rows[2] = L.n_chunks > 0 ? kv->chunk : 0;
  } else {
    rows[1] = L.n_chunks > 0 ? (L.n_chunks - 1) * kv->chunk : 0;
    rows[2] = L.n_chunks > 0 ? kv->chunk : 0;
  }
  return ISPA_OK;
}

int ispa_kv_bytes(const ispa_kv_cache* kv, int64_t* held_bytes, int64_t* reserved_bytes) {
  if (!kv || !held_bytes || !reserved_bytes) return ISPA_EINVAL;
  int64_t held = 0, mapped = 0;
  for (const auto& L : kv->layers) {
    held += 2 * kv->held_rows(L) * (int64_t)kv->row_bytes;
    mapped += (int64_t)(L.k.mapped + L.v.mapped);
  }
  *held_bytes = held;
  *reserved_bytes = mapped;
  return ISPA_OK;
}

}  // extern "C"
