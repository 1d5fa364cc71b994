// KV-cache manager: the per-layer K/V storage around the hot path (append each chunk's rows, drop the
// history of converted layers).  The operations, layouts and error behaviour are documented in
// include/ispa.h.
//
// The pages' inference stage keeps full attention (the whole growing cache) in the F-layers and only
// sink + current chunk in the converted L-layers (technical summary, section 2, stage 3
// "Memory-Efficient Inference"); the memory saving it reports is exactly the history rows those
// layers no longer hold.  Layout here: one device allocation per layer, K rows then V rows, each
// [capacity, d] row-major, rows in the attention calls' order (sink | history | current).  A full
// layer reserves sink + max_chunks * chunk rows up front -- appends never move data, and with 288 GB
// of HBM per GPU the reservation for a whole rollout fits -- while a converted layer is reallocated to
// sink + one chunk and overwrites its current chunk in place.
#include "../../include/ispa.h"

#include <hip/hip_runtime.h>

#include <new>
#include <vector>

struct ispa_kv_cache {
  struct Layer {
    char* base = nullptr;    // K rows [0, cap), then V rows [0, cap)
    int64_t cap = 0;         // rows reserved for K (and for V)
    int32_t n_chunks = 0;    // chunks appended so far (a converted layer holds at most one)
    bool local = false;      // history released: rows are sink + current chunk only
  };
  int d = 0, dtype = 0;
  int32_t sink = 0, chunk = 0, max_chunks = 0;
  size_t row_bytes = 0;      // bytes of one row of K (or V)
  std::vector<Layer> layers;

  char* k_ptr(const Layer& L, int64_t row) const { return L.base + row * row_bytes; }
  char* v_ptr(const Layer& L, int64_t row) const { return L.base + (L.cap + row) * row_bytes; }
  size_t alloc_bytes(int64_t cap) const { return 2 * (size_t)cap * row_bytes; }
  int64_t held_rows(const Layer& L) const {
    return L.local ? (int64_t)sink + (L.n_chunks > 0 ? chunk : 0) : (int64_t)sink + (int64_t)L.n_chunks * chunk;
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
  kv->d = d;
  kv->dtype = dtype;
  kv->sink = sink_rows;
  kv->chunk = chunk_rows;
  kv->max_chunks = max_chunks;
  kv->row_bytes = (size_t)d * elem_bytes(dtype);
  kv->layers.resize(n_layers);
  for (auto& L : kv->layers) {
    L.cap = cap;
    if (hipMalloc((void**)&L.base, kv->alloc_bytes(cap)) != hipSuccess) {
      L.base = nullptr;
      ispa_kv_destroy(kv);
      return ISPA_EHIP;
    }
  }
  *out = kv;
  return ISPA_OK;
}

int ispa_kv_destroy(ispa_kv_cache* kv) {
  if (!kv) return ISPA_OK;
  int st = ISPA_OK;
  for (auto& L : kv->layers)
    if (L.base && hipFree(L.base) != hipSuccess) st = ISPA_EHIP;
  delete kv;
  return st;
}

int ispa_kv_write_sink(ispa_kv_cache* kv, int layer, const void* k, const void* v, void* stream) {
  if (!valid_layer(kv, layer) || !k || !v) return ISPA_EINVAL;
  if (kv->sink == 0) return ISPA_OK;
  auto& L = kv->layers[layer];
  const size_t bytes = (size_t)kv->sink * kv->row_bytes;
  hipStream_t s = (hipStream_t)stream;
  if (hipMemcpyAsync(kv->k_ptr(L, 0), k, bytes, hipMemcpyDefault, s) != hipSuccess) return ISPA_EHIP;
  if (hipMemcpyAsync(kv->v_ptr(L, 0), v, bytes, hipMemcpyDefault, s) != hipSuccess) return ISPA_EHIP;
  return ISPA_OK;
}

int ispa_kv_append_chunk(ispa_kv_cache* kv, int layer, const void* k, const void* v, void* stream) {
  if (!valid_layer(kv, layer) || !k || !v) return ISPA_EINVAL;
  auto& L = kv->layers[layer];
  if (!L.local && L.n_chunks >= kv->max_chunks) return ISPA_EINVAL;
  // full layer: at the tail (the previous current chunk becomes history); converted: over the current chunk
  const int64_t row = L.local ? kv->sink : (int64_t)kv->sink + (int64_t)L.n_chunks * kv->chunk;
  const size_t bytes = (size_t)kv->chunk * kv->row_bytes;
  hipStream_t s = (hipStream_t)stream;
  if (hipMemcpyAsync(kv->k_ptr(L, row), k, bytes, hipMemcpyDefault, s) != hipSuccess) return ISPA_EHIP;
  if (hipMemcpyAsync(kv->v_ptr(L, row), v, bytes, hipMemcpyDefault, s) != hipSuccess) return ISPA_EHIP;
  L.n_chunks = L.local ? 1 : L.n_chunks + 1;
  return ISPA_OK;
}

int ispa_kv_release_history(ispa_kv_cache* kv, int layer, void* stream) {
  if (!valid_layer(kv, layer)) return ISPA_EINVAL;
  auto& L = kv->layers[layer];
  if (L.local) return ISPA_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  const int64_t cap = (int64_t)kv->sink + kv->chunk;
  char* nb = nullptr;
  if (hipMalloc((void**)&nb, kv->alloc_bytes(cap)) != hipSuccess) return ISPA_EHIP;
  ispa_kv_cache::Layer N = L;
  N.base = nb;
  N.cap = cap;
  N.local = true;
  N.n_chunks = L.n_chunks > 0 ? 1 : 0;
  const size_t sink_bytes = (size_t)kv->sink * kv->row_bytes, cur_bytes = (size_t)kv->chunk * kv->row_bytes;
  const int64_t cur_row = (int64_t)kv->sink + (int64_t)(L.n_chunks - 1) * kv->chunk;
  bool ok = true;
  if (sink_bytes) {
    ok = ok && hipMemcpyAsync(kv->k_ptr(N, 0), kv->k_ptr(L, 0), sink_bytes, hipMemcpyDeviceToDevice, s) == hipSuccess;
    ok = ok && hipMemcpyAsync(kv->v_ptr(N, 0), kv->v_ptr(L, 0), sink_bytes, hipMemcpyDeviceToDevice, s) == hipSuccess;
  }
  if (L.n_chunks > 0) {
    ok = ok && hipMemcpyAsync(kv->k_ptr(N, kv->sink), kv->k_ptr(L, cur_row), cur_bytes, hipMemcpyDeviceToDevice, s) ==
                   hipSuccess;
    ok = ok && hipMemcpyAsync(kv->v_ptr(N, kv->sink), kv->v_ptr(L, cur_row), cur_bytes, hipMemcpyDeviceToDevice, s) ==
                   hipSuccess;
  }
  // the old rows are read by the copies (and by any attention call queued before them): the stream
  // must reach this point before the old allocation can go
  ok = ok && hipStreamSynchronize(s) == hipSuccess;
  if (!ok) {
    (void)hipFree(nb);
    return ISPA_EHIP;
  }
  if (hipFree(L.base) != hipSuccess) {
    (void)hipFree(nb);
    return ISPA_EHIP;
  }
  L = N;
  return ISPA_OK;
}

int ispa_kv_layer(const ispa_kv_cache* kv, int layer, void** k, void** v, int32_t* rows) {
  if (!valid_layer(kv, layer) || !k || !v || !rows) return ISPA_EINVAL;
  const auto& L = kv->layers[layer];
  *k = kv->k_ptr(L, 0);
  *v = kv->v_ptr(L, 0);
  const int32_t cur = L.n_chunks > 0 ? kv->chunk : 0;
  rows[0] = kv->sink;
  rows[1] = L.local ? 0 : (L.n_chunks > 0 ? (L.n_chunks - 1) * kv->chunk : 0);
  rows[2] = cur;
  return ISPA_OK;
}

int ispa_kv_bytes(const ispa_kv_cache* kv, int64_t* held_bytes, int64_t* reserved_bytes) {
  if (!kv || !held_bytes || !reserved_bytes) return ISPA_EINVAL;
  int64_t held = 0, reserved = 0;
  for (const auto& L : kv->layers) {
    held += 2 * kv->held_rows(L) * (int64_t)kv->row_bytes;
    reserved += (int64_t)kv->alloc_bytes(L.cap);
  }
  *held_bytes = held;
  *reserved_bytes = reserved;
  return ISPA_OK;
}

}  // extern "C"
