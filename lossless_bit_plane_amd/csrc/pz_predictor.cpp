// Per-tensor compressibility predictor of the PlaneZip runtime (PlaneZip
// paper, §III-B "Compressibility Predictor"; accuracy in §V-B and Table IV).
//
// A saved tensor is named by a signature: where its producing operator sits
// in the sequence that every training iteration repeats, and which of that
// operator's outputs it is. The table
// keeps, per signature, the last measurement (raw bytes, compressed bytes):
// the size the engine reported for a swap, or a profiling-iteration
// measurement such as pz_compressed_size or pz_compressed_size_sampled. A new
// measurement overwrites the old one. A prediction scales the measured ratio
// to the asked size; a signature without a measurement predicts a ratio of 1.
//
// Host code only: open addressing over a power-of-two slot array of at least
// twice the capacity, one mutex per table.
#include "../../include/planezip.h"

#include <algorithm>
#include <cmath>
#include <mutex>
#include <new>
#include <vector>

struct pz_predictor {
  struct Slot {
    uint64_t sig;
    uint64_t raw;
    uint64_t comp;
    bool used;
  };
  std::mutex mu;
  size_t capacity = 0;
  size_t count = 0;
  std::vector<Slot> slots;

  static uint64_t mix(uint64_t x) {  // SplitMix64's finalizer (Steele, Lea, Flood 2014)
    x ^= x >> 30;
    x *= 0xBF58476D1CE4E5B9ull;
    x ^= x >> 27;
    x *= 0x94D049BB133111EBull;
    x ^= x >> 31;
    return x;
  }
  // The slot holding sig, or the empty slot where it would go.
  Slot &find(uint64_t sig) {
    const size_t mask = slots.size() - 1;
    size_t i = (size_t)mix(sig) & mask;
    while (slots[i].used && slots[i].sig != sig) i = (i + 1) & mask;
    return slots[i];
  }
};

extern "C" {

pz_predictor_t *pz_predictor_create(size_t capacity) {
  if (capacity == 0 || capacity > ((size_t)1 << 40)) return nullptr;
  pz_predictor *p = new (std::nothrow) pz_predictor;
  if (!p) return nullptr;
  size_t n = 2;
  while (n < 2 * capacity) n <<= 1;
  try {
    p->slots.assign(n, pz_predictor::Slot{0, 0, 0, false});
  } catch (...) {
    delete p;
    return nullptr;
  }
  p->capacity = capacity;
  return p;
}

void pz_predictor_destroy(pz_predictor_t *p) { delete p; }

pz_status_t pz_predictor_update(pz_predictor_t *p, uint64_t signature, uint64_t raw_bytes,
                                uint64_t comp_bytes) {
  if (!p || raw_bytes == 0 || comp_bytes == 0 || comp_bytes > PZ_MAX_COMPRESSED_BYTES(raw_bytes))
    return PZ_ERROR_INVALID_VALUE;
  std::lock_guard<std::mutex> lock(p->mu);
  pz_predictor::Slot &s = p->find(signature);
  if (!s.used) {
    if (p->count == p->capacity) return PZ_ERROR_INSUFFICIENT_BUFFER;
    s.used = true;
    s.sig = signature;
    ++p->count;
  }
  s.raw = raw_bytes;
  s.comp = comp_bytes;
  return PZ_SUCCESS;
}

pz_status_t pz_predictor_predict(pz_predictor_t *p, uint64_t signature, uint64_t raw_bytes,
                                 uint64_t *pred_bytes, int *measured) {
  if (!p || !pred_bytes) return PZ_ERROR_INVALID_VALUE;
  std::lock_guard<std::mutex> lock(p->mu);
  const pz_predictor::Slot &s = p->find(signature);
  if (measured) *measured = s.used ? 1 : 0;
  if (!s.used) {
    *pred_bytes = raw_bytes;
    return PZ_SUCCESS;
  }
  const unsigned __int128 num = (unsigned __int128)raw_bytes * s.comp;
  const unsigned __int128 q = (num + s.raw - 1) / s.raw;  // rounded up
  if (q > (unsigned __int128)UINT64_MAX) return PZ_ERROR_INVALID_VALUE;
  *pred_bytes = (uint64_t)q;
  return PZ_SUCCESS;
}

size_t pz_predictor_entries(pz_predictor_t *p) {
  if (!p) return 0;
  std::lock_guard<std::mutex> lock(p->mu);
  return p->count;
}

void pz_predictor_clear(pz_predictor_t *p) {
  if (!p) return;
  std::lock_guard<std::mutex> lock(p->mu);
  for (pz_predictor::Slot &s : p->slots) s.used = false;
  p->count = 0;
}

double pz_transfer_time(uint64_t raw_bytes, double ratio, double link_bytes_per_s, double engine_bytes_per_s) {
  const bool ok = std::isfinite(ratio) && std::isfinite(link_bytes_per_s) && std::isfinite(engine_bytes_per_s) &&
                  ratio > 0 && link_bytes_per_s > 0 && engine_bytes_per_s > 0;
  if (!ok) return -1.0;
  const double m = (double)raw_bytes;
  const double plain = m / link_bytes_per_s;  // the engine bypassed
  const double coded = std::max(m / (ratio * link_bytes_per_s), m / engine_bytes_per_s);
  return std::min(plain, coded);
}

}  // extern "C"
