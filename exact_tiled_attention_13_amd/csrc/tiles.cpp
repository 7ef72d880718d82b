// Launch-choice table: which of the compiled launch shapes a call uses.
//
// The NumPy tiled-attention build guide (Extending It) suggests choosing the
// tile configuration per head size and hardware by measurement, adapting it
// to the sequence length, and keeping the result.  Here the choices are
// runtime parameters of the compiled kernels, looked up per (operation,
// dtype, D, causal, sequence-length bucket, size bucket) in a table the
// caller sets (the Python binding loads it from a JSON file that the tuner
// writes).  Without a table, or for keys it does not cover, the built-in
// rule applies.  Every choice gives a correct result; only speed differs.
//
// Concurrency: launches read the table without taking a lock.  Every table
// is an immutable snapshot published through an atomic pointer; a new table
// replaces the pointer, and earlier snapshots stay allocated until the
// process ends (a launch may still be reading one), so no reader ever sees
// a partly written or freed table.  Snapshots hold exactly the entries they
// were given (at most 256 x 40 bytes each).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <memory>
#include <mutex>
#include <vector>

#include "../../include/miattn.h"
#include "launch.h"

namespace {

constexpr int kMaxEntries = 256;
constexpr int F = MIATTN_TILE_FIELDS;

struct Table {
  int n = 0;
  std::vector<int32_t> e;   // n * F fields
};

std::atomic<const Table*> g_cur{nullptr};

// Serialises the setters and owns every snapshot ever published.  Reachable
// from a global until exit on purpose: launches on other threads may still
// hold a pointer to an older snapshot.
std::mutex& set_mu() {
  static std::mutex* mu = new std::mutex;
  return *mu;
}
std::vector<std::unique_ptr<Table>>& snapshots() {
  static auto* all = new std::vector<std::unique_ptr<Table>>;
  return *all;
}

// first entry matching (op, dtype, D, causal, t_lo <= T <= t_hi,
// size_lo <= size <= size_hi), or nullptr
const int32_t* find(int op, int dtype, int D, int causal, long long T, long long size) {
  const Table* t = g_cur.load(std::memory_order_acquire);
  if (t == nullptr) return nullptr;
  for (int i = 0; i < t->n; ++i) {
    const int32_t* e = t->e.data() + (size_t)i * F;
    if (e[0] == op && e[1] == dtype && e[2] == D && e[3] == causal && T >= e[4] && T <= e[5] && size >= e[6] &&
        size <= e[7])
      return e;
  }
  return nullptr;
}

bool valid_entry(const int32_t* e) {
  const int op = e[0], dtype = e[1], D = e[2], causal = e[3];
  if (op != MIATTN_TILE_FWD && op != MIATTN_TILE_DECODE) return false;
  if (dtype != MIATTN_BF16 && dtype != MIATTN_E4M3) return false;
  if (D != 64 && D != 128) return false;
  if (causal != 0 && causal != 1) return false;
  if (e[4] < 0 || e[5] < e[4] || e[6] < 0 || e[7] < e[6]) return false;
  if (op == MIATTN_TILE_FWD) return (e[8] == 0 || e[8] == 1) && (e[9] >= -1 && e[9] <= 1);
  return e[8] >= 1 && e[8] <= 8 && e[9] == 0;
}

}  // namespace

namespace miattn {

FwdChoice choose_fwd(int dtype, int D, int causal, long long T, long long wg256) {
  if (const int32_t* e = find(MIATTN_TILE_FWD, dtype, D, causal, T, wg256)) return FwdChoice{e[8], e[9]};
  // built-in rule: 256-row workgroups once there are two per CU, else
  // 128-row workgroups with two key groups; zig-zag by its own rule
  return FwdChoice{wg256 >= kFwdSplitBelow ? 0 : 1, -1};
}

int choose_decode_wgs_per_cu(int dtype, int D, long long S_max, long long items) {
  if (const int32_t* e = find(MIATTN_TILE_DECODE, dtype, D, 1, S_max, items)) return e[8];
  return 2;
}

}  // namespace miattn

extern "C" {

int attn_set_tile_table(const int32_t* entries, int n) {
  if (n < 0 || n > kMaxEntries) return MIATTN_ERR_SHAPE;
  if (n > 0 && entries == nullptr) return MIATTN_ERR_NULL;
  for (int i = 0; i < n; ++i)
    if (!valid_entry(entries + (size_t)i * F)) return MIATTN_ERR_UNSUPPORTED;
  std::unique_ptr<Table> t(new Table);
  t->n = n;
  t->e.assign(entries, entries + (size_t)n * F);
  std::lock_guard<std::mutex> lk(set_mu());
  g_cur.store(t.get(), std::memory_order_release);
  snapshots().push_back(std::move(t));
  return MIATTN_OK;
}

int attn_tile_table_size(void) {
  const Table* t = g_cur.load(std::memory_order_acquire);
  return t == nullptr ? 0 : t->n;
}

int attn_tile_choice(int op, int dtype, int D, int causal, long long T, long long size, int32_t* out) {
  if (out == nullptr) return MIATTN_ERR_NULL;
  if (size < 0 || T < 0) return MIATTN_ERR_SHAPE;
  if ((op != MIATTN_TILE_FWD && op != MIATTN_TILE_DECODE) || (dtype != MIATTN_BF16 && dtype != MIATTN_E4M3) ||
      (D != 64 && D != 128) || (causal != 0 && causal != 1))
    return MIATTN_ERR_UNSUPPORTED;
  if (op == MIATTN_TILE_FWD) {
    const miattn::FwdChoice c = miattn::choose_fwd(dtype, D, causal, T, size);
    out[0] = c.shape;
    out[1] = c.zig;
  } else {
    out[0] = miattn::choose_decode_wgs_per_cu(dtype, D, T, size);
    out[1] = 0;
  }
  return MIATTN_OK;
}

}  // extern "C"
