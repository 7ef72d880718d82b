// Launch-choice table: which of the compiled launch shapes a call uses.
//
// The NumPy tiled-attention build guide (Extending It) suggests choosing the
// tile configuration per head size and hardware by measurement and keeping
// the result.  Here the choices are runtime parameters of the compiled
// kernels, looked up per (operation, dtype, D, causal, size bucket) in a
// table the caller sets (the Python binding loads it from a JSON file that
// the tuner writes).  Without a table, or for keys it does not cover, the
// built-in rule applies.  Every choice gives a correct result; only speed
// differs.
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>

#include "../../include/miattn.h"
#include "launch.h"

namespace {

constexpr int kMaxEntries = 256;

std::mutex g_mu;
int32_t g_tab[kMaxEntries][MIATTN_TILE_FIELDS];
int g_n = 0;

// first entry matching (op, dtype, D, causal, lo <= size <= hi), or nullptr;
// the caller holds g_mu
const int32_t* find(int op, int dtype, int D, int causal, long long size) {
  for (int i = 0; i < g_n; ++i) {
    const int32_t* e = g_tab[i];
    if (e[0] == op && e[1] == dtype && e[2] == D && e[3] == causal && size >= e[4] && size <= e[5]) return e;
  }
  return nullptr;
}

bool valid_entry(const int32_t* e) {
  const int op = e[0], dtype = e[1], D = e[2], causal = e[3];
  if (op != MIATTN_TILE_FWD && op != MIATTN_TILE_DECODE) return false;
  if (dtype != MIATTN_BF16 && dtype != MIATTN_E4M3) return false;
  if (D != 64 && D != 128) return false;
  if (causal != 0 && causal != 1) return false;
  if (e[4] < 0 || e[5] < e[4]) return false;
  if (op == MIATTN_TILE_FWD) return (e[6] == 0 || e[6] == 1) && (e[7] >= -1 && e[7] <= 1);
  return e[6] >= 1 && e[6] <= 8 && e[7] == 0;
}

}  // namespace

namespace miattn {

FwdChoice choose_fwd(int dtype, int D, int causal, long long wg256) {
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (const int32_t* e = find(MIATTN_TILE_FWD, dtype, D, causal, wg256)) return FwdChoice{e[6], e[7]};
  }
  // built-in rule: 256-row workgroups once there are two per CU, else
  // 128-row workgroups with two key groups; zig-zag by its own rule
  return FwdChoice{wg256 >= kFwdSplitBelow ? 0 : 1, -1};
}

int choose_decode_wgs_per_cu(int dtype, int D, long long items) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (const int32_t* e = find(MIATTN_TILE_DECODE, dtype, D, 1, items)) return e[6];
  return 2;
}

}  // namespace miattn

extern "C" {

int attn_set_tile_table(const int32_t* entries, int n) {
  if (n < 0 || n > kMaxEntries) return MIATTN_ERR_SHAPE;
  if (n > 0 && entries == nullptr) return MIATTN_ERR_NULL;
  for (int i = 0; i < n; ++i)
    if (!valid_entry(entries + (size_t)i * MIATTN_TILE_FIELDS)) return MIATTN_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_mu);
  if (n > 0) std::memcpy(g_tab, entries, sizeof(int32_t) * MIATTN_TILE_FIELDS * (size_t)n);
  g_n = n;
  return MIATTN_OK;
}

int attn_tile_table_size(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  return g_n;
}

int attn_tile_choice(int op, int dtype, int D, int causal, long long size, int32_t* out) {
  if (out == nullptr) return MIATTN_ERR_NULL;
  if (size < 0) return MIATTN_ERR_SHAPE;
  if ((op != MIATTN_TILE_FWD && op != MIATTN_TILE_DECODE) || (dtype != MIATTN_BF16 && dtype != MIATTN_E4M3) ||
      (D != 64 && D != 128) || (causal != 0 && causal != 1))
    return MIATTN_ERR_UNSUPPORTED;
  if (op == MIATTN_TILE_FWD) {
    const miattn::FwdChoice c = miattn::choose_fwd(dtype, D, causal, size);
    out[0] = c.shape;
    out[1] = c.zig;
  } else {
    out[0] = miattn::choose_decode_wgs_per_cu(dtype, D, size);
    out[1] = 0;
  }
  return MIATTN_OK;
}

}  // extern "C"
