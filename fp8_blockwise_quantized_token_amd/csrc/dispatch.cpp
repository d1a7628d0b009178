// dispatch.cpp -- per-shape choice among the GEMM variants (host only).
//
// The pages tune one GEMM per shape and pick the best variant and tile
// configuration for each (page "Helion: improving vLLM inference with
// autotuning", sections "Kernel Implementation", "Hybrid Dispatch" and
// "Per-shape Config Tuning").  Here the choice is a compiled-in table keyed
// on (N, K) and a bucket of M, measured on MI355X, with a heuristic for
// shapes the table does not hold (the pages fall back to a default config
// rather than failing when no tuned config exists).  Lookup is a binary
// search over the tabled weight shapes, then a scan of that shape's M
// buckets; deterministic; nothing is tuned at run time.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "../../include/fp8blk.h"
#include "dispatch.hpp"

namespace fp8blk {

bool standard_tile_supported(int tile_m, int tile_n, int stages, int kwaves);  // gemm_standard.hip

namespace {

struct Entry {
  int32_t n, k;       // weight shape
  int32_t m_lo, m_hi; // inclusive bucket of M
  fp8blk_gemm_config cfg;
};

#define CFG(v, tm, tn, sk, kw) {v, tm, tn, sk, kw, 0, 0, 0}
#define CFGS(v, tm, tn, sk, kw, ns) {v, tm, tn, sk, kw, ns, 0, 0}
#define CFGT(v, tm, tn, sk, kw, ns) {v, tm, tn, sk, kw, ns, 0, 1}  // split tail

// Measured table (MI355X).  Entries are checked in order; the first bucket
// containing M wins.
#include "dispatch_table.inc"

constexpr int kCUs = 256;
// Beyond this distance (a factor of about 4.5 in N times K) the nearest
// tabled shape says little and the heuristic decides.
constexpr double kMaxShapeDistance = 1.5;

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

void heuristic(int64_t M, int64_t N, int64_t K, fp8blk_gemm_config* c) {
  const int64_t kb = K / 128;
  *c = fp8blk_gemm_config{};
  if (M <= 64) {
    // Swap-AB: tokens on the 16-wide column side of the matrix core.
    c->variant = FP8BLK_SWAPAB;
    c->tile_m = M <= 16 ? 16 : (M <= 32 ? 32 : 64);
    c->tile_n = 16;
    c->kwaves = kb >= 8 ? 8 : (kb >= 4 ? 4 : (kb >= 2 ? 2 : 1));
    int64_t split = 1;
    const int64_t blocks = N / c->tile_n;
    while (blocks * split < 2 * kCUs && split * 2 * c->kwaves <= kb && split < 256) split *= 2;
    c->split_k = (int32_t)split;
    return;
  }
  c->variant = FP8BLK_STANDARD;
  const int64_t t256x256 = (N % 256 == 0) ? cdiv(M, 256) * (N / 256) : 0;
  const int64_t t256 = cdiv(M, 256) * (N / 128);
  const int64_t t128 = cdiv(M, 128) * (N / 128);
  if (t256x256 >= kCUs) {
    c->tile_m = 256;
    c->tile_n = 256;
  } else if (t256 >= kCUs) {
    c->tile_m = 256;
    c->tile_n = 128;
  } else if (t128 >= kCUs) {
    c->tile_m = 128;
    c->tile_n = 128;
  } else {
    c->tile_m = M <= 64 ? 64 : 128;
    c->tile_n = 128;
  }
  const int64_t tiles = cdiv(M, c->tile_m) * (N / c->tile_n);
  int64_t split = 1;
  while (tiles * split < kCUs && split * 2 * 4 <= kb && split < 256) split *= 2;
  c->split_k = (int32_t)split;
  c->kwaves = 1;
  // Whole rounds of 256x256 tiles plus a partial round of at most half the
  // CUs: split only that last round (one 256x256 workgroup per CU).
  const int64_t tail = tiles % kCUs;
  if (c->tile_m == 256 && c->tile_n == 256 && tiles > kCUs && tail > 0 && tail <= kCUs / 2) {
    const int64_t s = tail <= kCUs / 4 ? 4 : 2;
    if (s * 2 <= kb) {
      c->split_k = (int32_t)s;
      c->split_tail = 1;
    }
  }
}

// A tabled configuration is usable for another (M, N, K) when its tile
// divides N, its split fits K and its Swap-AB token tile holds M.
bool usable(const fp8blk_gemm_config& c, int64_t M, int64_t N, int64_t K) {
  const int64_t kb = K / 128;
  if (c.split_k > kb) return false;
  if (c.variant == FP8BLK_SWAPAB) return M <= c.tile_m;
  return N % c.tile_n == 0 && standard_tile_supported(c.tile_m, c.tile_n, c.stages, c.kwaves == 0 ? 1 : c.kwaves);
}

// The table's entries grouped by weight shape: one run per (N, K), its
// entries in table order, the runs in order of first appearance, plus an
// index of the runs sorted by (N, K) and the logarithms the nearest-shape
// rule needs.  Built once (thread-safe static initialization), read-only
// afterwards.
struct Run {
  int32_t n, k;
  double ln_n, ln_k;
  std::vector<const Entry*> entries;
};
struct Index {
  std::vector<Run> runs;
  std::vector<int> by_shape;  // run numbers sorted by (n, k)
};

const Index& table_index() {
  static const Index idx = [] {
    Index x;
    for (const Entry& e : kTable) {
      auto it = std::find_if(x.runs.begin(), x.runs.end(), [&](const Run& r) { return r.n == e.n && r.k == e.k; });
      if (it == x.runs.end()) {
        x.runs.push_back(Run{e.n, e.k, log((double)e.n), log((double)e.k), {}});
        it = x.runs.end() - 1;
      }
      it->entries.push_back(&e);
    }
    for (int i = 0; i < (int)x.runs.size(); ++i) x.by_shape.push_back(i);
    std::sort(x.by_shape.begin(), x.by_shape.end(), [&](int a, int b) {
      const Run &ra = x.runs[a], &rb = x.runs[b];
      return ra.n != rb.n ? ra.n < rb.n : ra.k < rb.k;
    });
    return x;
  }();
  return idx;
}

// The first entry of a run whose M bucket holds M (and, if asked, whose
// configuration is usable for the shape), or nullptr.
const Entry* bucket(const Run& r, int64_t M, int64_t N, int64_t K, bool need_usable) {
  for (const Entry* e : r.entries)
    if (M >= e->m_lo && M <= e->m_hi && (!need_usable || usable(e->cfg, M, N, K))) return e;
  return nullptr;
}

// The tabled entry for exactly (N, K) whose bucket holds M.
const Entry* exact(int64_t M, int64_t N, int64_t K) {
  const Index& x = table_index();
  auto it = std::lower_bound(x.by_shape.begin(), x.by_shape.end(), 0, [&](int a, int) {
    const Run& r = x.runs[a];
    return r.n != N ? r.n < N : r.k < K;
  });
  if (it == x.by_shape.end() || x.runs[*it].n != N || x.runs[*it].k != K) return nullptr;
  return bucket(x.runs[*it], M, N, K, false);
}

// Nearest tabled weight shape: the entry whose M bucket holds M and whose
// (N, K) is closest in |ln(N/n)| + |ln(K/k)| among the usable ones (the
// shape tabled first on ties).  Layers of other models of similar size get
// the configuration measured for their neighbour instead of the heuristic's.
bool nearest(int64_t M, int64_t N, int64_t K, fp8blk_gemm_config* out) {
  const Index& x = table_index();
  const double ln_n = log((double)N), ln_k = log((double)K);
  double best = 1e30;
  const Entry* pick = nullptr;
  for (const Run& r : x.runs) {
    const double d = fabs(ln_n - r.ln_n) + fabs(ln_k - r.ln_k);
    if (d >= best) continue;
    const Entry* e = bucket(r, M, N, K, true);
    if (e == nullptr) continue;
    best = d;
    pick = e;
  }
  if (pick == nullptr || best > kMaxShapeDistance) return false;
  *out = pick->cfg;
  return true;
}

}  // namespace

void select_config(int64_t M, int64_t N, int64_t K, uint32_t flags, fp8blk_gemm_config* out) {
  const Entry* e = exact(M, N, K);
  bool found = e != nullptr;
  if (found) *out = e->cfg;
  if (!found) found = nearest(M, N, K, out);
  if (!found) heuristic(M, N, K, out);
  // Power-of-two activation and weight scales: the Standard kernels apply
  // them in the matrix core (v_mfma_scale) instead of one VALU rescale per
  // K block.  Both operands must be powers of two for that.
  const uint32_t both = FP8BLK_FLAG_UE8M0 | FP8BLK_FLAG_WEIGHT_POW2;
  if ((flags & both) == both && out->variant == FP8BLK_STANDARD) out->scale_mode = FP8BLK_SCALES_POW2;
}

}  // namespace fp8blk
