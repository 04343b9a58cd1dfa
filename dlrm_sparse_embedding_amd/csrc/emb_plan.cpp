// Host-side planning of the dedup's radix sort (no device code): how many
// passes, how wide a digit, how large a tile, and whether each table's
// lookups are sorted as a segment of their own on their row bits. The host
// layer sizes the workspace from these plans before any launch; the sort
// kernels (k_keys_sort.hip) run them.
#include <algorithm>

#include "emb_internal.h"

namespace emb {

namespace {

int passes_for(int bits) { return bits <= kRadixMaxBits ? 1 : (bits + kRadixMaxBits - 1) / kRadixMaxBits; }

SortPlan make_plan(bool seg, int bits, int S, long long N) {
  SortPlan p{};
  p.seg = seg;
  p.bits = bits;
  p.passes = passes_for(bits);
  p.rb = std::min(kRadixMaxBits, std::max(8, (bits + p.passes - 1) / p.passes));
  p.S = seg ? S : 1;
  // larger tiles for large sorts: twice the items per digit run written,
  // half the per-tile counters to write and scan (small sorts keep more
  // tiles than the GPU has CUs)
  p.ipt = N >= kSortBigN ? 16 : 8;
  const long long tile = 256ll * p.ipt;
  const long long tiles = (N + tile - 1) / tile + (seg ? S : 0);
  p.nblk = (int)((tiles + 7) / 8 * 8);
  return p;
}

}  // namespace

SortPlan sort_plan_global(int bits, long long N) { return make_plan(false, bits, 1, N); }

// Per table when that takes fewer passes, or as many passes with narrower
// digits (fewer counters per tile to write and scan, longer runs per digit).
SortPlan sort_plan_dedup(const Geom& g, long long N) {
  const SortPlan glob = make_plan(false, g.key_bits, 1, N);
  if (g.T > kSegMaxTables) return glob;
  const SortPlan seg = make_plan(true, g.row_bits, g.T, N);
  return seg.passes < glob.passes || (seg.passes == glob.passes && seg.rb < glob.rb) ? seg : glob;
}

}  // namespace emb
