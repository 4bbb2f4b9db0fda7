// Launch plans and workspace sizes: plain host arithmetic on the shapes and
// the device's compute-unit count (no HIP calls), shared by the C ABI's size
// queries and its launches so the two always agree.
#include <algorithm>

#include "fa_internal.h"

namespace fa {

namespace {
inline size_t round256(size_t b) { return (b + 255) / 256 * 256; }
inline int pad_rows(int N) { return (N + kBwdQueryBlock - 1) / kBwdQueryBlock * kBwdQueryBlock; }
}  // namespace

// Plan of a forward launch.  Decode: when all query rows that read a key /
// value head fit one wave (group * Nq <= 32, d = 64 or 128) the packed-rows
// kernel runs, its keys split into ranges of at least 128 keys aiming at the
// one-wave workgroups per CU its three LDS stages allow (three at d = 128,
// 48 KiB each; four at d = 64).  Otherwise the tile kernels, whose keys are
// split only when the query tiles alone leave compute units idle (fewer
// workgroups than CUs): ranges of at least four 64-key tiles, two workgroups
// per CU.  Splitting needs the caller's workspace (has_ws).
FwdPlan fwd_plan(int BH, int group, int Nq, int Nk, int d, bool has_ws, int cus) {
  FwdPlan pl{0, 1, Nk};
  if (Nk <= 0 || BH <= 0 || Nq <= 0) return pl;
  const int bn = kFwdSplitKeys;
  const int nkt = (Nk + bn - 1) / bn;
  if ((d == 64 || d == 128) && (long long)group * Nq <= 32) {
    pl.decode = 1;
    if (!has_ws) return pl;
    const long long heads = BH / group;
    // one-wave workgroups per CU that the decode kernel's LDS stages allow
    const long long per_cu = d == 128 ? 3 : 4;
    int ns = (int)((per_cu * cus + heads - 1) / heads);
    ns = std::min(ns, std::max(1, Nk / 128));
    if (ns <= 1) return pl;
    const int tiles_per = (nkt + ns - 1) / ns;
    pl.klen = tiles_per * bn;
    pl.nsplit = (Nk + pl.klen - 1) / pl.klen;
    return pl;
  }
  if (!has_ws) return pl;
  const int bm = fwd_rows_per_tile(d);
  const long long tiles = (long long)BH * ((Nq + bm - 1) / bm);
  if (tiles >= cus) return pl;
  int ns = (int)((2LL * cus + tiles - 1) / tiles);
  ns = std::min(ns, nkt / 4);
  if (ns <= 1) return pl;
  const int tiles_per = (nkt + ns - 1) / ns;
  pl.klen = tiles_per * bn;
  pl.nsplit = (Nk + pl.klen - 1) / pl.klen;
  return pl;
}

size_t fwd_workspace_bytes(int BH, int group, int Nq, int Nk, int d, int cus) {
  const FwdPlan pl = fwd_plan(BH, group, Nq, Nk, d, true, cus);
  if (pl.nsplit <= 1) return 0;
  const size_t rows = (size_t)pl.nsplit * BH * Nq;
  return round256(rows * d * 4) + rows * 4;
}

size_t bwd_workspace_bytes(int BH, int N, int d) {
  // L2 and D rows; the fp32 dQ accumulator only where dQ is accumulated by
  // atomics (d = 64)
  return 2 * round256((size_t)BH * pad_rows(N) * 4) + (d == 64 ? (size_t)BH * N * d * 4 : 0);
}

int bwd_head_split(int BHkv, int group, int Nq, int Nk, int d, bool causal, int cus) {
  if (group < 2 || BHkv <= 0 || Nq <= 0 || Nk <= 0) return 1;
  // Workgroups run one per compute unit, so the key-tile kernel takes about
  // max(heaviest workgroup, total work / CUs).  Under causal masking the
  // first key tiles see every query block and the last almost none: with
  // few key / value heads the heaviest workgroup (all `group` heads of key
  // tile 0) then sets the time.  Take the smallest divisor s of the group
  // whose share (group / s heads) is no heavier than the average per CU.
  const int keys = bwd_keys_per_tile(d);
  const int nkt = (Nk + keys - 1) / keys;
  const int nqb = (Nq + kBwdQueryBlock - 1) / kBwdQueryBlock;
  long long sum = 0;
  int heaviest = 0;
  for (int kt = 0; kt < nkt; ++kt) {
    const int qb0 = causal ? std::max(0, kt * keys - (Nk - Nq)) / kBwdQueryBlock : 0;
    const int nit = std::max(0, nqb - qb0);
    sum += nit;
    heaviest = std::max(heaviest, nit);
  }
  const long long per_cu = ((long long)BHkv * group * sum + cus - 1) / cus;
  for (int s = 1; s < group; ++s)
    if (group % s == 0 && (long long)(group / s) * heaviest <= per_cu) return s;
  return group;
}

size_t bwd_split_bytes(int BHkv, int Nk, int d, int hsplit) {
  if (hsplit <= 1) return 0;
  return round256(2 * (size_t)hsplit * BHkv * (size_t)Nk * d * 4);
}

size_t bwd_kv_workspace_bytes(int BH, int group, int Nq, int Nk, int d, int cus) {
  const int BHkv = BH / group;
  const int s = std::max(bwd_head_split(BHkv, group, Nq, Nk, d, true, cus),
                         bwd_head_split(BHkv, group, Nq, Nk, d, false, cus));
  return bwd_workspace_bytes(BH, Nq, d) + bwd_split_bytes(BHkv, Nk, d, s);
}

}  // namespace fa
