// Host check of the stream-K split (no GPU). Compiled for the host only; it
// includes the kernels' own header and enumerates, for every workgroup of a
// launch, the work units sk_unit() hands it -- exactly what the stream-K
// kernel walks -- and checks over a sweep of launch shapes:
//
//  * every k-step pair of every tile is covered exactly once;
//  * the first W*G tiles come as whole units, one per workgroup per wave, in
//    the static order (workgroup w: w, w+G, ...);
//  * every range of tail pairs has length floor/ceil(S/Gs), so workgroups'
//    tail work differs by at most one pair;
//  * a unit is partial exactly when the fix-up's sk_owner() range for its
//    tile has two or more workgroups, and those workgroups are exactly the
//    ones whose units touch the tile, in ascending k order;
//  * the workspace slots w + s of partial units are distinct and below
//    Gs + R;
//  * units start and end on even k-steps (stage 0 of the ring);
//  * SkWalker, the incremental form the kernel runs, yields exactly the
//    same unit sequence as sk_unit().
//
// usage: sk_split_check  -> prints "ok <shapes checked>" or the first failure
#include <cstdio>
#include <cstdlib>
#include <set>
#include <vector>

#include "../persistent_tile_scheduling_macro_amd/csrc/device_common.h"

using namespace pgemm;

static int fail(const char* what, int T, int G, int Gs, int kp, int w, int q) {
  std::printf("FAIL %s: T=%d G=%d Gs=%d kp=%d w=%d q=%d\n", what, T, G, Gs, kp, w, q);
  return 1;
}

// One launch shape: T tiles, G = grid of the whole-tile phase (the
// workgroup count when W >= 1), Gs tail groups, kp pairs per tile.
static int check(int T, int G, int Gs, int kp) {
  const int W = T / G, R = T % G;
  const int grid = W >= 1 ? G : Gs;
  if (R == 0) Gs = 0;
  const int64_t S = (int64_t)R * kp;
  std::vector<int> cover((size_t)T * kp, 0);
  std::vector<std::vector<int>> touch(R);  // workgroups with a unit of tail tile s, in walk order
  std::vector<int> partial_of(R, -1);       // 1 if some unit of s is partial
  std::set<int> slots;
  for (int w = 0; w < grid; ++w) {
    int64_t tail_pairs = 0;
    SkWalker walk;
    walk.init(w, G, W, T, R, Gs, kp);
    for (int q = 0;; ++q) {
      int tile, kb, ke, wt, wkb, wke;
      const bool more = sk_unit(q, w, G, W, T, R, Gs, kp, &tile, &kb, &ke);
      const bool wmore = walk.next(&wt, &wkb, &wke);
      if (more != wmore || (more && (wt != tile || wkb != kb || wke != ke)))
        return fail("walker differs from sk_unit", T, G, Gs, kp, w, q);
      if (!more) break;
      if (q > W + R + 1) return fail("unit sequence does not end", T, G, Gs, kp, w, q);
      if (tile < 0 || tile >= T) return fail("tile out of range", T, G, Gs, kp, w, q);
      if ((kb & 1) || (ke & 1) || kb < 0 || ke > 2 * kp || kb >= ke)
        return fail("bad k-step range", T, G, Gs, kp, w, q);
      if (q < W) {
        if (tile != q * G + w || kb != 0 || ke != 2 * kp) return fail("whole-tile phase order", T, G, Gs, kp, w, q);
      } else {
        if (tile < T - R) return fail("tail unit on a whole tile", T, G, Gs, kp, w, q);
      }
      for (int pr = kb / 2; pr < ke / 2; ++pr) cover[(size_t)tile * kp + pr]++;
      if (tile >= T - R) {
        const int s = tile - (T - R);
        tail_pairs += (ke - kb) / 2;
        touch[s].push_back(w);
        const bool partial = kb != 0 || ke != 2 * kp;
        if (partial) {
          partial_of[s] = 1;
          const int slot = w + s;
          if (slot >= Gs + R) return fail("slot beyond workspace", T, G, Gs, kp, w, q);
          if (!slots.insert(slot).second) return fail("slot used twice", T, G, Gs, kp, w, q);
        }
      }
    }
    if (R > 0 && w < Gs) {
      const int64_t lo = S / Gs, hi = (S + Gs - 1) / Gs;
      if (lo < 1) return fail("empty tail range", T, G, Gs, kp, w, -1);
      if (tail_pairs < lo || tail_pairs > hi) return fail("unbalanced tail range", T, G, Gs, kp, w, -1);
    } else if (tail_pairs != 0) {
      return fail("tail work outside the tail groups", T, G, Gs, kp, w, -1);
    }
  }
  for (size_t i = 0; i < cover.size(); ++i)
    if (cover[i] != 1) return fail("pair not covered exactly once", T, G, Gs, kp, (int)(i / kp), (int)(i % kp));
  for (int s = 0; s < R; ++s) {
    const int w0 = sk_owner((int64_t)s * kp, S, Gs), w1 = sk_owner((int64_t)(s + 1) * kp - 1, S, Gs);
    const bool split = w0 != w1;
    if (split != (partial_of[s] == 1)) return fail("fix-up split test disagrees with the units", T, G, Gs, kp, -1, s);
    if ((int)touch[s].size() != w1 - w0 + 1) return fail("fix-up piece count", T, G, Gs, kp, -1, s);
    for (int i = 0; i < (int)touch[s].size(); ++i)
      if (touch[s][i] != w0 + i) return fail("fix-up pieces are not workgroups w0..w1", T, G, Gs, kp, -1, s);
  }
  return 0;
}

int main() {
  long shapes = 0;
  const int Ts[] = {1, 2, 3, 7, 16, 36, 64, 100, 255, 256, 257, 300, 511, 576, 1024, 1089, 4225};
  const int Gsz[] = {1, 3, 8, 97, 256, 512};
  const int kps[] = {1, 2, 3, 4, 5, 16, 33, 48, 65, 128};
  for (int T : Ts)
    for (int G : Gsz)
      for (int kp : kps) {
        const int R = T % G;
        const int64_t S = (int64_t)R * kp;
        // every tail-group count the planner could pick, and a few more
        std::set<int> gss = {1, G, (int)std::min<int64_t>(G, S)};
        for (int minp : {1, 2, 4, 8}) gss.insert((int)std::max<int64_t>(1, std::min<int64_t>(G, S / minp)));
        for (int Gs : gss) {
          if (R > 0 && (Gs < 1 || Gs > G || Gs > S)) continue; // the split's precondition
          if (check(T, G, Gs, kp)) return 1;
          ++shapes;
        }
      }
  std::printf("ok %ld\n", shapes);
  return 0;
}
