// Host race test of the claim protocol of the claiming tile schedulers.
//
// Compiled for the host only and linked with nothing from the library: it
// includes the kernels' own header and calls the same claim_tile() the
// claiming kernels call, from G std::threads that stand in for the G
// workgroups. In the dynamic mode each worker starts on tile w, then claims;
// in the cancel-and-reuse mode (G = T workers, started at staggered times)
// each worker claims its first tile too and stops at once if none is left.
// Either way a worker claims until a claim fails (KernelWiki "Persistent
// Kernels with Cluster Launch Control", intro: a failed request ends that
// worker's requests). Random sleeps vary the interleavings.
//
// usage: sched_sim <scenario> <dynamic|cancel> T G launches seed [arg]
//   scenario "race":    plain launches back to back on one counter
//   scenario "stall":   worker 0 sleeps `arg` ms after starting its first tile
//   scenario "corrupt": the counter is preset to `arg` before the first launch
// Prints one line of key=value pairs; the pytest wrapper checks them.
#include <atomic>
#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <string>
#include <thread>
#include <vector>

#include "../persistent_tile_scheduling_macro_amd/csrc/device_common.h"

int main(int argc, char** argv) {
  using namespace pgemm;
  if (argc < 7) {
    std::fprintf(stderr, "usage: %s race|stall|corrupt dynamic|cancel T G launches seed [arg]\n", argv[0]);
    return 2;
  }
  const std::string scenario = argv[1];
  const bool cancel = std::string(argv[2]) == "cancel";
  const int T = std::atoi(argv[3]);
  const int G = std::atoi(argv[4]);
  const int launches = std::atoi(argv[5]);
  const unsigned seed = (unsigned)std::strtoul(argv[6], nullptr, 10);
  const long arg = argc > 7 ? std::atol(argv[7]) : 0;
  if (T < 1 || G < 1 || G > T || launches < 1) {
    std::fprintf(stderr, "need 1 <= G <= T and launches >= 1\n");
    return 2;
  }
  const int offset = cancel ? claim_offset<kCancel>(G) : claim_offset<kDynamic>(G);
  const int total = cancel ? claim_total<kCancel>(T, G) : claim_total<kDynamic>(T, G);

  alignas(64) int counter = scenario == "corrupt" ? (int)arg : 0;
  std::vector<std::atomic<int>> visits(T);
  for (auto& v : visits) v.store(0);
  std::atomic<long> claims{0}, failed{0};
  std::vector<int> worker_tiles(G, 0);
  std::vector<int> counter_after(launches, 0);

  for (int l = 0; l < launches; ++l) {
    std::vector<std::thread> pool;
    pool.reserve(G);
    for (int w = 0; w < G; ++w) {
      pool.emplace_back([&, w, l] {
        std::mt19937 rng(seed * 7919u + (unsigned)w * 104729u + (unsigned)l);
        auto claim = [&]() {
          const int t = claim_tile(&counter, T, offset, total);
          claims.fetch_add(1);
          if (t >= T) failed.fetch_add(1);
          return t;
        };
        int t = w;  // dynamic: first tile without a claim
        if (cancel) {
          // workgroups start at different times; the first tile is claimed
          std::this_thread::sleep_for(std::chrono::microseconds(rng() % 2000));
          t = claim();
        }
        while (t < T) {
          visits[t].fetch_add(1);
          ++worker_tiles[w];
          if (scenario == "stall" && w == 0 && worker_tiles[w] == 1)
            std::this_thread::sleep_for(std::chrono::milliseconds(arg));
          else if (rng() % 4 == 0)
            std::this_thread::sleep_for(std::chrono::microseconds(rng() % 200));
          else
            std::this_thread::yield();
          t = claim();
        }
      });
    }
    for (auto& th : pool) th.join();
    counter_after[l] = __hip_atomic_load(&counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  int vmin = 1 << 30, vmax = 0;
  long unvisited = 0;
  for (int t = 0; t < T; ++t) {
    const int v = visits[t].load();
    vmin = v < vmin ? v : vmin;
    vmax = v > vmax ? v : vmax;
    if (v == 0) ++unvisited;
  }
  int wmin = 1 << 30, wmax = 0;
  for (int w = 0; w < G; ++w) {
    wmin = worker_tiles[w] < wmin ? worker_tiles[w] : wmin;
    wmax = worker_tiles[w] > wmax ? worker_tiles[w] : wmax;
  }
  std::printf("visits_min=%d visits_max=%d unvisited=%ld claims=%ld failed=%ld worker0_tiles=%d "
              "worker_tiles_min=%d worker_tiles_max=%d counter_after=",
              vmin, vmax, unvisited, claims.load(), failed.load(), worker_tiles[0], wmin, wmax);
  for (int l = 0; l < launches; ++l) std::printf(l ? ",%d" : "%d", counter_after[l]);
  std::printf("\n");
  return 0;
}
