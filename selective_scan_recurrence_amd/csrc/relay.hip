// Host side of the relay split (see relay.h).
#include <stdlib.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "relay.h"

namespace ssm {

RelaySplit relay_split(int64_t jobs, int64_t L, int tile, int cap, int n_cu, int max_jobs) {
    RelaySplit r;
    const char* env = getenv("SSM_RELAY");  // "0": never split (read at every launch)
    if (env && env[0] == '0') return r;
    if (n_cu <= 0 || jobs < n_cu || L < 2 || tile <= 0) return r;
    const int64_t full = jobs / n_cu, rem = jobs % n_cu;
    if (rem == 0 || cap < full + 1 || rem > max_jobs) return r;
    const int64_t k0 = n_cu / rem;
    if (k0 < 2) return r;
    int64_t len = (L + k0 - 1) / k0;
    len = (len + tile - 1) / tile * tile;
    const int64_t k = (L + len - 1) / len;
    if (k < 2) return r;
    r.full = (int)(full * n_cu);
    r.rem = (int)rem;
    r.k = (int)k;
    r.len = (int)len;
    return r;
}

RoundSplit round_split(int64_t jobs, int steps, int64_t slots, int min_len) {
    RoundSplit r;
    const char* env = getenv("SSM_RELAY");  // "0": never split (read at every launch)
    if (env && env[0] == '0') return r;
    if (jobs <= 0 || slots <= 0 || steps <= 0 || jobs <= slots) return r;
    int64_t best = -1;
    for (int k = 1; k <= 8; ++k) {
        const int len = (steps + k - 1) / k;
        if (k > 1 && len < min_len) break;
        const int kk = (steps + len - 1) / len;  // pieces actually needed
        const int64_t rounds = std::max<int64_t>((jobs * kk + slots - 1) / slots, kk);
        const int64_t t = rounds * (len + 1);
        if (best < 0 || t < best) {
            best = t;
            r.k = kk;
            r.len = len;
        }
    }
    if (r.k <= 1) r = RoundSplit{};
    return r;
}

int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cache[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

int resident_blocks(const void* fn, int threads) {
    struct Entry {
        int dev;
        const void* fn;
        int threads, blocks;
    };
    static std::mutex mu;
    static Entry table[256];
    static int used = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    std::lock_guard<std::mutex> lock(mu);
    for (int e = 0; e < used; ++e)
        if (table[e].dev == dev && table[e].fn == fn && table[e].threads == threads) return table[e].blocks;
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, fn, threads, 0) != hipSuccess) return 0;
    if (used < 256) table[used++] = Entry{dev, fn, threads, blocks};
    return blocks;
}

}  // namespace ssm
