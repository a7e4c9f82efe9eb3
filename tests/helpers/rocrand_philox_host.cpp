// Host-side wrapper around rocRAND's Philox4x32-10 engine, used only by the
// CPU tests to cross-check the oracle's independent Philox implementation.
// The engine is driven through its public constructor: seed -> key words,
// subsequence -> counter words 2..3, offset/4 -> counter words 0..1; next4()
// then returns the block function of that counter.
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdint>

extern "C" void rocrand_philox_blocks(const uint32_t* counters, uint64_t seed,
                                      uint32_t* out, int n) {
  for (int t = 0; t < n; ++t) {
    const uint32_t* c = counters + 4 * t;
    unsigned long long subseq = ((unsigned long long)c[3] << 32) | c[2];
    unsigned long long offset = (((unsigned long long)c[1] << 32) | c[0]) * 4ull;
    rocrand_device::philox4x32_10_engine eng(seed, subseq, offset);
    uint4 r = eng.next4();
    out[4 * t + 0] = r.x;
    out[4 * t + 1] = r.y;
    out[4 * t + 2] = r.z;
    out[4 * t + 3] = r.w;
  }
}
