// Test-only cross-check of the oracle's Philox4x32-10 against ROCm's open-source
// rocRAND implementation (header only). It is compiled for the host and run by
// tests/test_oracle_philox.py; nothing in the library or the oracle uses it.
// Reads lines "c0 c1 c2 c3 k0 k1" (hex) on stdin, prints the 4 output words.
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>

struct PhiloxProbe : rocrand_device::philox4x32_10_engine {
    uint4 block(uint4 ctr, uint2 key) { return ten_rounds(ctr, key); }
};

int main() {
    unsigned c0, c1, c2, c3, k0, k1;
    PhiloxProbe probe;
    while (std::scanf("%x %x %x %x %x %x", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
        uint4 r = probe.block(make_uint4(c0, c1, c2, c3), make_uint2(k0, k1));
        std::printf("%08x %08x %08x %08x\n", r.x, r.y, r.z, r.w);
    }
    return 0;
}
