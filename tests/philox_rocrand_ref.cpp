// Independent reference for the oracle's Philox-4x32-10: rocRAND's own engine
// (header-only, host-callable), reached through a subclass so a counter and key
// can be given directly.  Reads lines "c0 c1 c2 c3 k0 k1" (hex) from stdin and
// prints the four output words (hex) per line.
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

struct PhiloxProbe : rocrand_device::philox4x32_10_engine {
    uint4 block(uint4 ctr, uint2 key) { return this->ten_rounds(ctr, key); }
};

int main() {
    unsigned c0, c1, c2, c3, k0, k1;
    PhiloxProbe p;
    while (std::scanf("%x %x %x %x %x %x", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
        uint4 c = {c0, c1, c2, c3};
        uint2 k = {k0, k1};
        uint4 r = p.block(c, k);
        std::printf("%08x %08x %08x %08x\n", r.x, r.y, r.z, r.w);
    }
    return 0;
}
