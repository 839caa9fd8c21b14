// Host check of pack_bfp4 (the prefill down kernel's y format) against the
// format's plain definition: E = max(fp32 exponent field of the block's
// largest magnitude, 13), q = clamp(round-half-even(v * 2^(139 - E)), +-8191),
// bits [0,8) E, then four 14-bit two's-complement q; a block with a NaN or an
// infinity is (255, 0).  Prints the number of mismatching blocks.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>

#include "flint_internal.hpp"

static uint32_t bits(float f) { uint32_t u; std::memcpy(&u, &f, 4); return u; }
static float from_bits(uint32_t u) { float f; std::memcpy(&f, &u, 4); return f; }

static void reference(const float v[4], uint32_t out[2]) {
    uint32_t m = 0;
    for (int i = 0; i < 4; ++i) m = std::max(m, bits(v[i]) & 0x7FFFFFFFu);
    if (m >= 0x7F800000u) { out[0] = 255u; out[1] = 0u; return; }
    const uint32_t E = std::max(m >> 23, 13u);
    const double scale = std::ldexp(1.0, 139 - (int)E);
    int32_t q[4];
    for (int i = 0; i < 4; ++i) {
        const double x = (double)v[i] * scale;  // exact: a power-of-two scaling of a float
        double r = std::nearbyint(x);           // round half to even (default rounding mode)
        r = std::min(std::max(r, -8191.0), 8191.0);
        q[i] = (int32_t)r;
    }
    const uint64_t w = (uint64_t)E | ((uint64_t)((uint32_t)q[0] & 0x3FFFu) << 8) |
                       ((uint64_t)((uint32_t)q[1] & 0x3FFFu) << 22) | ((uint64_t)((uint32_t)q[2] & 0x3FFFu) << 36) |
                       ((uint64_t)((uint32_t)q[3] & 0x3FFFu) << 50);
    out[0] = (uint32_t)w;
    out[1] = (uint32_t)(w >> 32);
}

int main() {
    std::mt19937_64 rng(20261204);
    std::normal_distribution<float> nd(0.f, 1.f);
    std::uniform_int_distribution<uint32_t> ud;
    long bad = 0, n = 0;
    auto check = [&](const float v[4]) {
        uint32_t ref[2];
        reference(v, ref);
        const uint2 got = flint::pack_bfp4(v[0], v[1], v[2], v[3]);
        ++n;
        if (got.x != ref[0] || got.y != ref[1]) {
            if (bad < 5)
                std::printf("mismatch: %a %a %a %a -> %08x %08x, want %08x %08x\n", v[0], v[1], v[2], v[3], got.x,
                            got.y, ref[0], ref[1]);
            ++bad;
        }
    };
    float v[4];
    for (int it = 0; it < 2000000; ++it) {  // normal values over many binades
        const float sc = std::ldexp(1.f, (int)(ud(rng) % 200) - 100);
        for (int i = 0; i < 4; ++i) v[i] = nd(rng) * sc;
        check(v);
    }
    for (int it = 0; it < 2000000; ++it) {  // arbitrary bit patterns (NaN, infinities, subnormals)
        for (int i = 0; i < 4; ++i) v[i] = from_bits((uint32_t)ud(rng));
        check(v);
    }
    for (int it = 0; it < 2000000; ++it) {  // exact and near halfway points, the clamp at 2^13
        const int E = 13 + (int)(ud(rng) % 242);
        const float step = std::ldexp(1.f, E - 139);
        v[0] = std::ldexp(1.f, E - 127) * (1.f - std::ldexp(1.f, -24 + (int)(ud(rng) % 12)));  // near the top
        for (int i = 1; i < 4; ++i) {
            const int k = (int)(ud(rng) % 16383) - 8191;
            const int kind = (int)(ud(rng) % 3);
            float x = ((float)k + (kind == 0 ? 0.5f : kind == 1 ? 0.25f : 0.75f)) * step;
            if (ud(rng) & 1) x = std::nextafter(x, ud(rng) & 2 ? 1e30f : -1e30f);
            v[i] = x;
        }
        check(v);
    }
    const float specials[] = {0.f, -0.f, 1e-45f, -1e-45f, 1.17549435e-38f, 3.4028235e38f, -3.4028235e38f,
                              INFINITY, -INFINITY, NAN, 1.f, -1.f, 8191.5f, 0.5f};
    for (float a : specials)
        for (float b : specials)
            for (float c : specials) {
                v[0] = a; v[1] = b; v[2] = c; v[3] = 1.f;
                check(v);
            }
    std::printf("blocks %ld mismatches %ld\n", n, bad);
    return bad != 0;
}
