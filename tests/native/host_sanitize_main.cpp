// Runs the host core (rq_host.cpp: parameter tables, Lloyd-Max and polar
// codebooks, QR, slot tables, layouts) for every session kind and prints one
// FNV-1a digest per (bits, mode) over every table it builds.  The CPU test
// compiles this file together with rq_host.cpp under AddressSanitizer and
// UndefinedBehaviorSanitizer (no recovery), runs it, and compares the digests
// with the same tables read through the built library's rq_host_params.
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../kv_cache_vector_norm_amd/csrc/rq_host.h"

namespace {

uint64_t fnv(uint64_t h, const void* p, size_t n) {
    const unsigned char* b = static_cast<const unsigned char*>(p);
    for (size_t i = 0; i < n; ++i) {
        h ^= b[i];
        h *= 1099511628211ULL;
    }
    return h;
}

template <class T>
uint64_t fnv_vec(uint64_t h, const std::vector<T>& v) {
    return v.empty() ? h : fnv(h, v.data(), v.size() * sizeof(T));
}

}  // namespace

int main() {
    struct Case {
        int bits, mode;
    };
    const Case cases[] = {{1, 0}, {2, 0}, {3, 0}, {4, 0}, {1, 1}, {2, 1}, {3, 1}, {4, 1}, {5, 1},
                          {2, 2}, {3, 2}, {4, 2}, {3, 3}, {1, 3}, {4, 4}};
    int failures = 0;
    for (const Case& c : cases) {
        rqh::Tables t;
        std::string err;
        const int rc = rqh::make_tables(128, c.bits, 0, c.mode, &t, &err);
        if (rc != 0) {
            std::printf("FAIL bits=%d mode=%d rc=%d %s\n", c.bits, c.mode, rc, err.c_str());
            ++failures;
            continue;
        }
        uint64_t h = 1469598103934665603ULL;
        h = fnv_vec(h, t.rotors);
        h = fnv_vec(h, t.rotmats);
        h = fnv_vec(h, t.centroids);
        h = fnv_vec(h, t.boundaries);
        h = fnv_vec(h, t.pi);
        h = fnv_vec(h, t.s);
        std::printf("tables bits=%d mode=%d %016llx\n", c.bits, c.mode, static_cast<unsigned long long>(h));
    }
    // invalid and unsupported arguments take their error paths cleanly
    rqh::Layout lay;
    std::string err;
    if (rqh::make_layout(64, 3, 0, &lay, &err) != 2) ++failures;
    if (rqh::make_layout(128, 9, 0, &lay, &err) != 1) ++failures;
    if (rqh::make_layout(128, 3, 8, &lay, &err) != 1) ++failures;
    std::printf("failures %d\n", failures);
    return failures ? 1 : 0;
}
