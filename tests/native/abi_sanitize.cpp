// abi_sanitize.cpp -- drives the host side of the C ABI (argument checks,
// workspace sizing, status strings) with bad, empty and extreme arguments in
// a process where the library's host code is built with AddressSanitizer and
// UndefinedBehaviorSanitizer.  Every call here is refused or sized before
// any HIP call (each expects the status that says so), so no GPU is needed
// and none is touched.  Compiled and run by
// tests/test_sanitize_host.py.
#include "specverify.h"

#include <climits>
#include <cmath>
#include <cstdio>
#include <cstdlib>

static int g_calls = 0;

static void expect(int got, int want, int line)
{
    ++g_calls;
    if (got != want) {
        std::fprintf(stderr, "line %d: status %d, expected %d\n", line, got, want);
        std::exit(2);
    }
}
#define EXPECT(call, want) expect((call), (want), __LINE__)

// A 16-byte aligned address that is never dereferenced: validation returns first.
static void* fake(uintptr_t off = 0) { return reinterpret_cast<void*>(uintptr_t(0x10000) + off); }

template <typename T>
static T* fk(uintptr_t off = 0) { return static_cast<T*>(fake(off)); }

static int chain(int dt, int B, int N, int V, float T, const void* tq, int64_t qr, void* ws, size_t wsb,
                 int32_t* src = nullptr, int32_t* kvl = nullptr, const int32_t* kvin = nullptr,
                 int32_t* tok = fk<int32_t>(), int32_t* num = fk<int32_t>())
{
    return spec_verify_chain(tq, (int64_t(N) + 1) * qr, qr, fake(), int64_t(N) * qr, qr, dt, fk<int32_t>(), B, N, V,
                             1, 2, T, tok, num, nullptr, nullptr, nullptr, kvin, src, kvl, ws, wsb, nullptr,
                             nullptr);
}

int main()
{
    EXPECT(sv_abi_version() > 0, 1);
    for (int c = -3; c < 12; ++c) EXPECT(sv_status_string(c) != nullptr, 1);

    // workspace sizes: ordinary, refused and extreme shapes (no overflow)
    EXPECT(sv_chain_workspace_bytes(256, 7, 128256) > 0, 1);
    EXPECT(sv_chain_workspace_bytes(1, 65, 10) == 0, 1);
    const int ext[] = {-1, 0, 1, 7, 64, 1 << 20, INT_MAX};
    for (int B : ext)
        for (int N : ext)
            for (int V : ext) {
                (void)sv_chain_workspace_bytes(B, N, V);
                (void)sv_tree_workspace_bytes(B, N, V);
                g_calls += 2;
            }

    // chain: every refusal the header documents
    const size_t big = size_t(1) << 30;
    EXPECT(chain(7, 2, 3, 32, 1.0f, fake(), 32, fake(), big), SV_EDTYPE);
    EXPECT(chain(0, 2, 3, 32, 0.0f, fake(), 32, fake(), big), SV_EINVAL);
    EXPECT(chain(0, 2, 3, 32, -1.0f, fake(), 32, fake(), big), SV_EINVAL);
    EXPECT(chain(0, 2, 3, 32, NAN, fake(), 32, fake(), big), SV_EINVAL);
    EXPECT(chain(0, 2, 3, 32, INFINITY, fake(), 32, fake(), big), SV_EINVAL);
    EXPECT(chain(0, 2, 65, 32, 1.0f, fake(), 32, fake(), big), SV_ESHAPE);
    EXPECT(chain(0, 2, 3, 0, 1.0f, fake(), 32, fake(), big), SV_EINVAL);
    EXPECT(chain(0, -1, 3, 32, 1.0f, fake(), 32, fake(), big), SV_EINVAL);
    EXPECT(chain(0, 2, -1, 32, 1.0f, fake(), 32, fake(), big), SV_EINVAL);
    EXPECT(chain(0, 2, 3, 32, 1.0f, nullptr, 32, fake(), big), SV_EINVAL);
    EXPECT(chain(0, 2, 3, 32, 1.0f, fake(2), 32, fake(), big), SV_EALIGN);
    EXPECT(chain(1, 2, 3, 32, 1.0f, fake(1), 32, fake(), big), SV_EALIGN);
    EXPECT(chain(0, 2, 3, 32, 1.0f, fake(), -32, fake(), big), SV_EINVAL);
    EXPECT(chain(0, 2, 3, 32, 1.0f, fake(), 32, fake(), 16), SV_EWORKSPACE);
    EXPECT(chain(0, 2, 3, 32, 1.0f, fake(), 32, nullptr, big), SV_EWORKSPACE);
    EXPECT(chain(0, 2, 3, 32, 1.0f, fake(), 32, fake(), big, fk<int32_t>()), SV_EINVAL);
    EXPECT(chain(0, 2, 3, 32, 1.0f, fake(), 32, fake(), big, nullptr, fk<int32_t>()), SV_EINVAL);
    EXPECT(chain(0, 2, 3, 32, 1.0f, fake(), 32, fake(), big, nullptr, nullptr, nullptr, nullptr), SV_EINVAL);
    EXPECT(chain(0, 2, 3, 32, 1.0f, fake(), 32, fake(), big, nullptr, nullptr, nullptr, fk<int32_t>(), nullptr),
           SV_EINVAL);
    EXPECT(chain(0, 0, 3, 32, 1.0f, fake(), 32, fake(), big), SV_OK);
    // extreme sizes and strides are refused, never overflowed
    EXPECT(chain(1, INT_MAX, 64, INT_MAX, 1.0f, fake(), INT_MAX, fake(), big), SV_ESHAPE);
    EXPECT(chain(1, 1 << 20, 64, 1 << 20, 1.0f, fake(), 1 << 20, fake(), big), SV_ESHAPE);
    EXPECT(chain(0, 2, 3, 32, 1.0f, fake(), INT64_MAX / 4, fake(), big), SV_EINVAL);

    // the no-allocation entry point: sizes past its static scratch, empty, bad shape
    EXPECT(spec_verify_chain_noalloc(fake(), 8 * 128256, 128256, fake(), 8 * 128256, 128256, 1, fk<int32_t>(), 1024,
                                     7, 128256, 0, 0, 1.0f, fk<int32_t>(), fk<int32_t>(), nullptr, nullptr, nullptr,
                                     nullptr, nullptr, nullptr, nullptr, nullptr),
           SV_ESCRATCH);
    EXPECT(spec_verify_chain_noalloc(fake(), 8 * 32, 32, fake(), 8 * 32, 32, 0, fk<int32_t>(), 0, 3, 32, 0, 0, 1.0f,
                                     fk<int32_t>(), fk<int32_t>(), nullptr, nullptr, nullptr, nullptr, nullptr,
                                     nullptr, nullptr, nullptr),
           SV_OK);
    EXPECT(spec_verify_chain_noalloc(fake(), 8 * 32, 32, fake(), 8 * 32, 32, 0, fk<int32_t>(), 2, 65, 32, 0, 0, 1.0f,
                                     fk<int32_t>(), fk<int32_t>(), nullptr, nullptr, nullptr, nullptr, nullptr,
                                     nullptr, nullptr, nullptr),
           SV_ESHAPE);
    EXPECT(spec_verify_chain_noalloc(fake(), 8 * 32, 32, fake(), 8 * 32, 32, 0, fk<int32_t>(), INT_MAX, 64, INT_MAX,
                                     0, 0, 1.0f, fk<int32_t>(), fk<int32_t>(), nullptr, nullptr, nullptr, nullptr,
                                     nullptr, nullptr, nullptr, nullptr), SV_ESHAPE);

    // tree
    auto tree = [](int dt, int B, int T, int V, int md, int walk, float temp, const int32_t* par, int32_t* path,
                   size_t wsb, int32_t* src = nullptr, int32_t* kvl = nullptr) {
        return spec_verify_tree(fake(), (int64_t(T) + 1) * 32, 32, fake(), (int64_t(T) + 1) * 32, 32, dt, fk<int32_t>(),
                                par, 1, B, T, V, md, walk, 0, 0, temp, fk<int32_t>(), path, fk<int32_t>(), nullptr,
                                nullptr, nullptr, nullptr, src, kvl, fake(), wsb, nullptr, nullptr);
    };
    const size_t wsb = size_t(1) << 30;
    EXPECT(tree(0, 2, 1024, 32, 3, 0, 1.0f, fk<int32_t>(), fk<int32_t>(), wsb), SV_ESHAPE);
    EXPECT(tree(0, 2, 5, 32, 6, 0, 1.0f, fk<int32_t>(), fk<int32_t>(), wsb), SV_ESHAPE);
    EXPECT(tree(0, 2, 5, 32, -1, 0, 1.0f, fk<int32_t>(), fk<int32_t>(), wsb), SV_EINVAL);
    EXPECT(tree(0, 2, 5, 32, 3, 0, 1.0f, nullptr, fk<int32_t>(), wsb), SV_EINVAL);
    EXPECT(tree(0, 2, 5, 32, 3, 0, 1.0f, fk<int32_t>(), nullptr, wsb), SV_EINVAL);
    EXPECT(tree(0, 2, 5, 32, 3, 0, 0.0f, fk<int32_t>(), fk<int32_t>(), wsb), SV_EINVAL);
    EXPECT(tree(9, 2, 5, 32, 3, 0, 1.0f, fk<int32_t>(), fk<int32_t>(), wsb), SV_EDTYPE);
    EXPECT(tree(0, 2, 5, 32, 3, 0, 1.0f, fk<int32_t>(), fk<int32_t>(), 100), SV_EWORKSPACE);
    EXPECT(tree(0, 2, 5, 32, 3, 2, 1.0f, fk<int32_t>(), fk<int32_t>(), wsb), SV_EINVAL);
    EXPECT(tree(0, 2, 5, 32, 3, -1, 1.0f, fk<int32_t>(), fk<int32_t>(), wsb), SV_EINVAL);
    EXPECT(tree(0, 2, 5, 32, 3, 0, 1.0f, fk<int32_t>(), fk<int32_t>(), wsb, fk<int32_t>()), SV_EINVAL);
    EXPECT(tree(0, 0, 5, 32, 3, 1, 1.0f, fk<int32_t>(), fk<int32_t>(), wsb), SV_OK);
    EXPECT(tree(1, INT_MAX, 1023, INT_MAX, 1023, 0, 1.0f, fk<int32_t>(), fk<int32_t>(), wsb), SV_ESHAPE);
    EXPECT(tree(0, -5, -5, -5, -5, 0, 1.0f, fk<int32_t>(), fk<int32_t>(), wsb), SV_EINVAL);
    EXPECT(tree(0, 2, INT_MAX, 32, 3, 0, 1.0f, fk<int32_t>(), fk<int32_t>(), wsb), SV_ESHAPE);

    // KV compaction
    EXPECT(kv_compact_indices(nullptr, fk<int32_t>(), fk<int32_t>(), 2, -1, fk<int32_t>(), fk<int32_t>(), nullptr, 0,
                              0, 0, 0, 0, 0, nullptr),
           SV_EINVAL);
    EXPECT(kv_compact_indices(nullptr, nullptr, fk<int32_t>(), 2, 3, fk<int32_t>(), fk<int32_t>(), nullptr, 0, 0, 0,
                              0, 0, 0, nullptr),
           SV_EINVAL);
    EXPECT(kv_compact_indices(nullptr, fk<int32_t>(), fk<int32_t>(), 2, 3, fk<int32_t>(), fk<int32_t>(), fake(8), 64,
                              4096, 64, 64, 1, 0, nullptr),
           SV_EALIGN);
    EXPECT(kv_compact_indices(nullptr, fk<int32_t>(), fk<int32_t>(), 2, 3, fk<int32_t>(), fk<int32_t>(), fake(), 64,
                              4096, 64, 128, 1, 0, nullptr),
           SV_EINVAL);
    EXPECT(kv_compact_indices(nullptr, fk<int32_t>(), fk<int32_t>(), 70000, 3, fk<int32_t>(), fk<int32_t>(), fake(),
                              64, 4096, 64, 64, 1, 0, nullptr),
           SV_ESHAPE);
    EXPECT(kv_compact_indices(nullptr, fk<int32_t>(), fk<int32_t>(), 2, 3, fk<int32_t>(), fk<int32_t>(), fake(), 64,
                              4096, 64, 64, 70000, 0, nullptr),
           SV_ESHAPE);
    EXPECT(kv_compact_indices(nullptr, fk<int32_t>(), fk<int32_t>(), 0, 3, fk<int32_t>(), fk<int32_t>(), nullptr, 0,
                              0, 0, 0, 0, 0, nullptr),
           SV_OK);
    EXPECT(kv_compact_indices(nullptr, fk<int32_t>(), fk<int32_t>(), INT_MAX, INT_MAX, fk<int32_t>(), fk<int32_t>(),
                              fake(), INT_MAX, INT64_MAX, INT64_MAX, INT_MAX, INT_MAX, INT64_MAX, nullptr), SV_EALIGN);

    // tree mask, tree build, draft sampler, uniforms
    EXPECT(kv_compact_indices(nullptr, fk<int32_t>(), fk<int32_t>(), 60000, 3, fk<int32_t>(), fk<int32_t>(), fake(),
                              64, int64_t(1) << 52, 4096, 64, 4, int64_t(1) << 60, nullptr),
           SV_EINVAL);
    EXPECT(tree_attention_mask(fk<int32_t>(), 1, nullptr, 2, 1024, fk<uint64_t>(), fk<int32_t>(), nullptr),
           SV_ESHAPE);
    EXPECT(tree_attention_mask(fk<int32_t>(), 1, nullptr, 2, INT_MAX, fk<uint64_t>(), fk<int32_t>(), nullptr),
           SV_ESHAPE);
    EXPECT(tree_attention_mask(fk<int32_t>(), 1, nullptr, -1, 5, fk<uint64_t>(), fk<int32_t>(), nullptr), SV_EINVAL);
    EXPECT(tree_attention_mask(nullptr, 1, nullptr, 2, 5, fk<uint64_t>(), fk<int32_t>(), nullptr), SV_EINVAL);
    EXPECT(tree_attention_mask(fk<int32_t>(), 1, nullptr, 0, 5, fk<uint64_t>(), fk<int32_t>(), nullptr), SV_OK);
    auto ex = [](int dt, int B, int F, int V, int k, float T, int lvl, int nmax, int off, const void* rows) {
        return tree_expand(rows, int64_t(F) * V, V, dt, B, F, V, k, T, nullptr, nullptr, lvl, nmax, off,
                           fk<int32_t>(), fk<int32_t>(), fk<int32_t>(), fk<double>(), nullptr);
    };
    EXPECT(ex(5, 2, 3, 100, 10, 1.0f, 1, 30, 0, fake()), SV_EDTYPE);
    EXPECT(ex(1, 2, 3, 100, 17, 1.0f, 1, 30, 0, fake()), SV_ESHAPE);
    EXPECT(ex(1, 2, 3, 100, 0, 1.0f, 1, 30, 0, fake()), SV_ESHAPE);
    EXPECT(ex(1, 2, 3, 5, 10, 1.0f, 1, 30, 0, fake()), SV_ESHAPE);
    EXPECT(ex(1, 2, 3, 100, 10, 1.0f, 1, 30, 1, fake()), SV_ESHAPE);
    EXPECT(ex(1, 2, 3, 100, 10, 1.0f, 1, 4096, 0, fake()), SV_ESHAPE);
    EXPECT(ex(1, 2, 3, 100, 10, 0.0f, 1, 30, 0, fake()), SV_EINVAL);
    EXPECT(ex(1, 2, 3, 100, 10, 1.0f, 0, 30, 0, fake()), SV_EINVAL);
    EXPECT(ex(1, 2, 3, 100, 10, 1.0f, 1, 30, 0, nullptr), SV_EINVAL);
    EXPECT(ex(1, 2, 3, 100, 10, 1.0f, 1, 30, 0, fake(1)), SV_EALIGN);
    EXPECT(ex(1, 0, 3, 100, 10, 1.0f, 1, 30, 0, fake()), SV_OK);
    EXPECT(ex(1, INT_MAX, INT_MAX, INT_MAX, 16, 1.0f, INT_MAX, INT_MAX, INT_MAX, fake()), SV_ESHAPE);
    EXPECT(tree_select(fk<double>(), 2, 30, 0, 31, 10, fk<int32_t>(), fk<double>(), nullptr), SV_ESHAPE);
    EXPECT(tree_select(fk<double>(), 2, 30, 0, 20, 21, fk<int32_t>(), fk<double>(), nullptr), SV_EINVAL);
    EXPECT(tree_select(fk<double>(), 0, 30, 0, 20, 10, fk<int32_t>(), fk<double>(), nullptr), SV_OK);
    EXPECT(tree_select(fk<double>(), INT_MAX, INT_MAX, INT_MAX, INT_MAX, INT_MAX, fk<int32_t>(), fk<double>(),
                       nullptr), SV_ESHAPE);
    EXPECT(tree_finalize(fk<int32_t>(), fk<int32_t>(), fk<int32_t>(), fk<double>(), 2, 30, 30, 31, fk<int32_t>(),
                         fk<int32_t>(), fk<int32_t>(), fk<double>(), nullptr),
           SV_EINVAL);
    EXPECT(tree_finalize(fk<int32_t>(), fk<int32_t>(), fk<int32_t>(), fk<double>(), 2, 4096, 510, 60, fk<int32_t>(),
                         fk<int32_t>(), fk<int32_t>(), fk<double>(), nullptr),
           SV_ESHAPE);
    EXPECT(tree_finalize(fk<int32_t>(), fk<int32_t>(), fk<int32_t>(), fk<double>(), 2, 30, 30, 10, nullptr,
                         fk<int32_t>(), fk<int32_t>(), fk<double>(), nullptr),
           SV_EINVAL);
    auto sd = [](int dt, int B, int R, int V, float T, int pos0, const void* rows, int32_t* out) {
        return sv_sample_draft(rows, int64_t(R) * V, V, dt, B, R, V, T, 0, 0, pos0, out, nullptr, nullptr);
    };
    EXPECT(sd(3, 2, 3, 100, 1.0f, 0, fake(), fk<int32_t>()), SV_EDTYPE);
    EXPECT(sd(1, 2, 3, 0, 1.0f, 0, fake(), fk<int32_t>()), SV_EINVAL);
    EXPECT(sd(1, 2, 3, 524289, 1.0f, 0, fake(), fk<int32_t>()), SV_ESHAPE);
    EXPECT(sd(1, 2, 3, 100, 0.0f, 0, fake(), fk<int32_t>()), SV_EINVAL);
    EXPECT(sd(1, 2, 3, 100, INFINITY, 0, fake(), fk<int32_t>()), SV_EINVAL);
    EXPECT(sd(1, 2, 3, 100, 1.0f, -1, fake(), fk<int32_t>()), SV_EINVAL);
    EXPECT(sd(1, 2, 3, 100, 1.0f, 0, nullptr, fk<int32_t>()), SV_EINVAL);
    EXPECT(sd(1, 2, 3, 100, 1.0f, 0, fake(), nullptr), SV_EINVAL);
    EXPECT(sd(1, 2, 3, 100, 1.0f, 0, fake(1), fk<int32_t>()), SV_EALIGN);
    EXPECT(sd(1, 0, 3, 100, 1.0f, 0, fake(), fk<int32_t>()), SV_OK);
    EXPECT(sd(1, INT_MAX, INT_MAX, 524288, 1.0f, INT_MAX, fake(), fk<int32_t>()), SV_ESHAPE);
    EXPECT(sv_sample_draft(fake(), INT64_MAX / 2, 100, 1, 2, 3, 100, 1.0f, 0, 0, 0, fk<int32_t>(), nullptr, nullptr),
           SV_EINVAL);
    EXPECT(sv_sample_draft(fake(), int64_t(1) << 60, 100, 1, 3, 3, 100, 1.0f, 0, 0, 0, fk<int32_t>(), nullptr,
                           nullptr),
           SV_EINVAL);
    EXPECT(tree_expand(fake(), int64_t(1) << 61, 100, 1, 2, 3, 100, 10, 1.0f, nullptr, nullptr, 1, 30, 0,
                       fk<int32_t>(), fk<int32_t>(), fk<int32_t>(), fk<double>(), nullptr),
           SV_EINVAL);
    EXPECT(sv_philox_uniforms(0, 0, -1, 3, fk<double>(), nullptr, nullptr), SV_EINVAL);
    EXPECT(sv_philox_uniforms(0, 0, INT_MAX, INT_MAX, fk<double>(), nullptr, nullptr), SV_ESHAPE);

    std::printf("abi sanitize: %d calls clean\n", g_calls);
    return 0;
}
