// Host-side checks of libmhla's validation, workspace arithmetic and launch
// plans, built with AddressSanitizer and UndefinedBehaviorSanitizer on the
// host code (tests/test_abi_sanitized.py).  No GPU is used: every call here
// returns before any HIP call (validation errors, sizes, plans, empty
// problems, injected allocation failure).
#include <mhla.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

static int failures = 0;
#define CHECK(cond)                                                            \
    do {                                                                       \
        if (!(cond)) {                                                         \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            ++failures;                                                        \
        }                                                                      \
    } while (0)

static mhla_grid grid(int B, int H, int d, int dt, int nd, int e0, int e1, int e2, float eps = 1e-6f) {
    mhla_grid g;
    std::memset(&g, 0, sizeof(g));
    g.batch = B; g.heads = H; g.head_dim = d; g.dtype = dt; g.ndim = nd;
    g.extent[0] = e0; g.extent[1] = e1; g.extent[2] = e2;
    g.eps = eps;
    return g;
}
static mhla_block block(int e0, int e1, int e2 = 1) {
    mhla_block b;
    b.extent[0] = e0; b.extent[1] = e1; b.extent[2] = e2;
    return b;
}

int main() {
    const uintptr_t BIG = (uintptr_t)1 << 36;   // fake, aligned, never dereferenced
    auto P = [&](int k) { return reinterpret_cast<void*>(BIG * (uintptr_t)k); };
    // sweep of shapes: valid, ragged, invalid; every query function on each
    const int dims[] = {16, 32, 48, 64, 100, 128, 0, -3};
    const int blks[] = {1, 2, 3, 4, 5, 8, 16, 0, -1, 7};
    const int hds[] = {32, 64, 128, 16, 0};
    long valid = 0;
    for (int dt = 0; dt < 3; ++dt)
        for (int d : hds)
            for (int y : dims)
                for (int x : dims)
                    for (int by : blks)
                        for (int bx : blks) {
                            mhla_grid g = grid(2, 3, d, dt, 2, y, x, 0);
                            mhla_block b = block(by, bx);
                            int64_t M = -1, T = -1;
                            const mhla_status st = mhla_check_problem(&g, &b, &M, &T);
                            const size_t ws = mhla_workspace_bytes(&g, &b);
                            (void)mhla_backward_workspace_bytes(&g, &b);
                            (void)mhla_causal_backward_workspace_bytes(&g, &b);
                            (void)mhla_causal_stream_workspace_bytes(&g, &b);
                            (void)mhla_causal_state_bytes(&g, &b, 7);
                            (void)mhla_layer_workspace_bytes(&g, &b);
                            for (int path = 0; path < 4; ++path) {
                                int32_t n = -1;
                                const char* names[3] = {nullptr, nullptr, nullptr};
                                (void)mhla_launch_plan(&g, &b, path | (path == 0 ? MHLA_VARIANT_MIX_SPLIT : 0), &n, names);
                            }
                            if (st == MHLA_OK) {
                                ++valid;
                                CHECK(M >= 1 && T >= 1 && M * T == (int64_t)y * x);
                                CHECK(ws > 0);
                                // too-small workspace and misaligned pointers are rejected
                                CHECK(mhla_forward_ex(P(1), P(2), P(3), (const float*)P(4), &g, &b, P(5), P(6), ws - 1,
                                                      MHLA_PATH_3KERNEL, nullptr, nullptr) == MHLA_ERR_INVALID_ARG);
                                CHECK(mhla_forward_ex((char*)P(1) + 2, P(2), P(3), (const float*)P(4), &g, &b, P(5),
                                                      P(6), ws, MHLA_PATH_3KERNEL, nullptr, nullptr) ==
                                      MHLA_ERR_MISALIGNED);
                            } else {
                                CHECK(ws == 0);
                                CHECK(mhla_forward(P(1), P(2), P(3), (const float*)P(4), &g, &b, P(5), nullptr) == st);
                            }
                        }
    CHECK(valid > 100);
    // 3D grids
    {
        mhla_grid g = grid(1, 12, 128, MHLA_BF16, 3, 16, 64, 64);
        mhla_block b = block(4, 8, 8);
        int64_t M = 0, T = 0;
        CHECK(mhla_check_problem(&g, &b, &M, &T) == MHLA_OK && M == 256 && T == 256);
        CHECK(mhla_workspace_bytes(&g, &b) > 0);
    }
    // null structs, status strings
    CHECK(mhla_check_problem(nullptr, nullptr, nullptr, nullptr) == MHLA_ERR_INVALID_ARG);
    CHECK(mhla_workspace_bytes(nullptr, nullptr) == 0);
    for (int c = 0; c < 8; ++c) CHECK(mhla_status_string((mhla_status)c) != nullptr);
    // layer validation: missing parameters
    {
        mhla_grid g = grid(1, 6, 64, MHLA_BF16, 2, 64, 64, 0);
        mhla_block b = block(8, 8);
        mhla_layer_params lp;
        std::memset(&lp, 0, sizeof(lp));
        CHECK(mhla_layer_forward(P(1), (const float*)P(2), &g, &b, &lp, P(3), P(4), (size_t)1 << 40, nullptr,
                                 nullptr) == MHLA_ERR_INVALID_ARG);
        CHECK(mhla_layer_forward(P(1), (const float*)P(2), &g, &b, nullptr, P(3), P(4), (size_t)1 << 40, nullptr,
                                 nullptr) == MHLA_ERR_INVALID_ARG);
    }
    // causal streaming validation
    {
        mhla_grid g = grid(2, 3, 64, MHLA_BF16, 2, 1, 256, 0);
        mhla_block b = block(1, 64);
        CHECK(mhla_causal_stream(P(1), P(2), P(3), (const float*)P(4), 10, &g, &b, -1, (float*)P(6), 10, P(7), P(8),
                                 (size_t)1 << 30, nullptr) == MHLA_ERR_INVALID_ARG);
        CHECK(mhla_causal_stream(P(1), P(2), P(3), (const float*)P(4), 10, &g, &b, 7, (float*)P(6), 10, P(7), P(8),
                                 (size_t)1 << 30, nullptr) == MHLA_ERR_INVALID_ARG);
    }
    // no-alloc entry point: too large for the scratch, invalid, empty
    {
        mhla_grid g = grid(32, 6, 64, MHLA_BF16, 2, 64, 64, 0);
        mhla_block b = block(8, 8);
        CHECK(mhla_forward_noalloc(P(1), P(2), P(3), (const float*)P(4), &g, &b, P(5), nullptr) ==
              MHLA_ERR_UNSUPPORTED);
        mhla_grid e = grid(0, 6, 64, MHLA_BF16, 2, 64, 64, 0);
        CHECK(mhla_forward_noalloc(nullptr, nullptr, nullptr, nullptr, &e, &b, nullptr, nullptr) == MHLA_OK);
    }
    // injected allocation failure: the allocating entry points return MHLA_ERR_ALLOC
    {
        setenv("MHLA_FAIL_ALLOC", "1", 1);
        mhla_grid g = grid(1, 6, 64, MHLA_BF16, 2, 256, 256, 0);
        mhla_block b = block(16, 16);
        CHECK(mhla_forward(P(1), P(2), P(3), (const float*)P(4), &g, &b, P(5), nullptr) == MHLA_ERR_ALLOC);
        CHECK(mhla_backward(P(1), P(2), P(3), (const float*)P(4), P(5), &g, &b, P(6), P(7), P(8), (float*)P(9),
                            nullptr, 0, nullptr, nullptr) == MHLA_ERR_ALLOC);
        unsetenv("MHLA_FAIL_ALLOC");
    }
    if (failures) {
        std::fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    std::printf("OK %ld valid shapes\n", valid);
    return 0;
}
