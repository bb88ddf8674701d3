// Host-side checks of the convtile C ABI, built host-only with AddressSanitizer
// and UndefinedBehaviorSanitizer (no device code: nothing here launches).
// Exercises the argument checks, the config space and its legality check,
// the split enumerator, the tuning-log reader (resume order, cache load of
// well-formed and malformed lines, save), the ridge fit and guided search on
// host tables, and the status / variant introspection.  Exit status 0 when
// every check holds; a sanitizer report aborts the process.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "convtile.h"

static int g_fail = 0;
#define CHECK(cond)                                                         \
    do {                                                                    \
        if (!(cond)) {                                                      \
            std::fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond); \
            ++g_fail;                                                       \
        }                                                                   \
    } while (0)

static void write_file(const std::string& path, const std::string& text) {
    FILE* f = std::fopen(path.c_str(), "w");
    if (!f) return;
    std::fputs(text.c_str(), f);
    std::fclose(f);
}

int main(int argc, char** argv) {
    const std::string dir = argc > 1 ? argv[1] : "/tmp";
    // argument checks
    float y = 0;
    const int bad[][9] = {{0, 1, 1, 1, 1, 1, 1, 1, 0}, {1, 1, 1, 1, 1, 1, 1, 0, 0},
                          {1, 1, 1, 1, 1, 1, 1, 1, -1}, {1, 1, 1, 1, 1, 5, 5, 1, 0}};
    for (const auto& b : bad)
        CHECK(ct_conv2d_nchw_fwd(&y, &y, &y, b[0], b[1], b[2], b[3], b[4], b[5], b[6], b[7], b[8], CT_F32,
                                 CT_EPI_NONE, nullptr, nullptr, 1e-5f, nullptr) == CT_ERR_INVALID_ARG);
    CHECK(ct_conv2d_nchw_fwd(nullptr, &y, &y, 1, 1, 3, 3, 1, 3, 3, 1, 1, CT_F32, CT_EPI_NONE, nullptr, nullptr,
                             1e-5f, nullptr) == CT_ERR_INVALID_ARG);
    CHECK(ct_conv2d_nchw_fwd(&y, &y, &y, 1, 1, 3, 3, 1, 3, 3, 1, 1, 7, CT_EPI_NONE, nullptr, nullptr, 1e-5f,
                             nullptr) == CT_ERR_INVALID_ARG);
    CHECK(ct_conv2d_nchw_fwd(&y, &y, &y, 1, 1, 3, 3, 1, 3, 3, 1, 1, CT_F32, CT_EPI_BIAS, nullptr, nullptr, 1e-5f,
                             nullptr) == CT_ERR_INVALID_ARG);
    CHECK(std::strlen(ct_last_error()) > 0);
    CHECK(ct_gemm_fwd(&y, &y, &y, 0, 4, 4, CT_F32, 0, nullptr, nullptr, 1e-5f, nullptr) == CT_ERR_INVALID_ARG);
    CHECK(ct_broadcast_nchw(nullptr, &y, 1, 1, 1, 1, CT_F32, CT_BC_EXP, CT_BC_AUTO, nullptr) == CT_ERR_INVALID_ARG);
    ct_bcast_program prog{};
    prog.n_ops[0] = CT_CHAIN_MAX_OPS + 1;
    CHECK(ct_broadcast_chain(&prog, nullptr, nullptr, nullptr, nullptr, nullptr, &y, CT_F32, 1, 1, 1, CT_BC_AUTO,
                             nullptr) == CT_ERR_INVALID_ARG);
    CHECK(ct_conv2d_filter_prepared_bytes(40, 12, 3, 3, CT_F16) == 2LL * 40 * 64 * 9);
    CHECK(ct_conv2d_filter_prepared_bytes(40, 12, 3, 3, CT_F32) == CT_ERR_INVALID_ARG);

    // the config space of the final ResNet layer: every point decodes, the
    // legality check runs without a device, indices round-trip
    const int sh[11] = {1, 512, 7, 7, 512, 3, 3, 1, 1, CT_F32, CT_EPI_NONE};
    const long long n = ct_conv2d_space_size(sh[0], sh[1], sh[2], sh[3], sh[4], sh[5], sh[6], sh[7], sh[8], sh[9],
                                             sh[10]);
    CHECK(n > 0);
    long long n_legal = 0;
    for (long long i = 0; i < n; ++i) {
        ct_tile_config c{};
        int legal = -1;
        CHECK(ct_conv2d_space_entity(sh[0], sh[1], sh[2], sh[3], sh[4], sh[5], sh[6], sh[7], sh[8], sh[9], sh[10], i,
                                     &c, &legal) == CT_OK);
        CHECK(c.index == i && (legal == 0 || legal == 1));
        n_legal += legal;
    }
    CHECK(n_legal > 0);
    ct_tile_config c{};
    CHECK(ct_conv2d_space_entity(sh[0], sh[1], sh[2], sh[3], sh[4], sh[5], sh[6], sh[7], sh[8], sh[9], sh[10], n, &c,
                                 nullptr) == CT_ERR_INVALID_ARG);
    int from_cache = -1;
    CHECK(ct_conv2d_query(sh[0], sh[1], sh[2], sh[3], sh[4], sh[5], sh[6], sh[7], sh[8], sh[9], sh[10], &c,
                          &from_cache) == CT_OK);
    CHECK(from_cache == 0);

    // the split enumerator: the printed space lengths of the tutorial's run
    CHECK(ct_split_count(512, 4) == 220 && ct_split_count(7, 4) == 4 && ct_split_count(3, 3) == 3);
    long long e[4];
    for (long long i = 0; i < 220; ++i) {
        CHECK(ct_split_entity(512, 4, i, e) == CT_OK);
        CHECK(e[0] * e[1] * e[2] * e[3] == 512);
    }
    CHECK(ct_split_entity(512, 4, 220, e) == CT_ERR_INVALID_ARG);
    CHECK(ct_split_count(0, 2) < 0 && ct_split_count(8, 9) < 0);

    // the tutorial template's space: the printed size, a decode/encode round
    // trip over a stride of the space, and the best config's shared bytes
    CHECK(ct_tvm_space_size(1, 512, 7, 7, 512, 3, 3, 1, 1) == 10454400);
    for (long long i = 0; i < 10454400; i += 104543) {
        ct_tvm_config tc{};
        CHECK(ct_tvm_space_entity(1, 512, 7, 7, 512, 3, 3, 1, 1, i, &tc) == CT_OK);
        CHECK(ct_tvm_space_index(1, 512, 7, 7, 512, 3, 3, 1, 1, &tc) == i);
        long long nb = 0;
        int nt = 0;
        const int fits = ct_tvm_config_check(&tc, 1, CT_TVM_LIMITS_GFX950, &nb, &nt);
        CHECK((fits == 0 || fits == 1) && nb > 0 && nt > 0);
    }
    const ct_tvm_config best = {{8, 1, 64, 1}, {1, 7, 1, 1}, {1, 7, 1, 1}, {64, 2, 4}, {1, 1, 3}, {1, 3, 1}, 1500, 1};
    long long best_bytes = 0;
    CHECK(ct_tvm_config_check(&best, 1, CT_TVM_LIMITS_PAGE, &best_bytes, nullptr) == 1);
    CHECK(best_bytes == 4LL * (8 * 9 * 9 + 64 * 8 * 3 * 3));
    CHECK(ct_tvm_space_index(1, 512, 7, 7, 512, 3, 3, 1, 1, &best) == 9751545);
    CHECK(ct_tvm_config_check(nullptr, 1, CT_TVM_LIMITS_PAGE, nullptr, nullptr) == CT_ERR_INVALID_ARG);

    // tuning log: resume order, then a log with malformed lines loads the
    // fastest successful record and ignores the rest
    std::vector<long long> order(n);
    int n_order = 0;
    setenv("CT_CACHE_PATH", (dir + "/none.jsonl").c_str(), 1);
    CHECK(ct_conv2d_tune_order(sh[0], sh[1], sh[2], sh[3], sh[4], sh[5], sh[6], sh[7], sh[8], sh[9], sh[10], 0,
                               order.data(), (int)n, &n_order) == CT_OK);
    CHECK(n_order == n);
    ct_tile_config c0{}, c1{};
    CHECK(ct_conv2d_space_entity(sh[0], sh[1], sh[2], sh[3], sh[4], sh[5], sh[6], sh[7], sh[8], sh[9], sh[10],
                                 order[0], &c0, nullptr) == CT_OK);
    CHECK(ct_conv2d_space_entity(sh[0], sh[1], sh[2], sh[3], sh[4], sh[5], sh[6], sh[7], sh[8], sh[9], sh[10],
                                 order[1], &c1, nullptr) == CT_OK);
    ct_variant_desc d0{}, d1{};
    CHECK(ct_variant_info(c0.variant, &d0) == CT_OK && ct_variant_info(c1.variant, &d1) == CT_OK);
    auto rec = [&](const ct_tile_config& cf, const char* name, int err, double us) {
        char buf[512];
        std::snprintf(buf, sizeof(buf),
                      "{\"key\":\"1,512,7,7,512,3,3,1,1,0,0,gfx950,v1\",\"N\":1,\"CI\":512,\"H\":7,\"W\":7,\"CO\":512,"
                      "\"KH\":3,\"KW\":3,\"stride\":1,\"pad\":1,\"dtype\":0,\"epilogue\":0,\"arch\":\"gfx950\","
                      "\"variant\":\"%s\",\"split_k\":%d,\"stages\":%d,\"kc\":%d,\"index\":-1,\"us\":%g,"
                      "\"error_no\":%d,\"costs_us\":[%g,%g,%g],\"all_cost\":0.1,\"timestamp\":1}\n",
                      name, cf.split_k, cf.stages, cf.kc, us, err, us, us, us);
        return std::string(buf);
    };
    const std::string log = dir + "/log.jsonl";
    write_file(log, rec(c0, d0.name, 0, 9.0) + rec(c1, d1.name, 6, 1.0) + "{\"key\":\"trunc\n" + "\n" +
                        "{\"key\":\"1,512,7,7,512,3,3,1,1,0,0,gfx950,v1\",\"split_k\":\"x\"}\n" +
                        std::string(600, 'x') + "\n" + "[1,2,3]\n" + "{\"a\":[1,2\n");
    setenv("CT_CACHE_PATH", log.c_str(), 1);
    std::vector<long long> order2(n);
    int n2 = 0;
    CHECK(ct_conv2d_tune_order(sh[0], sh[1], sh[2], sh[3], sh[4], sh[5], sh[6], sh[7], sh[8], sh[9], sh[10], 0,
                               order2.data(), (int)n, &n2) == CT_OK);
    CHECK(n2 == n - 2 && order2[0] == order[2]);
    CHECK(ct_cache_clear() == CT_OK);
    CHECK(ct_cache_load(log.c_str()) == CT_OK);
    CHECK(ct_cache_size() == 1);
    CHECK(ct_conv2d_query(sh[0], sh[1], sh[2], sh[3], sh[4], sh[5], sh[6], sh[7], sh[8], sh[9], sh[10], &c,
                          &from_cache) == CT_OK);
    CHECK(from_cache == 1 && c.variant == c0.variant && c.split_k == c0.split_k);
    CHECK(ct_cache_save((dir + "/saved.jsonl").c_str()) == CT_OK);
    CHECK(ct_cache_load((dir + "/missing/none.jsonl").c_str()) == CT_ERR_IO);
    CHECK(ct_cache_load(nullptr) == CT_ERR_INVALID_ARG);
    CHECK(ct_cache_clear() == CT_OK && ct_cache_size() == 0);
    unsetenv("CT_CACHE_PATH");

    // ridge fit and guided search on host tables
    const int rows = 40, d = 3;
    std::vector<double> X(rows * d), yv(rows), wv(d);
    for (int i = 0; i < rows; ++i) {
        X[i * d] = 1.0;
        X[i * d + 1] = i;
        X[i * d + 2] = (i * 7) % 5;
        yv[i] = 2.0 - 0.5 * i + 0.25 * X[i * d + 2];
    }
    CHECK(ct_ridge_fit(X.data(), yv.data(), rows, d, 0.0, wv.data()) == CT_OK);
    CHECK(std::fabs(wv[0] - 2.0) < 1e-9 && std::fabs(wv[1] + 0.5) < 1e-9 && std::fabs(wv[2] - 0.25) < 1e-9);
    CHECK(ct_ridge_fit(X.data(), yv.data(), rows, 0, 0.0, wv.data()) == CT_ERR_INVALID_ARG);
    std::vector<double> cost(rows);
    for (int i = 0; i < rows; ++i) cost[i] = std::exp(yv[i] / 10.0);
    std::vector<int> ord(rows);
    int n_ord = 0;
    CHECK(ct_guided_search_table(X.data(), cost.data(), rows, d, 16, 4, 1, 7, 1e-3, ord.data(), &n_ord) == CT_OK);
    CHECK(n_ord == 16);
    CHECK(ct_guided_search_table(X.data(), cost.data(), rows, d, 16, 0, 1, 7, 1e-3, ord.data(), &n_ord) ==
          CT_ERR_INVALID_ARG);

    // introspection
    const int nv = ct_variant_count();
    CHECK(nv > 0);
    for (int v = 0; v < nv; ++v) {
        ct_variant_desc vd{};
        CHECK(ct_variant_info(v, &vd) == CT_OK && std::strlen(vd.name) > 0);
    }
    CHECK(ct_variant_info(nv, &d0) == CT_ERR_INVALID_ARG);
    for (int s = -7; s <= 1; ++s) CHECK(ct_status_string(s) != nullptr);
    CHECK(std::strstr(ct_version(), "gfx950") != nullptr);
    std::printf("host checks: %d failed\n", g_fail);
    return g_fail == 0 ? 0 : 1;
}
