// Host-side entry points of libbsa: error reporting, the tile permutation
// (plain and padded) and its inverse, the top-k budget, and the sliding-tile
// and same-label block lists.
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <utility>
#include <vector>

#include "common.h"

namespace bsa {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
}

void clear_error() { g_err[0] = '\0'; }

int check_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) BSA_FAIL(BSA_ERR_DEVICE, "%s: launch failed: %s", what, hipGetErrorString(e));
    return BSA_OK;
}

}  // namespace bsa

using namespace bsa;

extern "C" const char* bsa_last_error(void) { return g_err; }

extern "C" int bsa_version(void) { return (2 << 16) | 2; }

// Tile-contiguous order.  Permuted position p is (tile index) * vol + (offset
// inside the tile); both are counted T-major, so walking tiles in T-major
// order and their cells in T-major order lists the sources in permuted order.
extern "C" int bsa_tile_permutation(int T, int Hg, int Wg, int a, int b, int c, int32_t* perm) {
    clear_error();
    BSA_REQUIRE(T > 0 && Hg > 0 && Wg > 0, "grid %dx%dx%d must be positive", T, Hg, Wg);
    BSA_REQUIRE(a > 0 && b > 0 && c > 0, "tile %dx%dx%d must be positive", a, b, c);
    BSA_REQUIRE(T % a == 0 && Hg % b == 0 && Wg % c == 0, "tile %dx%dx%d does not divide grid %dx%dx%d",
                a, b, c, T, Hg, Wg);
    BSA_REQUIRE((int64_t)T * Hg * Wg <= INT32_MAX, "grid too large");
    BSA_REQUIRE(perm != nullptr, "perm is NULL");
    int64_t p = 0;
    for (int tt = 0; tt < T / a; ++tt)
        for (int ty = 0; ty < Hg / b; ++ty)
            for (int tx = 0; tx < Wg / c; ++tx)
                for (int rt = 0; rt < a; ++rt)
                    for (int ry = 0; ry < b; ++ry)
                        for (int rx = 0; rx < c; ++rx)
                            perm[p++] = (int32_t)(((int64_t)(tt * a + rt) * Hg + ty * b + ry) * Wg + tx * c + rx);
    return BSA_OK;
}

extern "C" int64_t bsa_padded_length(int T, int Hg, int Wg, int a, int b, int c) {
    clear_error();
    const int64_t n = padded_length(T, Hg, Wg, a, b, c);
    if (n < 0) set_error("grid %dx%dx%d and tile %dx%dx%d must be positive", T, Hg, Wg, a, b, c);
    return n;
}

extern "C" int bsa_tile_permutation_padded(int T, int Hg, int Wg, int a, int b, int c, int32_t* perm) {
    clear_error();
    const int64_t n = padded_length(T, Hg, Wg, a, b, c);
    BSA_REQUIRE(n > 0, "grid %dx%dx%d and tile %dx%dx%d must be positive", T, Hg, Wg, a, b, c);
    BSA_REQUIRE(n <= INT32_MAX, "grid too large");
    BSA_REQUIRE(perm != nullptr, "perm is NULL");
    const int nt = (T + a - 1) / a, ny = (Hg + b - 1) / b, nx = (Wg + c - 1) / c;
    int64_t p = 0;
    for (int tt = 0; tt < nt; ++tt)
        for (int ty = 0; ty < ny; ++ty)
            for (int tx = 0; tx < nx; ++tx)
                for (int rt = 0; rt < a; ++rt)
                    for (int ry = 0; ry < b; ++ry)
                        for (int rx = 0; rx < c; ++rx) {
                            const int t = tt * a + rt, y = ty * b + ry, x = tx * c + rx;
                            perm[p++] = (t < T && y < Hg && x < Wg)
                                            ? (int32_t)(((int64_t)t * Hg + y) * Wg + x)
                                            : -1;
                        }
    return BSA_OK;
}

extern "C" int bsa_video_labels(int T, int Hg, int Wg, int kind, int32_t* labels) {
    clear_error();
    BSA_REQUIRE(labels != nullptr, "bsa_video_labels: NULL labels");
    BSA_REQUIRE(T > 0 && Hg > 0 && Wg > 0, "bsa_video_labels: grid must be positive");
    const int64_t hw = (int64_t)Hg * Wg, S = (int64_t)T * hw;
    BSA_REQUIRE(S <= INT32_MAX, "bsa_video_labels: grid too large");
    if (kind == BSA_LABEL_SPATIAL) {
        for (int64_t s = 0; s < S; ++s) labels[s] = (int32_t)(s / hw);   // frame of a T-major token
    } else if (kind == BSA_LABEL_TEMPORAL) {
        for (int64_t p = 0; p < S; ++p) labels[p] = (int32_t)(p / T);   // position of tile order (T, 1, 1)
    } else {
        BSA_FAIL(BSA_ERR_INVALID_ARG, "bsa_video_labels: unknown kind %d", kind);
    }
    return BSA_OK;
}

extern "C" int bsa_label_block_list(const int32_t* labels, int64_t S, int block, int32_t* kv_idx, int32_t* kv_cnt,
                                    int max_kept) {
    clear_error();
    BSA_REQUIRE(labels != nullptr && kv_idx != nullptr && kv_cnt != nullptr, "NULL argument");
    BSA_REQUIRE(S > 0 && block >= 1 && S % block == 0, "block %d must divide S=%lld", block, (long long)S);
    BSA_REQUIRE(max_kept >= 1, "max_kept must be >= 1");
    const int64_t nb = S / block;
    BSA_REQUIRE(nb <= 16384, "too many blocks (%lld)", (long long)nb);
    // (label, block) pairs sorted by label: every run of one label links all its blocks
    std::vector<std::pair<int32_t, int32_t>> lb;
    lb.reserve((size_t)S);
    for (int64_t s = 0; s < S; ++s)
        if (labels[s] >= 0) lb.emplace_back(labels[s], (int32_t)(s / block));
    std::sort(lb.begin(), lb.end());
    lb.erase(std::unique(lb.begin(), lb.end()), lb.end());
    std::vector<uint8_t> keep((size_t)(nb * nb), 0);
    for (size_t i = 0; i < lb.size();) {
        size_t j = i;
        while (j < lb.size() && lb[j].first == lb[i].first) ++j;
        for (size_t u = i; u < j; ++u)
            for (size_t w = i; w < j; ++w) keep[(size_t)lb[u].second * nb + lb[w].second] = 1;
        i = j;
    }
    for (int64_t I = 0; I < nb; ++I) {
        int cnt = 0;
        for (int64_t J = 0; J < nb; ++J)
            if (keep[(size_t)(I * nb + J)]) {
                BSA_REQUIRE(cnt < max_kept, "query block %lld keeps more than max_kept=%d blocks", (long long)I,
                            max_kept);
                kv_idx[I * max_kept + cnt++] = (int32_t)J;
            }
        for (int i = cnt; i < max_kept; ++i) kv_idx[I * max_kept + i] = -1;
        kv_cnt[I] = cnt;
    }
    return BSA_OK;
}

extern "C" int bsa_invert_permutation(const int32_t* perm, int64_t S, int32_t* inv) {
    clear_error();
    BSA_REQUIRE(perm != nullptr && inv != nullptr, "NULL argument");
    BSA_REQUIRE(S > 0 && S <= INT32_MAX, "S=%lld out of range", (long long)S);
    std::vector<char> seen((size_t)S, 0);
    for (int64_t p = 0; p < S; ++p) {
        int32_t s = perm[p];
        BSA_REQUIRE(s >= 0 && s < S && !seen[(size_t)s], "perm is not a permutation (entry %lld = %d)",
                    (long long)p, s);
        seen[(size_t)s] = 1;
    }
    for (int64_t p = 0; p < S; ++p) inv[perm[p]] = (int32_t)p;
    return BSA_OK;
}

extern "C" int bsa_budget(double frac, int n_blocks) {
    clear_error();
    if (!(frac > 0.0 && frac <= 1.0) || n_blocks < 1) {
        set_error("budget fraction %g must be in (0, 1] and n_blocks %d >= 1", frac, n_blocks);
        return -1;
    }
    double k = std::floor(frac * (double)n_blocks);
    return k < 1.0 ? 1 : (int)k;
}

extern "C" int bsa_sliding_tile_block_list(int nt, int nh, int nw, int rt, int rh, int rw,
                                           int32_t* kv_idx, int32_t* kv_cnt, int max_kept) {
    clear_error();
    BSA_REQUIRE(nt > 0 && nh > 0 && nw > 0, "tile grid must be positive");
    BSA_REQUIRE(rt >= 0 && rh >= 0 && rw >= 0, "radii must be >= 0");
    BSA_REQUIRE(kv_idx != nullptr && kv_cnt != nullptr, "NULL argument");
    const int64_t n = (int64_t)nt * nh * nw;
    BSA_REQUIRE(n <= (1 << 24), "tile grid too large");
    const int64_t widest = (int64_t)std::min(nt, 2 * rt + 1) * std::min(nh, 2 * rh + 1) * std::min(nw, 2 * rw + 1);
    BSA_REQUIRE(max_kept >= widest, "max_kept %d < %lld kept blocks of the widest row", max_kept, (long long)widest);
    for (int t = 0; t < nt; ++t)
        for (int y = 0; y < nh; ++y)
            for (int x = 0; x < nw; ++x) {
                const int64_t I = ((int64_t)t * nh + y) * nw + x;
                int32_t* row = kv_idx + I * max_kept;
                int cnt = 0;
                // neighbours in ascending T-major index order
                for (int t2 = std::max(0, t - rt); t2 <= std::min(nt - 1, t + rt); ++t2)
                    for (int y2 = std::max(0, y - rh); y2 <= std::min(nh - 1, y + rh); ++y2)
                        for (int x2 = std::max(0, x - rw); x2 <= std::min(nw - 1, x + rw); ++x2)
                            row[cnt++] = (int32_t)(((int64_t)t2 * nh + y2) * nw + x2);
                for (int i = cnt; i < max_kept; ++i) row[i] = -1;
                kv_cnt[I] = cnt;
            }
    return BSA_OK;
}
