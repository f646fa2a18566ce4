// Synchronous checks of device-resident indices: bsa_validate_block_list and
// bsa_validate_indices.  The asynchronous calls trust the lists they are
// given; these report a violated invariant as a status instead
// ([ADR-0001, shared conventions: validation]: RuntimeError for invariants;
// [FastVideo windowed_attention.py, `windowed_attention`]: a query block with
// no keys is such a violation).
#include "common.h"

namespace bsa {
namespace {

// flag[0] = number of bad rows, flag[1] = first bad row (or index)
__global__ void init_flag(unsigned long long* flag) {
    flag[0] = 0;
    flag[1] = ~0ull;
}

__global__ void check_lists(const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt, uint64_t rows,
                            int nk, int max_kept, unsigned long long* flag) {
    const uint64_t r = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= rows) return;
    const int c = cnt[r];
    bool bad = c < 1 || c > max_kept;
    if (!bad) {
        int prev = -1;
        for (int i = 0; i < c; ++i) {
            const int j = idx[r * max_kept + i];
            if (j <= prev || j >= nk) {
                bad = true;
                break;
            }
            prev = j;
        }
    }
    if (bad) {
        atomicAdd(&flag[0], 1ull);
        atomicMin(&flag[1], (unsigned long long)r);
    }
}

__global__ void check_range(const int32_t* __restrict__ v, uint64_t n, int lo, int hi, unsigned long long* flag) {
    const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int x = v[i];
    if (x < lo || x >= hi) {
        atomicAdd(&flag[0], 1ull);
        atomicMin(&flag[1], (unsigned long long)i);
    }
}

// Runs `launch` against a fresh two-word flag and returns the flag.
template <typename F>
int run_check(hipStream_t st, F launch, unsigned long long out[2], const char* name) {
    unsigned long long* flag = nullptr;
    if (hipMalloc(&flag, 2 * sizeof(unsigned long long)) != hipSuccess)
        BSA_FAIL(BSA_ERR_DEVICE, "%s: hipMalloc failed", name);
    init_flag<<<1, 1, 0, st>>>(flag);
    launch(flag);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = hipMemcpyAsync(out, flag, 2 * sizeof(unsigned long long), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    (void)hipFree(flag);
    if (e != hipSuccess) BSA_FAIL(BSA_ERR_DEVICE, "%s: %s", name, hipGetErrorString(e));
    return BSA_OK;
}

}  // namespace
}  // namespace bsa

using namespace bsa;

extern "C" int bsa_validate_block_list(const int32_t* kv_idx, const int32_t* kv_cnt, int64_t B, int64_t H, int Nq,
                                       int Nk, int max_kept, bsa_stream_t stream) {
    clear_error();
    const char* name = "bsa_validate_block_list";
    BSA_REQUIRE(kv_idx && kv_cnt, "%s: NULL argument", name);
    BSA_REQUIRE(B >= 1 && H >= 1 && Nq >= 1 && Nk >= 1 && max_kept >= 1, "%s: sizes must be >= 1", name);
    const uint64_t rows = (uint64_t)B * H * Nq;
    unsigned long long res[2] = {0, 0};
    hipStream_t st = (hipStream_t)stream;
    int rc = run_check(
        st,
        [&](unsigned long long* flag) {
            check_lists<<<(unsigned)((rows + 255) / 256), 256, 0, st>>>(kv_idx, kv_cnt, rows, Nk, max_kept, flag);
        },
        res, name);
    if (rc) return rc;
    if (res[0]) {
        const unsigned long long r = res[1];
        BSA_FAIL(BSA_ERR_INVARIANT,
                 "%s: %llu bad row(s); first is row %llu (b*H*Nq + h*Nq + I): count outside [1, %d] or indices not "
                 "ascending inside [0, %d)",
                 name, res[0], r, max_kept, Nk);
    }
    return BSA_OK;
}

extern "C" int bsa_validate_indices(const int32_t* v, int64_t n, int lo, int hi, bsa_stream_t stream) {
    clear_error();
    const char* name = "bsa_validate_indices";
    BSA_REQUIRE(v != nullptr, "%s: NULL argument", name);
    BSA_REQUIRE(n >= 1, "%s: n must be >= 1", name);
    unsigned long long res[2] = {0, 0};
    hipStream_t st = (hipStream_t)stream;
    int rc = run_check(
        st,
        [&](unsigned long long* flag) {
            check_range<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(v, (uint64_t)n, lo, hi, flag);
        },
        res, name);
    if (rc) return rc;
    if (res[0]) BSA_FAIL(BSA_ERR_INVARIANT, "%s: %llu value(s) outside [%d, %d); first at %llu", name, res[0], lo, hi, res[1]);
    return BSA_OK;
}
