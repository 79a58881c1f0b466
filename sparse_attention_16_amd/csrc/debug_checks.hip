// debug_checks.hip — on-device validation of a selection (the top-k output)
// against its contract, for the library's debug mode.
//
// Page "Техотчёт DeepSeek-V3.2 (2025): разреженное внимание DSA и
// масштабирование RL", section "Отбор и основное внимание": a query row's
// selection is Top-k over its visible keys.  Whatever the scores, the output
// of a row that sees n keys therefore holds exactly min(k, n) distinct
// visible positions, in ascending order, and -1 in every slot after them.
// idx_check_kernel counts the rows that break this; the host reads the count
// after the stream has drained.
#include "dsa_device.h"
#include "kernels.h"

namespace dsa {

namespace {

// Rows that broke the contract since the last reset, one counter per GPU (each
// GPU holds its own copy; host code takes the address with hipGetSymbolAddress).
__device__ int bad_rows;

constexpr int CHK_T = 256;

__global__ __launch_bounds__(CHK_T) void idx_check_reset_kernel(int *bad) { *bad = 0; }

// One workgroup per query row.
__global__ __launch_bounds__(CHK_T) void idx_check_kernel(const int32_t *cu_q, const int64_t *cu_kv,
                                                          const int32_t *pos0, int B, int64_t total_kv, int max_kv,
                                                          const int32_t *idx, int k, int *bad) {
    __shared__ int fail;
    const int t = blockIdx.x;
    if (threadIdx.x == 0) fail = 0;
    __syncthreads();
    const RowInfo ri = row_info(cu_q, cu_kv, pos0, B, total_kv, max_kv, t);
    const int want = ri.nvis < k ? ri.nvis : k;
    const int32_t *row = idx + (int64_t)t * k;
    for (int j = threadIdx.x; j < k; j += CHK_T) {
        const int32_t v = row[j];
        bool ok;
        if (j < want)
            ok = v >= 0 && v < ri.nvis && (j == 0 || row[j - 1] < v);
        else
            ok = v == -1;
        if (!ok) fail = 1;
    }
    __syncthreads();
    if (threadIdx.x == 0 && fail) atomicAdd(bad, 1);
}

}  // namespace

hipError_t check_selection(const int32_t *cu_q, const int64_t *cu_kv, const int32_t *pos0, int B, int64_t total_kv,
                           int max_kv, int T, const int32_t *idx, int k, hipStream_t s, int *bad_out) {
    *bad_out = 0;
    if (T <= 0) return hipSuccess;
    int *bad = nullptr;
    hipError_t e = hipGetSymbolAddress(reinterpret_cast<void **>(&bad), HIP_SYMBOL(bad_rows));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(idx_check_reset_kernel, dim3(1), dim3(1), 0, s, bad);
    hipLaunchKernelGGL(idx_check_kernel, dim3(T), dim3(CHK_T), 0, s, cu_q, cu_kv, pos0, B, total_kv, max_kv, idx, k,
                       bad);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = hipMemcpyAsync(bad_out, bad, sizeof(int), hipMemcpyDeviceToHost, s)) != hipSuccess) return e;
    return hipStreamSynchronize(s);
}

}  // namespace dsa
