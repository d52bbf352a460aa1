// sv_kv.hip -- KV rollback indices and in-place KV compaction gather.
//
// [PT] "Decodificacao Especulativa e EAGLE-3", Implementando, Passo 4 and
// "Reversao de KV cache": the logical KV length is truncated after the
// accepted prefix; [ZH] "投机解码与 EAGLE", section 3: after acceptance the KV
// rows of the accepted path are copied together and the other branches
// dropped.
//
// Node n of a round was written at KV row L0 + n.  Keeping the accepted path
// 0 = path[0] < path[1] < ... < path[k] means moving row L0 + path[i] to row
// L0 + i.  Because the path is strictly increasing from 0, path[i] >= i and
// every later source row L0 + path[j] (j > i) lies above every earlier
// destination L0 + i; so a thread that owns one 16-byte column of all rows
// and copies i = 1..k in ascending order never overwrites a row it still has
// to read, and threads owning different columns never touch the same bytes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "specverify.h"
#include "sv_host.h"

namespace sv {

// One thread per sequence: source rows, logical length, validity.
__global__ void k_kv_indices(const int32_t* __restrict__ path_nodes, const int32_t* __restrict__ num_accepted,
                             const int32_t* __restrict__ kv_len_in, int B, int max_depth, int kv_rows,
                             int32_t* __restrict__ src_rows, int32_t* __restrict__ kv_len)
{
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    const int width = max_depth + 1;
    const int k = num_accepted[b];
    const int L0 = kv_len_in[b];
    int32_t* out = src_rows + (int64_t)b * width;
    if (k < 0 || k > max_depth) {
        for (int i = 0; i < width; ++i) out[i] = -1;
        kv_len[b] = L0;
        return;
    }
    // validate: path strictly increasing from node 0, every row in range
    bool ok = L0 >= 0 && (int64_t)L0 + k < (int64_t)kv_rows;
    int prev = -1;
    for (int i = 0; i <= k && ok; ++i) {
        const int node = path_nodes ? path_nodes[(int64_t)b * width + i] : i;
        if ((i == 0 && node != 0) || node <= prev || (int64_t)L0 + node >= (int64_t)kv_rows) ok = false;
        prev = node;
    }
    for (int i = 0; i < width; ++i) {
        int32_t v = -1;
        if (ok && i <= k) v = L0 + (path_nodes ? path_nodes[(int64_t)b * width + i] : i);
        out[i] = v;
    }
    kv_len[b] = ok ? L0 + k + 1 : -1;
}

// grid (column tiles, planes, sequences); a thread copies one 16-byte column
// of rows 1..k of its sequence and plane, in ascending order.
__global__ void k_kv_gather(char* __restrict__ kv, int64_t seq_stride, int64_t row_stride, int ncols,
                            int64_t plane_stride, int max_depth, const int32_t* __restrict__ src_rows,
                            const int32_t* __restrict__ kv_len)
{
    const int col = blockIdx.x * blockDim.x + threadIdx.x;
    const int plane = blockIdx.y;
    const int b = blockIdx.z;
    if (col >= ncols) return;
    const int width = max_depth + 1;
    const int32_t* src = src_rows + (int64_t)b * width;
    const int len = kv_len[b];
    const int L0 = src[0];
    if (len < 0 || L0 < 0) return;
    const int k = len - L0 - 1;
    char* base = kv + (int64_t)plane * plane_stride + (int64_t)b * seq_stride + (int64_t)col * 16;
    for (int i = 1; i <= k; ++i) {
        const int from = src[i];
        const int to = L0 + i;
        if (from == to) continue;
        const uint4 v = *reinterpret_cast<const uint4*>(base + (int64_t)from * row_stride);
        *reinterpret_cast<uint4*>(base + (int64_t)to * row_stride) = v;
    }
}

}  // namespace sv

extern "C" int kv_compact_indices(const int32_t* path_nodes, const int32_t* num_accepted, const int32_t* kv_len_in,
                                  int B, int max_depth, int32_t* out_src_rows, int32_t* out_kv_len, void* kv,
                                  int kv_rows, int64_t seq_stride, int64_t row_stride, int row_bytes, int n_planes,
                                  int64_t plane_stride, hipStream_t stream)
{
    if (B < 0 || max_depth < 0 || kv_rows < 0) return SV_EINVAL;
    if (B == 0) return SV_OK;
    if (!num_accepted || !kv_len_in || !out_src_rows || !out_kv_len) return SV_EINVAL;
    if (kv) {
        if (n_planes < 0 || row_bytes < 0 || seq_stride < 0 || row_stride < 0 || plane_stride < 0) return SV_EINVAL;
        if (((uintptr_t)kv & 15u) || (seq_stride & 15) || (row_stride & 15) || (row_bytes & 15) ||
            (plane_stride & 15))
            return SV_EALIGN;
        if ((int64_t)row_bytes > row_stride) return SV_EINVAL;
        if (!sv::span_fits(n_planes, plane_stride, B, seq_stride, kv_rows, row_stride, row_bytes)) return SV_EINVAL;
        // the gather's grid: planes and sequences are grid dimensions
        if (n_planes > 0 && row_bytes > 0 && (B > 65535 || n_planes > 65535)) return SV_ESHAPE;
    }
    const int threads = 64;
    sv::k_kv_indices<<<dim3((B + threads - 1) / threads), dim3(threads), 0, stream>>>(
        path_nodes, num_accepted, kv_len_in, B, max_depth, kv ? kv_rows : 0x7FFFFFFF, out_src_rows, out_kv_len);
    if (hipGetLastError() != hipSuccess) return SV_EHIP;
    if (kv && n_planes > 0 && row_bytes > 0) {
        const int ncols = row_bytes / 16;
        const dim3 grid((ncols + threads - 1) / threads, n_planes, B);
        sv::k_kv_gather<<<grid, dim3(threads), 0, stream>>>(static_cast<char*>(kv), seq_stride, row_stride, ncols,
                                                              plane_stride, max_depth, out_src_rows, out_kv_len);
        if (hipGetLastError() != hipSuccess) return SV_EHIP;
    }
    return SV_OK;
}
