// sv_tree.hip -- the tree attention mask and position ids of a flattened
// draft tree ("投机解码与 EAGLE", section 3: each node attends to itself and
// its ancestors only).  gfx950, wave64.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "specverify.h"

namespace sv {

constexpr int kTreeBlock = 256;
constexpr int kTreeMaxNodes = 1024;  // T + 1

// Block b: the mask rows and position ids of sequence b; thread t takes nodes
// t, t + 256, ...  Node n walks its ancestor chain once.  Parents have lower
// indices than their children, so the chain visits node indices in
// decreasing order and the words of row n are finished from the highest
// (the one holding n) down to word 0: each word is stored when the walk
// leaves it, words above n's are 0.
__global__ __launch_bounds__(kTreeBlock) void k_tree_mask(const int32_t* __restrict__ parents, int parents_shared,
                                                         const int32_t* __restrict__ kv_len_in, int T,
                                                         uint64_t* __restrict__ out_mask,
                                                         int32_t* __restrict__ out_positions)
{
    __shared__ int s_par[kTreeMaxNodes];
    const int b = blockIdx.x;
    const int nn = T + 1;
    const int W = (nn + 63) >> 6;
    const int32_t* par = parents_shared ? parents : parents + (int64_t)b * nn;
    int bad = 0;
    for (int n = threadIdx.x; n < nn; n += kTreeBlock) {
        const int p = par[n];
        s_par[n] = p;
        bad |= n == 0 ? (p != -1) : (p < 0 || p >= n);
    }
    bad = __syncthreads_or(bad);
    const int L0 = kv_len_in ? kv_len_in[b] : 0;
    uint64_t* mask = out_mask + (int64_t)b * nn * W;
    int32_t* pos = out_positions + (int64_t)b * nn;
    for (int n = threadIdx.x; n < nn; n += kTreeBlock) {
        uint64_t* row = mask + (int64_t)n * W;
        if (bad) {
            for (int w = 0; w < W; ++w) row[w] = 0;
            pos[n] = -1;
            continue;
        }
        for (int w = W - 1; w > (n >> 6); --w) row[w] = 0;
        int w = n >> 6;
        uint64_t word = 0;
        int depth = 0;
        for (int j = n; j >= 0; j = s_par[j]) {
            while ((j >> 6) < w) {  // the walk left word w: store it
                row[w--] = word;
                word = 0;
            }
            word |= 1ull << (j & 63);
            depth += j != n;
        }
        row[w] = word;  // holds the root (word 0)
        pos[n] = L0 + depth;
    }
}

}  // namespace sv

extern "C" int tree_attention_mask(const int32_t* parents, int parents_shared, const int32_t* kv_len_in, int B,
                                   int T, uint64_t* out_mask, int32_t* out_positions, hipStream_t stream)
{
    if (B < 0 || T < 0) return SV_EINVAL;
    if (T + 1 > sv::kTreeMaxNodes) return SV_ESHAPE;
    if (B == 0) return SV_OK;
    if (!parents || !out_mask || !out_positions) return SV_EINVAL;
    hipLaunchKernelGGL(sv::k_tree_mask, dim3((unsigned)B), dim3(sv::kTreeBlock), 0, stream, parents, parents_shared,
                       kv_len_in, T, out_mask, out_positions);
    return hipGetLastError() == hipSuccess ? SV_OK : SV_EHIP;
}
