// sv_draft.hip -- draft-token sampling on the device: d ~ softmax(z / T)
// for every row of a batch of draft logits ([PT] "Decodificacao
// Especulativa e EAGLE-3", O Conceito and Implementando, Passo 1: the draft
// proposes d ~ p; [ZH] "投机解码与 EAGLE" section 2: each draft token is drawn
// from the draft model's softmax in turn).  The draw is the inverse CDF in
// token order of the verify step's sampling (first token whose running
// weight exceeds u*W, W the total weight, accumulated in double; the last
// token of positive weight when rounding leaves none), with the uniform of
// Philox stream 1.  gfx950, wave64.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "specverify.h"
#include "sv_device.h"

namespace sv {

constexpr int kDraftPerLane = 16;                    // logits per lane per chunk
constexpr int kDraftChunk = 64 * kDraftPerLane;      // 1024 logits per chunk (one wave)
constexpr int kDraftMaxChunks = 512;                 // V <= 524288

struct DraftArgs {
    const char* rows;
    int64_t seq_stride, row_stride;  // elements
    int R, V, pos0;
    double invT;
    float c;  // log2(e) / T
    uint64_t seed, round;
    int32_t* out_tokens;
    double* out_logprob;
};

// The uniform of a draft draw: Philox block (position, sequence, round lo,
// (round hi) << 4 | stream 1), words 0 and 1.
__device__ __forceinline__ double draft_uniform(uint64_t seed, uint64_t round, uint32_t seq, uint32_t pos)
{
    const Words4 w = philox4x32_10(pos, seq, (uint32_t)round, ((uint32_t)(round >> 32) << 4) | 1u, (uint32_t)seed,
                                   (uint32_t)(seed >> 32));
    return u53(w.w0, w.w1);
}

// A lane's kDraftPerLane logits of chunk c (contiguous, token order), as raw
// 16-byte vectors; padding past V is masked when decoded.
template <int DT>
struct ChunkRegs {
    static constexpr int NV = kDraftPerLane * (DT == DT_BF16 ? 2 : 4) / 16;
    uint4 v[NV];
};

template <int DT>
__device__ __forceinline__ void load_lane_chunk(const char* row, int V, int c, int lane, ChunkRegs<DT>& r)
{
    constexpr int EB = DT == DT_BF16 ? 2 : 4;
    constexpr int EPV = 16 / EB;
    const int64_t e0 = (int64_t)c * kDraftChunk + (int64_t)lane * kDraftPerLane;
    const bool vec = ((((uintptr_t)row) & 15u) == 0) && e0 + kDraftPerLane <= V;
    if (vec) {
        const uint4* p = reinterpret_cast<const uint4*>(row + e0 * EB);
#pragma unroll
        for (int i = 0; i < ChunkRegs<DT>::NV; ++i) r.v[i] = stream_load16(p + i);
    } else {
        // ragged tail or unaligned row: element by element, -inf past V
        float x[kDraftPerLane];
#pragma unroll
        for (int j = 0; j < kDraftPerLane; ++j) x[j] = (e0 + j < V) ? load_logit<DT>(row, e0 + j) : -INFINITY;
#pragma unroll
        for (int i = 0; i < ChunkRegs<DT>::NV; ++i) r.v[i] = encode16<DT>(x + i * EPV);
    }
}

template <int DT>
__device__ __forceinline__ void decode_lane_chunk(const ChunkRegs<DT>& r, float* x)
{
    constexpr int EPV = DT == DT_BF16 ? 8 : 4;
#pragma unroll
    for (int i = 0; i < ChunkRegs<DT>::NV; ++i) decode16<DT>(r.v[i], x + i * EPV);
}

__device__ __forceinline__ double wave_sum_d(double v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

__device__ __forceinline__ float wave_max_fl(float v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

// Exclusive prefix sum over the wave's lanes (lane order), and the total.
__device__ __forceinline__ double wave_exclusive(double v, int lane, double* total)
{
    double x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    *total = __shfl(x, 63, 64);
    return x - v;
}

// Block (b, r): one draw from row r of sequence b.
//  1. Each wave takes chunks w, w + NW, ... (1024 logits, 16 contiguous per
//     lane, the next two chunks' loads in flight): a reference m_c and s_c = sum
//     of the weights 2^((x - m_c) c), c = log2(e)/T, each an fp32 exp2
//     (about 1e-7 relative) summed in double, into LDS.
//  2. Wave 0: M = max m_c, chunk weights s_c exp((m_c - M)/T), W, u*W, and
//     the chunk where the running weight passes u*W (8 chunks per lane, an
//     exclusive scan over lanes).
//  3. Wave 0 rescans that chunk in token order with the same weights (the
//     same fp32 values), so the draw is the exact inverse CDF of the fp32
//     weights: within about 1e-7 relative of the exact softmax CDF.
// A row holding NaN or +inf, or only -inf, gives token -1 and NaN.
// NW = 8 waves per block for large batches, 16 for small ones (a row's
// chunks spread over more waves); at 84 VGPRs five waves fit per SIMD.
template <int DT, int NW>
__global__ __launch_bounds__(NW * 64, 4) void k_draft_sample(DraftArgs A)
{
    __shared__ double s_tab[kExpTabN];
    __shared__ float s_m[kDraftMaxChunks];
    __shared__ double s_s[kDraftMaxChunks];
    __shared__ float s_e[kDraftMaxChunks];
    const int row_id = blockIdx.x;
    const int b = row_id / A.R, r = row_id - b * A.R;
    const char* row = A.rows + ((int64_t)b * A.seq_stride + (int64_t)r * A.row_stride) * (DT == DT_BF16 ? 2 : 4);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nch = (A.V + kDraftChunk - 1) / kDraftChunk;
    fill_exp_table(s_tab);
    __syncthreads();
    const lds_dptr tab = (lds_dptr)s_tab;
    const double invT = A.invT;

    // 1. chunk sums.  The wave's reference ref (uniform) lags its running
    // maximum by under 2 in the exponent, so most chunks skip the wave-wide
    // maximum; a term is 2^(fma(x, c, -p)), p = RN(ref c), which is
    // 2^((x - ref) c) times 2^e, e = ref c - p (exact in fp32), shed in
    // step 2.  NaN and +inf reach the sum as NaN (while ref is -inf, p = 0
    // keeps every term 0 or NaN).
    float ref = -INFINITY, lim = -INFINITY, pf = 0.0f, ef = 0.0f;
    auto take = [&](const ChunkRegs<DT>& regs, int c) {
        float x[kDraftPerLane];
        decode_lane_chunk<DT>(regs, x);
        float lm = -INFINITY;
#pragma unroll
        for (int j = 0; j < kDraftPerLane; ++j) lm = fmaxf(lm, x[j]);
        if (__ballot(lm > lim)) {
            const float wm = wave_max_fl(lm);
            ref = wm;
            lim = wm + 2.0f / A.c;
            pf = wm * A.c;
            ef = __builtin_fmaf(wm, A.c, -pf);
        }
        double s = 0.0;
#pragma unroll
        for (int j = 0; j < kDraftPerLane; ++j) s += (double)__builtin_amdgcn_exp2f(__builtin_fmaf(x[j], A.c, -pf));
        s = wave_sum_d(s);
        if (lane == 0) {
            s_m[c] = ref;
            s_e[c] = ef;
            s_s[c] = s;
        }
    };
    // three register sets, loads two chunks ahead; a set is never copied
    // (a copy would wait for its loads), and a load past the row's chunks
    // is skipped (wave-uniform)
    ChunkRegs<DT> ra, rb, rc;
    auto load = [&](ChunkRegs<DT>& regs, int c) {
        if (c < nch) load_lane_chunk<DT>(row, A.V, c, lane, regs);
    };
    load(ra, wave);
    load(rb, wave + NW);
    for (int c = wave; c < nch; c += 3 * NW) {
        load(rc, c + 2 * NW);
        take(ra, c);
        if (c + NW >= nch) break;
        load(ra, c + 3 * NW);
        take(rb, c + NW);
        if (c + 2 * NW >= nch) break;
        load(rb, c + 4 * NW);
        take(rc, c + 2 * NW);
    }
    __syncthreads();
    if (wave != 0) return;

    // 2. total weight and the chunk of the draw
    const int64_t oi = (int64_t)b * A.R + r;
    float M = -INFINITY;
    int bad = 0;
    for (int c = lane; c < nch; c += 64) {
        M = fmaxf(M, s_m[c]);
        bad |= s_s[c] != s_s[c];
    }
    M = wave_max_fl(M);
    if (__ballot(bad) || M == -INFINITY) {
        if (lane == 0) {
            A.out_tokens[oi] = -1;
            if (A.out_logprob) A.out_logprob[oi] = NAN;
        }
        return;
    }
    // chunk c's weight: s_c 2^(-e_c) exp((ref_c - M)/T)
    auto chunk_scale = [&](int c) {
        return exp_rel(((double)s_m[c] - (double)M) * invT - (double)s_e[c] * 0.69314718055994530942, tab);
    };
    constexpr int CPL = kDraftMaxChunks / 64;  // chunks per lane, consecutive
    double cw[CPL];
    double lsum = 0.0;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = lane * CPL + i;
        cw[i] = (c < nch && s_m[c] != -INFINITY) ? s_s[c] * chunk_scale(c) : 0.0;
        lsum += cw[i];
    }
    double W;
    const double lbase = wave_exclusive(lsum, lane, &W);
    const double u = draft_uniform(A.seed, A.round, (uint32_t)b, (uint32_t)(A.pos0 + r));
    const double target = u * W;
    // the first lane whose running weight passes the target; else (rounding)
    // the last lane with positive weight, whose last positive chunk is taken
    const uint64_t pass = __ballot(lsum > 0.0 && lbase + lsum > target);
    const uint64_t pos = __ballot(lsum > 0.0);
    const bool fallback = pass == 0;
    const int owner = fallback ? 63 - __clzll((long long)pos) : __ffsll((unsigned long long)pass) - 1;
    int cs = -1;
    double cbase = 0.0;
    if (lane == owner) {
        double cum = lbase;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = lane * CPL + i;
            if (cw[i] > 0.0) {
                if (!fallback && cs < 0 && cum + cw[i] > target) {
                    cs = c;
                    cbase = cum;
                }
                if (fallback) {
                    cs = c;
                    cbase = cum;
                }
            }
            cum += cw[i];
        }
    }
    cs = __shfl(cs, owner, 64);
    cbase = __shfl(cbase, owner, 64);
    const float mc = s_m[cs];
    const float pc = mc * A.c;  // the chunk's p, as pass 1 formed it
    const double scale = chunk_scale(cs);
    const double local = fallback ? INFINITY : (target - cbase) / scale;

    // 3. rescan the chunk in token order
    ChunkRegs<DT> rr;
    load_lane_chunk<DT>(row, A.V, cs, lane, rr);
    float x[kDraftPerLane];
    decode_lane_chunk<DT>(rr, x);
    // the weights are recomputed below (the same fp32 values) rather than held
    double tsum = 0.0;
#pragma unroll
    for (int j = 0; j < kDraftPerLane; ++j) tsum += (double)__builtin_amdgcn_exp2f(__builtin_fmaf(x[j], A.c, -pc));
    double ctot;
    const double tbase = wave_exclusive(tsum, lane, &ctot);
    const uint64_t cand = __ballot(tsum > 0.0 && tbase + tsum > local);
    const uint64_t posl = __ballot(tsum > 0.0);
    const int own = cand ? __ffsll((unsigned long long)cand) - 1 : 63 - __clzll((long long)posl);
    if (lane == own) {
        double cum = tbase;
        int pick = -1, last = -1;
        float xpick = 0.0f, xlast = 0.0f;
#pragma unroll
        for (int j = 0; j < kDraftPerLane; ++j) {
            const double wj = (double)__builtin_amdgcn_exp2f(__builtin_fmaf(x[j], A.c, -pc));
            if (wj > 0.0) {
                last = j;
                xlast = x[j];
                if (pick < 0 && cum + wj > local) {
                    pick = j;
                    xpick = x[j];
                }
            }
            cum += wj;
        }
        if (pick < 0) {
            pick = last;
            xpick = xlast;
        }
        A.out_tokens[oi] = cs * kDraftChunk + lane * kDraftPerLane + pick;
        if (A.out_logprob) A.out_logprob[oi] = ((double)xpick - (double)M) * invT - log(W);
    }
}

}  // namespace sv

extern "C" int sv_sample_draft(const void* logits, int64_t seq_stride, int64_t row_stride, int dtype, int B, int R,
                               int V, float temperature, uint64_t seed, uint64_t round, int pos0,
                               int32_t* out_tokens, double* out_logprob, hipStream_t stream)
{
    if (dtype != SV_F32 && dtype != SV_BF16) return SV_EDTYPE;
    if (B < 0 || R < 0 || V < 1 || pos0 < 0 || seq_stride < 0 || row_stride < 0) return SV_EINVAL;
    if (!(temperature > 0.0f) || !(temperature < INFINITY)) return SV_EINVAL;
    if (V > sv::kDraftMaxChunks * sv::kDraftChunk || (int64_t)pos0 + R > 0xFFFFFFFFll) return SV_ESHAPE;
    if ((int64_t)B * R > 0x7FFFFFFF) return SV_ESHAPE;
    if (B == 0 || R == 0) return SV_OK;
    if (!logits || !out_tokens) return SV_EINVAL;
    const int es = dtype == SV_BF16 ? 2 : 4;
    if (((uintptr_t)logits) % es) return SV_EALIGN;
    sv::DraftArgs A;
    A.rows = static_cast<const char*>(logits);
    A.seq_stride = seq_stride;
    A.row_stride = row_stride;
    A.R = R;
    A.V = V;
    A.pos0 = pos0;
    A.invT = 1.0 / (double)temperature;
    A.c = (float)(1.4426950408889634074 / (double)temperature);
    A.seed = seed;
    A.round = round;
    A.out_tokens = out_tokens;
    A.out_logprob = out_logprob;
    const dim3 grid((unsigned)(B * R));
    const bool few = (int64_t)B * R < 512;  // under two blocks per CU: spread each row over 16 waves
    if (dtype == SV_BF16) {
        if (few) hipLaunchKernelGGL((sv::k_draft_sample<1, 16>), grid, dim3(1024), 0, stream, A);
        else hipLaunchKernelGGL((sv::k_draft_sample<1, 8>), grid, dim3(512), 0, stream, A);
    } else {
        if (few) hipLaunchKernelGGL((sv::k_draft_sample<0, 16>), grid, dim3(1024), 0, stream, A);
        else hipLaunchKernelGGL((sv::k_draft_sample<0, 8>), grid, dim3(512), 0, stream, A);
    }
    return hipGetLastError() == hipSuccess ? SV_OK : SV_EHIP;
}
