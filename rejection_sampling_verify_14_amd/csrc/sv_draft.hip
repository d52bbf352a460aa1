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
#include "sv_host.h"
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
    float T;
    int use_tab;      // bf16 rows: the temperature has a bf16-grid table
    uint32_t tab_lo;  // its first magnitude key
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

// Weights.  bf16 rows whose temperature gives a bf16-grid table (see
// kTabKeys) take E(z) = exp(z/T) from the block's LDS copy of it, summed
// without a reference (logits outside the table add exp_rel(z/T)); a row
// with a logit above 700 T (its exp(z/T) would overflow) or whose total
// weight falls below 1e-280 (every logit far below zero) is redone by the
// reference path.  The reference path (f32 rows, and those rows) sums
// exp((z - ref)/T) by exp_rel against a running reference per wave, as in
// the verify step's sampling.  Either way the weights are double, ~1e-11
// relative (exp_rel) or one rounding (table), so the draw is the inverse CDF
// of softmax(z/T) to far below the comparison band.
constexpr int kDraftTabPath = 1, kDraftRefPath = 2;
constexpr double kDraftOverflowArg = 700.0;  // exp_rel's arguments stay below this
constexpr double kDraftTinyTotal = 1e-280;

// Block (b, r): one draw from row r of sequence b.
//  1. Each wave takes chunks w, w + NW, ... (1024 logits, 16 contiguous per
//     lane, the next two chunks' loads in flight) and stores the chunk's
//     weight sum (and, on the reference path, its reference) in LDS.
//  2. Wave 0: total W, u*W, and the chunk where the running weight passes
//     u*W (8 chunks per lane, an exclusive scan over lanes).
//  3. Wave 0 rescans that chunk in token order with the same weights, so
//     the draw is the exact inverse CDF of the weights.
// A row holding NaN or +inf, or only -inf, gives token -1 and NaN.
// NW = 8 waves per block for large batches, 16 for small ones (a row's
// chunks spread over more waves); bf16 at least six waves per SIMD (the
// LDS table fits three 8-wave blocks per CU), f32 four (exp_rel's registers
// without spills).
template <int DT, int NW>
__global__ __launch_bounds__(NW * 64, DT == DT_BF16 ? 6 : 4) void k_draft_sample(DraftArgs A)
{
    constexpr bool TAB = DT == DT_BF16;
    __shared__ double s_etab[kExpTabN];
    __shared__ __align__(16) double s_tab[TAB ? kTabEntries : 2];
    __shared__ float s_m[kDraftMaxChunks];
    __shared__ double s_s[kDraftMaxChunks];
    __shared__ int s_flags;
    const int row_id = blockIdx.x;
    const int b = row_id / A.R, r = row_id - b * A.R;
    const char* row = A.rows + ((int64_t)b * A.seq_stride + (int64_t)r * A.row_stride) * (DT == DT_BF16 ? 2 : 4);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nch = (A.V + kDraftChunk - 1) / kDraftChunk;
    const double invT = A.invT;
    if (tid == 0) s_flags = 0;
    bool tab_path = false;
    if constexpr (TAB) tab_path = A.use_tab != 0;
    const lds_dptr etab = (lds_dptr)s_etab;
    const lds_cptr tabc = (lds_cptr)s_tab;

    // three register sets, loads two chunks ahead; a set is never copied
    // (a copy would wait for its loads), and a load past the row's chunks
    // is skipped (wave-uniform).  `before` runs (in every wave, so it may
    // hold barriers) once the first loads are in flight.
    auto stream_row = [&](auto&& take, auto&& before) {
        ChunkRegs<DT> ra, rb, rc;
        auto load = [&](ChunkRegs<DT>& regs, int c) {
            if (c < nch) load_lane_chunk<DT>(row, A.V, c, lane, regs);
        };
        load(ra, wave);
        load(rb, wave + NW);
        before();
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
    };

    // 1a. table path: chunk sums of E(z) = exp(z/T)
    if constexpr (TAB) {
        if (tab_path) {
            const u16x2 lo2 = {(unsigned short)A.tab_lo, (unsigned short)A.tab_lo};
            int flags = 0;  // 1: NaN or +inf, 2: a logit above 700 T
            auto take = [&](const ChunkRegs<DT>& regs, int c) {
                double sum = 0.0;
                u16x2 worst = {0, 0};
                const uint32_t w[8] = {regs.v[0].x, regs.v[0].y, regs.v[0].z, regs.v[0].w,
                                       regs.v[1].x, regs.v[1].y, regs.v[1].z, regs.v[1].w};
                // two halves of eight table reads (the halves keep the live
                // table values to 16 registers)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    double v[8];
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) {
                        uint32_t a0, a1;
                        tab_offsets(w[4 * h + kk], lo2, a0, a1, worst);
                        v[2 * kk] = lds_f64(tabc, a0);
                        v[2 * kk + 1] = lds_f64(tabc, a1);
                    }
#pragma unroll
                    for (int j = 0; j < 8; ++j) sum += v[j];
                    asm volatile("" : "+v"(sum));
                }
                if (__any(max((uint32_t)worst.x, (uint32_t)worst.y) >= (uint32_t)kTabKeys)) {
                    // logits outside the table went in as zeros
#pragma unroll 1
                    for (int i = 0; i < 16; ++i) {
                        const int k = i >> 1;
                        uint32_t x = w[0];
#pragma unroll
                        for (int q = 1; q < 8; ++q) x = k == q ? w[q] : x;
                        const float z = (i & 1) ? bf16_hi(x) : bf16_lo(x);
                        if (tab_index(z, A.tab_lo) >= 0 || z == -INFINITY) continue;
                        if (!(z < INFINITY)) {
                            flags |= 1;  // NaN or +inf
                            continue;
                        }
                        const double arg = (double)z * invT;
                        if (arg > kDraftOverflowArg) flags |= 2;
                        else sum += exp_rel(arg, etab);
                    }
                }
                sum = wave_sum_d(sum);
                if (lane == 0) s_s[c] = sum;
            };
            // the block's table, built while the first loads are in flight:
            // entry s (kTabKeys + 1) + t = exp(z/T) (exp_rel) for the bf16 z
            // of magnitude bits lo + t and sign s (t = kTabKeys: 0)
            auto build_table = [&]() {
                fill_exp_table(s_etab);
                __syncthreads();
                for (int i = tid; i < kTabEntries; i += NW * 64) {
                    const int sgn = i >= kTabHalf ? 1 : 0;
                    const int t = i - sgn * kTabHalf;
                    double v = 0.0;
                    if (t < kTabKeys) {
                        const uint32_t key = (A.tab_lo + (uint32_t)t) | ((uint32_t)sgn << 15);
                        v = exp_rel((double)__uint_as_float(key << 16) * invT, etab);
                    }
                    s_tab[i] = v;
                }
                __syncthreads();
            };
            stream_row(take, build_table);
            flags = (__any(flags & 1) ? 1 : 0) | (__any(flags & 2) ? 2 : 0);
            if (lane == 0 && flags) atomicOr(&s_flags, flags);
        }
    }

    // 1b. reference path (f32 rows; bf16 rows without the table; rows the
    // table path hands over): sums of exp((z - ref_c)/T) against a
    // reference that lags the wave's running maximum by less than 2 ln2 T.
    // NaN and +inf reach the sum as NaN.
    auto ref_path = [&]() {
        float ref = -INFINITY, lim = -INFINITY;
        const float step = (float)(2.0 * 0.69314718055994530942 / invT);
        auto take = [&](const ChunkRegs<DT>& regs, int c) {
            float x[kDraftPerLane];
            decode_lane_chunk<DT>(regs, x);
            float lm = -INFINITY;
            int bad = 0;
#pragma unroll
            for (int j = 0; j < kDraftPerLane; ++j) {
                lm = fmaxf(lm, x[j]);
                bad |= !(x[j] < INFINITY) && x[j] != -INFINITY;
            }
            if (__ballot(lm > lim)) {
                const float wm = wave_max_fl(lm);
                ref = wm;
                lim = wm + step;
            }
            double sum = 0.0;
            if (ref != -INFINITY) {
#pragma unroll
                for (int j = 0; j < kDraftPerLane; ++j)
                    sum += exp_rel(((double)x[j] - (double)ref) * invT, etab);
            }
            sum = __any(bad) ? NAN : wave_sum_d(sum);
            if (lane == 0) {
                s_m[c] = ref;
                s_s[c] = sum;
            }
        };
        stream_row(take, [] {});
    };
    bool use_ref = !tab_path;
    if (use_ref) {
        fill_exp_table(s_etab);
        __syncthreads();
    }
    if (!use_ref) {
        __syncthreads();
        const int fl = s_flags;
        if (fl & 1) {
            // NaN or +inf: the row fails
            if (tid == 0) {
                const int64_t oi = (int64_t)b * A.R + r;
                A.out_tokens[oi] = -1;
                if (A.out_logprob) A.out_logprob[oi] = NAN;
            }
            return;
        }
        double tot = 0.0;
        for (int c = lane; c < nch; c += 64) tot += s_s[c];
        tot = wave_sum_d(tot);
        use_ref = (fl & 2) || !(tot >= kDraftTinyTotal);
        __syncthreads();  // every wave read s_s before the reference path rewrites it
    }
    if (use_ref) {
        ref_path();
    }
    __syncthreads();
    if (wave != 0) return;

    // 2. total weight and the chunk of the draw
    const int64_t oi = (int64_t)b * A.R + r;
    float M = -INFINITY;
    if (use_ref) {
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
    }
    // chunk c's weight: the table path's sum as is; the reference path's
    // s_c exp((ref_c - M)/T)
    auto chunk_scale = [&](int c) { return use_ref ? exp_rel(((double)s_m[c] - (double)M) * invT, etab) : 1.0; };
    constexpr int CPL = kDraftMaxChunks / 64;  // chunks per lane, consecutive
    double cw[CPL];
    double lsum = 0.0;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = lane * CPL + i;
        cw[i] = (c < nch && (!use_ref || s_m[c] != -INFINITY)) ? s_s[c] * chunk_scale(c) : 0.0;
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
    const double mc = use_ref ? (double)s_m[cs] : 0.0;
    const double scale = chunk_scale(cs);
    const double local = fallback ? INFINITY : (target - cbase) / scale;

    // 3. rescan the chunk in token order, the same weights as step 1
    ChunkRegs<DT> rr;
    load_lane_chunk<DT>(row, A.V, cs, lane, rr);
    float x[kDraftPerLane];
    decode_lane_chunk<DT>(rr, x);
    // the weight of token j of the lane (computed again where needed rather
    // than held: the same value both times)
    auto weight = [&](int j) -> double {
        if (!use_ref) {
            const int ti = TAB ? tab_index(x[j], A.tab_lo) : -1;
            return ti >= 0 ? ((lds_dptr)s_tab)[ti]
                           : (x[j] == -INFINITY ? 0.0 : exp_rel((double)x[j] * invT, etab));
        }
        return exp_rel(((double)x[j] - mc) * invT, etab);
    };
    double tsum = 0.0;
#pragma unroll
    for (int j = 0; j < kDraftPerLane; ++j) tsum += weight(j);
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
            const double wj = weight(j);
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
        // ln p = z/T - ln W (table path, W in units of exp(z/T)), or
        // (z - M)/T - ln W (reference path, W relative to M)
        if (A.out_logprob)
            A.out_logprob[oi] = (use_ref ? ((double)xpick - (double)M) * invT : (double)xpick * invT) - log(W);
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
    if (seq_stride > INT64_MAX / es || row_stride > INT64_MAX / es ||
        !sv::span_fits(B, seq_stride * es, R, row_stride * es, 1, 0, (int64_t)V * es))
        return SV_EINVAL;
    sv::DraftArgs A;
    A.rows = static_cast<const char*>(logits);
    A.seq_stride = seq_stride;
    A.row_stride = row_stride;
    A.R = R;
    A.V = V;
    A.pos0 = pos0;
    A.invT = 1.0 / (double)temperature;
    A.T = temperature;
    // the bf16-grid table of T: binades [2^(e-12), 2^(e+7)), e = floor(log2 T)
    int e2 = 0;
    frexp((double)temperature, &e2);
    const int blo = 127 + (e2 - 1) - 12;
    A.use_tab = dtype == SV_BF16 && blo >= 1 && blo + sv::kTabBinades <= 255;
    A.tab_lo = A.use_tab ? (uint32_t)blo << 7 : 0u;
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
