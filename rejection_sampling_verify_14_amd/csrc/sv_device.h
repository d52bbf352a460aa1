// sv_device.h -- device helpers of the gfx950 verify library: Philox4x32-10,
// 53-bit uniforms, logit decoding, wave64/block reductions, and the shared
// workspace records.  CDNA4 only (wave64, 256-thread blocks).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kBlock = 256;          // threads per block in every kernel
constexpr int kWaves = kBlock / 64;  // wave64
constexpr int kChunk = 4096;         // elements per sampling chunk (16 per thread)
constexpr int kPerThread = kChunk / kBlock;
constexpr int DT_F32 = 0;
constexpr int DT_BF16 = 1;

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of the 4x32
// S-box with multipliers 0xD2511F53 / 0xCD9E8D57; the key is bumped by the
// Weyl constants 0x9E3779B9 / 0xBB67AE85 before every round but the first.
// ---------------------------------------------------------------------------
struct Words4 {
    uint32_t w0, w1, w2, w3;
};

__device__ __forceinline__ Words4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                                uint32_t k1)
{
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint32_t a_lo = 0xD2511F53u * c0;
        const uint32_t a_hi = __umulhi(0xD2511F53u, c0);
        const uint32_t b_lo = 0xCD9E8D57u * c2;
        const uint32_t b_hi = __umulhi(0xCD9E8D57u, c2);
        const uint32_t n0 = b_hi ^ c1 ^ k0;
        const uint32_t n2 = a_hi ^ c3 ^ k1;
        c0 = n0;
        c1 = b_lo;
        c2 = n2;
        c3 = a_lo;
    }
    return {c0, c1, c2, c3};
}

// 53-bit uniform in [0, 1): (a >> 5) * 2^26 + (b >> 6), scaled by 2^-53; exact.
__device__ __forceinline__ double u53(uint32_t a, uint32_t b)
{
    return ((double)(a >> 5) * 67108864.0 + (double)(b >> 6)) * 0x1.0p-53;
}

// Block of the verify stream: key = seed, counter = (pos, seq, round lo,
// (round hi) << 4 | stream 0).
__device__ __forceinline__ Words4 verify_block(uint64_t seed, uint64_t round, uint32_t seq, uint32_t pos)
{
    return philox4x32_10(pos, seq, (uint32_t)round, (uint32_t)(round >> 32) << 4, (uint32_t)seed,
                         (uint32_t)(seed >> 32));
}

__device__ __forceinline__ double accept_uniform(uint64_t seed, uint64_t round, uint32_t seq, uint32_t pos)
{
    Words4 w = verify_block(seed, round, seq, pos);
    return u53(w.w0, w.w1);
}

__device__ __forceinline__ double sample_uniform(uint64_t seed, uint64_t round, uint32_t seq, uint32_t slot)
{
    Words4 w = verify_block(seed, round, seq, slot);
    return u53(w.w2, w.w3);
}

// ---------------------------------------------------------------------------
// Logits
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <int DT>
__device__ __forceinline__ float load_logit(const char* row, int64_t t)
{
    if constexpr (DT == DT_BF16) {
        const uint32_t h = ((const uint16_t*)row)[t];
        return __uint_as_float(h << 16);
    } else {
        return ((const float*)row)[t];
    }
}

template <int DT>
constexpr int elem_bytes()
{
    return DT == DT_BF16 ? 2 : 4;
}

// Decode one 16-byte vector into 8 (bf16) or 4 (f32) floats.
template <int DT>
__device__ __forceinline__ void decode16(const uint4 v, float* x)
{
    if constexpr (DT == DT_BF16) {
        x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x);
        x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
        x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z);
        x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
    } else {
        x[0] = __uint_as_float(v.x); x[1] = __uint_as_float(v.y);
        x[2] = __uint_as_float(v.z); x[3] = __uint_as_float(v.w);
    }
}

// ---------------------------------------------------------------------------
// Workspace records
// ---------------------------------------------------------------------------
// Statistics of one logit row: s = sum_t exp((z_t - m) / T) (accumulated in
// double) with m a reference logit no more than 64 binary orders of
// magnitude below the row maximum (the maximum itself unless the row is
// pathological).  lse = m / T + log(s).
struct __align__(16) RowStat {
    double s;
    float m;
    int pad;
};

// What the sampling kernels need to know about one sequence.
struct __align__(16) SeqState {
    int64_t q_off;    // element offset of the q row to sample from
    int64_t p_off;    // element offset of the p row (residual only)
    double sq;        // pass-1 sums of the q / p rows (residual only)
    double sp;
    double u;         // sampling uniform
    float mq;         // pass-1 references of the q / p rows (residual only)
    float mp;
    // q_t > p_t  <=>  zq_t - zp_t > theta, theta from the pass-1 statistics.
    // Tokens with zq - zp above thr_hi certainly have q > p, below thr_lo
    // certainly q < p; the band between is resolved exactly by the sampler.
    float thr_lo;
    float thr_hi;
    int k;            // accepted count (= slot of the sampled token)
    int status;       // 0 ok, 1 data error
    int mode;         // 0 residual, 1 bonus
    int pad[3];
};
static_assert(sizeof(SeqState) == 80, "SeqState layout");

// Per-chunk sums of the sampled row(s).  Residual: sa = sum a, sb = sum b
// (a = exp((zq - mq)/T), b = exp((zp - mp)/T)); pa, pb = the same over the
// tokens certainly in {q > p}; na, nb = over the near-threshold tokens, whose
// smallest and largest zq - zp are dmin, dmax.  Bonus: sa = chunk maximum of
// z, sb = sum exp((z - sa)/T), pa = 1 if the chunk holds NaN or +inf.
struct __align__(16) ChunkSums {
    double sa, sb, pa, pb, na, nb;
    float dmin, dmax;
    double pad;
};
static_assert(sizeof(ChunkSums) == 64, "ChunkSums layout");

constexpr int kMaxChunks = 1024;  // V <= kMaxChunks * kChunk

constexpr int kModeResidual = 0;
constexpr int kModeBonus = 1;

// ---------------------------------------------------------------------------
// Reductions (wave64 via shuffles, block via LDS)
// ---------------------------------------------------------------------------
__device__ __forceinline__ double wave_sum(double v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

// Sum over the block; the result is valid in every thread.  `red` holds
// kWaves doubles of LDS.
__device__ __forceinline__ double block_sum(double v, double* red)
{
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) t += red[w];
    return t;
}

__device__ __forceinline__ float block_max(float v, float* red)
{
    v = wave_max(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float t = red[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) t = fmaxf(t, red[w]);
    return t;
}

// Exclusive prefix sum over the block in thread order; returns the prefix of
// this thread and writes the block total.  `scan` holds kWaves doubles.
__device__ __forceinline__ double block_exclusive_scan(double v, double* scan, double* total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    double incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
    }
    double excl = __shfl_up(incl, 1, 64);
    if (lane == 0) excl = 0.0;
    __syncthreads();
    if (lane == 63) scan[wave] = incl;
    __syncthreads();
    double base = 0.0, all = 0.0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        if (w < wave) base += scan[w];
        all += scan[w];
    }
    *total = all;
    return base + excl;
}

}  // namespace sv
