// sv_device.h -- device helpers of the gfx950 verify library: Philox4x32-10,
// 53-bit uniforms, logit decoding, wave64/block reductions, and the shared
// workspace records.  CDNA4 only (wave64, 256-thread blocks).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sv_exp_table.h"

namespace sv {

constexpr int kBlock = 256;          // threads per block in every kernel

constexpr int kWaves = kBlock / 64;  // wave64
constexpr int kChunk = 2048;         // elements per sampling chunk (8 per thread)
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
// exp(x) in double by Tang's table-driven method (P.T.P. Tang, ACM TOMS
// 15(2), 1989), with a table of kExpTabN = 64 (or 32, SV_EXP_TAB) entries
// 2^(j/N): n = round(N x/ln2), r = x - n ln2/N, so |r| <= ln2/(2N) up to
// rounding, and exp(x) = 2^(n>>log2 N) 2^((n&(N-1))/N) exp(r).  The 2^(j/N)
// come from the block's LDS copy of the table (fill_exp_table).  exp(r) - 1
// is r g(r) with g from its Chebyshev interpolant of degree 2 on
// |r| <= ln2/128 (N = 64; below 1e-11 relative), or r times the Taylor
// polynomial of degree 3 of g (N = 32; truncation below 1.3e-12 relative).
//
// r is formed by one fma against ln2/N rounded to a double: the product is
// exact inside the fma, and the rounding of the constant shifts r by at most
// |n| * 1.2e-18 * 32/N, below 1e-14 relative for |x| <= 40 and below 8e-14
// over the whole clamped range.  n is the low word of N x/ln2 + 1.5 * 2^52.
// x is clamped below at -1000, where the final ldexp underflows to exactly
// 0, so a masked logit (-inf) contributes nothing; terms between exp(-745)
// and exp(-708) come out as denormals.  x must not exceed 700 (callers' x are
// relative to their row's reference, so at most 6T or so).  NaN is not
// propagated (callers screen it).  14 (N = 64) or 15 full-rate operations.
// ---------------------------------------------------------------------------
#ifndef SV_EXP_TAB
#define SV_EXP_TAB 64
#endif
constexpr int kExpTabN = SV_EXP_TAB;
static_assert(kExpTabN == 32 || kExpTabN == 64, "exp table of 32 or 64 entries");
typedef const double __attribute__((address_space(3)))* lds_dptr;  // LDS-typed: ds_read, 32-bit address

__device__ __forceinline__ double exp_rel(double x, lds_dptr tab)
{
    constexpr double kRound = 0x1.8p52;
    x = fmax(x, -1000.0);
    if constexpr (kExpTabN == 64) {
        const double kd = fma(x, k64ByLn2, kRound);
        const int n = (int)(uint32_t)__double_as_longlong(kd);
        const double r = fma(kd - kRound, -kLn2By64, x);
        double p = fma(r, kExpG2, kExpG1);
        p = fma(r, p, 1.0);
        p *= r;
        const double t = tab[n & 63];
        return ldexp(fma(t, p, t), n >> 6);
    } else {
        const double kd = fma(x, k32ByLn2, kRound);
        const int n = (int)(uint32_t)__double_as_longlong(kd);
        const double r = fma(kd - kRound, -kLn2By32, x);
        double p = fma(r, 1.0 / 24.0, 1.0 / 6.0);
        p = fma(r, p, 0.5);
        p = fma(r, p, 1.0);
        p *= r;
        const double t = tab[n & 31];
        return ldexp(fma(t, p, t), n >> 5);
    }
}

// The block's LDS copy of the 2^(j/N) table (its N doubles; publish it with
// a barrier before the first exp_rel).
__device__ __forceinline__ void fill_exp_table(double* tab)
{
    if (threadIdx.x < kExpTabN) tab[threadIdx.x] = kExpTabN == 64 ? kExp2Table64[threadIdx.x] : kExp2Table32[threadIdx.x & 31];
}

// ---------------------------------------------------------------------------
// exp(z/T) over the bf16 grid
// ---------------------------------------------------------------------------
// A bf16 logit has 8 significant bits, so the logits of a row take few
// distinct values.  A call with bf16 logits fills a table E of exp(z/T) in
// double (the math library's exp, one rounding of z/T before it) for every
// bf16 z whose magnitude lies in the kTabBinades binades [2^(e-12), 2^(e+7)),
// e = floor(log2 T): there |z|/T lies in (2^-13, 2^7).  Entry s (kTabKeys +
// 1) + t holds the value with magnitude bits (lo + t) and sign s, lo = (127 +
// e - 12) << 7; entries t = kTabKeys are zero.  exp((z - m)/T) is then
// E(z) * R with R = exp(-m/T), for rows whose reference has |m/T| <=
// kTabRefLimit (both factors and the product stay far inside the double
// range).  Logits outside the table (tiny or huge magnitudes, -inf, NaN) take
// exp_rel.  The table is split by sign, kTabKeys + 1 entries each (so the
// logits of one sign, the common case, spread over every LDS bank).
constexpr int kTabBinades = 19;
constexpr int kTabKeys = kTabBinades * 128;
constexpr int kTabHalf = kTabKeys + 1;
constexpr int kTabEntries = 2 * kTabHalf;
constexpr double kTabRefLimit = 512.0;

// Entry index of a bf16 logit (decoded to a float), or -1 outside the table.
__host__ __device__ __forceinline__ int tab_index(float z, uint32_t lo)
{
    const uint32_t key = __builtin_bit_cast(uint32_t, z) >> 16;
    const uint32_t t = (key & 0x7FFFu) - lo;
    return t < (uint32_t)kTabKeys ? (int)(t + (key >> 15) * (uint32_t)kTabHalf) : -1;
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef const char __attribute__((address_space(3)))* lds_cptr;

// LDS byte offsets (8 * entry index) of the two bf16 logits packed in w, low
// half first, both formed by 16-bit packed arithmetic; a magnitude outside
// the table maps to a zero entry.  `worst` keeps the largest unclamped index
// t per half: a value of kTabKeys or more marks an element outside the table.
static_assert(8 * kTabEntries < 65536, "byte offsets fit 16 bits");
__host__ __device__ __forceinline__ void tab_offsets(uint32_t w, u16x2 lo2, uint32_t& a0, uint32_t& a1,
                                                     u16x2& worst)
{
    const u16x2 t = __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu) - lo2;
    worst = __builtin_elementwise_max(worst, t);
    const u16x2 c = __builtin_elementwise_min(t, u16x2{(unsigned short)kTabKeys, (unsigned short)kTabKeys});
    const u16x2 c8 = c << (unsigned short)3;
    // the sign bit spread over its half (arithmetic shift), masked to the
    // second half's byte offset
    typedef short i16x2 __attribute__((ext_vector_type(2)));
    const i16x2 sgn = __builtin_bit_cast(i16x2, w) >> (short)15;
    // (a 32-bit add of the packed halves: each half's sum stays below 2^16,
    // so no carry crosses into the other)
    constexpr uint32_t kHalfOff = 8u * kTabHalf;
    const uint32_t a = (__builtin_bit_cast(uint32_t, sgn) & (kHalfOff | (kHalfOff << 16))) +
                       __builtin_bit_cast(uint32_t, c8);
    a0 = a & 0xFFFFu;
    a1 = a >> 16;
}

__device__ __forceinline__ double lds_f64(lds_cptr base, uint32_t byte_off)
{
    return *reinterpret_cast<lds_dptr>(base + byte_off);
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

// 16-byte streaming load of pass-1 rows, with the nontemporal hint by
// default (SV_STREAM_NT): pass 1 reads every row once, and the rows a
// sequence samples from (a few percent) are re-read from HBM either way.
// With the row kernel's loads kept in flight across batches the hint lifts
// its stream from ~6.0 to ~6.8 TB/s (B=256 N=7 V=128256 bf16 chains).
#ifndef SV_STREAM_NT
#define SV_STREAM_NT 1
#endif
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 stream_load16(const uint4* p)
{
#if SV_STREAM_NT
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
#else
    return *p;
#endif
}

// 16-byte streaming load through a buffer resource: `voff` per lane,
// `soff` uniform; an access past the resource's size reads zeros.
__device__ __forceinline__ uint4 stream_buf16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, SV_STREAM_NT ? 2 : 0);
    return make_uint4(v.x, v.y, v.z, v.w);
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

// Inverse of decode16 for values that are exactly representable (bf16 values
// decoded from bf16 storage, or -inf).
template <int DT>
__device__ __forceinline__ uint4 encode16(const float* x)
{
    if constexpr (DT == DT_BF16) {
        auto w = [&](int k) { return (__float_as_uint(x[2 * k]) >> 16) | (__float_as_uint(x[2 * k + 1]) & 0xFFFF0000u); };
        return make_uint4(w(0), w(1), w(2), w(3));
    } else {
        return make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3]));
    }
}

// ---------------------------------------------------------------------------
// Records passed between blocks of one launch
// ---------------------------------------------------------------------------
// A record is a whole number of 16-byte atoms whose last word is a tag:
// tag = epoch ^ hash(every other word), with epoch the low word of the
// call's number (a 64-bit count of the library's calls that starts at a
// value taken from the clock when the library is loaded).  Writers store
// the atoms with agent-coherent (sc1) 16-byte buffer stores; readers load
// all atoms with coherent loads and take the record once the tag matches
// what they loaded.  A record left by an earlier call fails the check (its
// tag carries another call's number), and so does a record read while its
// stores are still landing (the hash no longer matches the mixture), so no
// ordering between the stores is needed.  Coherent accesses
// go to the level shared by all XCDs: no cache-wide write-back or
// invalidation is involved.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCpolSc1 = 16;  // agent-coherent access: misses the CU cache, served by L2
constexpr int kCpolNT = 2;    // nontemporal: the line is not kept for reuse

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ void put_atom(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, kCpolSc1);
}

// Not volatile: a volatile access is widened to system scope, which sends it
// past L2; loops that poll a record re-read it after a compiler barrier
// instead (wait_record).
__device__ __forceinline__ u32x4 get_atom(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCpolSc1);
}

// Word hash of the record tags: per word an xor, an odd multiply and an
// xor-shift (each a bijection of h, and each with a scalar instruction, so a
// wave-uniform record is tagged by the scalar unit), then a final avalanche.
__device__ __forceinline__ uint32_t hash_step(uint32_t h, uint32_t w)
{
    h = (h ^ w) * 0x9e3779b1u;
    return h ^ (h >> 15);
}

__device__ __forceinline__ uint32_t hash_final(uint32_t h)
{
    h ^= h >> 15;
    h *= 0xc2b2ae3du;
    h ^= h >> 13;
    h *= 0x165667b1u;
    return h ^ (h >> 16);
}

template <int K>
__device__ __forceinline__ uint32_t record_tag(const u32x4* a, uint32_t epoch)
{
    uint32_t h = 0x6a09e667u;
#pragma unroll
    for (int i = 0; i < K; ++i) {
        h = hash_step(h, a[i].x);
        h = hash_step(h, a[i].y);
        h = hash_step(h, a[i].z);
        if (i + 1 < K) h = hash_step(h, a[i].w);
    }
    return epoch ^ hash_final(h);
}

template <int K>
__device__ __forceinline__ void put_record(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4* a, uint32_t epoch)
{
    a[K - 1].w = record_tag<K>(a, epoch);
#pragma unroll
    for (int i = 0; i < K; ++i) put_atom(r, off + 16u * i, a[i]);
}

template <int K>
__device__ __forceinline__ bool try_record(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4* a, uint32_t epoch)
{
#pragma unroll
    for (int i = 0; i < K; ++i) a[i] = get_atom(r, off + 16u * i);
    return a[K - 1].w == record_tag<K>(a, epoch);
}

__device__ __forceinline__ uint32_t lo32(double d) { return (uint32_t)__double_as_longlong(d); }
__device__ __forceinline__ uint32_t hi32(double d) { return (uint32_t)((uint64_t)__double_as_longlong(d) >> 32); }
__device__ __forceinline__ double d64(uint32_t lo, uint32_t hi)
{
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Plain coherent accesses (tree paths, outputs read back by later items).
template <typename T>
__device__ __forceinline__ void cput(T* p, T v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T>
__device__ __forceinline__ T cget(const T* p)
{
    return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// All of this thread's memory operations have completed.
__device__ __forceinline__ void ops_complete() { __builtin_amdgcn_s_waitcnt(0); }

// Statistics of one segment of one logit row: s = sum_t exp((z_t - m) / T)
// (accumulated in double) with m a reference logit at most one binary order
// of magnitude (in units of the scaled logits) below the segment maximum.
// One atom.
struct RowStat {
    double s;
    float m;
};

// What the sampling work of one sequence needs from its accept step.  Four
// atoms.
struct SeqState {
    double sq, sp;    // pass-1 sums of the q / p rows (residual only)
    double u;         // sampling uniform
    float mq, mp;     // pass-1 references of the q / p rows (residual only)
    // q_t > p_t  <=>  zq_t - zp_t > theta, theta from the pass-1 statistics.
    // Tokens with zq - zp above thr_hi certainly have q > p, below thr_lo
    // certainly q < p; the band between is resolved exactly by the sampler.
    float thr_lo, thr_hi;
    int k;            // accepted count (= slot of the sampled token)
    int node;         // row sampled from: chain position k, tree stop node
    int status;       // 0 ok, 1 data error
    int mode;         // 0 residual, 1 bonus
    int bonus_ref;    // bonus: mq is the pass-1 reference of the bonus row
    uint32_t tag;     // record tag (the state is stored as a four-atom record)
};
static_assert(sizeof(SeqState) == 64, "SeqState is four 16-byte atoms");

// Per-chunk sums of the sampled row(s).  Residual: sa = sum a, sb = sum b
// (a = exp((zq - mq)/T), b = exp((zp - mp)/T)); pa, pb = the same over the
// tokens certainly in {q > p}; na, nb = over the near-threshold tokens, whose
// smallest and largest zq - zp are dmin, dmax.  Bonus: sa = the reference the
// chunk is summed against (the chunk maximum of z, or the row's pass-1
// reference when known), sb = sum exp((z - sa)/T).  flags: bit 0 NaN/+inf in the chunk, bit 1
// the sequence state never arrived.  Four atoms.
struct ChunkSums {
    double sa, sb, pa, pb, na, nb;
    float dmin, dmax;
    uint32_t flags;
};

constexpr uint32_t kRowStatBytes = 16, kChunkSumsBytes = 64, kSeqStateBytes = 64;

__device__ __forceinline__ void pack(const RowStat& v, u32x4* a)
{
    a[0] = u32x4{lo32(v.s), hi32(v.s), __float_as_uint(v.m), 0u};
}
__device__ __forceinline__ RowStat unpack_rowstat(const u32x4* a)
{
    return RowStat{d64(a[0].x, a[0].y), __uint_as_float(a[0].z)};
}

__device__ __forceinline__ void pack(const SeqState& v, u32x4* a)
{
    a[0] = u32x4{lo32(v.sq), hi32(v.sq), lo32(v.sp), hi32(v.sp)};
    a[1] = u32x4{lo32(v.u), hi32(v.u), __float_as_uint(v.mq), __float_as_uint(v.mp)};
    a[2] = u32x4{__float_as_uint(v.thr_lo), __float_as_uint(v.thr_hi), (uint32_t)v.k, (uint32_t)v.node};
    a[3] = u32x4{(uint32_t)v.status, (uint32_t)v.mode, (uint32_t)v.bonus_ref, 0u};
}
__device__ __forceinline__ SeqState unpack_state(const u32x4* a)
{
    SeqState v;
    v.sq = d64(a[0].x, a[0].y);
    v.sp = d64(a[0].z, a[0].w);
    v.u = d64(a[1].x, a[1].y);
    v.mq = __uint_as_float(a[1].z);
    v.mp = __uint_as_float(a[1].w);
    v.thr_lo = __uint_as_float(a[2].x);
    v.thr_hi = __uint_as_float(a[2].y);
    v.k = (int)a[2].z;
    v.node = (int)a[2].w;
    v.status = (int)a[3].x;
    v.mode = (int)a[3].y;
    v.bonus_ref = (int)a[3].z;
    return v;
}

__device__ __forceinline__ void pack(const ChunkSums& v, u32x4* a)
{
    a[0] = u32x4{lo32(v.sa), hi32(v.sa), lo32(v.sb), hi32(v.sb)};
    a[1] = u32x4{lo32(v.pa), hi32(v.pa), lo32(v.pb), hi32(v.pb)};
    a[2] = u32x4{lo32(v.na), hi32(v.na), lo32(v.nb), hi32(v.nb)};
    a[3] = u32x4{__float_as_uint(v.dmin), __float_as_uint(v.dmax), v.flags, 0u};
}
__device__ __forceinline__ ChunkSums unpack_chunk(const u32x4* a)
{
    ChunkSums c;
    c.sa = d64(a[0].x, a[0].y);
    c.sb = d64(a[0].z, a[0].w);
    c.pa = d64(a[1].x, a[1].y);
    c.pb = d64(a[1].z, a[1].w);
    c.na = d64(a[2].x, a[2].y);
    c.nb = d64(a[2].z, a[2].w);
    c.dmin = __uint_as_float(a[3].x);
    c.dmax = __uint_as_float(a[3].y);
    c.flags = a[3].z;
    return c;
}

constexpr uint32_t kFlagBad = 1u;
constexpr int kModeResidual = 0;
constexpr int kModeBonus = 1;
constexpr int kMaxChunks = 1024;  // V <= kMaxChunks * kChunk

// ---------------------------------------------------------------------------
// Reductions (wave64 via shuffles, block via LDS)
// ---------------------------------------------------------------------------
__device__ __forceinline__ double wave_sum(double v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// A double that every lane holds the same value of, taken from lane `src`
// as a wave-uniform (scalar) value.
__device__ __forceinline__ double lane_value(double v, int src)
{
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)__double_as_longlong(v), src);
    const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(__double_as_longlong(v) >> 32), src);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Sums over the wave of four doubles at once, returned wave-uniform.  The
// first two exchanges halve the data each (lanes 32..63 keep the last two
// sums, then lanes 16..31 and 48..63 the odd ones), so 7 additions do the
// work of 24; the totals end in lanes 0, 16, 32 and 48.
__device__ __forceinline__ void wave_sum4(double a0, double a1, double a2, double a3, double* out)
{
    const int lane = threadIdx.x & 63;
    const bool h32 = (lane & 32) != 0, h16 = (lane & 16) != 0;
    double k0 = h32 ? a2 : a0, k1 = h32 ? a3 : a1;
    k0 += __shfl_xor(h32 ? a0 : a2, 32, 64);
    k1 += __shfl_xor(h32 ? a1 : a3, 32, 64);
    double k = h16 ? k1 : k0;
    k += __shfl_xor(h16 ? k0 : k1, 16, 64);
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) k += __shfl_xor(k, off, 64);
    out[0] = lane_value(k, 0);
    out[1] = lane_value(k, 16);
    out[2] = lane_value(k, 32);
    out[3] = lane_value(k, 48);
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

// Sum of K doubles over the block in one LDS round trip; results valid in
// every thread.  `red` holds kWaves * K doubles.
template <int K>
__device__ __forceinline__ void block_sum_n(double* v, double* red)
{
#pragma unroll
    for (int i = 0; i < K; ++i) v[i] = wave_sum(v[i]);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) {
#pragma unroll
        for (int i = 0; i < K; ++i) red[wave * K + i] = v[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < K; ++i) {
        double t = 0.0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) t += red[w * K + i];
        v[i] = t;
    }
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
// Exclusive prefix sum over the lanes of a wave (Hillis-Steele); *total gets
// the wave's sum in every lane.
__device__ __forceinline__ double wave_exclusive_scan(double v, double* total)
{
    const int lane = threadIdx.x & 63;
    double incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
    }
    *total = __shfl(incl, 63, 64);
    const double excl = __shfl_up(incl, 1, 64);
    return lane == 0 ? 0.0 : excl;
}

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
