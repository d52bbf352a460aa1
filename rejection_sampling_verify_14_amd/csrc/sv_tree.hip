// sv_tree.hip -- draft-tree kernels: the tree attention mask and position
// ids of a flattened draft tree ("投机解码与 EAGLE", section 3: each node
// attends to itself and its ancestors only), and the EAGLE-2 dynamic draft
// tree build (section 4, eagle_round steps 1-2: expand the frontier's top-k
// children by cumulative log-probability, keep the best budget nodes),
// as expand / select / finalize launches.  gfx950, wave64.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "specverify.h"
#include "sv_host.h"

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

// ---------------------------------------------------------------------------
// EAGLE-2 dynamic draft tree ("投机解码与 EAGLE", section 4, eagle_round step
// 2; section 5, the dynamic tree).  Candidates live in a caller-owned table
// of n_max entries per sequence: token, parent candidate id (-1 = the
// root), level, log-score (the sum of ln p along the path: the logarithm of
// the pages' product of probabilities).
// ---------------------------------------------------------------------------
constexpr int kTopkMax = 16;
constexpr int kTreeMaxCand = 2048;
constexpr int kExpandFewRows = 512;  // below this many rows an expand block has 16 waves
#ifndef SV_TREE_BATCH
#define SV_TREE_BATCH 2  // 16-byte loads per lane per batch (2: 80 VGPRs, 5 waves per SIMD)
#endif

// A 64-bit key ordering (logit desc, token asc): the logit's bits made
// order-preserving in the high word, the token inverted in the low word.
__device__ __forceinline__ uint64_t topk_key(float x, int t)
{
    const uint32_t u = __float_as_uint(x);
    const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)o << 32) | (uint32_t)~(uint32_t)t;
}

__device__ __forceinline__ float key_value(uint64_t k)
{
    const uint32_t o = (uint32_t)(k >> 32);
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

__device__ __forceinline__ int key_token(uint64_t k) { return (int)~(uint32_t)k; }

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const uint64_t o = __shfl_xor(v, off, 64);
        v = o > v ? o : v;
    }
    return v;
}

struct ExpandArgs {
    const char* rows;
    int64_t seq_stride, row_stride;  // elements
    const int32_t* frontier_ids;     // [B, F] or null (the root)
    const double* frontier_score;    // [B, F] or null (0)
    int F, V, topk, level, n_max, offset;
    float invT;
    double invTd, c;                  // 1/T, log2(e)/T
    int32_t *cand_token, *cand_parent, *cand_level;
    double* cand_score;
};

template <int DT>
__device__ __forceinline__ float logit_of(const char* row, int64_t t)
{
    if constexpr (DT == 1) return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(row)[t] << 16);
    else return reinterpret_cast<const float*>(row)[t];
}

// 16-byte load with the nontemporal hint: a draft row is read once.
__device__ __forceinline__ uint4 load_nt16(const uint4* p)
{
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Element i (0 .. 16/es - 1) of a 16-byte vector of logits.
template <int DT>
__device__ __forceinline__ float vec_elem(const uint4& w, int i)
{
    const uint32_t ws = i / (DT == 1 ? 2 : 1) == 0 ? w.x : i / (DT == 1 ? 2 : 1) == 1 ? w.y
                      : i / (DT == 1 ? 2 : 1) == 2 ? w.z : w.w;
    if constexpr (DT == 1) return __uint_as_float((i & 1) ? (ws & 0xFFFF0000u) : (ws << 16));
    else return __uint_as_float(ws);
}

__device__ __forceinline__ float wave_max_f(float v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

// The k-th largest (k <= 64, wave-uniform) of the 64 lanes' values, in
// every lane: a bitonic sort across the wave into descending lane order.
__device__ __forceinline__ float wave_kth_largest(float v, int lane, int k)
{
#pragma unroll
    for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            const float o = __shfl_xor(v, j, 64);
            const bool desc = (lane & k) == 0, lower = (lane & j) == 0;
            v = (lower == desc) ? fmaxf(v, o) : fminf(v, o);
        }
    }
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), k - 1));
}

// One wave's running state over its share of a row.  A term is
// 2^(fma(x, cf, -p)) with p = RN(ref * cf): 2^((x - ref) cf) times 2^e,
// e = ref * cf - p (exact in fp32), a factor common to every term that the
// sum sheds when ref moves and at the end.
struct ExpandWave {
    float ref = -INFINITY;  // wave-uniform reference: the wave's maximum when last moved
    float lim = -INFINITY;  // ref moves once a logit passes lim (= ref + 2 / cf)
    float p = 0.0f, e = 0.0f;
    double s = 0.0;         // this lane's exp terms against ref, times 2^e
    uint64_t bad = 0;       // wave-uniform: lanes whose sum met NaN or +inf
    uint64_t L = 0;         // lane j < K: the wave's j-th best key (0 = none yet)
    uint64_t tau = 0;       // wave-uniform: the wave's K-th best key
    float tauv = -INFINITY; // its value
    float theta = -INFINITY;  // wave-uniform: a value at or below the K-th best seen
    int K;                  // the list's length: the k of the top-k
};

// Insert every key k of the wave above tau into the sorted list, one lane
// at a time (a wave-uniform loop): each insert shifts the list by one lane
// from the new key's place down.
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}

// Lane j of each 16-lane row receives lane j - 1's value (DPP row_shr:1);
// lane 0 of a row receives ~0, above every key.
__device__ __forceinline__ uint64_t row_shift_up_u64(uint64_t v)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)(uint32_t)v, 0x111, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)(uint32_t)(v >> 32), 0x111, 0xF, 0xF, false);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ void insert_keys(ExpandWave& st, uint64_t k)
{
    uint64_t cm = __ballot(k > st.tau);
    while (cm) {
        const int l = __ffsll((unsigned long long)cm) - 1;
        const uint64_t kn = readlane_u64(k, l);  // wave-uniform, not yet held, above tau
        // the list lives in lanes 0..15 (the other lanes hold junk)
        const uint64_t prev = row_shift_up_u64(st.L);
        st.L = st.L > kn ? st.L : (prev > kn ? kn : prev);
        st.tau = readlane_u64(st.L, st.K - 1);
        st.tauv = st.tau == 0 ? -INFINITY : key_value(st.tau);
        cm = __ballot(k > st.tau) & (~0ull << l << 1);
    }
}

// Raise the wave's reference to wm (> ref): rescale the sum to the new
// reference and offset.
__device__ __forceinline__ void raise_ref(ExpandWave& st, float wm, float cf)
{
    const float p = wm * cf;
    const float e = __builtin_fmaf(wm, cf, -p);
    st.s = (st.ref == -INFINITY) ? st.s * 0.0  // 0, or NaN kept
                                 : st.s * exp2(((double)st.ref - (double)wm) * (double)cf + (double)(e - st.e));
    st.ref = wm;
    st.lim = wm + 2.0f / cf;
    st.p = p;
    st.e = e;
}

// A batch of U 16-byte vectors per lane (vector u of this lane starts at
// token t0[u]; real[u] false: padding that adds nothing and offers no key).
template <int DT, int U, int NW>
__device__ __forceinline__ void expand_batch(ExpandWave& st, const uint4 (&w)[U], const int (&t0)[U],
                                             const bool (&real)[U], float cf, int lane, float* s_thr, int wave)
{
    constexpr int EPV = DT == 1 ? 8 : 4;
    float vm[U];
    float lm = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        vm[u] = -INFINITY;
#pragma unroll
        for (int i = 0; i < EPV; ++i) {
            vm[u] = fmaxf(vm[u], vec_elem<DT>(w[u], i));
        }
        vm[u] = real[u] ? vm[u] : -INFINITY;
        lm = fmaxf(lm, vm[u]);
    }
    // ref lags the maximum by less than 2 in the exponent (terms below 4,
    // so the fma's rounding stays near that of a term at 1)
    if (__ballot(lm > st.lim)) raise_ref(st, wave_max_f(lm), cf);
    // NaN and +inf show as a NaN sum: a NaN term, or inf - inf.  While
    // ref is -inf (p = 0) every term is 0 or NaN.
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float g = 0.0f;
#pragma unroll
        for (int i = 0; i < EPV; ++i) g += __builtin_amdgcn_exp2f(__builtin_fmaf(vec_elem<DT>(w[u], i), cf, -st.p));
        st.s += real[u] ? (double)g : 0.0;
    }
    // At the start (no K keys held, no bound yet), K lanes' batch maxima
    // bound the K-th best from below: K distinct keys reach that bound, so a
    // value under it can never be among the K best.  (A wave whose keys the
    // shared threshold keeps out may never hold K keys; it seeds once.)
    if (st.tau == 0 && st.theta == -INFINITY) st.theta = wave_kth_largest(lm, lane, st.K);
    float thr = fmaxf(st.tauv, st.theta);
#pragma unroll
    for (int q = 0; q < NW; ++q) thr = fmaxf(thr, __hip_atomic_load(s_thr + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
    if (!__ballot(lm >= thr)) return;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (!__ballot(vm[u] >= thr)) continue;
#pragma unroll
        for (int i = 0; i < EPV; ++i) {
            // thr only rises while keys go in, so the test against its
            // value at the batch's start passes every key that may insert
            const float x = vec_elem<DT>(w[u], i);
            if (__ballot(real[u] && x >= thr)) insert_keys(st, (real[u] && x >= thr) ? topk_key(x, t0[u] + i) : 0);
        }
    }
    // publish this wave's threshold (other waves read it without a barrier:
    // any value it has held is a valid bound)
    if (lane == 0) __hip_atomic_store(s_thr + wave, fmaxf(st.tauv, st.theta), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Block (b, f) of NW waves: one pass over frontier row f of sequence b: its
// log-sum-exp and its top-k tokens by (logit desc, token asc); then k
// candidates at offset + f*k of the table.  A row holding NaN or +inf, or
// only -inf, gives NaN scores (the finalize step fails the sequence).
//
// Every decision that could diverge inside a wave is taken wave-uniformly:
// - log-sum-exp: the terms of a 16-byte vector are fp32 exp2 against a
//   reference that is the wave's running maximum (it moves, with an fp64
//   rescale of the double sums, only when a batch raises it), each vector's
//   sum added in double;
// - top-k: the wave holds one sorted list of its K = k best keys spread
//   over lanes 0..K-1, and its K-th key tau is a wave-uniform threshold.  A
//   vector whose largest value is below tau's is skipped; otherwise each key
//   above tau is inserted, one lane at a time, by a parallel shift.  A key at
//   or below tau is never among the K best of what the wave has seen (K
//   distinct keys exceed it), so nothing is lost.  Before K keys are held
//   the threshold is the K-th largest lane maximum of the batch, so the
//   first batch inserts a few dozen keys, not every one it holds.  (Lanes
//   K..15 keep keys shifted out of the list: real logits of the row, so the
//   block's merge may count them.)  After each batch a wave publishes its
//   threshold in LDS, and every wave filters by the largest published one:
//   a logit below another wave's threshold has K distinct keys of that
//   wave above it, so it is not among the block's K best either.
// NW = 16 serves levels with few rows (the root), NW = 4 the wide ones.
template <int DT, int NW>
__global__ __launch_bounds__(NW * 64, NW == 4 ? 4 : 1) void k_tree_expand(ExpandArgs A)
{
    constexpr int NT = NW * 64;
    const int b = (int)blockIdx.x / A.F, f = (int)blockIdx.x - b * A.F;
    constexpr int EB = DT == 1 ? 2 : 4;
    constexpr int EPV = 16 / EB;
    constexpr int U = SV_TREE_BATCH;  // 16-byte loads per lane in flight
    const char* row = A.rows + ((int64_t)b * A.seq_stride + (int64_t)f * A.row_stride) * EB;
    const float cf = (float)A.c;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    ExpandWave st;
    st.K = A.topk;
    __shared__ float s_thr[NW];  // each wave's published filter threshold
    if (threadIdx.x < NW) s_thr[threadIdx.x] = -INFINITY;
    __syncthreads();
    const bool vec = ((((uintptr_t)row) & 15u) == 0);
    const int nvec = vec ? A.V / EPV : 0;
    // whole batches of U vectors per lane, then one vector per lane, then
    // single logits (each lane's tokens increase along the row)
    const int nb = nvec / (U * NT);
    const int nfull = nb * (U * NT);
    // two register sets: batch i + 1 is in flight while batch i is taken
    // (a set is never copied, which would wait for its loads); a load past
    // the last batch reads the last batch again and is not taken
    const uint4* rv = reinterpret_cast<const uint4*>(row) + threadIdx.x;
    bool real[U];
    int ta[U], tb[U];
    uint4 wa[U], wb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) real[u] = true;
    auto load = [&](uint4 (&w)[U], int (&t)[U], int bi) {
        const int v0 = min(bi, nb - 1) * (U * NT);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            w[u] = load_nt16(rv + v0 + u * NT);
            t[u] = (v0 + u * NT + (int)threadIdx.x) * EPV;
        }
    };
    if (nb > 0) load(wa, ta, 0);
    for (int bi = 0; bi < nb; bi += 2) {
        load(wb, tb, bi + 1);
        expand_batch<DT, U, NW>(st, wa, ta, real, cf, lane, s_thr, wave);
        if (bi + 1 >= nb) break;
        load(wa, ta, bi + 2);
        expand_batch<DT, U, NW>(st, wb, tb, real, cf, lane, s_thr, wave);
    }
    for (int v0 = nfull; v0 < nvec; v0 += NT) {
        const int v = v0 + (int)threadIdx.x;
        constexpr uint32_t kNegInf = DT == 1 ? 0xFF80FF80u : 0xFF800000u;  // -inf logits
        uint4 w[1] = {make_uint4(kNegInf, kNegInf, kNegInf, kNegInf)};
        if (v < nvec) w[0] = reinterpret_cast<const uint4*>(row)[v];
        const int t0[1] = {v * EPV};
        const bool real[1] = {v < nvec};
        expand_batch<DT, 1, NW>(st, w, t0, real, cf, lane, s_thr, wave);
    }
    for (int t0 = nvec * EPV; t0 < A.V; t0 += NT) {
        // one logit per lane (unaligned rows, or the tail past the vectors);
        // lanes past V hold -inf, add nothing and offer no key
        const int t = t0 + (int)threadIdx.x;
        const float x0 = t < A.V ? logit_of<DT>(row, t) : -INFINITY;
        const float wm = wave_max_f(x0);
        if (wm > st.ref) raise_ref(st, wm, cf);
        st.s += (double)__builtin_amdgcn_exp2f(__builtin_fmaf(x0, cf, -st.p));  // 0 past V
        insert_keys(st, t < A.V ? topk_key(x0, t) : 0);
    }
    // the wave's sum against ref (every lane shares ref, p and e)
    st.bad |= __ballot(st.s != st.s);
    double s = st.ref == -INFINITY ? 0.0 : st.s * exp2(-(double)st.e);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    __shared__ uint64_t s_keys[NW * kTopkMax];
    __shared__ float s_m[NW];
    __shared__ double s_s[NW];
    if (lane < kTopkMax) s_keys[wave * kTopkMax + lane] = st.L;
    if (lane == 0) {
        s_m[wave] = st.ref;
        s_s[wave] = s;
    }
    const int bad = __syncthreads_or(st.bad != 0);
    // the row's log-sum-exp and the block's top-k by rank among the waves' lists
    if (threadIdx.x >= NW * kTopkMax) return;
    double S = 0.0;
    float M = -INFINITY;
    for (int q = 0; q < NW; ++q) M = fmaxf(M, s_m[q]);
    for (int q = 0; q < NW; ++q)
        if (s_m[q] != -INFINITY) S += s_m[q] == M ? s_s[q] : s_s[q] * exp2(((double)s_m[q] - (double)M) * (double)cf);
    const uint64_t mine = s_keys[threadIdx.x];
    int rank = 0;
#pragma unroll 8
    for (int j = 0; j < NW * kTopkMax; ++j) rank += s_keys[j] > mine;
    if (rank < A.topk) {
        const double lse = (double)M * A.invTd + log(S);
        const bool fail = bad || M == -INFINITY || mine == 0;
        const int64_t at = (int64_t)b * A.n_max + A.offset + (int64_t)f * A.topk + rank;
        const double fs = A.frontier_score ? A.frontier_score[(int64_t)b * A.F + f] : 0.0;
        A.cand_token[at] = fail ? -1 : key_token(mine);
        A.cand_parent[at] = A.frontier_ids ? A.frontier_ids[(int64_t)b * A.F + f] : -1;
        A.cand_level[at] = A.level;
        A.cand_score[at] = fail ? NAN : fs + ((double)key_value(mine) * A.invTd - lse);
    }
}

// NaN-safe order of (score desc, id asc): NaN ranks as -inf.
__device__ __forceinline__ double order_score(double v) { return v != v ? -INFINITY : v; }

// Block b: the k best of candidates [offset, offset + count) of sequence b by
// (score desc, id asc), in that order: their ids and scores.
__global__ __launch_bounds__(256) void k_tree_select(const double* __restrict__ cand_score, int n_max, int offset,
                                                     int count, int k, int32_t* __restrict__ out_ids,
                                                     double* __restrict__ out_score)
{
    __shared__ double s_sc[kTreeMaxCand];
    const int b = blockIdx.x;
    const double* sc = cand_score + (int64_t)b * n_max + offset;
    for (int i = threadIdx.x; i < count; i += 256) s_sc[i] = order_score(sc[i]);
    __syncthreads();
    for (int i = threadIdx.x; i < count; i += 256) {
        const double v = s_sc[i];
        int rank = 0;
#pragma unroll 8
        for (int j = 0; j < count; ++j) {  // branch-free: bitwise, not short-circuit
            const double sj = s_sc[j];
            rank += (int)(sj > v) | ((int)(sj == v) & (int)(j < i));
        }
        if (rank < k) {
            out_ids[(int64_t)b * k + rank] = offset + i;
            out_score[(int64_t)b * k + rank] = sc[i];
        }
    }
}

// An order-preserving 64-bit image of a double (NaN excluded): larger
// values give larger keys, -0 and +0 the same key.
__device__ __forceinline__ uint64_t double_key(double v)
{
    const uint64_t u = (uint64_t)__double_as_longlong(v + 0.0);  // -0 + 0 = +0
    return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

constexpr int kFinalizeBlock = 1024;

// Bitonic sort of P (a power of two, <= the block) pairs held one per thread
// (thread e holds element e; threads >= P hold padding that is never read)
// into the order `first` (a precedes b).  Strides below 64 exchange inside
// the wave by shuffles; wider ones go through LDS (s_k, s_i), with a barrier
// on each side.  Every thread of the block calls it.
template <typename First>
__device__ __forceinline__ void block_bitonic(uint64_t& key, int& id, int P, uint64_t* s_k, int* s_i, First first)
{
    const int e = threadIdx.x;
    for (int k = 2; k <= P; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            uint64_t ko;
            int io;
            if (j >= 64) {
                if (e < P) {
                    s_k[e] = key;
                    s_i[e] = id;
                }
                __syncthreads();
                if (e < P) {
                    ko = s_k[e ^ j];
                    io = s_i[e ^ j];
                }
                __syncthreads();
            } else {
                ko = ((uint64_t)(uint32_t)__shfl_xor((int)(key >> 32), j, 64) << 32) |
                     (uint32_t)__shfl_xor((int)(uint32_t)key, j, 64);
                io = __shfl_xor(id, j, 64);
            }
            if (e < P) {
                const bool lower = (e & j) == 0;
                const uint64_t ki = lower ? key : ko, kl = lower ? ko : key;
                const int ii = lower ? id : io, il = lower ? io : id;
                if (first(kl, il, ki, ii) == ((e & k) == 0)) {
                    key = ko;
                    id = io;
                }
            }
        }
    }
}

// Block b: the kept set of sequence b -- the `budget` best candidates by
// (score desc, id asc) -- numbered 1..budget by (level asc, score desc, id
// asc), and the flattened tree: parents (node 0: -1), tokens (0), depth (0),
// log-scores (0).  A NaN score, or a kept candidate whose parent is not kept
// (never for tables the expand step wrote), fails the sequence: -1 in every
// slot.
//
// Two bitonic sorts in LDS, one compare-exchange per thread and stage: the
// n candidates (padded to a power of two) by (score desc, id asc), whose
// first `budget` are the kept set; then the kept ranks by (level asc, rank
// asc), whose order is the node numbering.
__global__ __launch_bounds__(kFinalizeBlock) void k_tree_finalize(
    const int32_t* __restrict__ cand_token, const int32_t* __restrict__ cand_parent,
    const int32_t* __restrict__ cand_level, const double* __restrict__ cand_score, int n_max, int n, int budget,
    int32_t* __restrict__ out_parents, int32_t* __restrict__ out_tokens, int32_t* __restrict__ out_depth,
    double* __restrict__ out_score)
{
    __shared__ uint64_t s_key[kTreeMaxCand];
    __shared__ int s_id[kTreeMaxCand];
    __shared__ int s_node[kTreeMaxCand];  // candidate id -> node number (0: not kept)
    const int b = blockIdx.x, tid = threadIdx.x;
    const int64_t base = (int64_t)b * n_max;
    const int nn = budget + 1;
    int P = 1;
    while (P < n) P <<= 1;
    int bad = 0;
    for (int i = tid; i < P; i += kFinalizeBlock) {
        uint64_t key = 0;  // padding: below every score's key (-inf's is 0x000F...)
        if (i < n) {
            const double v = cand_score[base + i];
            bad |= v != v;
            key = double_key(order_score(v));
            s_node[i] = 0;
        }
        s_key[i] = key;
        s_id[i] = i;  // padding ids follow every real one
    }
    bad = __syncthreads_or(bad);
    // sort 1: descending by (key, -id)
    auto by_score = [](uint64_t ka, int ia, uint64_t kb, int ib) { return (ka > kb) | ((ka == kb) & (ia < ib)); };
    if (P <= kFinalizeBlock) {
        uint64_t key = tid < P ? s_key[tid] : 0;
        int id = tid < P ? s_id[tid] : 0;
        __syncthreads();
        block_bitonic(key, id, P, s_key, s_id, by_score);
        if (tid < P) {
            s_key[tid] = key;
            s_id[tid] = id;
        }
        __syncthreads();
    } else {
        for (int k = 2; k <= P; k <<= 1) {
            for (int j = k >> 1; j > 0; j >>= 1) {
                for (int t = tid; t < (P >> 1); t += kFinalizeBlock) {
                    const int i = ((t & ~(j - 1)) << 1) | (t & (j - 1)), l = i + j;
                    const uint64_t ki = s_key[i], kl = s_key[l];
                    const int ii = s_id[i], il = s_id[l];
                    if (by_score(kl, il, ki, ii) == ((i & k) == 0)) {
                        s_key[i] = kl;
                        s_key[l] = ki;
                        s_id[i] = il;
                        s_id[l] = ii;
                    }
                }
                __syncthreads();
            }
        }
    }
    // sort 2: the kept ranks r < budget, ascending by (level, r)
    int P2 = 1;
    while (P2 < budget) P2 <<= 1;
    auto by_level = [](uint64_t ka, int, uint64_t kb, int) { return ka < kb; };
    if (P2 <= kFinalizeBlock) {
        uint64_t key = tid < budget ? ((uint64_t)((uint32_t)cand_level[base + s_id[tid]] ^ 0x80000000u) << 32) |
                                          (uint32_t)tid
                                    : ~0ull;
        int id = 0;
        block_bitonic(key, id, P2, s_key, s_node, by_level);  // s_node as scratch for the ids
        __syncthreads();
        if (tid < P2) s_key[tid] = key;
        for (int i = tid; i < n; i += kFinalizeBlock) s_node[i] = 0;
        __syncthreads();
    } else {
        for (int r = tid; r < P2; r += kFinalizeBlock)
            s_key[r] = r < budget ? ((uint64_t)((uint32_t)cand_level[base + s_id[r]] ^ 0x80000000u) << 32) | (uint32_t)r
                                  : ~0ull;
        __syncthreads();
        for (int k = 2; k <= P2; k <<= 1) {
            for (int j = k >> 1; j > 0; j >>= 1) {
                for (int t = tid; t < (P2 >> 1); t += kFinalizeBlock) {
                    const int i = ((t & ~(j - 1)) << 1) | (t & (j - 1)), l = i + j;
                    const uint64_t ki = s_key[i], kl = s_key[l];
                    if (by_level(kl, 0, ki, 0) == ((i & k) == 0)) {
                        s_key[i] = kl;
                        s_key[l] = ki;
                    }
                }
                __syncthreads();
            }
        }
    }
    for (int q = tid; q < budget; q += kFinalizeBlock) s_node[s_id[(uint32_t)s_key[q]]] = q + 1;
    __syncthreads();
    int32_t* Po = out_parents + (int64_t)b * nn;
    int32_t* K = out_tokens + (int64_t)b * nn;
    int32_t* D = out_depth + (int64_t)b * nn;
    double* S = out_score + (int64_t)b * nn;
    for (int q = tid; q < budget && !bad; q += kFinalizeBlock) {
        const int i = s_id[(uint32_t)s_key[q]];
        const int node = q + 1;
        const int par = cand_parent[base + i];
        int pnode = 0;
        if (par >= 0) pnode = (par < i && s_node[par] > 0) ? s_node[par] : -1;
        Po[node] = pnode;
        K[node] = cand_token[base + i];
        D[node] = cand_level[base + i];
        S[node] = cand_score[base + i];
        if (pnode < 0) bad = 1;
    }
    bad = __syncthreads_or(bad);
    if (tid == 0 && !bad) {
        Po[0] = -1;
        K[0] = 0;
        D[0] = 0;
        S[0] = 0.0;
    }
    if (bad)
        for (int i = tid; i < nn; i += kFinalizeBlock) {
            Po[i] = K[i] = D[i] = -1;
            S[i] = 0.0;
        }
}

}  // namespace sv

extern "C" int tree_attention_mask(const int32_t* parents, int parents_shared, const int32_t* kv_len_in, int B,
                                   int T, uint64_t* out_mask, int32_t* out_positions, hipStream_t stream)
{
    if (B < 0 || T < 0) return SV_EINVAL;
    if (T >= sv::kTreeMaxNodes) return SV_ESHAPE;
    if (B == 0) return SV_OK;
    if (!parents || !out_mask || !out_positions) return SV_EINVAL;
    hipLaunchKernelGGL(sv::k_tree_mask, dim3((unsigned)B), dim3(sv::kTreeBlock), 0, stream, parents, parents_shared,
                       kv_len_in, T, out_mask, out_positions);
    return hipGetLastError() == hipSuccess ? SV_OK : SV_EHIP;
}

extern "C" int tree_expand(const void* frontier_logits, int64_t seq_stride, int64_t row_stride, int dtype, int B,
                           int F, int V, int topk, float temperature, const int32_t* frontier_ids,
                           const double* frontier_score, int level, int n_max, int offset, int32_t* cand_token,
                           int32_t* cand_parent, int32_t* cand_level, double* cand_score, hipStream_t stream)
{
    if (dtype != SV_F32 && dtype != SV_BF16) return SV_EDTYPE;
    if (B < 0 || F < 1 || V < 1 || level < 1 || offset < 0 || seq_stride < 0 || row_stride < 0) return SV_EINVAL;
    if (!(temperature > 0.0f) || !(temperature < INFINITY)) return SV_EINVAL;
    if (topk < 1 || topk > sv::kTopkMax || topk > V) return SV_ESHAPE;
    if (n_max > sv::kTreeMaxCand || (int64_t)offset + (int64_t)F * topk > n_max) return SV_ESHAPE;
    if (B == 0) return SV_OK;
    if (!frontier_logits || !cand_token || !cand_parent || !cand_level || !cand_score) return SV_EINVAL;
    const int es = dtype == SV_BF16 ? 2 : 4;
    if (((uintptr_t)frontier_logits) % es) return SV_EALIGN;
    if ((int64_t)B * F > 0x7FFFFFFF) return SV_ESHAPE;
    if (seq_stride > INT64_MAX / es || row_stride > INT64_MAX / es ||
        !sv::span_fits(B, seq_stride * es, F, row_stride * es, 1, 0, (int64_t)V * es))
        return SV_EINVAL;
    sv::ExpandArgs A;
    A.rows = static_cast<const char*>(frontier_logits);
    A.seq_stride = seq_stride;
    A.row_stride = row_stride;
    A.frontier_ids = frontier_ids;
    A.frontier_score = frontier_score;
    A.F = F;
    A.V = V;
    A.topk = topk;
    A.level = level;
    A.n_max = n_max;
    A.offset = offset;
    A.invT = 1.0f / temperature;
    A.invTd = 1.0 / (double)temperature;
    A.c = 1.4426950408889634074 / (double)temperature;
    A.cand_token = cand_token;
    A.cand_parent = cand_parent;
    A.cand_level = cand_level;
    A.cand_score = cand_score;
    // few rows (the root level): 16 waves per row, else 4
    const bool wide = (int64_t)B * F < sv::kExpandFewRows;
    const dim3 grid((unsigned)(B * F));
    if (dtype == SV_BF16) {
        if (wide) hipLaunchKernelGGL((sv::k_tree_expand<1, 16>), grid, dim3(1024), 0, stream, A);
        else hipLaunchKernelGGL((sv::k_tree_expand<1, 4>), grid, dim3(256), 0, stream, A);
    } else {
        if (wide) hipLaunchKernelGGL((sv::k_tree_expand<0, 16>), grid, dim3(1024), 0, stream, A);
        else hipLaunchKernelGGL((sv::k_tree_expand<0, 4>), grid, dim3(256), 0, stream, A);
    }
    return hipGetLastError() == hipSuccess ? SV_OK : SV_EHIP;
}

extern "C" int tree_select(const double* cand_score, int B, int n_max, int offset, int count, int k,
                           int32_t* out_ids, double* out_score, hipStream_t stream)
{
    if (B < 0 || offset < 0 || count < 1 || k < 1 || k > count) return SV_EINVAL;
    if (n_max > sv::kTreeMaxCand || (int64_t)offset + count > n_max) return SV_ESHAPE;
    if (B == 0) return SV_OK;
    if (!cand_score || !out_ids || !out_score) return SV_EINVAL;
    hipLaunchKernelGGL(sv::k_tree_select, dim3((unsigned)B), dim3(256), 0, stream, cand_score, n_max, offset, count, k,
                       out_ids, out_score);
    return hipGetLastError() == hipSuccess ? SV_OK : SV_EHIP;
}

extern "C" int tree_finalize(const int32_t* cand_token, const int32_t* cand_parent, const int32_t* cand_level,
                             const double* cand_score, int B, int n_max, int n, int budget, int32_t* out_parents,
                             int32_t* out_tokens, int32_t* out_depth, double* out_score, hipStream_t stream)
{
    if (B < 0 || n < 1 || budget < 1 || budget > n || n > n_max) return SV_EINVAL;
    if (n_max > sv::kTreeMaxCand) return SV_ESHAPE;
    if (B == 0) return SV_OK;
    if (!cand_token || !cand_parent || !cand_level || !cand_score || !out_parents || !out_tokens || !out_depth ||
        !out_score)
        return SV_EINVAL;
    hipLaunchKernelGGL(sv::k_tree_finalize, dim3((unsigned)B), dim3(sv::kFinalizeBlock), 0, stream, cand_token, cand_parent,
                       cand_level, cand_score, n_max, n, budget, out_parents, out_tokens, out_depth, out_score);
    return hipGetLastError() == hipSuccess ? SV_OK : SV_EHIP;
}
